// Backward of the masked attention for float32 ("Why attention must compute
// the max first", section 3.3: dS = P (dP - rowsum(P dP)); the row maximum
// carries no gradient). Same parameters, mask rules, workspace and flags as
// the 16-bit kernels in mha_bwd.hpp.
//
// These run for D = 128, where the MFMA kernels' float32 tiles and fragments
// do not fit a CU's LDS and a lane's registers (smaller D use the MFMA
// kernels of mha_bwd.hpp). They use the vector ALUs: one wave per
// query row (dQ, the row's log-sum-exp and Delta) or per key row (dK, dV),
// four rows per workgroup. For the scores, lane l takes the keys (queries)
// l, l + 64, ... and forms its dot products against the wave's own row, staged
// once in LDS and read by every lane at the same address. For the products,
// lane l takes features l and l + 64, and each chunk's 64 weights are
// broadcast from their lanes one at a time (v_readlane). Rows of a workgroup
// have different causal ranges, so no workgroup barrier is used: every wave
// syncs only with itself.
#pragma once

#include "mha_bwd.hpp"

namespace mha {

// LDS written by some lanes of a wave and then read by others of the same wave.
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline float wave_max_f32(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ inline float wave_sum_f32(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ inline float lane_value(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Entry (row, key) of the head's float32 mask slab (both in range).
__device__ inline float mask_at_f32(const BwdParams& p, int bh, int row, int key) {
  const int64_t slab = p.mask_heads == 1 ? bh / p.H : bh;
  return static_cast<const float*>(p.mask)[(slab * p.Lq + row) * (int64_t)p.Lk + key];
}

// a . b over D features: a from LDS (the same address in every lane), b a row
// of this lane's own.
template <int D>
__device__ inline float dot_row(const float* a, const float* b) {
  float s = 0.f;
#pragma unroll
  for (int f = 0; f < D; f += 4) {
    const float4 x = *reinterpret_cast<const float4*>(a + f);
    const float4 y = *reinterpret_cast<const float4*>(b + f);
    s = __builtin_fmaf(x.x, y.x, s);
    s = __builtin_fmaf(x.y, y.y, s);
    s = __builtin_fmaf(x.z, y.z, s);
    s = __builtin_fmaf(x.w, y.w, s);
  }
  return s;
}

// ---- dQ and the row statistics: one wave per query row ----------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_f32_dq_kernel(const BwdParams p) {
  constexpr int FPL = (D + 63) / 64;  // features per lane in the dQ product
  __shared__ __attribute__((aligned(16))) float rows[4][2][D];  // [wave][q, dO]
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nrg = (p.Lq + 3) / 4;
  const int bh = blockIdx.x / nrg;
  const int qi = (blockIdx.x % nrg) * 4 + wv;
  if (qi >= p.Lq) return;
  bool bad = false;
  const int kend = bwd_len(p, bh / p.H, &bad);
  const int kmax = p.causal ? min(kend, qi + 1) : kend;  // keys of this row: [0, kmax)
  const float* q = static_cast<const float*>(p.q) + ((int64_t)bh * p.Lq + qi) * D;
  const float* go = static_cast<const float*>(p.dout) + ((int64_t)bh * p.Lq + qi) * D;
  const float* K = static_cast<const float*>(p.k) + (int64_t)bh * p.Lk * D;
  const float* V = static_cast<const float*>(p.v) + (int64_t)bh * p.Lk * D;
  for (int f = lane; f < D; f += 64) {
    rows[wv][0][f] = q[f];
    rows[wv][1][f] = go[f];
  }
  wave_lds_sync();
  // logit of key j in log2 units, or -inf (j < kmax)
  auto logit = [&](int j, float s) {
    float x = s * p.c;
    if (p.mask) x = masked_logit(p, x, mask_at_f32(p, bh, qi, j));
    return x;
  };

  // pass 1: per lane running maximum m, sum l of 2^(x - m), sum a of 2^(x - m) dP
  float m = -INFINITY, l = 0.f, a = 0.f;
  for (int j = lane; j < kmax; j += 64) {
    const float x = logit(j, dot_row<D>(rows[wv][0], K + (int64_t)j * D));
    if (x == -INFINITY) continue;
    const float dp = dot_row<D>(rows[wv][1], V + (int64_t)j * D);
    const float mn = fmaxf(m, x);
    const float alpha = exp2_fast(m - mn), e = exp2_fast(x - mn);
    l = l * alpha + e;
    a = a * alpha + e * dp;
    m = mn;
  }
  const float M = wave_max_f32(m);
  const float w = (M == -INFINITY) ? 0.f : exp2_fast(m - M);
  const float L = wave_sum_f32(l * w), A = wave_sum_f32(a * w);
  const float lse = (L == 0.f) ? -INFINITY : M + __log2f(L);
  const float delta = (L == 0.f) ? 0.f : A / L;
  if (lane == 0) {
    p.lse2[(int64_t)bh * p.Lq + qi] = lse;
    p.delta[(int64_t)bh * p.Lq + qi] = delta;
  }

  // pass 2: dS_j = P_j (dP_j - Delta) per lane, then dQ += dS_j K_j over the
  // chunk with lanes on features
  float acc[FPL];
#pragma unroll
  for (int r = 0; r < FPL; ++r) acc[r] = 0.f;
  const int kdo = __builtin_amdgcn_readfirstlane((lse == -INFINITY) ? 0 : kmax);  // wave-uniform
  for (int j0 = 0; j0 < kdo; j0 += 64) {
    const int j = j0 + lane;
    float ds = 0.f;
    if (j < kdo) {
      const float x = logit(j, dot_row<D>(rows[wv][0], K + (int64_t)j * D));
      if (x != -INFINITY) {
        const float dp = dot_row<D>(rows[wv][1], V + (int64_t)j * D);
        ds = exp2_fast(x - lse) * (dp - delta);
      }
    }
    const int nj = min(64, kdo - j0);
    for (int jj = 0; jj < nj; ++jj) {
      const float d = lane_value(ds, jj);
      const float* kr = K + (int64_t)(j0 + jj) * D;
#pragma unroll
      for (int r = 0; r < FPL; ++r)
        if (lane + 64 * r < D) acc[r] = __builtin_fmaf(d, kr[lane + 64 * r], acc[r]);
    }
  }
  float* dq = static_cast<float*>(p.dq) + ((int64_t)bh * p.Lq + qi) * D;
  bool nonfinite = false;
#pragma unroll
  for (int r = 0; r < FPL; ++r)
    if (lane + 64 * r < D) {
      const float y = acc[r] * p.scale;
      dq[lane + 64 * r] = y;
      nonfinite |= !__builtin_isfinite(y);
    }
  const uint64_t nf = __ballot(nonfinite);
  if (lane == 0) {
    const uint32_t fl = (nf ? F_NONFINITE : 0u) | (lse == -INFINITY ? F_FULLY_MASKED_ROW : 0u) |
                        (bad ? F_BAD_LENGTH : 0u);
    if (fl) atomicOr(p.flags, fl);
  }
}

// ---- dK and dV: one wave per key row ------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_f32_dkv_kernel(const BwdParams p) {
  constexpr int FPL = (D + 63) / 64;
  __shared__ __attribute__((aligned(16))) float rows[4][2][D];  // [wave][k, v]
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nrg = (p.Lk + 3) / 4;
  const int bh = blockIdx.x / nrg;
  const int kj = (blockIdx.x % nrg) * 4 + wv;
  if (kj >= p.Lk) return;
  bool bad = false;
  const int kend = bwd_len(p, bh / p.H, &bad);
  // rows that see this key: from the key on (causal), none past the length
  const int i_lo = kj >= kend ? p.Lq : (p.causal ? kj : 0);
  const float* Q = static_cast<const float*>(p.q) + (int64_t)bh * p.Lq * D;
  const float* G = static_cast<const float*>(p.dout) + (int64_t)bh * p.Lq * D;
  const float* k = static_cast<const float*>(p.k) + ((int64_t)bh * p.Lk + kj) * D;
  const float* v = static_cast<const float*>(p.v) + ((int64_t)bh * p.Lk + kj) * D;
  const float* lse2 = p.lse2 + (int64_t)bh * p.Lq;
  const float* dlt = p.delta + (int64_t)bh * p.Lq;
  for (int f = lane; f < D; f += 64) {
    rows[wv][0][f] = k[f];
    rows[wv][1][f] = v[f];
  }
  wave_lds_sync();

  float ak[FPL], av[FPL];
#pragma unroll
  for (int r = 0; r < FPL; ++r) ak[r] = av[r] = 0.f;
  for (int i0 = i_lo; i0 < p.Lq; i0 += 64) {
    const int i = i0 + lane;
    float pr = 0.f, ds = 0.f;
    if (i < p.Lq) {
      const float lse = lse2[i];
      if (lse != -INFINITY) {
        float x = dot_row<D>(rows[wv][0], Q + (int64_t)i * D) * p.c;
        if (p.mask) x = masked_logit(p, x, mask_at_f32(p, bh, i, kj));
        if (x != -INFINITY) {
          const float dp = dot_row<D>(rows[wv][1], G + (int64_t)i * D);
          pr = exp2_fast(x - lse);
          ds = pr * (dp - dlt[i]);
        }
      }
    }
    const int ni = min(64, p.Lq - i0);
    for (int ii = 0; ii < ni; ++ii) {
      const float wp = lane_value(pr, ii), wd = lane_value(ds, ii);
      const float* qr = Q + (int64_t)(i0 + ii) * D;
      const float* gr = G + (int64_t)(i0 + ii) * D;
#pragma unroll
      for (int r = 0; r < FPL; ++r)
        if (lane + 64 * r < D) {
          av[r] = __builtin_fmaf(wp, gr[lane + 64 * r], av[r]);
          ak[r] = __builtin_fmaf(wd, qr[lane + 64 * r], ak[r]);
        }
    }
  }
  float* dk = static_cast<float*>(p.dk) + ((int64_t)bh * p.Lk + kj) * D;
  float* dv = static_cast<float*>(p.dv) + ((int64_t)bh * p.Lk + kj) * D;
  bool nonfinite = false;
#pragma unroll
  for (int r = 0; r < FPL; ++r)
    if (lane + 64 * r < D) {
      const float a = ak[r] * p.scale, b = av[r];
      dk[lane + 64 * r] = a;
      dv[lane + 64 * r] = b;
      nonfinite |= !__builtin_isfinite(a) || !__builtin_isfinite(b);
    }
  if (__ballot(nonfinite) && lane == 0) atomicOr(p.flags, F_NONFINITE);
}

template <int D>
hipError_t launch_bwd_f32(const BwdParams& p, hipStream_t stream) {
  const long long gq = (long long)p.B * p.H * ((p.Lq + 3) / 4);  // 4 query rows per workgroup
  const long long gk = (long long)p.B * p.H * ((p.Lk + 3) / 4);  // 4 key rows per workgroup
  if (gq > 0x7fffffffLL || gk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (gq > 0) hipLaunchKernelGGL(bwd_f32_dq_kernel<D>, dim3((unsigned)gq), dim3(256), 0, stream, p);
  if (gk > 0) hipLaunchKernelGGL(bwd_f32_dkv_kernel<D>, dim3((unsigned)gk), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mha
