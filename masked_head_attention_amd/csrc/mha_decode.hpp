// mha_decode.hpp -- the decode shape of masked multi-head attention for
// gfx950 (CDNA4): one new query row per (batch, head) against a key/value
// cache with per-sequence lengths, with the keys split across waves and the
// partial results merged by log-sum-exp.
//
// Sources (web pages, cited by title and section):
//   [MMHA] "masked multi head attention" CUDA implementation notes
//          (2kiu.com/news/6063113), 6.1: the kernel called from an inference
//          engine's key/value-cache update with one new token per sequence.
//   [MAX]  "Why attention must compute the max first" (gsyq.cn/news/340375),
//          2.3-2.4: the online softmax (running maximum, rescaled running sum,
//          weights multiplied into the output accumulator); two running
//          states combine exactly by rescaling both to the larger maximum.
//
// With one query row the two contractions are matrix-vector products: every
// key and value byte is used once, so the work is bound by HBM and runs on
// the vector ALUs (there is no dense contraction for the matrix cores).
//
// Split kernel: one wave owns `chunk` consecutive keys of one (b, h) head.
//   * A key row of D elements is RB = D*esize bytes = LPK 16-byte pieces;
//     LPK lanes share a key, so one load instruction moves G = 64/LPK whole
//     consecutive rows (1 KiB, contiguous). U loads of K and U of V are in
//     flight per iteration.
//   * Each lane forms the partial dot product of its 16-byte piece of q and
//     k; a butterfly over the LPK lanes (DPP within a 16-lane row, a lane
//     swap across rows) leaves the full score in every lane of the group,
//     bitwise identical (each step adds the same two values).
//   * Each lane keeps the online softmax state of its key group: running
//     maximum m, running sum l and the unnormalised output of its features.
//     Scores are in log2 units (q.k * scale * log2 e), exponentials are 2^x.
//   * At the end the G groups of the wave are merged by log-sum-exp.
//   * Keys at or past the sequence length are outside the buffer range of
//     K and V, so their loads return zeros and move no data; the split's own
//     range test masks them.
// With one split per head the wave normalises and stores the row (and its
// log-sum-exp). Otherwise each split stores (m, l, O) in float32 and the
// merge kernel combines the splits of a head:
//   M = max m_s,  L = sum l_s 2^(m_s - M),  O = sum O_s 2^(m_s - M) / L,
//   lse = (M + log2 L) ln 2   (natural log of the sum of exp(scaled scores)).
#pragma once

#include "mha_common.hpp"

namespace mha {

struct DecodeParams {
  const void* q;        // [B,H,D]
  const void* k;        // [B,H,Lk,D]
  const void* v;        // [B,H,Lk,D]
  const int32_t* lens;  // [B] or null (every key legal)
  void* out;            // [B,H,D]
  float* lse;           // [B,H] or null
  float* part_o;        // [B*H, nsplit, D] float32 (nsplit > 1)
  float* part_ml;       // [B*H, nsplit, 2] float32: (m, l) in log2 units
  int B, H, Lk;
  int chunk;            // keys per split (a multiple of DecCfg::KPI)
  int nsplit;           // splits per head
  float c;              // scale * log2(e)
  uint32_t* flags;
};

template <typename T, int D>
struct DecCfg {
  static constexpr int E = sizeof(T);
  static constexpr int RB = D * E;      // bytes per key row
  static constexpr int LPK = RB / 16;   // lanes per key row
  static constexpr int G = 64 / LPK;    // key rows per load instruction
  static constexpr int EPL = 16 / E;    // features per lane
  static constexpr int U = 4;           // loads of K (and of V) in flight per iteration
  static constexpr int KPI = G * U;     // keys per iteration
  static_assert(LPK >= 2 && LPK <= 32, "a key row spans 2..32 lanes");
};

// Keys per iteration of the split kernel for a dtype size and D (host side).
inline int decode_keys_per_iter(int D, int esize) { return 4 * 1024 / (D * esize); }

template <int CTRL>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over the LPK-lane group of each lane (groups are aligned runs of LPK
// lanes); every lane of a group receives the same value.
template <int LPK>
__device__ inline float group_sum(float x) {
  if constexpr (LPK >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (LPK >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (LPK >= 8) x += dpp<0x141>(x);  // row_half_mirror: the other quad of 8
  if constexpr (LPK >= 16) x += dpp<0x140>(x); // row_mirror: the other 8 of the row
  if constexpr (LPK >= 32) {                   // the neighbouring 16-lane row
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                              false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return x;
}

// Partial dot product of a lane's 16-byte pieces of q and k, float32 sum.
__device__ inline float dot16(const uint4 q, const uint4 k, _Float16*) {
  float a = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, q.x), __builtin_bit_cast(f16x2, k.x),
                                   0.f, false);
  a = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, q.y), __builtin_bit_cast(f16x2, k.y), a,
                             false);
  a = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, q.z), __builtin_bit_cast(f16x2, k.z), a,
                             false);
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, q.w), __builtin_bit_cast(f16x2, k.w), a,
                                false);
}
__device__ inline float dot16(const uint4 q, const uint4 k, __bf16*) {
  float a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.x),
                                            __builtin_bit_cast(bf16x2, k.x), 0.f, false);
  a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.y),
                                      __builtin_bit_cast(bf16x2, k.y), a, false);
  a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.z),
                                      __builtin_bit_cast(bf16x2, k.z), a, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.w),
                                         __builtin_bit_cast(bf16x2, k.w), a, false);
}
__device__ inline float dot16(const uint4 q, const uint4 k, float*) {
  float a = __uint_as_float(q.x) * __uint_as_float(k.x);
  a = __builtin_fmaf(__uint_as_float(q.y), __uint_as_float(k.y), a);
  a = __builtin_fmaf(__uint_as_float(q.z), __uint_as_float(k.z), a);
  return __builtin_fmaf(__uint_as_float(q.w), __uint_as_float(k.w), a);
}

// The features of a lane's 16-byte piece of a row, as float32.
template <typename T>
__device__ inline void piece_to_f32(const uint4 u, float (&x)[16 / sizeof(T)]) {
  if constexpr (sizeof(T) == 4) {
    x[0] = __uint_as_float(u.x); x[1] = __uint_as_float(u.y);
    x[2] = __uint_as_float(u.z); x[3] = __uint_as_float(u.w);
  } else {
    T* tag = nullptr;
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = lo_f(w[i], tag);
      x[2 * i + 1] = hi_f(w[i], tag);
    }
  }
}

// EPL float32 values packed into a 16-byte piece of T (nearest even).
template <typename T>
__device__ inline uint4 f32_pack_piece(const float (&x)[16 / sizeof(T)]) {
  if constexpr (sizeof(T) == 4) {
    return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                      __float_as_uint(x[3]));
  } else {
    T* tag = nullptr;
    return make_uint4(pack2(x[0], x[1], tag), pack2(x[2], x[3], tag), pack2(x[4], x[5], tag),
                      pack2(x[6], x[7], tag));
  }
}

// Length of sequence b clamped to [0, Lk]; *bad is set when it was outside.
__device__ inline int decode_len(const DecodeParams& p, int b, bool* bad) {
  if (!p.lens) {
    *bad = false;
    return p.Lk;
  }
  const int l = p.lens[b];
  *bad = l < 0 || l > p.Lk;
  return l < 0 ? 0 : (l > p.Lk ? p.Lk : l);
}

template <typename T, int D>
// Four waves per SIMD: registers for two K/V buffers per wave, which keeps
// the compiler from trading the prefetch for occupancy.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void
decode_split_kernel(const DecodeParams p) {
  using C = DecCfg<T, D>;
  constexpr int EPL = C::EPL, U = C::U, G = C::G, LPK = C::LPK, RB = C::RB;
  const int lane = threadIdx.x & 63;
  // (head, split) of this wave; wave-uniform, so the buffer resources are
  // scalar. The host keeps B*H*nsplit below 2^31.
  const uint32_t wid =
      blockIdx.x * 4u + (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (wid >= (uint32_t)(p.B * p.H * p.nsplit)) return;  // whole waves only
  // the split index is the slow one: consecutive workgroups take the same
  // split of neighbouring heads, so the CUs that the round-robin placement
  // feeds each receive a mix of early (always legal) and late splits
  const uint32_t nbh = (uint32_t)(p.B * p.H);
  const int s = (int)(wid / nbh);
  const uint32_t bh32 = wid - (uint32_t)s * nbh;
  const int64_t bh = bh32;
  bool bad = false;
  const int len = decode_len(p, (int)(bh32 / (uint32_t)p.H), &bad);
  const int start = s * p.chunk;
  const bool direct = p.nsplit == 1;
  if (!direct && start >= len) return;  // no legal key in this split: the merge skips it
  const int end = min(start + p.chunk, len);
  const int g = lane / LPK, sub = lane % LPK;

  const char* kh = static_cast<const char*>(p.k) + bh * (int64_t)p.Lk * RB;
  const char* vh = static_cast<const char*>(p.v) + bh * (int64_t)p.Lk * RB;
  // rows at or past the split's end read as zeros and move no data, so the
  // prefetch of the iteration after the last one is free
  const auto krs = make_rsrc(kh, (uint32_t)end * RB);
  const auto vrs = make_rsrc(vh, (uint32_t)end * RB);
  const uint4 qv =
      *reinterpret_cast<const uint4*>(static_cast<const char*>(p.q) + bh * RB + sub * 16);
  T* tag = nullptr;

  float m = -INFINITY, l = 0.f, o[EPL];
#pragma unroll
  for (int f = 0; f < EPL; ++f) o[f] = 0.f;

  // Every cache byte is read once per call, so the loads carry the
  // non-temporal hint (cache-policy bit `nt`): the lines they bring in are
  // the first to be replaced and do not push out other data.
  constexpr int NT = 2;
  auto issue = [&](int kb, uint4 (&kr)[U], uint4 (&vr)[U]) {
    const uint32_t off0 = (uint32_t)(kb + g) * RB + sub * 16;
#pragma unroll
    for (int u = 0; u < U; ++u)
      kr[u] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, off0 + u * G * RB, 0, NT));
#pragma unroll
    for (int u = 0; u < U; ++u)
      vr[u] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(vrs, off0 + u * G * RB, 0, NT));
  };
  auto consume = [&](int kb, const uint4 (&kr)[U], const uint4 (&vr)[U]) {
    float t[U];
    float mx = m;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float sc = group_sum<LPK>(dot16(qv, kr[u], tag)) * p.c;
      t[u] = (kb + u * G + g < end) ? sc : -INFINITY;
      mx = fmaxf(mx, t[u]);
    }
    const float mu = (mx == -INFINITY) ? 0.f : mx;  // no legal key yet: weights stay 0
    const float alpha = exp2_fast(m - mu);
    l *= alpha;
#pragma unroll
    for (int f = 0; f < EPL; ++f) o[f] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float pu = exp2_fast(t[u] - mu);
      l += pu;
      float vf[EPL];
      piece_to_f32<T>(vr[u], vf);
#pragma unroll
      for (int f = 0; f < EPL; ++f) o[f] = __builtin_fmaf(pu, vf[f], o[f]);
    }
    m = mx;
  };

  // two register buffers: the next iteration's loads are in flight while the
  // current one is consumed
  uint4 ka[U], va[U], kb2[U], vb2[U];
  if (start < end) issue(start, ka, va);
  for (int kb = start; kb < end; kb += 2 * C::KPI) {
    issue(kb + C::KPI, kb2, vb2);
    consume(kb, ka, va);
    if (kb + C::KPI >= end) break;
    issue(kb + 2 * C::KPI, ka, va);
    consume(kb + C::KPI, kb2, vb2);
  }

  // merge the G key groups of the wave (log-sum-exp), lanes with equal `sub`
#pragma unroll
  for (int x = LPK; x < 64; x <<= 1) {
    const float mo = __shfl_xor(m, x, 64);
    const float lo = __shfl_xor(l, x, 64);
    const float M = fmaxf(m, mo);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    const float a = exp2_fast(m - Mu), b = exp2_fast(mo - Mu);
    l = l * a + lo * b;
#pragma unroll
    for (int f = 0; f < EPL; ++f) o[f] = o[f] * a + __shfl_xor(o[f], x, 64) * b;
    m = M;
  }
  if (g != 0) return;  // lanes 0 .. LPK-1 hold the wave's result

  if (!direct) {
    const int64_t slot = bh * p.nsplit + s;
    float* po = p.part_o + slot * D + sub * EPL;
#pragma unroll
    for (int f = 0; f < EPL; f += 4)
      *reinterpret_cast<float4*>(po + f) = make_float4(o[f], o[f + 1], o[f + 2], o[f + 3]);
    if (sub == 0) *reinterpret_cast<float2*>(p.part_ml + 2 * slot) = make_float2(m, l);
    return;
  }
  // one split: normalise and store the row
  const float inv = (l == 0.f) ? 0.f : 1.0f / l;  // no legal key: output 0
  float y[EPL];
  bool nonfinite = false;
#pragma unroll
  for (int f = 0; f < EPL; ++f) {
    y[f] = o[f] * inv;
  }
  const uint4 packed = f32_pack_piece<T>(y);
  float back[EPL];
  piece_to_f32<T>(packed, back);
#pragma unroll
  for (int f = 0; f < EPL; ++f) nonfinite |= !__builtin_isfinite(back[f]);
  *reinterpret_cast<uint4*>(static_cast<char*>(p.out) + bh * RB + sub * 16) = packed;
  const uint64_t nf = __ballot(nonfinite);
  if (sub == 0) {
    if (p.lse) p.lse[bh] = (l == 0.f) ? -INFINITY : (m + __log2f(l)) * 0.6931471805599453f;
    uint32_t fl = (l == 0.f ? F_FULLY_MASKED_ROW : 0u) | (bad ? F_BAD_LENGTH : 0u) |
                  (nf ? F_NONFINITE : 0u);
    if (fl) atomicOr(p.flags, fl);
  }
}

// Merge of the splits of each head: one wave per (b, h).
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(const DecodeParams p) {
  constexpr int FPL = (D + 63) / 64;  // features per lane
  const int lane = threadIdx.x & 63;
  const uint32_t bh32 =
      blockIdx.x * 4u + (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (bh32 >= (uint32_t)(p.B * p.H)) return;
  const int64_t bh = bh32;
  bool bad = false;
  const int len = decode_len(p, (int)(bh32 / (uint32_t)p.H), &bad);
  const int ns = (len + p.chunk - 1) / p.chunk;  // splits holding a legal key
  const float* ml = p.part_ml + bh * p.nsplit * 2;
  const float* po = p.part_o + bh * p.nsplit * D;
  // split s's (m, l) is read by lane s % 64; maxima and sums are wave reductions
  float M = -INFINITY, L = 0.f, O[FPL];
#pragma unroll
  for (int r = 0; r < FPL; ++r) O[r] = 0.f;
  constexpr int NH = 32;  // up to NH splits: every load of the head issued at once
  if (ns <= NH) {
    float2 v = make_float2(-INFINITY, 0.f);
    if (lane < ns) v = *reinterpret_cast<const float2*>(ml + 2 * lane);
    float x[NH][FPL];
#pragma unroll
    for (int j = 0; j < NH; ++j)
#pragma unroll
      for (int r = 0; r < FPL; ++r) {
        const int f = lane + 64 * r;
        x[j][r] = (j < ns && f < D) ? po[(int64_t)j * D + f] : 0.f;
      }
    M = v.x;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    const float Mu = (M == -INFINITY) ? 0.f : M;
    const float w = (lane < ns) ? exp2_fast(v.x - Mu) : 0.f;  // weight of split `lane`
    L = v.y * w;
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
#pragma unroll
      for (int r = 0; r < FPL; ++r) O[r] = __builtin_fmaf(x[j][r], wj, O[r]);
    }
  } else {
    for (int s = lane; s < ns; s += 64) M = fmaxf(M, ml[2 * s]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    const float Mu = (M == -INFINITY) ? 0.f : M;
    constexpr int SB = 8;  // splits whose partial outputs are loaded together
    for (int s0 = 0; s0 < ns; s0 += 64) {
      const int n = min(64, ns - s0);
      float w = 0.f;  // weight of split s0 + lane
      if (lane < n) {
        const float2 v = *reinterpret_cast<const float2*>(ml + 2 * (s0 + lane));
        w = exp2_fast(v.x - Mu);
        L = __builtin_fmaf(v.y, w, L);
      }
      for (int j0 = 0; j0 < n; j0 += SB) {
        float x[SB][FPL];
#pragma unroll
        for (int j = 0; j < SB; ++j)
#pragma unroll
          for (int r = 0; r < FPL; ++r) {
            const int f = lane + 64 * r;
            x[j][r] = (j0 + j < n && f < D) ? po[(int64_t)(s0 + j0 + j) * D + f] : 0.f;
          }
#pragma unroll
        for (int j = 0; j < SB; ++j) {
          const float wj =
              (j0 + j < n) ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j0 + j))
                           : 0.f;
#pragma unroll
          for (int r = 0; r < FPL; ++r) O[r] = __builtin_fmaf(x[j][r], wj, O[r]);
        }
      }
    }
  }
#pragma unroll
  for (int x = 32; x > 0; x >>= 1) L += __shfl_xor(L, x, 64);
  const float inv = (L == 0.f) ? 0.f : 1.0f / L;
  bool nonfinite = false;
  T* out = static_cast<T*>(p.out) + bh * D;
#pragma unroll
  for (int r = 0; r < FPL; ++r) {
    const int f = lane + 64 * r;
    if (f < D) {
      const T y = (T)(O[r] * inv);  // round to nearest even
      out[f] = y;
      nonfinite |= !__builtin_isfinite((float)y);
    }
  }
  const uint64_t nf = __ballot(nonfinite);
  if (lane == 0) {
    if (p.lse) p.lse[bh] = (L == 0.f) ? -INFINITY : (M + __log2f(L)) * 0.6931471805599453f;
    uint32_t fl = (ns == 0 ? F_FULLY_MASKED_ROW : 0u) | (bad ? F_BAD_LENGTH : 0u) |
                  (nf ? F_NONFINITE : 0u);
    if (fl) atomicOr(p.flags, fl);
  }
}

template <typename T, int D>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream) {
  const long long waves = (long long)p.B * p.H * p.nsplit;
  if (waves <= 0) return hipSuccess;
  const long long grid = (waves + 3) / 4;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((decode_split_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  if (p.nsplit > 1) {
    const long long mgrid = ((long long)p.B * p.H + 3) / 4;
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((unsigned)mgrid), dim3(256), 0, stream,
                       p);
  }
  return hipGetLastError();
}

}  // namespace mha
