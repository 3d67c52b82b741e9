// mha_bwd.hpp -- backward of the fused masked multi-head attention forward for
// gfx950 (CDNA4), float16 and bfloat16 (and float32 up to D = 64): the
// gradients dQ, dK, dV for an upstream gradient dO.
//
// Source (web page, cited by title and section):
//   [MAX] "Why attention must compute the max first" (gsyq.cn/news/340375),
//         3.3: the softmax Jacobian dp_j/ds_k = p_j (delta_jk - p_k); the row
//         maximum carries no gradient, so the weights can be rebuilt from the
//         row's log-sum-exp.
// With P = softmax(scale Q K^T) over the legal keys:
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - Delta),
//   Delta_i = sum_j P_ij dP_ij (the Jacobian's row term),  dQ = scale dS K,
//   dK = scale dS^T Q.
//
// Two kernels, two waves per 32-row block (each takes alternate tiles of the
// other dimension and the two add their sums), all contractions on 32x32x16 MFMA
// with float32 accumulation:
//   * dq kernel (a query block): pass 1 computes each row's log-sum-exp from
//     S^T = K Q^T and, with dP^T = V dO^T, Delta (a running maximum with the
//     rescaled sums of the weights and of weight * dP per lane, as in the
//     forward's online softmax); pass 2 rebuilds P and dP, forms dS and
//     accumulates dQ = dS K. It also stores the log-sum-exp and Delta of
//     each row for the second kernel. Delta is formed from P and dP in
//     float32, not from the stored 16-bit output O (whose rounding would
//     shift every dS of a row).
//   * dkv kernel (a key block): S = Q K^T and dP = dO V^T per query tile,
//     P from the stored log-sum-exp, then dV += P^T dO and dK += dS^T Q.
// Operand layouts (32x32x16 MFMA): lane l supplies row/column l % 32 and the
// 8 consecutive k-slots 8 (l / 32) .. +7; accumulator register i of lane l
// holds row 8 (i / 4) + 4 (l / 32) + i % 4 of column l % 32. Rows of a
// score tile are loaded through keymap (mha_common.hpp), so a lane's 16
// score accumulators are two runs of 8 consecutive keys (or queries): they
// are the k-slots of the next contraction's A operand as they stand. The B
// operands that need 8 consecutive rows of one feature (K for dQ, dO and Q
// for dV and dK) go through a row-major copy of the tile in LDS, read with
// the transposing ds_read_b64_tr_b16.
// P and dS enter the MFMAs as a pair of 16-bit values (the rounded value
// and the rounded remainder), so the products keep about 16 significant
// bits beyond the 16-bit type.
// float32 runs the same kernels: a 16-element slice is 8 steps of
// v_mfma_f32_32x32x2_f32 with the same slot assignment, fragments are 32
// bytes, the B operands are 4-byte reads (no transposing read for 32-bit
// elements), and P and dS enter as they are.
#pragma once

#include "mha_common.hpp"

namespace mha {

struct BwdParams {
  const void* q;        // [B,H,Lq,D]
  const void* k;        // [B,H,Lk,D]
  const void* v;        // [B,H,Lk,D]
  const void* dout;     // [B,H,Lq,D]
  const int32_t* lens;  // [B] (PADDING) or null
  const void* mask;     // [B,Hm,Lq,Lk] additive or keep mask in the element type, or null
  int mask_heads;       // Hm: 1 (shared by the heads) or H (one slab per head)
  int keep;             // the mask tensor is a keep-mask (0 masks a key; values not added)
  void* dq;             // [B,H,Lq,D]
  void* dk;             // [B,H,Lk,D]
  void* dv;             // [B,H,Lk,D]
  float* lse2;          // [B*H*Lq] row log-sum-exp, log2 units of c*q.k (workspace)
  float* delta;         // [B*H*Lq] sum_j P_ij dP_ij (workspace)
  int B, H, Lq, Lk;
  int nqblk, nkblk;     // 32-row blocks of queries and of keys
  int causal;
  float c;              // scale * log2(e)
  float scale;
  uint32_t* flags;
};

// Key (or query) offset within a 32-row tile held by accumulator register i
// of a lane in half hh, for a tile whose rows were loaded through keymap.
__device__ inline int run_off(int i, int hh) { return i < 8 ? 8 * hh + i : 16 + 8 * hh + (i - 8); }

// A operand frag (k-block kk of a 32-wide contraction) from accumulator
// values: registers 8kk .. 8kk+7, as the rounded value and its remainder.
template <typename T>
__device__ inline void split_frag(const float* x, Frag8<T>& hi, Frag8<T>& lo) {
  float h[8], r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = (float)(T)x[e];
    r[e] = x[e] - h[e];
  }
  hi = pack8<T>(h);
  lo = pack8<T>(r);
}

// float16: each pair rounded in one packed conversion, then each remainder
// x - hi (exact before its one rounding) in one mixed-precision FMA that
// reads hi's half straight from the packed word. Left to itself the compiler
// rounds every value a second time to feed that FMA.
template <>
__device__ inline void split_frag<_Float16>(const float* x, Frag8<_Float16>& hi,
                                            Frag8<_Float16>& lo) {
  _Float16* tag = nullptr;
  uint32_t h[4], l[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    h[k] = pack2(x[2 * k], x[2 * k + 1], tag);
    asm("v_fma_mixlo_f16 %0, %1, 1.0, -%2 op_sel_hi:[0,0,1]" : "=v"(l[k]) : "v"(x[2 * k]), "v"(h[k]));
    asm("v_fma_mixhi_f16 %0, %1, 1.0, -%2 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
        : "+v"(l[k])
        : "v"(x[2 * k + 1]), "v"(h[k]));
  }
  hi.u[0] = make_uint4(h[0], h[1], h[2], h[3]);
  lo.u[0] = make_uint4(l[0], l[1], l[2], l[3]);
}

// LDS tiles are row-major, 32 rows of D elements, RS bytes apart. The row
// padding spreads the rows of one read over the banks; of 16, 32, 48 and 64
// bytes, 48 measured fastest (backward workload 402.8 us; 409.6, 412.5, 447.8).
template <typename T, int D>
constexpr int tile_rs() { return D * (int)sizeof(T) + 48; }

// Eight consecutive elements (one A or B operand fragment) in LDS.
template <typename T>
__device__ inline Frag8<T> lds_frag(const char* p) {
  Frag8<T> f;
  f.u[0] = lds_load16(p);
  if constexpr (sizeof(T) == 4) f.u[1] = lds_load16(p + 16);
  return f;
}
template <typename T>
__device__ inline void lds_put_frag(char* p, const Frag8<T>& f) {
  *reinterpret_cast<uint4*>(p) = f.u[0];
  if constexpr (sizeof(T) == 4) *reinterpret_cast<uint4*>(p + 16) = f.u[1];
}

// float32: the 32 x 32 product over a 16-element slice as 8 steps of
// v_mfma_f32_32x32x2_f32. In step j a lane of half hh supplies its element j,
// contraction index 8 hh + j: the same slot assignment as the 16-bit slice.
__device__ inline f32x16 mma8(const Frag8<float>& a, const Frag8<float>& b, f32x16 c) {
  const uint32_t av[8] = {a.u[0].x, a.u[0].y, a.u[0].z, a.u[0].w,
                          a.u[1].x, a.u[1].y, a.u[1].z, a.u[1].w};
  const uint32_t bv[8] = {b.u[0].x, b.u[0].y, b.u[0].z, b.u[0].w,
                          b.u[1].x, b.u[1].y, b.u[1].z, b.u[1].w};
#pragma unroll
  for (int j = 0; j < 8; ++j)
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(av[j]), __uint_as_float(bv[j]), c, 0,
                                             0, 0);
  return c;
}

typedef __fp16 bwd_f16x4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __bf16 bwd_bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
template <typename T>
__device__ inline uint2 bwd_read_tr(const char* p);
template <>
__device__ inline uint2 bwd_read_tr<_Float16>(const char* p) {
  return __builtin_bit_cast(uint2,
                            __builtin_amdgcn_ds_read_tr16_b64_v4f16(MHA_LDS_PTR(bwd_f16x4, p)));
}
template <>
__device__ inline uint2 bwd_read_tr<__bf16>(const char* p) {
  return __builtin_bit_cast(uint2,
                            __builtin_amdgcn_ds_read_tr16_b64_v4bf16(MHA_LDS_PTR(bwd_bf16x4, p)));
}

// B operand frag: feature 32 fb + l % 32, rows 16 kk + 8 (l / 32) .. +7 of
// the tile, by two transposing reads. ds_read_b64_tr_b16: within a group of
// 16 lanes, lane i receives element i % 4 of the 8 bytes addressed by lane
// 4 j + i / 4 as its element j. Lane 4 j + c addresses row j, features
// 4 c .. 4 c + 3 of its group's 16, so lane i gets 4 consecutive rows of
// feature i.
// float32 (no transposing read for 32-bit elements): eight 4-byte reads, rows
// 16 kk + 8 (l / 32) + e of feature 32 fb + l % 32.
template <typename T, int D>
__device__ inline Frag8<T> load_tr_frag(const char* t, int fb, int kk, int lane) {
  Frag8<T> f;
  if constexpr (sizeof(T) == 4) {
    const char* a = t + (16 * kk + 8 * (lane >> 5)) * tile_rs<T, D>() + (32 * fb + (lane & 31)) * 4;
    uint32_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = *reinterpret_cast<const uint32_t*>(a + e * tile_rs<T, D>());
    f.u[0] = make_uint4(v[0], v[1], v[2], v[3]);
    f.u[1] = make_uint4(v[4], v[5], v[6], v[7]);
  } else {
    const int g = lane >> 4, j = (lane >> 2) & 3, c = lane & 3;
    const char* a = t + (16 * kk + 8 * (g >> 1) + j) * tile_rs<T, D>() +
                    (32 * fb + 16 * (g & 1) + 4 * c) * 2;
    const uint2 lo = bwd_read_tr<T>(a), hi = bwd_read_tr<T>(a + 4 * tile_rs<T, D>());
    f.u[0] = make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
  return f;
}

template <typename T, int D>
__device__ inline void load_rows(const __amdgpu_buffer_rsrc_t rs, int row, int hh,
                                 Frag8<T> (&f)[D / 16]) {
  constexpr int ES = sizeof(T);
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb)
#pragma unroll
    for (int w = 0; w < Frag8<T>::W; ++w)
      f[kb].u[w] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(
                     rs, (uint32_t)row * (D * ES) + (16 * kb + 8 * hh) * ES + 16 * w, 0, 0));
}

// Workgroup -> (head, block group) for a grid that runs in rounds (one
// workgroup per CU). Workgroups are dealt to the 8 XCDs round-robin; this map
// keeps every block of a head on one XCD, so the tiles that all blocks of the
// head stream (K and V, or Q and dO) stay in that XCD's L2. An XCD's
// workgroups go in block-group order, all its heads' group 0 first, and a CU
// takes the next one of its XCD when its current one ends: with the longest
// groups first, a CU that held a long group takes a short one. Heads beyond
// the last complete group of 8 keep the plain order.
__device__ inline void xcd_lpt(int nbh, int nblk, int* bh, int* blk) {
  const int i = blockIdx.x;
  const int hpx = nbh / 8;  // heads per XCD among the complete groups of 8
  const int full = hpx * 8 * nblk;
  if (i < full) {
    const int x = i % 8, j = i / 8;
    *blk = j / hpx;
    *bh = (j % hpx) * 8 + x;
  } else {
    *bh = i / nblk;
    *blk = i - *bh * nblk;
  }
}

// Entry (row, key) of the head's mask slab as float32 (0 for rows and keys
// outside the tensor).
template <typename T>
__device__ inline float mask_at(const BwdParams& p, int bh, int row, int key) {
  if (row >= p.Lq || key >= p.Lk) return 0.f;
  const int64_t slab = p.mask_heads == 1 ? bh / p.H : bh;
  const int64_t at = (slab * p.Lq + row) * (int64_t)p.Lk + key;
  if constexpr (sizeof(T) == 4) {
    return static_cast<const float*>(p.mask)[at];
  } else {
    const uint16_t u = static_cast<const uint16_t*>(p.mask)[at];
    T* tag = nullptr;
    return lo_f((uint32_t)u, tag);
  }
}

// A legal score in log2 units, or -inf: the mask tensor's decision and (for
// an additive mask) its value, added after scaling and not scaled.
__device__ inline float masked_logit(const BwdParams& p, float x, float m) {
  if (p.keep) return m == 0.f ? -INFINITY : x;
  return m == -INFINITY ? -INFINITY : __builtin_fmaf(m, 1.4426950408889634f, x);
}

__device__ inline int bwd_len(const BwdParams& p, int b, bool* bad) {
  if (!p.lens) {
    *bad = false;
    return p.Lk;
  }
  const int l = p.lens[b];
  *bad = l < 0 || l > p.Lk;
  return l < 0 ? 0 : (l > p.Lk ? p.Lk : l);
}

// ---- dQ (and the row statistics) per group of 4 query blocks --------------
// Eight waves, two per 32-query block. Each step stages two K/V tiles through
// LDS: each thread loads its 16-byte pieces of the next step's tiles into
// registers while the waves work on the current ones, and stores them into the
// other LDS buffer before the step's barrier. The first wave of a query block
// takes the even key tiles and the second the odd ones, so a causal group's
// chain of tiles is half as long; the two merge their row statistics through
// LDS after pass 1 (in one fixed order, so both get the same values) and add
// their dQ after pass 2, each finishing half of the 32-feature blocks. The A
// operands (K and V rows through keymap) are LDS reads, and dQ's B operand
// (8 consecutive keys of one feature) is a transposing read of the same
// row-major K tile.
// One workgroup per CU (at most 256 registers per lane: at D = 128 the
// compiler fits it without spills), so the grid runs in rounds; the
// workgroups of an XCD are dealt longest first (xcd_lpt).
// The dQ product runs at raised wave priority, so the SIMD's other wave fills
// the matrix core's gaps with its vector work (around the S and dP products,
// which both passes share, this lost).
template <typename T, int D, bool TM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void
bwd_dq_kernel(const BwdParams p) {
  // 32-feature blocks of the dQ accumulators (D = 16: one block whose upper
  // 16 columns read the LDS tile's row padding and are never stored)
  constexpr int FB = (D + 31) / 32;
  constexpr int SB = (FB + 1) / 2;  // blocks a wave hands to its partner (at most)
  constexpr int ES = sizeof(T);      // element bytes
  constexpr int RS = tile_rs<T, D>();
  constexpr int TB = 32 * RS;       // bytes of one staged 32-row tile
  constexpr int CPR = D * ES / 16;  // 16-byte pieces per row
  constexpr int PPT = 32 * CPR;     // pieces per 32-row tile
  constexpr int PPS = (2 * PPT + 511) / 512;  // pieces per thread and tensor of a step
  // LDS: staged tiles [buffer][tile][K, V], then each wave's row statistics
  // (m, l, a for its 32 rows); after pass 2 the staged tiles' space holds the
  // partial dQ handed over, [wave][block], 4 KB each
  constexpr int STAGE = 8 * TB, XST = 8 * 32 * 3 * 4, XCH = 8 * SB * 4096;
  constexpr int LDS = (STAGE + XST) > XCH ? (STAGE + XST) : XCH;
  __shared__ __attribute__((aligned(16))) char smem[LDS];
  char* const stg = smem;
  float* const xst = reinterpret_cast<float*>(smem + STAGE);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wq = wv & 3, half = wv >> 2;
  const int n = lane & 31, hh = lane >> 5;
  const int ngrp = (p.nqblk + 3) / 4;
  int bh = 0, qg = 0;
  xcd_lpt(p.B * p.H, ngrp, &bh, &qg);
  if (p.causal) qg = ngrp - 1 - qg;  // the longest rows (most key tiles) first
  const int q0 = (4 * qg + wq) * 32;  // this wave's query block
  bool bad = false;
  const int kend = bwd_len(p, bh / p.H, &bad);
  const int qi = q0 + n;  // this lane's query (column of S^T)
  const int64_t qoff = (int64_t)bh * p.Lq * D * ES, koff = (int64_t)bh * p.Lk * D * ES;
  const uint32_t qbytes = (uint32_t)p.Lq * D * ES;
  const auto qrs = make_rsrc(static_cast<const char*>(p.q) + qoff, qbytes);
  const auto grs = make_rsrc(static_cast<const char*>(p.dout) + qoff, qbytes);
  const auto krs = make_rsrc(static_cast<const char*>(p.k) + koff, (uint32_t)kend * D * ES);
  const auto vrs = make_rsrc(static_cast<const char*>(p.v) + koff, (uint32_t)kend * D * ES);

  Frag8<T> qf[D / 16], gf[D / 16];
  load_rows<T, D>(qrs, qi, hh, qf);
  load_rows<T, D>(grs, qi, hh, gf);
  // keys past a block's last query are illegal for all its rows (causal);
  // the group streams the tiles of its last block, each wave computes its own
  const int kmax = p.causal ? min(kend, q0 + 32) : kend;
  const int ntile = q0 < p.Lq ? (kmax + 31) / 32 : 0;
  const int kmax_g = p.causal ? min(kend, 4 * qg * 32 + 128) : kend;
  const int nstep = ((kmax_g + 31) / 32 + 1) / 2;  // step s stages tiles 2s, 2s + 1

  // staged copy of a step's K/V tiles: piece u = tid + 512 i is tile u / PPT,
  // row (u % PPT) / CPR, 16-byte chunk u % CPR; rows past the key range read
  // as zeros
  uint4 rk[PPS], rv[PPS];
  auto gload = [&](int s) {
#pragma unroll
    for (int i = 0; i < PPS; ++i) {
      const int u = tid + 512 * i;
      if ((2 * PPT) % 512 == 0 || u < 2 * PPT) {
        const int tl = u / PPT, w = u % PPT;
        const uint32_t off = (uint32_t)(32 * (2 * s + tl) + w / CPR) * (D * ES) + (w % CPR) * 16;
        rk[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0));
        rv[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0));
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PPS; ++i) {
      const int u = tid + 512 * i;
      if ((2 * PPT) % 512 == 0 || u < 2 * PPT) {
        const int tl = u / PPT, w = u % PPT;
        const int o = (buf * 2 + tl) * 2 * TB + (w / CPR) * RS + (w % CPR) * 16;
        *reinterpret_cast<uint4*>(stg + o) = rk[i];
        *reinterpret_cast<uint4*>(stg + o + TB) = rv[i];
      }
    }
  };
  // this wave's K tile of the step in buffer buf (V follows it)
  auto ktile = [&](int buf) { return stg + (buf * 2 + half) * 2 * TB; };
  // S^T and dP^T of the tile in buffer buf (K and V rows through keymap)
  auto tile = [&](int buf, f32x16& sa, f32x16& da) {
    const char* kr = ktile(buf) + keymap(n) * RS + 8 * hh * ES;
    const char* vr = kr + TB;
    sa = f32x16{};
    da = f32x16{};
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
      const Frag8<T> kf = lds_frag<T>(kr + 16 * kb * ES), vf = lds_frag<T>(vr + 16 * kb * ES);
      sa = mma8(kf, qf[kb], sa);
      da = mma8(vf, gf[kb], da);
    }
  };
  auto legal = [&](int key) { return key < kend && !(p.causal && key > qi); };
  // one streaming pass over the group's key tiles; body(t, buf) runs for the
  // tiles of this wave's share of its block's range
  auto stream = [&](auto&& body) {
    if (nstep > 0) {
      gload(0);
      lstore(0);
    }
    __syncthreads();
    for (int s = 0; s < nstep; ++s) {
      const int buf = s & 1;
      if (s + 1 < nstep) gload(s + 1);
      const int t = 2 * s + half;
      if (t < ntile) body(t, buf);
      if (s + 1 < nstep) lstore(buf ^ 1);  // last read at step s - 1, before its barrier
      __syncthreads();
    }
  };

  // Only a tile that reaches the key length or (causal) the block's diagonal
  // tests each key; the others are legal throughout (wave-uniform choice).
  auto edge = [&](int t) { return 32 * t + 31 >= kend || (p.causal && 32 * t >= q0); };

  // pass 1: log-sum-exp (log2 units) and Delta = sum_j P_j dP_j of each row:
  // running maximum m, sum l of 2^(s - m) and sum a of 2^(s - m) dP
  float m = -INFINITY, l = 0.f, a = 0.f;
  stream([&](int t, int buf) {
    f32x16 sa, da;
    tile(buf, sa, da);
    float s[16], mx = m;
    auto logits = [&](auto edge_tag) {
      constexpr bool EDGE = decltype(edge_tag)::value;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 32 * t + run_off(i, hh);
        float x = sa[i] * p.c;
        if constexpr (TM) x = masked_logit(p, x, mask_at<T>(p, bh, qi, key));
        s[i] = (!EDGE || legal(key)) ? x : -INFINITY;
        mx = fmaxf(mx, s[i]);
      }
    };
    if (edge(t))
      logits(std::true_type{});
    else
      logits(std::false_type{});
    const float mu = (mx == -INFINITY) ? 0.f : mx;
    const float alpha = exp2_fast(m - mu);
    l *= alpha;
    a *= alpha;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = exp2_fast(s[i] - mu);
      l += e;
      a = __builtin_fmaf(e, da[i], a);
    }
    m = mx;
  });
  float lse, delta;
  {
    // this wave's keys: the two lanes of a query, then the block's other wave
    const float M = pair_max(m);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    const float w = exp2_fast(m - Mu);
    const float L = pair_sum(l * w);
    const float A = pair_sum(a * w);
    if (hh == 0) {
      xst[(wv * 32 + n) * 3 + 0] = M;
      xst[(wv * 32 + n) * 3 + 1] = L;
      xst[(wv * 32 + n) * 3 + 2] = A;
    }
    __syncthreads();
    const float* x0 = xst + (wq * 32 + n) * 3;        // the even tiles' wave
    const float* x1 = xst + ((wq + 4) * 32 + n) * 3;  // the odd tiles'
    const float M0 = x0[0], M1 = x1[0];
    const float Mx = fmaxf(M0, M1);
    const float Mxu = (Mx == -INFINITY) ? 0.f : Mx;
    // a wave without legal keys has M = -inf and L = A = 0: its weight is 0
    const float w0 = exp2_fast(M0 - Mxu), w1 = exp2_fast(M1 - Mxu);
    const float Lt = x0[1] * w0 + x1[1] * w1;
    const float At = x0[2] * w0 + x1[2] * w1;
    lse = (Lt == 0.f) ? -INFINITY : Mxu + __log2f(Lt);
    delta = (Lt == 0.f) ? 0.f : At / Lt;
  }
  const bool row_ok = qi < p.Lq;
  if (half == 0 && hh == 0 && row_ok) {
    p.lse2[(int64_t)bh * p.Lq + qi] = lse;
    p.delta[(int64_t)bh * p.Lq + qi] = delta;
  }

  // pass 2: dS and dQ = dS K
  f32x16 dqa[FB];
#pragma unroll
  for (int fb = 0; fb < FB; ++fb) dqa[fb] = f32x16{};
  // a row without weight (lse = -inf) subtracts +inf: 2^-inf = 0
  const float lse_w = lse == -INFINITY ? INFINITY : lse;
  stream([&](int t, int buf) {
    f32x16 sa, da;
    tile(buf, sa, da);
    float ds[16];
    auto grads = [&](auto edge_tag) {
      constexpr bool EDGE = decltype(edge_tag)::value;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 32 * t + run_off(i, hh);
        float x = sa[i] * p.c;
        if constexpr (TM) x = masked_logit(p, x, mask_at<T>(p, bh, qi, key));
        float pr = exp2_fast(x - lse_w);
        if constexpr (EDGE) pr = legal(key) ? pr : 0.f;
        ds[i] = pr * (da[i] - delta);
      }
    };
    if (edge(t))
      grads(std::true_type{});
    else
      grads(std::false_type{});
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      Frag8<T> hi, lo;
      split_frag<T>(ds + 8 * kk, hi, lo);
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        const Frag8<T> kb = load_tr_frag<T, D>(ktile(buf), fb, kk, lane);
        dqa[fb] = mma8(hi, kb, dqa[fb]);
        if constexpr (ES == 2) dqa[fb] = mma8(lo, kb, dqa[fb]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  });

  // The two waves of a block add their sums: wave half h finishes the
  // feature blocks fb with fb % 2 == h (with one block, the first wave) and
  // hands the others over, lane l's values in 4 quads of 16 bytes, quad q at
  // float offset 4 (64 q + l). The staged tiles are free: every wave passed
  // pass 2's last barrier after its last read.
  float* const xs = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
    if ((fb & 1) != half) {
      float* o = xs + (wv * SB + (fb >> 1)) * 1024;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(o + 4 * (64 * q + lane)) =
            make_float4(dqa[fb][4 * q], dqa[fb][4 * q + 1], dqa[fb][4 * q + 2], dqa[fb][4 * q + 3]);
    }
  __syncthreads();
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
    if ((fb & 1) == half) {
      const float* o = xs + ((wv ^ 4) * SB + (fb >> 1)) * 1024;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(o + 4 * (64 * q + lane));
        dqa[fb][4 * q] += v.x;
        dqa[fb][4 * q + 1] += v.y;
        dqa[fb][4 * q + 2] += v.z;
        dqa[fb][4 * q + 3] += v.w;
      }
    }

  // dQ: lane holds feature 32 fb + n of rows 8 (i / 4) + 4 hh + i % 4
  T* dq = static_cast<T*>(p.dq) + (int64_t)bh * p.Lq * D;
  bool nonfinite = false;
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
    if ((fb & 1) == half) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = q0 + 8 * (i >> 2) + 4 * hh + (i & 3);
        if (row < p.Lq && 32 * fb + n < D) {
          const T y = (T)(dqa[fb][i] * p.scale);
          dq[(int64_t)row * D + 32 * fb + n] = y;
          nonfinite |= !__builtin_isfinite((float)y);
        }
      }
    }
  const bool empty_row = half == 0 && row_ok && lse == -INFINITY;
  const uint64_t nf = __ballot(nonfinite), em = __ballot(empty_row);
  if (lane == 0) {
    const uint32_t fl = (nf ? F_NONFINITE : 0u) | (em ? F_FULLY_MASKED_ROW : 0u) |
                        (bad ? F_BAD_LENGTH : 0u);
    if (fl) atomicOr(p.flags, fl);
  }
}

// ---- dK and dV per group of 4 key blocks -------------------------------------
// Eight waves, two per 32-key block (K in registers, V in an LDS tile the two
// share). Each step stages two query tiles -- Q and dO rows and the rows'
// statistics -- through LDS, one step ahead as in the dq kernel; the first
// wave of a key block takes the even query tiles and the second the odd ones,
// so a causal group's chain of tiles is half as long. At the end the two
// waves of a block add their dK and dV through LDS, each finishing half of
// the 32-feature blocks. The A operands (Q and dO rows through keymap) are LDS
// reads; the B operands of dV += P^T dO and dK += dS^T Q are transposing reads
// of the same row-major tiles.
// One workgroup per CU (at most 256 registers per lane, 128 KB of LDS at
// D = 128), so the grid runs in rounds; the workgroups of an XCD are dealt
// longest first (xcd_lpt), and a CU whose long group ends early takes a short
// one next.
// Both MFMA blocks run at raised wave priority, as the dq kernel's dQ product.
template <typename T, int D, bool TM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void
bwd_dkv_kernel(const BwdParams p) {
  constexpr int FB = (D + 31) / 32;  // 32-feature blocks of the dK, dV accumulators
  constexpr int SB = (FB + 1) / 2;   // blocks a wave hands to its partner (at most)
  constexpr int ES = sizeof(T);      // element bytes
  constexpr int RS = tile_rs<T, D>();
  constexpr int TB = 32 * RS;        // bytes of one staged 32-row tile
  constexpr int CPR = D * ES / 16;
  constexpr int PPT = 32 * CPR;
  constexpr int PPS = (2 * PPT + 511) / 512;  // pieces per thread and tensor of a step
  // LDS during the tile loop: staged tiles [buffer][tile][Q, dO], the four
  // blocks' V rows, row statistics [buffer][tile][lse x32, Delta x32]; after
  // it, the partial dK, dV handed over: [wave][block][dK, dV], 4 KB each
  constexpr int STAGE = 8 * TB, VT = 4 * TB, STATS = 2 * 128 * 4;
  constexpr int XCH = 8 * SB * 2 * 4096;
  constexpr int LDS = (STAGE + VT + STATS) > XCH ? (STAGE + VT + STATS) : XCH;
  __shared__ __attribute__((aligned(16))) char smem[LDS];
  char* const stg = smem;
  char* const vt = smem + STAGE;
  float* const st = reinterpret_cast<float*>(smem + STAGE + VT);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int kw = wv & 3, half = wv >> 2;
  const int n = lane & 31, hh = lane >> 5;
  const int ngrp = (p.nkblk + 3) / 4;
  int bh = 0, kgp = 0;
  xcd_lpt(p.B * p.H, ngrp, &bh, &kgp);
  const int k0 = (4 * kgp + kw) * 32;  // this wave's key block
  bool bad = false;
  const int kend = bwd_len(p, bh / p.H, &bad);
  const int kj = k0 + n;  // this lane's key (column of S)
  const int64_t qoff = (int64_t)bh * p.Lq * D * ES, koff = (int64_t)bh * p.Lk * D * ES;
  const uint32_t qbytes = (uint32_t)p.Lq * D * ES;
  const auto qrs = make_rsrc(static_cast<const char*>(p.q) + qoff, qbytes);
  const auto grs = make_rsrc(static_cast<const char*>(p.dout) + qoff, qbytes);
  const auto krs = make_rsrc(static_cast<const char*>(p.k) + koff, (uint32_t)kend * D * ES);
  const auto vrs = make_rsrc(static_cast<const char*>(p.v) + koff, (uint32_t)kend * D * ES);
  const float* lse2 = p.lse2 + (int64_t)bh * p.Lq;
  const float* dlt = p.delta + (int64_t)bh * p.Lq;

  Frag8<T> kf[D / 16];
  load_rows<T, D>(krs, kj, hh, kf);
  if (half == 0) {
    // the block's V rows, row-major in its LDS tile (read by both of its
    // waves after the barrier that precedes the tile loop)
    Frag8<T> v0[D / 16];
    load_rows<T, D>(vrs, kj, hh, v0);
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb)
      lds_put_frag<T>(vt + kw * TB + n * RS + (16 * kb + 8 * hh) * ES, v0[kb]);
  }
  f32x16 dka[FB], dva[FB];
#pragma unroll
  for (int fb = 0; fb < FB; ++fb) dka[fb] = dva[fb] = f32x16{};

  // queries before a block's first key see none of its keys (causal); a
  // block past the key length gets zeros. The group streams from its first
  // block's first query tile (an even tile); each wave computes from its own.
  const int k0g = 4 * kgp * 32;
  const int t0 = p.causal ? k0 / 32 : 0;
  const int t0g = p.causal ? k0g / 32 : 0;
  const bool active = k0 < kend;
  const int ntile = (k0g < kend) ? (p.Lq + 31) / 32 : 0;
  const int s0 = t0g / 2, nstep = (ntile + 1) / 2;  // step s stages tiles 2s, 2s + 1
  const bool kcut = k0 + 32 > kend;  // the block straddles the key length

  uint4 rq[PPS], rg[PPS];
  float rs = 0.f;  // thread tid < 128: lse or Delta of row tid % 32 of the step's tile tid / 64
  auto gload = [&](int s) {
#pragma unroll
    for (int i = 0; i < PPS; ++i) {
      const int u = tid + 512 * i;
      if ((2 * PPT) % 512 == 0 || u < 2 * PPT) {
        const int tl = u / PPT, w = u % PPT;
        const uint32_t off = (uint32_t)(32 * (2 * s + tl) + w / CPR) * (D * ES) + (w % CPR) * 16;
        rq[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0));
        rg[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(grs, off, 0, 0));
      }
    }
    if (tid < 128) {  // rows past Lq or fully masked: no weight (+inf) and no Delta
      const int row = 32 * (2 * s + (tid >> 6)) + (tid & 31);
      if ((tid & 32) == 0) {
        const float v = row < p.Lq ? lse2[row] : INFINITY;
        rs = v == -INFINITY ? INFINITY : v;
      } else {
        rs = row < p.Lq ? dlt[row] : 0.f;
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PPS; ++i) {
      const int u = tid + 512 * i;
      if ((2 * PPT) % 512 == 0 || u < 2 * PPT) {
        const int tl = u / PPT, w = u % PPT;
        const int o = (buf * 2 + tl) * 2 * TB + (w / CPR) * RS + (w % CPR) * 16;
        *reinterpret_cast<uint4*>(stg + o) = rq[i];
        *reinterpret_cast<uint4*>(stg + o + TB) = rg[i];
      }
    }
    if (tid < 128) st[buf * 128 + tid] = rs;
  };

  if (nstep > s0) {
    gload(s0);
    lstore(0);
  }
  __syncthreads();
  for (int s = s0; s < nstep; ++s) {
    const int buf = (s - s0) & 1;
    if (s + 1 < nstep) gload(s + 1);
    const int t = 2 * s + half;  // this wave's query tile
    if (active && t >= t0 && t < ntile) {
      const char* qt = stg + (buf * 2 + half) * 2 * TB;  // Q rows; dO rows follow
      const char* gt = qt + TB;
      const float* sr = st + buf * 128 + half * 64;
      const char* vr = vt + kw * TB + n * RS + 8 * hh * ES;
      // S = Q K^T and dP = dO V^T (Q and dO rows through keymap)
      const char* qr = qt + keymap(n) * RS + 8 * hh * ES;
      const char* gr = gt + keymap(n) * RS + 8 * hh * ES;
      __builtin_amdgcn_s_setprio(1);
      f32x16 sa = f32x16{}, da = f32x16{};
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb) {
        const Frag8<T> qa = lds_frag<T>(qr + 16 * kb * ES), ga = lds_frag<T>(gr + 16 * kb * ES);
        const Frag8<T> vb = lds_frag<T>(vr + 16 * kb * ES);
        sa = mma8(qa, kf[kb], sa);
        da = mma8(ga, vb, da);
      }
      __builtin_amdgcn_s_setprio(0);
      // P from the row's log-sum-exp. A row without weight holds +inf (staged
      // so), which gives 2^-inf = 0 without a per-element test; the tests of
      // keys past the length and of the causal diagonal run only on a tile
      // that needs them (a wave-uniform branch). One run of 8 rows at a time:
      // its P and dS are the A operands of one 16-row step of dV += P^T dO
      // and dK += dS^T Q.
      const bool diag = p.causal && t == t0;
      const bool fix = __builtin_amdgcn_readfirstlane((int)(diag || kcut)) != 0;
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float pr[8], ds[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float x = sa[8 * kk + e] * p.c;
          if constexpr (TM)
            x = masked_logit(p, x, mask_at<T>(p, bh, 32 * t + 16 * kk + 8 * hh + e, kj));
          pr[e] = exp2_fast(x - sr[16 * kk + 8 * hh + e]);
        }
        if (fix) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 16 * kk + 8 * hh + e;  // row 32 t + r; key k0 + n after it
            if ((diag && n > r) || kj >= kend) pr[e] = 0.f;
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) ds[e] = pr[e] * (da[8 * kk + e] - sr[32 + 16 * kk + 8 * hh + e]);
        Frag8<T> phi, plo, shi, slo;
        split_frag<T>(pr, phi, plo);
        split_frag<T>(ds, shi, slo);
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) {
          const Frag8<T> gb = load_tr_frag<T, D>(gt, fb, kk, lane);
          dva[fb] = mma8(phi, gb, dva[fb]);
          if constexpr (ES == 2) dva[fb] = mma8(plo, gb, dva[fb]);
          const Frag8<T> qb = load_tr_frag<T, D>(qt, fb, kk, lane);
          dka[fb] = mma8(shi, qb, dka[fb]);
          if constexpr (ES == 2) dka[fb] = mma8(slo, qb, dka[fb]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    }
    if (s + 1 < nstep) lstore(buf ^ 1);  // last read at step s - 1, before its barrier
    __syncthreads();
  }

  // The two waves of a block add their sums: wave half h finishes the
  // feature blocks fb with fb % 2 == h (with one block, the first wave) and
  // hands the others over; lane l's value of a block sits in 4 quads of 16
  // bytes, quad q at float offset 4 (64 q + l). The staged tiles are free:
  // every wave passed the loop's last barrier after its last read.
  float* const xs = reinterpret_cast<float*>(smem);
  auto slot = [&](int w, int j, int which) { return xs + ((w * SB + j) * 2 + which) * 1024; };
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
    if ((fb & 1) != half) {
      float* ok = slot(wv, fb >> 1, 0);
      float* ov = slot(wv, fb >> 1, 1);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        *reinterpret_cast<float4*>(ok + 4 * (64 * q + lane)) =
            make_float4(dka[fb][4 * q], dka[fb][4 * q + 1], dka[fb][4 * q + 2], dka[fb][4 * q + 3]);
        *reinterpret_cast<float4*>(ov + 4 * (64 * q + lane)) =
            make_float4(dva[fb][4 * q], dva[fb][4 * q + 1], dva[fb][4 * q + 2], dva[fb][4 * q + 3]);
      }
    }
  __syncthreads();
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
    if ((fb & 1) == half) {
      const float* ik = slot(wv ^ 4, fb >> 1, 0);
      const float* iv = slot(wv ^ 4, fb >> 1, 1);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 a = *reinterpret_cast<const float4*>(ik + 4 * (64 * q + lane));
        const float4 b = *reinterpret_cast<const float4*>(iv + 4 * (64 * q + lane));
        dka[fb][4 * q] += a.x;
        dka[fb][4 * q + 1] += a.y;
        dka[fb][4 * q + 2] += a.z;
        dka[fb][4 * q + 3] += a.w;
        dva[fb][4 * q] += b.x;
        dva[fb][4 * q + 1] += b.y;
        dva[fb][4 * q + 2] += b.z;
        dva[fb][4 * q + 3] += b.w;
      }
    }

  // lane holds feature 32 fb + n of keys 8 (i / 4) + 4 hh + i % 4
  T* dk = static_cast<T*>(p.dk) + (int64_t)bh * p.Lk * D;
  T* dv = static_cast<T*>(p.dv) + (int64_t)bh * p.Lk * D;
  bool nonfinite = false;
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
    if ((fb & 1) == half) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 8 * (i >> 2) + 4 * hh + (i & 3);
        if (key < p.Lk && 32 * fb + n < D) {
          const T a = (T)(dka[fb][i] * p.scale), b = (T)dva[fb][i];
          dk[(int64_t)key * D + 32 * fb + n] = a;
          dv[(int64_t)key * D + 32 * fb + n] = b;
          nonfinite |= !__builtin_isfinite((float)a) || !__builtin_isfinite((float)b);
        }
      }
    }
  if (__ballot(nonfinite) && lane == 0) atomicOr(p.flags, F_NONFINITE);
}

template <typename T, int D, bool TM>
hipError_t launch_bwd_m(const BwdParams& p, hipStream_t stream) {
  const long long gq = (long long)p.B * p.H * ((p.nqblk + 3) / 4);  // groups of 4 query blocks
  const long long gk = (long long)p.B * p.H * ((p.nkblk + 3) / 4);  // groups of 4 key blocks
  if (gq > 0x7fffffffLL || gk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (gq > 0)
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, TM>), dim3((unsigned)gq), dim3(512), 0, stream, p);
  if (gk > 0)
    hipLaunchKernelGGL((bwd_dkv_kernel<T, D, TM>), dim3((unsigned)gk), dim3(512), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t stream) {
  return p.mask ? launch_bwd_m<T, D, true>(p, stream) : launch_bwd_m<T, D, false>(p, stream);
}

}  // namespace mha
