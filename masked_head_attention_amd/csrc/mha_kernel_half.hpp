// mha_kernel_half.hpp -- fused masked multi-head attention forward for gfx950
// (CDNA4), float16 / bfloat16 variant.
//
// Sources (web pages, cited by title and section):
//   [MMHA]  "masked multi head attention" CUDA implementation notes (2kiu.com/news/6063113)
//   [MAX]   "Why attention must compute the max first" (gsyq.cn/news/340375)
//   [LNXA]  "How to fuse cross-attention and layer-norm into a single CUDA kernel?"
//           (cms365.cn question page)
//
// Same method as the float32 kernel (mha_kernel_f32.hpp) -- S = scale*QK^T,
// mask before the softmax, online softmax, O += P V with S/P in registers
// [MAX 2.3, 2.4; MMHA 2] -- arranged for throughput on 16-bit inputs:
//   * K and V tiles go straight from HBM into LDS with buffer_load ... lds
//     (16 bytes per lane, no register staging). Rows past Lk come back as
//     zeros from the buffer's range check, so there are no guards or
//     branches on the loads. The XOR swizzle is applied by choosing which
//     global chunk each lane fetches, since the LDS side of these loads is
//     lane-ordered;
//   * V stays row-major in LDS and is read transposed with
//     ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
//     (i & 3) of the 8 bytes addressed by lane 4j + (i >> 2) in slot j. With
//     the addresses chosen below, each lane gets 4 consecutive keys at its own
//     feature index -- the k-slots of the A operand of O^T = V^T P^T;
//   * a tile whose keys sit strictly inside every row's legal range runs a
//     path with no per-element mask tests; only tiles that straddle the
//     causal diagonal, the padding length or Lk pay for them;
//   * the running maximum is raised only when a row's new maximum exceeds the
//     current one by more than 2^8 in probability (8 in log2 units), so the
//     O rescale is rare; weights of up to 2^8 stay exact in fp32 and are
//     normalised by the same running sum [MAX 2.3];
//   * up to two workgroups per CU (launch bound: 2 waves per SIMD) so one
//     wave's softmax overlaps another's MFMAs;
//   * causal masks run two key splits per query group (8 waves), which halves
//     the heaviest query block's serial chain; the splits' (m, l, O) states
//     merge through LDS at the end;
//   * bfloat16 V is rewritten once per tile into a float16 copy in LDS, so P V
//     runs as one float16 MFMA (a tile with a value beyond the float16 range
//     falls back to P split into two bfloat16 parts);
//   * where P is float16, the row sum adds the packed weights the MFMA
//     consumes (v_dot2), so numerator and normaliser see the same values.
#pragma once

#include "mha_common.hpp"

namespace mha {

typedef __fp16 lds_f16x4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __bf16 lds_bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));

template <typename T>
__device__ inline uint2 lds_read_tr(const char* p);
template <>
__device__ inline uint2 lds_read_tr<_Float16>(const char* p) {
  return __builtin_bit_cast(uint2,
                            __builtin_amdgcn_ds_read_tr16_b64_v4f16(MHA_LDS_PTR(lds_f16x4, p)));
}
template <>
__device__ inline uint2 lds_read_tr<__bf16>(const char* p) {
  return __builtin_bit_cast(uint2,
                            __builtin_amdgcn_ds_read_tr16_b64_v4bf16(MHA_LDS_PTR(lds_bf16x4, p)));
}

// Sum of the eight float16 values in w, added to acc in float32 (v_dot2 with
// (1, 1): each product is exact).
__device__ inline float row_sum_f16x8(const uint4 w, float acc) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w.x), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w.y), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w.z), one, acc, false);
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w.w), one, acc, false);
}

// LDS swizzles, in 16-byte chunks (16 chunks = 64 banks x 4 bytes). A K
// operand read has 16 lanes hitting 16 different rows at one logical chunk;
// a transposed V read has 32 lanes hitting 4 consecutive rows x 4 chunks.
// Both place every lane of such a phase in a distinct chunk slot mod 16.
template <int CPR>
__device__ inline int swz_k16(int row) {
  return CPR >= 16 ? (row & 15) : ((row / (16 / CPR)) & (CPR - 1));
}
template <int CPR>
__device__ inline int swz_v16(int row) {
  // rows r..r+3 (r % 4 == 0), chunks c..c+3 (c % 4 == 0)
  if constexpr (CPR >= 16) return 4 * (row & 3);
  else if constexpr (CPR == 8) return 4 * ((row >> 1) & 1);
  else return 0;
}

// Float16 copies of K and V for bfloat16 pre-LN calls (a workspace): the
// copy kernel below writes them with one flag per sub-range of a head, and
// the attention kernel runs twice over the same grid.
//   mode 0: no copies (every other call);
//   mode 1: p.k and p.v are the float16 copies (KV16 instantiation): the
//           launch serves the heads whose flags are all clear, with each
//           token's LayerNorm statistics read from `stats`;
//   mode 2: p.k and p.v are the bfloat16 tensors: the launch serves the heads
//           with a flag set, rewriting tiles in LDS as without a workspace.
// flags[(b*H + h)*nsub + s] != 0: sub-range s of head (b, h) holds a value of
// magnitude above 65504, which float16 cannot hold.
struct KvPre {
  const int* flags;
  int nsub;
  int mode;
  const float2* stats;  // mode 1: [B*Lq] (mean, 1/sqrt(var + eps)) of each token
};

struct KvConvParams {
  const void* k;   // [B,H,Lk,D] bfloat16
  const void* v;
  void* k16;       // [B,H,Lk,D] float16
  void* v16;
  int* flags;      // [B*H, nsub]
  int64_t n16;     // 16-byte chunks of one head's K (or V): Lk*D/8
  int nsub;        // workgroups per head
  int nstat;       // workgroups computing statistics (first); the rest copy, B*H*nsub
  const void* x;   // [B*Lq, F] bfloat16 tokens
  float2* stats;   // [B*Lq] (mean, 1/sqrt(var + eps))
  int64_t ntok;    // B*Lq
  int F;           // H*D features per token
  float eps;
};

// The first nstat workgroups: the LayerNorm statistics of the tokens [LNXA
// answer step 2], mean then mean squared deviation over the F features in
// float32. The others: one per sub-range of a head's K and V, bfloat16 ->
// float32 -> float16 (nearest even: the rewrite the attention kernel applies
// to its LDS tiles, so both give the same float16 values). Sources are read
// once, with the non-temporal hint; the copies are read next by the attention
// kernel. The statistics come first in the grid so that their loads overlap
// the copy's.
template <typename T>
__global__ __launch_bounds__(256) void mha_half_kernel_kv16_copy(const KvConvParams c) {
  if ((int)blockIdx.x < c.nstat) {
    // 16 lanes per token, 4 tokens per wave and pass; up to 128 chunks of 16
    // bytes per token (F <= 1024) stay in registers, all loads in flight at
    // once, and both sums run from them; longer rows are read twice
    constexpr int XC = 8;
    const int lane = threadIdx.x & 63, g16 = lane >> 4, l16 = lane & 15;
    const int nch = c.F / 8;
    const float invF = 1.0f / (float)c.F;
    T* tag = nullptr;
    const int64_t step = (int64_t)c.nstat * 16;  // tokens per pass of the whole grid
    for (int64_t t0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4; t0 < c.ntok; t0 += step) {
      const int64_t tok = t0 + g16;
      const bool valid = tok < c.ntok;
      const char* xr = static_cast<const char*>(c.x) +
                       (valid ? tok : 0) * (int64_t)c.F * (int64_t)sizeof(T);
      float sum = 0.f, v2 = 0.f;
      if (nch <= 16 * XC) {
        uint4 u[XC];
#pragma unroll
        for (int j = 0; j < XC; ++j) {
          const int ch = l16 + 16 * j;
          u[j] = (valid && ch < nch) ? *reinterpret_cast<const uint4*>(xr + 16 * ch)
                                     : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int j = 0; j < XC; ++j) {
          const uint32_t w[4] = {u[j].x, u[j].y, u[j].z, u[j].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) sum += lo_f(w[i], tag) + hi_f(w[i], tag);
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) sum += __shfl_xor(sum, o, 64);
        const float mean = sum * invF;
#pragma unroll
        for (int j = 0; j < XC; ++j) {
          if (l16 + 16 * j >= nch) continue;
          const uint32_t w[4] = {u[j].x, u[j].y, u[j].z, u[j].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float a0 = lo_f(w[i], tag) - mean, a1 = hi_f(w[i], tag) - mean;
            v2 += a0 * a0 + a1 * a1;
          }
        }
        sum = mean;
      } else {
        for (int ch = l16; ch < nch; ch += 16) {
          if (!valid) break;
          const uint4 u = *reinterpret_cast<const uint4*>(xr + 16 * ch);
          const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) sum += lo_f(w[i], tag) + hi_f(w[i], tag);
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) sum += __shfl_xor(sum, o, 64);
        const float mean = sum * invF;
        for (int ch = l16; ch < nch; ch += 16) {
          if (!valid) break;
          const uint4 u = *reinterpret_cast<const uint4*>(xr + 16 * ch);
          const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float a0 = lo_f(w[i], tag) - mean, a1 = hi_f(w[i], tag) - mean;
            v2 += a0 * a0 + a1 * a1;
          }
        }
        sum = mean;
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) v2 += __shfl_xor(v2, o, 64);
      if (valid && l16 == 0) c.stats[tok] = make_float2(sum, 1.0f / sqrtf(v2 * invF + c.eps));
    }
    return;
  }
  const int64_t blk = (int64_t)blockIdx.x - c.nstat;  // a copy workgroup
  const int64_t bh = blk / c.nsub;
  const int s = (int)(blk % c.nsub);
  const int64_t lo = c.n16 * s / c.nsub, hi = c.n16 * (s + 1) / c.nsub;
  bool big = false;
  T* tb = nullptr;
  _Float16* th = nullptr;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const char* src = static_cast<const char*>(m ? c.v : c.k) + bh * c.n16 * 16;
    char* dst = static_cast<char*>(m ? c.v16 : c.k16) + bh * c.n16 * 16;
    for (int64_t i = lo + threadIdx.x; i < hi; i += 256) {
      const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + 16 * i));
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
      uint32_t r[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = lo_f(w[j], tb), b = hi_f(w[j], tb);
        big |= fmaxf(fabsf(a), fabsf(b)) > 65504.f;
        r[j] = pack2(a, b, th);
      }
      *reinterpret_cast<uint4*>(dst + 16 * i) = make_uint4(r[0], r[1], r[2], r[3]);
    }
  }
  const int any = __syncthreads_or(big ? 1 : 0);
  if (threadIdx.x == 0) c.flags[blk] = any ? 1 : 0;
}

// NK = 1: 4 waves, each 32 query rows against every key tile.
// NK = 2 (causal masks): 8 waves, two per query group, taking alternate key
// tiles; the heaviest query block's serial chain halves and one workgroup
// fills a CU, so the heaviest-first launch order balances the causal
// triangle. The two partial (m, l, O) states merge through LDS.
// AM: the mask tensor's form -- 0 none, 1 rows of 16-byte multiples (read as
// 16-byte vectors), 2 any other row length (read element by element). The
// two read paths are separate instantiations so that the element-wise one's
// scalar loads and waits never enter the vector kernel's schedule.
// KV16: the float16 copies of a bfloat16 pre-LN call (mode 1 above).
template <typename T, int D, int AM, bool PRENORM, int NK, bool KV16 = false>
__global__ __launch_bounds__((256 * NK), 2) void mha_half_kernel(const Params p, const KvPre kp) {
  static_assert(sizeof(T) == 2, "16-bit element types only");
  static_assert(AM >= 0 && AM <= 2, "mask form");
  static_assert(!KV16 || (PRENORM && AM == 0 && std::is_same<T, __bf16>::value),
                "float16 K/V copies serve bfloat16 pre-LN calls without a mask tensor");
  constexpr bool ADD = AM != 0;
  constexpr int E = 2;
  constexpr int NQ = 4, NW = NQ * NK, NT = 64 * NW, BM = 128, BN = 64, NB32 = 2;
  constexpr int NC = D / 16;                  // 16-feature slices of QK^T
  constexpr int DP = D < 32 ? 32 : D;         // O^T rows, padded to 32
  constexpr int ND = DP / 32;
  constexpr int CPR = D / 8;                  // 16-byte chunks per K/V row
  constexpr int RB = D * E;                   // bytes per K/V row
  constexpr int TILE_BYTES = BN * RB;
  constexpr int SPLIT_BYTES = 2 * TILE_BYTES; // K tile then V tile of one key split
  constexpr int BUF_BYTES = NK * SPLIT_BYTES;
  constexpr int NCHUNK = NK * BN * CPR;       // 16-byte chunks per matrix per buffer
  constexpr int NLD = (NCHUNK + NT - 1) / NT;
  // two key splits (NK = 2): each wave finishes half of the 32-feature O
  // blocks and hands the other half, with its (m, l), to its partner
  constexpr int HALF = ND / 2;
  constexpr bool SPLIT_FINISH = NK == 2 && ND >= 2;
  constexpr int PART_BYTES = 64 * 8 + HALF * 4 * 64 * 16;  // (m, l) + HALF blocks of 16 floats, per lane
  constexpr int MERGE_BYTES = SPLIT_FINISH ? NQ * NK * PART_BYTES
                              : NK > 1 ? NQ * (NK - 1) * 64 * (ND * 16 + 2) * 4 : 0;
  constexpr int TILE_REGION = 2 * BUF_BYTES > MERGE_BYTES ? 2 * BUF_BYTES : MERGE_BYTES;
  constexpr int STAT_BYTES = PRENORM ? NQ * 32 * 8 : 16;
  constexpr bool SPLIT_P = std::is_same<T, __bf16>::value;
  // bfloat16: each landed V tile is rewritten once into float16 (exact for
  // |v| <= 65280; bf16 has 8 significant bits, f16 11), so P V runs as one
  // f16 MFMA with P in f16 instead of two bf16 MFMAs with P split into hi + lo.
  // A tile holding a larger finite value falls back to the split. Only where
  // the extra LDS keeps the occupancy (2 workgroups per CU for NK = 1).
  constexpr int VC_BYTES = 2 * NK * TILE_BYTES;
  constexpr bool CONV_V = SPLIT_P && !KV16 && (TILE_REGION + VC_BYTES + STAT_BYTES + 16) <= (NK == 1 ? 80 : 160) * 1024;
  constexpr float LOG2E = 1.4426950408889634f;
  constexpr float RESCALE_GAP = 8.0f;         // log2 units
  constexpr bool LS = PRENORM;                // scores leave the MFMAs in log2 units, less m
  // Pre-LN: the normalised query is rounded once, to float16 (11 significant
  // bits), whatever the call dtype; bfloat16 K tiles are rewritten into
  // float16 in place once landed, so Q K^T is one float16 MFMA per 16
  // features. A tile holding a finite |k| > 65504 is re-loaded as bfloat16
  // and multiplied by the same float16 query split exactly into two
  // bfloat16 parts.
  constexpr bool CONV_K = PRENORM && SPLIT_P && !KV16;
  using QT = std::conditional_t<PRENORM, _Float16, T>;  // type of the Q fragments
  static_assert(NCHUNK % 64 == 0, "tile chunks must fill whole waves");

  __shared__ __attribute__((aligned(16))) char smem[TILE_REGION + (CONV_V ? VC_BYTES : 0) + STAT_BYTES + 16];
  char* const vc_lds = smem + TILE_REGION;                              // converted V, [buf][split]
  char* const stat_lds = smem + TILE_REGION + (CONV_V ? VC_BYTES : 0);
  int* const vflag = reinterpret_cast<int*>(stat_lds + STAT_BYTES);    // [buf]: tag of a tile that fell back
  int* const kflag = vflag + 2;                                          // [buf]: same for K

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = (tid >> 6) % NQ, ks = (tid >> 6) / NQ;  // query group, key split
  const int n = lane & 31, hh = lane >> 5;

  // Workgroup -> work item.
  //  * causal: every (b, head) of the heaviest query block first, the
  //    lightest last, in dispatch order (work per block grows with its index);
  //  * otherwise: consecutive workgroup ids go to different XCDs (8 of them,
  //    each with its own L2), so ids are remapped to put the query blocks of
  //    one (b, head group) -- which read the same K/V (and, for pre-LN, the
  //    same x rows across head groups) -- on one XCD.
  int b, hg, qblk;
  {
    const int G = (int)gridDim.x;
    const int bid = (int)blockIdx.x;
    const int ngrp = PRENORM ? p.H / p.hg : p.H;
    int grp;
    if (p.kind & K_CAUSAL) {
      grp = bid % (p.B * ngrp);
      qblk = p.nqblk - 1 - bid / (p.B * ngrp);
    } else {
      const int L = (G % 8 == 0) ? (bid & 7) * (G >> 3) + (bid >> 3) : bid;
      qblk = L % p.nqblk;
      grp = L / p.nqblk;
    }
    b = grp / ngrp;
    hg = grp % ngrp;
  }
  // the heads of the group this launch serves (bit hl), from the copy flags
  const int nheads = PRENORM ? p.hg : 1;
  unsigned serve = (1u << nheads) - 1u;
  if (kp.mode != 0) {
    serve = 0u;
    for (int hl = 0; hl < nheads; ++hl) {
      const int* f = kp.flags + ((int64_t)b * p.H + (PRENORM ? hg * p.hg + hl : hg)) * kp.nsub;
      int any = 0;
      for (int s2 = 0; s2 < kp.nsub; ++s2) any |= f[s2];
      if ((any != 0) == (kp.mode == 2)) serve |= 1u << hl;
    }
    if (serve == 0u) return;  // the other launch serves every head of the group
  }
  const int Lq = p.Lq, Lk = p.Lk, H = p.H;
  const int q0 = qblk * BM;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + n;
  const bool row_ok = qi < Lq;
  const bool wave_active = qw0 < Lq;
  const bool causal = (p.kind & K_CAUSAL) != 0;

  int kpad = Lk;
  if (p.kind & K_PADDING) {
    const int L = p.lens[b];
    kpad = L < 0 ? 0 : (L > Lk ? Lk : L);
    if ((L < 0 || L > Lk) && hg == 0 && qblk == 0 && tid == 0) atomicOr(p.flags, F_BAD_LENGTH);
  }
  int kend_w = kpad;
  if (causal) kend_w = min(kend_w, min(qw0 + 31, Lq - 1) + 1);
  if (!wave_active) kend_w = 0;
  int kend_g = kpad;
  if (causal) kend_g = min(kend_g, min(q0 + BM - 1, Lq - 1) + 1);
  const int ntiles = (kend_g + NK * BN - 1) / (NK * BN);

  // ---- pre-LN: token statistics, once per workgroup for all its heads ----
  float2 ms = make_float2(0.f, 0.f);
  if constexpr (KV16) {
    // statistics computed by the copy kernel
    if (row_ok) ms = kp.stats[(int64_t)b * Lq + qi];
  } else if constexpr (PRENORM) {
    // token statistics over F = H*D features [LNXA answer step 2]: 16 lanes per
    // token, 4 tokens per pass, mean then mean squared deviation
    const int F = H * D;
    const int nch = F / 8;
    const int g16 = lane >> 4, l16 = lane & 15;
    float2* st = reinterpret_cast<float2*>(stat_lds) + wave * 32;
    // A lane's chunks of one token are ch = l16, l16 + 16, ... When they fit
    // in XC registers (F <= 128 * XC), the loads of two 4-token passes are
    // issued together and both sums run from registers; otherwise each sum
    // streams the row (one load in flight at a time, the row read twice).
    constexpr int XC = 8;
    const float invF = 1.0f / (float)F;
    auto finish = [&](float s, float v2, int r) {  // s, v2: this lane's partial sums of token r
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) v2 += __shfl_xor(v2, o, 64);
      if (l16 == 0) st[r] = make_float2(s, 1.0f / sqrtf(v2 * invF + p.eps));
    };
    T* tag = nullptr;
    if (nch <= 16 * XC) {
      for (int r0 = 0; r0 < (ks == 0 ? 32 : 0); r0 += 8) {
        uint4 u[2][XC];
        bool valid[2];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const int row = qw0 + r0 + 4 * pp + g16;
          valid[pp] = row < Lq;
          const char* xr =
              (const char*)p.x + ((int64_t)b * Lq + (valid[pp] ? row : 0)) * (int64_t)F * E;
#pragma unroll
          for (int i = 0; i < XC; ++i) {
            const int ch = l16 + 16 * i;
            u[pp][i] = (valid[pp] && ch < nch) ? *reinterpret_cast<const uint4*>(xr + 16 * ch)
                                               : make_uint4(0u, 0u, 0u, 0u);  // absent: adds 0
          }
        }
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          float s = 0.f, v2 = 0.f;
#pragma unroll
          for (int i = 0; i < XC; ++i) {
            const uint32_t w[4] = {u[pp][i].x, u[pp][i].y, u[pp][i].z, u[pp][i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) s += lo_f(w[j], tag) + hi_f(w[j], tag);
          }
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o, 64);
          const float mean = s * invF;
#pragma unroll
          for (int i = 0; i < XC; ++i) {
            if (!(valid[pp] && l16 + 16 * i < nch)) continue;
            const uint32_t w[4] = {u[pp][i].x, u[pp][i].y, u[pp][i].z, u[pp][i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float a0 = lo_f(w[j], tag) - mean, a1 = hi_f(w[j], tag) - mean;
              v2 += a0 * a0 + a1 * a1;
            }
          }
          finish(mean, v2, r0 + 4 * pp + g16);
        }
      }
    } else {
      for (int r0 = 0; r0 < (ks == 0 ? 32 : 0); r0 += 4) {
        const int row = qw0 + r0 + g16;
        const bool valid = row < Lq;
        const char* xr = (const char*)p.x + ((int64_t)b * Lq + (valid ? row : 0)) * (int64_t)F * E;
        float s = 0.f, v2 = 0.f;
        if (valid) {
          for (int ch = l16; ch < nch; ch += 16) {
            const uint4 u = *reinterpret_cast<const uint4*>(xr + 16 * ch);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) s += lo_f(w[i], tag) + hi_f(w[i], tag);
          }
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o, 64);
        const float mean = s * invF;
        if (valid) {
          for (int ch = l16; ch < nch; ch += 16) {
            const uint4 u = *reinterpret_cast<const uint4*>(xr + 16 * ch);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float a0 = lo_f(w[i], tag) - mean, a1 = hi_f(w[i], tag) - mean;
              v2 += a0 * a0 + a1 * a1;
            }
          }
        }
        finish(mean, v2, r0 + g16);
      }
    }
    __syncthreads();
    ms = st[n];
  }

  // ---- per-lane constants ----
  const float c = p.c;
  int krow_off[NB32], ksw[NB32];
#pragma unroll
  for (int blk = 0; blk < NB32; ++blk) {
    const int row = blk * 32 + keymap(n);
    krow_off[blk] = row * RB;
    ksw[blk] = swz_k16<CPR>(row);
  }
  // transposed V reads: lane = 16*G + 4*j + r; key = blk*32 + 16*tt + 8*(G>>1) + 4*t + j,
  // feature = 32*db + 16*(G&1) + 8*(r&1) + 4*(r>>1) (the keymap order of the O^T rows)
  const int vG = lane >> 4, vj = (lane >> 2) & 3, vr = lane & 3;
  const int vkey0 = 8 * (vG >> 1) + vj;
  const int vfeat0 = 16 * (vG & 1) + 8 * (vr & 1) + 4 * (vr >> 1);

  for (int hl = 0; hl < nheads; ++hl) {
  if (!((serve >> hl) & 1u)) continue;
  const bool first_head = (serve & ((1u << hl) - 1u)) == 0u;  // no earlier head served
  const int h = PRENORM ? hg * p.hg + hl : hg;
  const int64_t bh = (int64_t)b * H + h;

  // ---- Q fragments: Q[qi][16c + 8hh + j] (B operand of S^T = K Q^T) ----
  // Pre-LN: the normalised query [LNXA answer step 2] is formed in fp32,
  // multiplied by scale * log2(e) (so the scores come out of the MFMAs in
  // log2 units) and rounded once to float16, whose 11 significant bits keep
  // it within a small part of the tolerance for either call dtype; bfloat16
  // (8 bits) would not.
  Frag8<QT> qf[NC];
  if constexpr (!PRENORM) {
    const char* qrow = (const char*)p.q + ((bh * Lq + (row_ok ? qi : 0)) * D) * E;
#pragma unroll
    for (int c2 = 0; c2 < NC; ++c2)
      qf[c2] = row_ok ? ld_global8<T>(qrow + (16 * c2 + 8 * hh) * E) : zero8<T>();
  } else {
    const int F = H * D;
    const char* xrow = (const char*)p.x + (((int64_t)b * Lq + (row_ok ? qi : 0)) * F + h * D) * E;
    const char* grow = (const char*)p.gamma + (int64_t)h * D * E;
    const char* brow = (const char*)p.beta + (int64_t)h * D * E;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      const int off = (16 * cc + 8 * hh) * E;
      if (!row_ok) { qf[cc] = zero8<QT>(); continue; }
      float xv[8], gv[8], bv[8], qv[8];
      unpack8(ld_global8<T>(xrow + off), xv);
      unpack8(ld_global8<T>(grow + off), gv);
      unpack8(ld_global8<T>(brow + off), bv);
#pragma unroll
      for (int j = 0; j < 8; ++j) qv[j] = ((xv[j] - ms.x) * ms.y * gv[j] + bv[j]) * c;
      qf[cc] = pack8<QT>(qv);
    }
  }

  // ---- K/V tiles: HBM -> LDS directly. The buffers end at the padding
  // length (Lk without PADDING): key rows past a sequence's length are never
  // fetched and read as zeros, so whatever that memory holds cannot reach a
  // legal output [MMHA 3.1: keys past the length do not take part] ----
  const __amdgpu_buffer_rsrc_t krs =
      make_rsrc((const char*)p.k + bh * (int64_t)Lk * RB, (uint32_t)((int64_t)kpad * RB));
  const __amdgpu_buffer_rsrc_t vrs =
      make_rsrc((const char*)p.v + bh * (int64_t)Lk * RB, (uint32_t)((int64_t)kpad * RB));
  const int wid = tid >> 6;  // wave index in the workgroup
  // only_k: the K chunks alone (a K tile fetched again)
  auto issue_tile = [&](int kt0, int buf, bool only_k) {
#pragma unroll
    for (int it = 0; it < NLD; ++it) {
      const int u0 = it * NT + wid * 64;
      if (NCHUNK % NT != 0 && u0 >= NCHUNK) break;  // whole waves only
      const int sp = u0 / (BN * CPR);               // key split of this wave's chunks
      const int u1 = u0 - sp * (BN * CPR);
      char* kl = smem + buf * BUF_BYTES + sp * SPLIT_BYTES;
      char* vl = kl + TILE_BYTES;
      const int u = u1 + lane;
      const int row = u / CPR, phys = u % CPR;
      const uint32_t goff = (uint32_t)(kt0 + sp * BN + row) * RB;
      const int lck = phys ^ swz_k16<CPR>(row);
      const int lcv = phys ^ swz_v16<CPR>(row);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, MHA_LDS_PTR(void, kl + 16 * u1), 16,
                                               goff + 16 * lck, 0, 0, 0);
      if (!only_k)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, MHA_LDS_PTR(void, vl + 16 * u1), 16,
                                                 goff + 16 * lcv, 0, 0, 0);
    }
  };

  // additive mask: raw 16-byte groups for this lane's 2 x NB32 key runs.
  // One buffer per wave, based at its first query row (64-bit arithmetic), so
  // 32-bit offsets only span the wave's 32 rows; rows past Lq fall outside it
  const char* addrow = nullptr;
  __amdgpu_buffer_rsrc_t ars;
  uint32_t arow_off = 0;
  if constexpr (ADD) {
    // [B,1,Lq,Lk] shared by the heads, or one [Lq,Lk] slab per head
    const int64_t slab = (p.kind & K_PER_HEAD) ? (int64_t)b * H + h : (int64_t)b;
    const char* abase = (const char*)p.add + slab * Lq * (int64_t)Lk * E;
    addrow = abase + (int64_t)(row_ok ? qi : 0) * Lk * E;
    // the wave index comes from the thread id, so the compiler cannot see that
    // qw0 is the same in every lane; a descriptor built from it would sit in
    // vector registers and every load through it would loop over lanes
    const int qwu = __builtin_amdgcn_readfirstlane(qw0);
    const int wrows = Lq - qwu < 0 ? 0 : (Lq - qwu > 32 ? 32 : Lq - qwu);
    const int wbytes = __builtin_amdgcn_readfirstlane(wrows * Lk * E);
    ars = make_rsrc(abase + (int64_t)qwu * Lk * E, (uint32_t)wbytes);
    arow_off = (uint32_t)n * (uint32_t)Lk * E;
  }
  uint4 am_raw[NB32][2], am_nxt[NB32][2];
  auto load_mask = [&](int kt0, uint4 (&dst)[NB32][2]) {
#pragma unroll
    for (int blk = 0; blk < NB32; ++blk)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int key0 = kt0 + blk * 32 + 16 * g + 8 * hh;
        if constexpr (AM == 1) {
          dst[blk][g] = __builtin_bit_cast(
              uint4, __builtin_amdgcn_raw_buffer_load_b128(ars, arow_off + (uint32_t)key0 * E, 0, 0));
        } else {
          uint32_t w[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int k0 = key0 + 2 * jj;
            const uint32_t lo = (row_ok && k0 < Lk) ? reinterpret_cast<const uint16_t*>(addrow)[k0] : 0u;
            const uint32_t hi =
                (row_ok && k0 + 1 < Lk) ? reinterpret_cast<const uint16_t*>(addrow)[k0 + 1] : 0u;
            w[jj] = lo | (hi << 16);
          }
          dst[blk][g] = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
  };

  // a keep-mask (0 masks a key) as the additive form the tile code reads:
  // +-0 -> -inf, anything else -> +0
  auto to_additive = [&](uint4 (&m)[NB32][2]) {
    constexpr uint16_t NEG = std::is_same<T, __bf16>::value ? 0xFF80 : 0xFC00;
#pragma unroll
    for (int blk = 0; blk < NB32; ++blk)
#pragma unroll
      for (int g = 0; g < 2; ++g) m[blk][g] = keep_to_additive(m[blk][g], NEG);
  };

  // bf16 -> f16 rewrite of the V tile in buffer b (all key splits), same
  // swizzled layout; a finite |v| > 65504 marks the tile with `tag`
  auto convert_v = [&](int b, int tag) {
    bool big = false;
#pragma unroll
    for (int it = 0; it < NLD; ++it) {
      const int u = it * NT + tid;
      if (NCHUNK % NT != 0 && u >= NCHUNK) break;
      const int sp = u / (BN * CPR), u1 = u - sp * (BN * CPR);
      const uint4 x = lds_load16(smem + b * BUF_BYTES + sp * SPLIT_BYTES + TILE_BYTES + 16 * u1);
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
      uint32_t r[4];
      __bf16* tb = nullptr;
      _Float16* th = nullptr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = lo_f(w[i], tb), c2 = hi_f(w[i], tb);
        big |= fmaxf(fabsf(a), fabsf(c2)) > 65504.f;
        r[i] = pack2(a, c2, th);
      }
      *reinterpret_cast<uint4*>(vc_lds + (b * NK + sp) * TILE_BYTES + 16 * u1) =
          make_uint4(r[0], r[1], r[2], r[3]);
    }
    if (__ballot(big) != 0 && lane == 0) vflag[b] = tag;
  };

  // bf16 -> f16 rewrite in place of the K tile in buffer b (pre-LN): each
  // thread rewrites the chunks it loaded itself; a finite |k| > 65504 marks
  // the tile with `tag`
  auto convert_k = [&](int b, int tag) {
    bool big = false;
#pragma unroll
    for (int it = 0; it < NLD; ++it) {
      const int u = it * NT + tid;
      if (NCHUNK % NT != 0 && u >= NCHUNK) break;
      const int sp = u / (BN * CPR), u1 = u - sp * (BN * CPR);
      char* const a = smem + b * BUF_BYTES + sp * SPLIT_BYTES + 16 * u1;
      const uint4 x = lds_load16(a);
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
      uint32_t r[4];
      __bf16* tb = nullptr;
      _Float16* th = nullptr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a0 = lo_f(w[i], tb), a1 = hi_f(w[i], tb);
        big |= fmaxf(fabsf(a0), fabsf(a1)) > 65504.f;
        r[i] = pack2(a0, a1, th);
      }
      *reinterpret_cast<uint4*>(a) = make_uint4(r[0], r[1], r[2], r[3]);
    }
    if (__ballot(big) != 0 && lane == 0) kflag[b] = tag;
  };

  f32x16 o[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  int ncomp = 0;

  if (ntiles > 0) {
    issue_tile(0, 0, false);
    if constexpr (ADD) {
      load_mask(ks * BN, am_raw);
      if (p.kind & K_KEEP) to_additive(am_raw);
    }
    if constexpr (CONV_V || CONV_K) {
      if (first_head && tid < 4) vflag[tid] = -1;  // vflag[0..1], kflag[0..1]
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's loads have landed
    __syncthreads();
    if constexpr (CONV_V) {
      convert_v(0, hl << 16);
      __syncthreads();
    }
  }

  for (int t = 0; t < ntiles; ++t) {
    const int kt0 = t * NK * BN;
    const int buf = t & 1;
    if (t + 1 < ntiles) {
      issue_tile(kt0 + NK * BN, buf ^ 1, false);
      if constexpr (ADD) load_mask(kt0 + NK * BN + ks * BN, am_nxt);
    }
    const char* kl = smem + buf * BUF_BYTES + ks * SPLIT_BYTES;
    const char* vl = kl + TILE_BYTES;
    const char* vcl = KV16 ? vl : vc_lds + (buf * NK + ks) * TILE_BYTES;  // float16 V
    const bool vconv = CONV_V && vflag[buf] != ((hl << 16) | t);  // f16 copy of V is usable
    // K tiles stay bfloat16 (kbf): tile 0, which the rewrite at the end of a
    // tile never reaches (a second rewrite site, before the loop, costs ~40
    // registers), and a tile that did not fit float16, fetched again (the
    // wait also covers the next tile's loads; rare)
    bool kbf = false;
    if constexpr (CONV_K) {
      if (t > 0 && kflag[buf] == ((hl << 16) | t)) {
        issue_tile(kt0, buf, true);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        kbf = true;
      }
      kbf |= t == 0;
    }
    const int kb0 = kt0 + ks * BN;  // this wave's 64 keys
    bool comp = kb0 < kend_w;
    const bool edge = (kb0 + BN > kpad) || (causal && kb0 + BN - 1 > qw0);

    // additive mask, masked entries -inf [MMHA 1: -inf before normalisation].
    // Interior tiles keep the raw 16-bit values: the skip is decided on the
    // bits (a pair equal to two -inf holds no legal key) and each value is
    // widened inside the FMA that adds it. Edge tiles widen here and apply the
    // key limits.
    float am[NB32][16];
    if constexpr (ADD) {
      bool any = false;
      if (!edge) {
        constexpr uint32_t NEG2 = std::is_same<T, __bf16>::value ? 0xFF80FF80u : 0xFC00FC00u;
#pragma unroll
        for (int blk = 0; blk < NB32; ++blk)
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const uint4 w = am_raw[blk][g];
            any |= (w.x != NEG2) | (w.y != NEG2) | (w.z != NEG2) | (w.w != NEG2);
          }
      } else {
#pragma unroll
        for (int blk = 0; blk < NB32; ++blk)
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            Frag8<T> f;
            f.u[0] = am_raw[blk][g];
            float mv[8];
            unpack8(f, mv);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int key = kb0 + blk * 32 + 16 * g + 8 * hh + j;
              const float a = (key >= kpad || (causal && key > qi)) ? -INFINITY : mv[j];
              am[blk][8 * g + j] = a;
              any |= a != -INFINITY;
            }
          }
      }
      comp = __ballot(comp && row_ok && any) != 0;
    }

    // One 64-key tile. EDGE: per-element key limits (causal diagonal,
    // padding length, Lk); VCONV: P V from the float16 copy of V. Both are
    // uniform over the workgroup, so the body below has a single branch (the
    // rare rescale) and the scheduler can run one 32-key block's
    // exponentials under the other block's MFMAs.
    auto tile = [&](auto edge_tag, auto vconv_tag) {
      constexpr bool EDGE = decltype(edge_tag)::value;
      constexpr bool VCONV = decltype(vconv_tag)::value;
      // S^T = K Q^T; the two 32-key accumulator chains are interleaved.
      // Pre-LN (LS): Q carries scale * log2(e), and the accumulators start at
      // -m_ref, the running reference, so each score leaves the MFMAs as the
      // exponent of its weight, c*s - m, with no FMA per element.
      const float m_ref = (m_run == -INFINITY) ? 0.f : m_run;
      f32x16 s[NB32];
#pragma unroll
      for (int blk = 0; blk < NB32; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[blk][i] = LS ? -m_ref : 0.f;
      // both MFMA blocks run at raised wave priority: the SIMD's other wave
      // then fills the matrix core's gaps with its softmax arithmetic
      __builtin_amdgcn_s_setprio(1);
      if (CONV_K && kbf) {
        // bfloat16 K: the float16 query as two bfloat16 parts (hi + lo holds
        // its 11 significant bits exactly)
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
          // the copy's opaque update keeps the split inside this rare branch:
          // hoisted out of the tile loop it would hold 8 * NC more registers
          Frag8<QT> qc = qf[cc];
          asm volatile("" : "+v"(qc.u[0].x), "+v"(qc.u[0].y), "+v"(qc.u[0].z), "+v"(qc.u[0].w));
          float f[8], h[8];
          unpack8(qc, f);
          const Frag8<T> qh = pack8<T>(f);
          unpack8(qh, h);
#pragma unroll
          for (int j = 0; j < 8; ++j) f[j] -= h[j];
          const Frag8<T> ql = pack8<T>(f);
#pragma unroll
          for (int blk = 0; blk < NB32; ++blk) {
            Frag8<T> kf;
            kf.u[0] = lds_load16(kl + krow_off[blk] + 16 * ((2 * cc + hh) ^ ksw[blk]));
            s[blk] = mma8(kf, qh, s[blk]);
            s[blk] = mma8(kf, ql, s[blk]);
          }
        }
      } else {
#pragma unroll
        for (int cc = 0; cc < NC; ++cc)
#pragma unroll
          for (int blk = 0; blk < NB32; ++blk) {
            Frag8<QT> kf;  // float16 after the rewrite (pre-LN), else the call dtype
            kf.u[0] = lds_load16(kl + krow_off[blk] + 16 * ((2 * cc + hh) ^ ksw[blk]));
            s[blk] = mma8(kf, qf[cc], s[blk]);
          }
      }
      __builtin_amdgcn_s_setprio(0);
      // online softmax over the tile [MAX 2.3]. ADD: s becomes the logit
      // scale*s + mask (natural units); otherwise s stays raw (scale > 0
      // commutes with the max) and the scale is applied in the exponent's FMA
      float mt = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < NB32; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float u = s[blk][i];
          if constexpr (ADD) {
            float mv;
            if constexpr (EDGE) {
              mv = am[blk][i];
            } else {
              const uint32_t w = (&am_raw[blk][i >> 3].x)[(i & 7) >> 1];
              T* tag = nullptr;
              mv = (i & 1) ? hi_f(w, tag) : lo_f(w, tag);
            }
            u = LS ? __builtin_fmaf(mv, LOG2E, u) : __builtin_fmaf(u, p.scale, mv);
          } else if constexpr (EDGE) {
            const int key = kb0 + blk * 32 + (i < 8 ? 8 * hh + i : 8 + 8 * hh + i);
            if (key >= kpad || (causal && key > qi)) u = -INFINITY;
          }
          s[blk][i] = u;
          mt = fmaxf(mt, u);
        }
      mt = pair_max(mt);
      if constexpr (LS) mt = (mt == -INFINITY) ? -INFINITY : m_ref + mt;  // to absolute log2 units
      else if constexpr (ADD) mt *= LOG2E;  // to log2 units
      else mt = (mt == -INFINITY) ? -INFINITY : mt * c;
      // raise the reference maximum only when exceeded by more than the gap
      if (__ballot(mt > m_run + RESCALE_GAP) != 0) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = (m_new == -INFINITY) ? 1.0f : exp2_fast(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
        if constexpr (LS) {
          // the exponents were taken against m_ref: move them to m_new
          const float shift = (m_new == -INFINITY) ? 0.f : m_new - m_ref;
#pragma unroll
          for (int blk = 0; blk < NB32; ++blk)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[blk][i] -= shift;
        }
        m_run = m_new;
      }
      const float m_use = (ADD || EDGE) ? (m_run == -INFINITY ? 0.f : m_run) : m_run;
      // P in float16 (f16 inputs, or bf16 with the float16 V copy): the row
      // sum is taken from the packed P the MFMA consumes, two weights per
      // v_dot2 with float32 accumulation
      constexpr bool SUM_PACKED = VCONV || !SPLIT_P;
      float rs = 0.f;
#pragma unroll
      for (int blk = 0; blk < NB32; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float e;
          if constexpr (LS) {
            e = exp2_fast(s[blk][i]);  // -inf -> 0
          } else if constexpr (ADD) {
            e = exp2_fast(__builtin_fmaf(s[blk][i], LOG2E, -m_use));  // -inf -> 0
          } else {
            e = exp2_fast(__builtin_fmaf(s[blk][i], c, -m_use));
            if constexpr (EDGE) e = (s[blk][i] == -INFINITY) ? 0.f : e;  // also when scale = 0
          }
          s[blk][i] = e;
          if constexpr (!SUM_PACKED) rs += e;
        }
      // O^T += V^T P^T, 16 keys per MFMA k-step
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int blk = 0; blk < NB32; ++blk)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          float pv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) pv[j] = s[blk][8 * tt + j];
          const int key_a = blk * 32 + 16 * tt + vkey0;  // + 4 for the second read
          const int sw = swz_v16<CPR>(key_a);            // key_a and key_a + 4 share it
          if constexpr (VCONV) {
            // P and V in float16, one MFMA per 32 features
            const Frag8<_Float16> ph = pack8<_Float16>(pv);
            rs = row_sum_f16x8(ph.u[0], rs);
#pragma unroll
            for (int db = 0; db < ND; ++db) {
              const int feat = (32 * db + vfeat0) & (D - 1);
              const char* a0 = vcl + key_a * RB + 16 * ((feat >> 3) ^ sw) + (feat & 7) * E;
              const uint2 lo4 = lds_read_tr<_Float16>(a0);
              const uint2 hi4 = lds_read_tr<_Float16>(a0 + 4 * RB);
              Frag8<_Float16> vf;
              vf.u[0] = make_uint4(lo4.x, lo4.y, hi4.x, hi4.y);
              o[db] = mma8(vf, ph, o[db]);
            }
          } else {
            const Frag8<T> pf = pack8<T>(pv);
            if constexpr (SUM_PACKED) rs = row_sum_f16x8(pf.u[0], rs);
            Frag8<T> pf_lo;
            if constexpr (SPLIT_P) {
              float hi[8], lo[8];
              unpack8(pf, hi);
#pragma unroll
              for (int j = 0; j < 8; ++j) lo[j] = pv[j] - hi[j];
              pf_lo = pack8<T>(lo);
            }
#pragma unroll
            for (int db = 0; db < ND; ++db) {
              const int feat = (32 * db + vfeat0) & (D - 1);
              const char* a0 = vl + key_a * RB + 16 * ((feat >> 3) ^ sw) + (feat & 7) * E;
              const uint2 lo4 = lds_read_tr<T>(a0);
              const uint2 hi4 = lds_read_tr<T>(a0 + 4 * RB);
              Frag8<T> vf;
              vf.u[0] = make_uint4(lo4.x, lo4.y, hi4.x, hi4.y);
              o[db] = mma8(vf, pf, o[db]);
              if constexpr (SPLIT_P) o[db] = mma8(vf, pf_lo, o[db]);
            }
          }
        }
      __builtin_amdgcn_s_setprio(0);
      l_run += rs;
    };

    if (comp) {
      ++ncomp;
      using TT = std::true_type;
      using FF = std::false_type;
      constexpr bool VF16 = CONV_V || KV16;  // a float16 V tile exists
      if (KV16 || (CONV_V && vconv)) {
        if (edge) tile(TT{}, std::integral_constant<bool, VF16>{});
        else tile(FF{}, std::integral_constant<bool, VF16>{});
      } else {
        if (edge) tile(TT{}, FF{});
        else tile(FF{}, FF{});
      }
    }

    if constexpr (ADD) {
#pragma unroll
      for (int blk = 0; blk < NB32; ++blk)
#pragma unroll
        for (int g = 0; g < 2; ++g) am_raw[blk][g] = am_nxt[blk][g];
      if (p.kind & K_KEEP) to_additive(am_raw);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's share of the next tile is in LDS
    if constexpr (CONV_V) {
      // each thread rewrites exactly the V chunks it loaded itself, so its own
      // wait suffices; the barrier below publishes the copy with the tile.
      // Nothing reads buffer buf ^ 1 any more: its last readers (tile t - 1)
      // passed the previous barrier.
      asm volatile("" ::: "memory");
      if (t + 1 < ntiles) convert_v(buf ^ 1, (hl << 16) | (t + 1));
    }
    if constexpr (CONV_K) {
      asm volatile("" ::: "memory");
      if (t + 1 < ntiles) convert_k(buf ^ 1, (hl << 16) | (t + 1));  // this thread's own chunks
    }
    __syncthreads();
  }

  if (p.counters && wave_active && lane == 0) {
    const int nsub = (Lk + BN - 1) / BN;  // key tiles; this split owns those with index % NK == ks
    const int mine = nsub > ks ? (nsub - ks + NK - 1) / NK : 0;
    atomicAdd(p.counters + 0, (unsigned long long)ncomp);
    atomicAdd(p.counters + 1, (unsigned long long)(mine - ncomp));
  }

  // ---- merge the key splits of each query group (log-sum-exp) ----
  if constexpr (SPLIT_FINISH) {
    // wave (w, ks) finishes O blocks [ks*HALF, ks*HALF + HALF) and hands the
    // others to (w, ks^1); both combine the two states in the same order
    // (split 0's terms first), so the halves of a row share one l
    char* const out_part = smem + (wave * NK + ks) * PART_BYTES;
    const char* const in_part = smem + (wave * NK + (ks ^ 1)) * PART_BYTES;
    auto merge = [&](auto ks_c) {
      constexpr int KS = decltype(ks_c)::value;
      constexpr int GIVE = (KS ^ 1) * HALF, KEEP = KS * HALF;
      reinterpret_cast<float2*>(out_part)[lane] = make_float2(m_run, l_run);
      float4* const po = reinterpret_cast<float4*>(out_part + 512);
#pragma unroll
      for (int hb = 0; hb < HALF; ++hb)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          po[(hb * 4 + q) * 64 + lane] = make_float4(o[GIVE + hb][4 * q], o[GIVE + hb][4 * q + 1],
                                                     o[GIVE + hb][4 * q + 2], o[GIVE + hb][4 * q + 3]);
      __syncthreads();
      const float2 ml = reinterpret_cast<const float2*>(in_part)[lane];
      const float m0 = KS == 0 ? m_run : ml.x, m1 = KS == 0 ? ml.x : m_run;
      const float l0 = KS == 0 ? l_run : ml.y, l1 = KS == 0 ? ml.y : l_run;
      const float M = fmaxf(m0, m1);
      const float s0 = (M == -INFINITY) ? 0.f : exp2_fast(m0 - M);
      const float s1 = (M == -INFINITY) ? 0.f : exp2_fast(m1 - M);
      l_run = l0 * s0 + l1 * s1;
      const float4* const pi = reinterpret_cast<const float4*>(in_part + 512);
#pragma unroll
      for (int hb = 0; hb < HALF; ++hb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 f = pi[(hb * 4 + q) * 64 + lane];
          const float g[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = o[KEEP + hb][4 * q + r];
            o[KEEP + hb][4 * q + r] = KS == 0 ? x * s0 + g[r] * s1 : g[r] * s0 + x * s1;
          }
        }
    };
    if (ks == 0) merge(std::integral_constant<int, 0>{});
    else merge(std::integral_constant<int, 1>{});
    __syncthreads();  // the merge area is the next head's tile buffer
  } else if constexpr (NK > 1) {
    float* mg = reinterpret_cast<float*>(smem);
    constexpr int REGS = ND * 16 + 2;
    if (ks > 0) {
      float* dst = mg + ((wave * (NK - 1) + (ks - 1)) * REGS) * 64;
      dst[lane] = m_run;
      dst[64 + lane] = l_run;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[(2 + db * 16 + i) * 64 + lane] = o[db][i];
    }
    __syncthreads();
    if (ks == 0) {
      float M = m_run;
#pragma unroll
      for (int k2 = 1; k2 < NK; ++k2)
        M = fmaxf(M, mg[((wave * (NK - 1) + (k2 - 1)) * REGS) * 64 + lane]);
      const float s0 = (M == -INFINITY) ? 0.f : exp2_fast(m_run - M);
      l_run *= s0;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= s0;
#pragma unroll
      for (int k2 = 1; k2 < NK; ++k2) {
        const float* src = mg + ((wave * (NK - 1) + (k2 - 1)) * REGS) * 64;
        const float sk = (M == -INFINITY) ? 0.f : exp2_fast(src[lane] - M);
        l_run += src[64 + lane] * sk;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] += src[(2 + db * 16 + i) * 64 + lane] * sk;
      }
    }
    __syncthreads();  // the merge area is the next head's tile buffer
  }

  // ---- epilogue: O / l, residual, flags, 16-byte stores. With two key
  // splits each wave stores the O blocks it finished; otherwise the first
  // split stores them all ----
  const int db_lo = SPLIT_FINISH ? ks * HALF : 0;
  const int db_hi = SPLIT_FINISH ? db_lo + HALF : ND;
  if (SPLIT_FINISH || ks == 0) {
  const float l_tot = pair_sum(l_run);
  const bool fully = row_ok && !(l_tot != 0.f);
  const float inv = (l_tot != 0.f) ? 1.0f / l_tot : 0.f;
  bool nonfinite = false;
  if (row_ok) {
    char* orow;
    const char* rrow = nullptr;
    if constexpr (PRENORM) {
      const int64_t off = (((int64_t)b * Lq + qi) * (H * D) + h * D) * E;
      orow = (char*)p.out + off;
      if (p.residual) rrow = (const char*)p.residual + off;
    } else {
      orow = (char*)p.out + ((bh * Lq + qi) * D) * E;
    }
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int d0 = db * 32 + 16 * g + 8 * hh;
        if (d0 >= D || db < db_lo || db >= db_hi) continue;
        float ov[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) ov[j] = o[db][8 * g + j] * inv;
        if constexpr (PRENORM) {
          if (rrow) {
            float rv[8];
            unpack8(ld_global8<T>(rrow + d0 * E), rv);
#pragma unroll
            for (int j = 0; j < 8; ++j) ov[j] += rv[j];
          }
        }
        const Frag8<T> f = pack8<T>(ov);
        float back[8];
        unpack8(f, back);
#pragma unroll
        for (int j = 0; j < 8; ++j) nonfinite |= !__builtin_isfinite(back[j]);
        *reinterpret_cast<uint4*>(orow + d0 * E) = f.u[0];
      }
  }
  const unsigned long long fm = __ballot(fully && hh == 0 && ks == 0);  // one split reports rows
  const unsigned long long nf = __ballot(nonfinite);
  if (lane == 0) {
    const uint32_t fl = (fm ? F_FULLY_MASKED_ROW : 0u) | (nf ? F_NONFINITE : 0u);
    if (fl) atomicOr(p.flags, fl);
    if (p.counters && fm) atomicAdd(p.counters + 2, (unsigned long long)__popcll(fm));
  }
  }
  }  // heads of the group
}

}  // namespace mha
