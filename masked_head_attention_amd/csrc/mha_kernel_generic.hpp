// mha_kernel_generic.hpp -- fused masked multi-head attention forward for gfx950
// (CDNA4), register-staged variant (used for float32).
//
// Sources (web pages, cited by title and section):
//   [MMHA]  "masked multi head attention" CUDA implementation notes (2kiu.com/news/6063113)
//   [MAX]   "Why attention must compute the max first" (gsyq.cn/news/340375)
//   [LNXA]  "How to fuse cross-attention and layer-norm into a single CUDA kernel?"
//           (cms365.cn question page)
//
// One kernel computes, per (batch, head, block of query rows):
//   S = scale * Q K^T -> mask (causal / key padding / additive, before the
//   softmax) -> online softmax (running max m, rescaled running sum l)
//   -> O += P V, with S and P living only in registers [MAX 2.3, 2.4; MMHA 2].
//
// Mapping to CDNA4 (this is not the pages' CUDA layout):
//   * a wavefront owns 32 query rows; the contractions are 32x32 MFMAs
//     (v_mfma_f32_32x32x16_{f16,bf16} for half types, v_mfma_f32_32x32x2_f32
//     for float) with fp32 accumulation;
//   * the score tile is computed transposed, S^T = K Q^T, so that each lane
//     holds one query row's scores. The row max and sum are then reductions
//     inside a lane plus one exchange with the lane 32 apart
//     (v_permlane32_swap), and the probabilities are already laid out as the
//     B operand of the second contraction O^T = V^T P^T -- no trip through
//     LDS, no 16-lane shuffles;
//   * the MFMA row index m of S^T is mapped to key keymap(m) so that every
//     lane's 16 accumulator values are two runs of 8 consecutive keys; the
//     same map on the rows of V^T makes the 16 output values two runs of 8
//     consecutive features, so P packs straight into 16-byte operands and O
//     leaves in 16-byte stores;
//   * K and V tiles are staged in LDS (K row-major, V transposed), XOR
//     swizzled per 16-byte chunk so the MFMA operand reads hit distinct
//     banks, double-buffered through registers so the next tile's global
//     loads overlap this tile's math;
//   * exp is v_exp_f32 (2^x) with log2(e) folded into the score scale;
//   * masked tiles are skipped whole: the key loop stops at the causal
//     diagonal / the padding length, and with an additive mask a wave skips a
//     tile whose entries are all -inf (one ballot) [MMHA 2, 3.1];
//   * the pre-LayerNorm variant computes each token's mean and variance in
//     the prologue and forms Q = (x - mean) * rstd * gamma + beta in
//     registers; the epilogue adds the residual [LNXA answer steps 2, 4].
#pragma once

#include "mha_common.hpp"

namespace mha {

// ---------------------------------------------------------------------------
template <typename T, int D, bool ADD, bool PRENORM>
__global__ __launch_bounds__((64 * TileCfg<T, D>::NQ * TileCfg<T, D>::NK))
void mha_fwd_kernel(const Params p) {
  using Cfg = TileCfg<T, D>;
  constexpr int NQ = Cfg::NQ, NK = Cfg::NK, BN = Cfg::BN, NBUF = Cfg::NBUF;
  constexpr int E = sizeof(T);
  constexpr int EPC = 16 / E;                 // elements per 16-byte chunk
  constexpr int NW = NQ * NK;
  constexpr int NT = 64 * NW;
  constexpr int BM = 32 * NQ;                 // query rows per workgroup
  constexpr int BNT = BN * NK;                // keys per LDS tile
  constexpr int NB32 = BN / 32;               // 32-key blocks per wave sub-tile
  constexpr int NC = D / 16;                  // 16-feature slices of the QK^T contraction
  constexpr int DP = D < 32 ? 32 : D;         // O^T rows (features), padded to 32
  constexpr int ND = DP / 32;
  constexpr int CPR_K = D * E / 16;           // chunks per K row
  constexpr int CPR_V = BNT * E / 16;         // chunks per V^T row
  constexpr int KT_BYTES = BNT * D * E;
  constexpr int VT_BYTES = DP * BNT * E;
  constexpr int BUF_BYTES = KT_BYTES + VT_BYTES;
  constexpr int MERGE_BYTES = NK > 1 ? NQ * (NK - 1) * 64 * (ND * 16 + 2) * 4 : 0;
  constexpr int TILE_REGION = NBUF * BUF_BYTES > MERGE_BYTES ? NBUF * BUF_BYTES : MERGE_BYTES;
  constexpr int STAT_BYTES = PRENORM ? NQ * 32 * 8 : 16;
  static_assert(BN % 32 == 0 && D % 16 == 0, "tile shape");
  constexpr int KUNITS = BNT * CPR_K;         // 16-byte K chunks per tile
  constexpr int NLK = (KUNITS + NT - 1) / NT;
  constexpr int VUNITS = (E == 2) ? (BNT / 2) * CPR_K : BNT * CPR_K;
  constexpr int NLV = (VUNITS + NT - 1) / NT;
  constexpr int VW = (E == 2) ? 2 : 1;        // 16-byte loads per V unit
  // float32: Q is pre-multiplied by scale*log2(e), so scores arrive in log2
  // units and the row maximum's own weight is exactly 2^0 = 1. Half types keep
  // Q as given and apply the factor in the exponent's FMA.
  constexpr bool PRESCALE = (E == 4);
  // bfloat16 probabilities carry only 8 significant bits; P is split into
  // hi + lo bf16 parts (two MFMAs) so P V keeps ~16 bits.
  constexpr bool SPLIT_P = std::is_same<T, __bf16>::value;

  __shared__ __attribute__((aligned(16))) char smem[TILE_REGION + STAT_BYTES];
  char* const stat_lds = smem + TILE_REGION;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qg = wave % NQ, ks = wave / NQ;
  const int n = lane & 31, hh = lane >> 5;

  // ---- workgroup -> (b, h, query block) ----
  int b, h, qblk;
  {
    const int bid = blockIdx.x;
    if constexpr (PRENORM) {
      // heads fastest: the workgroups sharing x rows run side by side
      h = bid % p.H;
      const int r = bid / p.H;
      qblk = r % p.nqblk;
      b = r / p.nqblk;
    } else {
      // the last (for causal: heaviest) query blocks first
      const int nbh = p.B * p.H;
      const int bh = bid % nbh;
      qblk = p.nqblk - 1 - bid / nbh;
      b = bh / p.H;
      h = bh % p.H;
    }
  }
  const int Lq = p.Lq, Lk = p.Lk, H = p.H;
  const int q0 = qblk * BM;
  const int qw0 = q0 + qg * 32;
  const int qi = qw0 + n;
  const bool row_ok = qi < Lq;
  const bool wave_active = qw0 < Lq;
  const bool causal = (p.kind & K_CAUSAL) != 0;
  const int64_t bh = (int64_t)b * H + h;

  // ---- key limits (mask decisions that are whole ranges) ----
  int kpad = Lk;
  if (p.kind & K_PADDING) {
    const int L = p.lens[b];
    kpad = L < 0 ? 0 : (L > Lk ? Lk : L);
    if ((L < 0 || L > Lk) && h == 0 && qblk == 0 && tid == 0) atomicOr(p.flags, F_BAD_LENGTH);
  }
  int kend_w = kpad;  // this wave: keys >= kend_w are masked for all its rows
  if (causal) {
    const int qlast = min(qw0 + 31, Lq - 1);
    kend_w = min(kend_w, qlast + 1);
  }
  if (!wave_active) kend_w = 0;
  int kend_g = kpad;  // workgroup bound
  if (causal) kend_g = min(kend_g, min(q0 + BM - 1, Lq - 1) + 1);
  const int ntiles = (kend_g + BNT - 1) / BNT;

  // ---- Q fragments (B operand of S^T = K Q^T): Q[qi][16c + 8hh + j] ----
  Frag8<T> qf[NC];
  if constexpr (!PRENORM) {
    const char* qrow = (const char*)p.q + ((bh * Lq + (row_ok ? qi : 0)) * D) * E;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qf[c] = row_ok ? ld_global8<T>(qrow + (16 * c + 8 * hh) * E) : zero8<T>();
      if constexpr (PRESCALE) {
        float qv[8];
        unpack8(qf[c], qv);
#pragma unroll
        for (int j = 0; j < 8; ++j) qv[j] *= p.c;
        qf[c] = pack8<T>(qv);
      }
    }
  } else {
    // Token statistics over all F = H*D features [LNXA answer step 2]:
    // 16 lanes per token, 4 tokens at a time, two passes (mean, then the mean
    // squared deviation) read through the cache.
    const int F = H * D;
    const int nch = F / EPC;
    const int g16 = lane >> 4, l16 = lane & 15;
    float2* st = reinterpret_cast<float2*>(stat_lds) + qg * 32;
    if (ks == 0) {
      for (int r0 = 0; r0 < 32; r0 += 4) {
        const int row = qw0 + r0 + g16;
        // every lane takes part in the 16-lane reductions; rows past Lq add zeros
        const bool valid = row < Lq;
        const char* xr = (const char*)p.x + ((int64_t)b * Lq + (valid ? row : 0)) * (int64_t)F * E;
        float s = 0.f;
        if (valid) {
          for (int ch = l16; ch < nch; ch += 16) {
            const uint4 u = *reinterpret_cast<const uint4*>(xr + 16 * ch);
            if constexpr (E == 4) {
              s += __uint_as_float(u.x) + __uint_as_float(u.y) + __uint_as_float(u.z) +
                   __uint_as_float(u.w);
            } else {
              T* tag = nullptr;
              const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
              for (int i = 0; i < 4; ++i) s += lo_f(w[i], tag) + hi_f(w[i], tag);
            }
          }
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o, 64);
        const float mean = s / (float)F;
        float v2 = 0.f;
        if (valid) {
          for (int ch = l16; ch < nch; ch += 16) {
            const uint4 u = *reinterpret_cast<const uint4*>(xr + 16 * ch);
            if constexpr (E == 4) {
              const float a0 = __uint_as_float(u.x) - mean, a1 = __uint_as_float(u.y) - mean;
              const float a2 = __uint_as_float(u.z) - mean, a3 = __uint_as_float(u.w) - mean;
              v2 += a0 * a0 + a1 * a1 + a2 * a2 + a3 * a3;
            } else {
              T* tag = nullptr;
              const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float a0 = lo_f(w[i], tag) - mean, a1 = hi_f(w[i], tag) - mean;
                v2 += a0 * a0 + a1 * a1;
              }
            }
          }
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) v2 += __shfl_xor(v2, o, 64);
        const float rstd = 1.0f / sqrtf(v2 / (float)F + p.eps);
        if (l16 == 0) st[r0 + g16] = make_float2(mean, rstd);
      }
    }
    __syncthreads();
    const float2 ms = st[n];
    const char* xrow = (const char*)p.x + (((int64_t)b * Lq + (row_ok ? qi : 0)) * F + h * D) * E;
    const char* grow = (const char*)p.gamma + (int64_t)h * D * E;
    const char* brow = (const char*)p.beta + (int64_t)h * D * E;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int off = (16 * c + 8 * hh) * E;
      if (!row_ok) { qf[c] = zero8<T>(); continue; }
      float xv[8], gv[8], bv[8], qv[8];
      unpack8(ld_global8<T>(xrow + off), xv);
      unpack8(ld_global8<T>(grow + off), gv);
      unpack8(ld_global8<T>(brow + off), bv);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        qv[j] = (xv[j] - ms.x) * ms.y * gv[j] + bv[j];
        if constexpr (PRESCALE) qv[j] *= p.c;
      }
      qf[c] = pack8<T>(qv);
    }
  }

  // ---- K/V tile staging: global -> registers -> LDS ----
  const char* kbase = (const char*)p.k + bh * Lk * (int64_t)D * E;
  const char* vbase = (const char*)p.v + bh * Lk * (int64_t)D * E;
  uint4 kreg[NLK];
  uint4 vreg[NLV][VW];

  auto load_tile = [&](int kt0) {
#pragma unroll
    for (int it = 0; it < NLK; ++it) {
      const int u = tid + it * NT;
      const int row = u / CPR_K, ch = u % CPR_K;
      const int key = kt0 + row;
      kreg[it] = (KUNITS % NT == 0 || u < KUNITS) && key < Lk ? *reinterpret_cast<const uint4*>(kbase + ((int64_t)key * D) * E + 16 * ch)
                          : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int it = 0; it < NLV; ++it) {
      const int u = tid + it * NT;
      const int ch = u % CPR_K, pr = u / CPR_K;
#pragma unroll
      for (int w = 0; w < VW; ++w) {
        const int key = kt0 + pr * VW + w;
        vreg[it][w] = (VUNITS % NT == 0 || u < VUNITS) && key < Lk
                          ? *reinterpret_cast<const uint4*>(vbase + ((int64_t)key * D) * E + 16 * ch)
                          : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  auto store_tile = [&](int buf) {
    char* kl = smem + buf * BUF_BYTES;
    char* vl = kl + KT_BYTES;
#pragma unroll
    for (int it = 0; it < NLK; ++it) {
      const int u = tid + it * NT;
      if (KUNITS % NT != 0 && u >= KUNITS) break;
      const int row = u / CPR_K, ch = u % CPR_K;
      *reinterpret_cast<uint4*>(kl + row * (D * E) + 16 * (ch ^ (swz_k(row) & (CPR_K - 1)))) =
          kreg[it];
    }
#pragma unroll
    for (int it = 0; it < NLV; ++it) {
      const int u = tid + it * NT;
      if (VUNITS % NT != 0 && u >= VUNITS) break;
      const int ch = u % CPR_K, pr = u / CPR_K;
      if constexpr (E == 2) {
        // keys 2pr and 2pr+1, features 8ch .. 8ch+7: one dword per feature
        const uint32_t a[4] = {vreg[it][0].x, vreg[it][0].y, vreg[it][0].z, vreg[it][0].w};
        const uint32_t c2[4] = {vreg[it][1].x, vreg[it][1].y, vreg[it][1].z, vreg[it][1].w};
        const int key = 2 * pr;
        const int kc = key / EPC, kb = (key % EPC) * E;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int d = ch * 8 + j;
          const uint32_t lo = (j & 1) ? (a[j >> 1] >> 16) : (a[j >> 1] & 0xffffu);
          const uint32_t hi = (j & 1) ? (c2[j >> 1] & 0xffff0000u) : (c2[j >> 1] << 16);
          *reinterpret_cast<uint32_t*>(vl + d * (BNT * E) + 16 * (kc ^ (swz_v(d) & (CPR_V - 1))) +
                                       kb) = lo | hi;
        }
      } else {
        const uint32_t a[4] = {vreg[it][0].x, vreg[it][0].y, vreg[it][0].z, vreg[it][0].w};
        const int key = pr;
        const int kc = key / EPC, kb = (key % EPC) * E;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = ch * 4 + j;
          *reinterpret_cast<uint32_t*>(vl + d * (BNT * E) + 16 * (kc ^ (swz_v(d) & (CPR_V - 1))) +
                                       kb) = a[j];
        }
      }
    }
  };
  auto lds_frag = [&](const char* base, int row, int row_bytes, int chunk0, int swz,
                      int cmask) -> Frag8<T> {
    Frag8<T> f;
#pragma unroll
    for (int w = 0; w < Frag8<T>::W; ++w)
      f.u[w] = *reinterpret_cast<const uint4*>(base + row * row_bytes +
                                               16 * ((chunk0 + w) ^ (swz & cmask)));
    return f;
  };

  // ---- running state ----
  f32x16 o[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  int ncomp = 0;
  const float c = PRESCALE ? 1.0f : p.c;
  const int krow_l = keymap(n);   // K tile row (within a 32-key block) read by this lane
  const int vrow_l = keymap(n);   // V^T tile row (within a 32-feature block) read by this lane
  const char* addrow = nullptr;
  if constexpr (ADD)
    addrow = (const char*)p.add + ((int64_t)b * Lq + (row_ok ? qi : 0)) * (int64_t)Lk * E;

  if (NBUF == 2 && ntiles > 0) {
    load_tile(0);
    store_tile(0);
    __syncthreads();
  }

  for (int t = 0; t < ntiles; ++t) {
    const int kt0 = t * BNT;
    const int buf = NBUF == 2 ? (t & 1) : 0;
    if constexpr (NBUF == 2) {
      if (t + 1 < ntiles) load_tile(kt0 + BNT);
    } else {
      load_tile(kt0);
      store_tile(0);
      __syncthreads();
    }
    const char* kl = smem + buf * BUF_BYTES;
    const char* vl = kl + KT_BYTES;
    const int kb0 = kt0 + ks * BN;  // this wave's sub-tile

    bool comp = kb0 < kend_w;
    // additive mask values for this lane's 16*NB32 scores (in log2 units)
    float am[NB32][16];
    if constexpr (ADD) {
      bool any = false;
      if (comp) {
#pragma unroll
        for (int blk = 0; blk < NB32; ++blk)
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const int key0 = kb0 + blk * 32 + 16 * g + 8 * hh;
            float mv[8];
            if (row_ok && p.add_vec && key0 + 8 <= Lk) {
              unpack8(ld_global8<T>(addrow + (int64_t)key0 * E), mv);
            } else {
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const int key = key0 + j;
                float val = -INFINITY;
                if (row_ok && key < Lk) {
                  if constexpr (E == 4) {
                    val = reinterpret_cast<const float*>(addrow)[key];
                  } else {
                    const uint16_t bits = reinterpret_cast<const uint16_t*>(addrow)[key];
                    T* tag = nullptr;
                    val = lo_f((uint32_t)bits, tag);
                  }
                }
                mv[j] = val;
              }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int key = key0 + j;
              const bool msk = !row_ok || key >= kpad || (causal && key > qi) || mv[j] == -INFINITY;
              am[blk][8 * g + j] = msk ? -INFINITY : mv[j] * 1.4426950408889634f;
              any |= !msk;
            }
          }
      }
      comp = __ballot(any) != 0;  // the whole wave skips a tile with no legal pair
    }

    if (comp) {
      ++ncomp;
      // S^T = K Q^T for NB32 blocks of 32 keys
      f32x16 s[NB32];
#pragma unroll
      for (int blk = 0; blk < NB32; ++blk) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[blk][i] = 0.f;
        const int krow = ks * BN + blk * 32 + krow_l;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc)
          s[blk] = mma8(lds_frag(kl, krow, D * E, (16 * cc + 8 * hh) / EPC, swz_k(krow), CPR_K - 1),
                        qf[cc], s[blk]);
      }
      // mask, then the online softmax update [MAX 2.3, 4.2]
      const bool edge = ADD || (kb0 + BN > kpad) || (causal && kb0 + BN - 1 > qw0);
      float mt = -INFINITY;
      if constexpr (ADD) {
#pragma unroll
        for (int blk = 0; blk < NB32; ++blk)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            s[blk][i] = __builtin_fmaf(s[blk][i], c, am[blk][i]);  // -inf stays -inf
            mt = fmaxf(mt, s[blk][i]);
          }
      } else {
        if (edge) {
#pragma unroll
          for (int blk = 0; blk < NB32; ++blk)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = kb0 + blk * 32 + (i < 8 ? 8 * hh + i : 8 + 8 * hh + i);
              if (key >= kpad || (causal && key > qi)) s[blk][i] = -INFINITY;
            }
        }
#pragma unroll
        for (int blk = 0; blk < NB32; ++blk)
#pragma unroll
          for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[blk][i]);
      }
      mt = pair_max(mt);
      float mt_s = mt;
      if constexpr (!ADD) mt_s = (mt == -INFINITY) ? -INFINITY : mt * c;
      const float m_new = fmaxf(m_run, mt_s);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2_fast(m_run - m_use);
      m_run = m_new;
      float rs = 0.f;
      float pv[NB32][16];
#pragma unroll
      for (int blk = 0; blk < NB32; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float e;
          if constexpr (ADD) {
            e = exp2_fast(s[blk][i] - m_use);
          } else {
            e = exp2_fast(__builtin_fmaf(s[blk][i], c, -m_use));
            if (edge) e = (s[blk][i] == -INFINITY) ? 0.f : e;
          }
          pv[blk][i] = e;
          rs += e;
        }
      l_run = l_run * alpha + rs;
      if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      }
      // O^T += V^T P^T
#pragma unroll
      for (int blk = 0; blk < NB32; ++blk)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const Frag8<T> pf = pack8<T>(&pv[blk][8 * tt]);
          Frag8<T> pf_lo;
          if constexpr (SPLIT_P) {
            float hi[8], lo[8];
            unpack8(pf, hi);
#pragma unroll
            for (int j = 0; j < 8; ++j) lo[j] = pv[blk][8 * tt + j] - hi[j];
            pf_lo = pack8<T>(lo);
          }
          const int vchunk = (ks * BN + blk * 32 + 16 * tt + 8 * hh) / EPC;
#pragma unroll
          for (int db = 0; db < ND; ++db) {
            const int vrow = db * 32 + vrow_l;
            const Frag8<T> vf = lds_frag(vl, vrow, BNT * E, vchunk, swz_v(vrow), CPR_V - 1);
            o[db] = mma8(vf, pf, o[db]);
            if constexpr (SPLIT_P) o[db] = mma8(vf, pf_lo, o[db]);
          }
        }
    }

    if constexpr (NBUF == 2) {
      if (t + 1 < ntiles) store_tile((t + 1) & 1);
    }
    __syncthreads();
  }

  // ---- merge the NK key splits of each query group (log-sum-exp) ----
  if constexpr (NK > 1) {
    float* mg = reinterpret_cast<float*>(smem);
    constexpr int REGS = ND * 16 + 2;
    if (ks > 0) {
      float* dst = mg + ((qg * (NK - 1) + (ks - 1)) * REGS) * 64;
      dst[0 * 64 + lane] = m_run;
      dst[1 * 64 + lane] = l_run;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[(2 + db * 16 + i) * 64 + lane] = o[db][i];
    }
    __syncthreads();
    if (ks == 0) {
      float M = m_run;
#pragma unroll
      for (int k2 = 1; k2 < NK; ++k2) M = fmaxf(M, mg[((qg * (NK - 1) + (k2 - 1)) * REGS) * 64 + lane]);
      const float Mu = (M == -INFINITY) ? 0.f : M;
      const float s0 = exp2_fast(m_run - Mu);
      l_run *= s0;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= s0;
#pragma unroll
      for (int k2 = 1; k2 < NK; ++k2) {
        const float* src = mg + ((qg * (NK - 1) + (k2 - 1)) * REGS) * 64;
        const float sk = exp2_fast(src[lane] - Mu);
        l_run += src[64 + lane] * sk;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] += src[(2 + db * 16 + i) * 64 + lane] * sk;
      }
    }
  }

  // ---- debug counters: computed / skipped wave tiles ----
  if (p.counters && wave_active && lane == 0) {
    const int nsub = (Lk + BN - 1) / BN;  // wave sub-tiles across the key range
    const int mine = nsub > ks ? (nsub - ks + NK - 1) / NK : 0;  // those with index % NK == ks
    atomicAdd(p.counters + 0, (unsigned long long)ncomp);
    atomicAdd(p.counters + 1, (unsigned long long)(mine - ncomp));
  }

  if (ks != 0) return;

  // ---- epilogue: O / l, pre-LN residual, flags, 16-byte stores ----
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
        if (d0 >= D) continue;
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
#pragma unroll
        for (int w = 0; w < Frag8<T>::W; ++w)
          *reinterpret_cast<uint4*>(orow + d0 * E + 16 * w) = f.u[w];
      }
  }
  const unsigned long long fm = __ballot(fully && hh == 0);
  const unsigned long long nf = __ballot(nonfinite);
  if (lane == 0) {
    uint32_t fl = (fm ? F_FULLY_MASKED_ROW : 0u) | (nf ? F_NONFINITE : 0u);
    if (fl) atomicOr(p.flags, fl);
    if (p.counters && fm) atomicAdd(p.counters + 2, (unsigned long long)__popcll(fm));
  }
}

}  // namespace mha
