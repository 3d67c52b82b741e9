// mha_kernel_f32.hpp -- fused masked multi-head attention forward for gfx950
// (CDNA4), float32 variant.
//
// Sources (web pages, cited by title and section):
//   [MMHA]  "masked multi head attention" CUDA implementation notes (2kiu.com/news/6063113)
//   [MAX]   "Why attention must compute the max first" (gsyq.cn/news/340375)
//   [LNXA]  "How to fuse cross-attention and layer-norm into a single CUDA kernel?"
//           (cms365.cn question page)
//
// One kernel computes, per (batch, head, block of 16 query rows):
//   S = scale * Q K^T -> mask (causal / key padding / additive, before the
//   softmax) -> online softmax (running max m, rescaled running sum l)
//   -> O += P V, with S and P living only in registers [MAX 2.3, 2.4; MMHA 2].
//
// Float32 has no fast matrix path on CDNA4: v_mfma_f32_16x16x4_f32 gives
// 256 flop/cycle per CU, a sixteenth of the 16-bit rate, so the contractions
// bound the short sequences this type is used for, and the design spreads
// them over as many SIMDs as possible:
//   * a workgroup owns 16 query rows and NK waves; wave w takes keys
//     [32w, 32w + 32) of every NK*32-key step (two 16-key MFMA tiles), so the
//     per-wave chain is a quarter of the row block's work, and a short
//     sequence fills the chip with B*H*Lq/16 workgroups. The NK partial
//     (m, l, O) states are merged through LDS by log-sum-exp, each wave
//     finishing a slice of the output features;
//   * the score tile is computed transposed, S^T = K Q^T (16 keys x 16 rows):
//     lane (g, n) = (lane / 16, lane % 16) holds row n's scores for keys
//     4g .. 4g+3, which are exactly the k-slots that lane supplies as the B
//     operand of O^T = V^T P^T. P never leaves the registers; the row max and
//     sum need two exchanges (lanes 16 and 32 apart, v_permlane16/32_swap);
//   * Q is pre-multiplied by scale*log2(e), so the scores arrive in log2 units,
//     exp is v_exp_f32 (2^x) without a further multiply, and a row's maximum
//     has weight exactly 1;
//   * each wave loads exactly the K and V rows it consumes, from HBM into its
//     own LDS slice with buffer_load ... lds (16 bytes per lane, no register
//     staging), double-buffered, and waits only on its own loads (vmcnt): the
//     key loop has no workgroup barrier, K is waited for before V so QK^T
//     starts while V lands, and a wave whose keys are all masked loads
//     nothing. Rows past Lk come back as zeros from the buffer's range check.
//     The first tile is requested before the mask lengths are read, so the
//     two latencies overlap;
//   * XOR swizzles on 16-byte chunks keep both LDS read patterns free of bank
//     conflicts: K is read as 16 rows x one chunk (one b128 per lane), V as 4
//     rows x 16 consecutive features (one b32 per lane and k-slot);
//   * masked tiles are skipped whole at 16x16 granularity: the key loop stops
//     at the causal diagonal / the padding length, and with an additive mask a
//     wave skips a 16-key tile whose entries are all -inf (one ballot)
//     [MMHA 2, 3.1];
//   * the pre-LayerNorm variant computes the 16 tokens' mean and variance in
//     the prologue and forms Q = (x - mean) * rstd * gamma + beta in
//     registers; the epilogue adds the residual [LNXA answer steps 2, 4].
#pragma once

#include "mha_common.hpp"

namespace mha {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D>
struct F32Cfg {
  static constexpr int NK = D >= 128 ? 2 : 4;  // key-split waves per workgroup
  static constexpr int BM = 16;                // query rows per workgroup
  static constexpr int BN = 32;                // keys per wave per tile
  static constexpr int SUB = 16;               // keys per skip decision (one MFMA tile)
};

// Reductions over the four lanes l, l^16, l^32, l^48 that share a query row.
// Each swap returns the value of lane l and of its partner in an order that
// makes max/sum of the pair the same on both lanes.
__device__ inline float quad_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return pair_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ inline float quad_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return pair_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

template <int D, bool ADD, bool PRENORM>
__global__ __launch_bounds__(64 * F32Cfg<D>::NK) void mha_f32_kernel(const Params p) {
  using Cfg = F32Cfg<D>;
  constexpr int NK = Cfg::NK, BM = Cfg::BM, BN = Cfg::BN;
  constexpr int BNT = NK * BN;               // keys per step of the key loop
  constexpr int E = 4;
  constexpr int CPR = D / 4;                 // 16-byte chunks per K/V row
  constexpr int RB = D * E;                  // bytes per K/V row
  constexpr int NSB = D / 16;                // 16-feature slices: QK^T k-blocks, O^T tiles
  constexpr int MAT_BYTES = BN * RB;         // one wave's K (or V) rows of one step
  constexpr int WAVE_BYTES = 4 * MAT_BYTES;  // K and V, two buffers
  constexpr int NLD = MAT_BYTES / 1024;      // 1 KiB load instructions per matrix
  constexpr int MA = ADD ? 2 : 0;            // additive-mask loads per step
  constexpr int MO_BYTES = NK * NSB * 64 * 16;
  constexpr int QB = BM * RB;                // Q tile bytes
  constexpr int NQL = QB / 1024;             // 1 KiB load instructions for Q
  constexpr int MML_BYTES = NK * 64 * 8;
  constexpr int STAT_BYTES = PRENORM ? BM * 8 : 16;
  constexpr int KM = CPR - 1 < 15 ? CPR - 1 : 15;       // K swizzle mask (chunks)
  constexpr int VM = NSB - 1 < 3 ? NSB - 1 : 3;         // V swizzle mask (4-chunk groups)
  constexpr float LOG2E = 1.4426950408889634f;
  static_assert(MAT_BYTES % 1024 == 0, "a wave's rows must fill whole load instructions");
  static_assert(NLD + MA + 2 * NLD < 64, "vmcnt range");

  __shared__ __attribute__((aligned(16))) char smem[NK * WAVE_BYTES + MO_BYTES + MML_BYTES + QB + STAT_BYTES];
  f32x4* const mo = reinterpret_cast<f32x4*>(smem + NK * WAVE_BYTES);
  float2* const mml = reinterpret_cast<float2*>(smem + NK * WAVE_BYTES + MO_BYTES);
  char* const qlds = smem + NK * WAVE_BYTES + MO_BYTES + MML_BYTES;
  float2* const stat = reinterpret_cast<float2*>(qlds + QB);

  const int tid = threadIdx.x, lane = tid & 63;
  const int ks = __builtin_amdgcn_readfirstlane(tid >> 6);  // key split
  const int g = lane >> 4, n = lane & 15;
  const int Lq = p.Lq, Lk = p.Lk, H = p.H;
  const bool causal = (p.kind & K_CAUSAL) != 0;
  char* const wlds = smem + ks * WAVE_BYTES;  // this wave's K/V buffers

  // Workgroup -> (b, h, query block).
  //  * pre-LN: heads fastest, so the workgroups reading the same x rows run
  //    side by side;
  //  * causal: every (b, h) of the heaviest query block first, the lightest
  //    last (work grows with the block index);
  //  * otherwise: consecutive ids go to different XCDs (8, each with its own
  //    L2), so ids are remapped to keep the query blocks of one (b, h), which
  //    read the same K/V, on one XCD.
  int b, h, qblk;
  {
    const int G = (int)gridDim.x, bid = (int)blockIdx.x;
    const int nbh = p.B * H;
    int bh;
    if constexpr (PRENORM) {
      h = bid % H;
      const int r = bid / H;
      qblk = r % p.nqblk;
      b = r / p.nqblk;
      bh = b * H + h;
    } else if (causal) {
      bh = bid % nbh;
      qblk = p.nqblk - 1 - bid / nbh;
    } else {
      const int L = (G % 8 == 0) ? (bid & 7) * (G >> 3) + (bid >> 3) : bid;
      qblk = L % p.nqblk;
      bh = L / p.nqblk;
    }
    b = bh / H;
    h = bh % H;
  }
  const int64_t bh = (int64_t)b * H + h;
  const int q0 = qblk * BM;
  const int qi = q0 + n;
  const bool row_ok = qi < Lq;
  const float c = p.c;

  // ---- Q tile: HBM -> LDS, each wave a share of it ----
  // Loaded like K (same swizzle) and first, so that a wait that leaves only
  // this wave's step-0 loads in flight covers it; rows past Lq come back as
  // zeros. Loads are issued through the compiler-invisible LDS path, so no
  // compiler-inserted vmcnt wait serialises them with the K/V loads.
  if constexpr (!PRENORM) {
    const __amdgpu_buffer_rsrc_t qrs =
        make_rsrc((const char*)p.q + (bh * Lq + q0) * RB, (uint32_t)(min(Lq - q0, BM) * RB));
#pragma unroll
    for (int it = ks; it < NQL; it += NK) {
      const int u = it * 64 + lane;
      const int row = u / CPR, phys = u % CPR;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, MHA_LDS_PTR(void, qlds + 1024 * it), 16,
                                               (uint32_t)(row * RB + 16 * (phys ^ (row & KM))), 0,
                                               0, 0);
    }
  }

  // ---- key limits (mask decisions that are whole ranges) ----
  // The padding length is read before any K/V load: the buffers below end at
  // it, so key rows past a sequence's length are never fetched (they read as
  // zeros) and whatever that memory holds cannot reach a legal output
  // [MMHA 3.1: keys past the length do not take part].
  int kpad = Lk;
  if (p.kind & K_PADDING) {
    const int L = p.lens[b];
    kpad = L < 0 ? 0 : (L > Lk ? Lk : L);
    if ((L < 0 || L > Lk) && h == 0 && qblk == 0 && tid == 0) atomicOr(p.flags, F_BAD_LENGTH);
  }

  // ---- this wave's K/V rows and additive-mask entries of a step ----
  const __amdgpu_buffer_rsrc_t krs =
      make_rsrc((const char*)p.k + bh * (int64_t)Lk * RB, (uint32_t)((int64_t)kpad * RB));
  const __amdgpu_buffer_rsrc_t vrs =
      make_rsrc((const char*)p.v + bh * (int64_t)Lk * RB, (uint32_t)((int64_t)kpad * RB));
  // additive mask: 4 consecutive keys per lane and 16-key tile, one buffer per
  // workgroup (wave-uniform); rows past Lq fall outside it. Loads are
  // 16 bytes at 4-byte alignment; entries at keys >= Lk (the next row's) are
  // replaced by -inf when used.
  __amdgpu_buffer_rsrc_t ars;
  uint32_t arow_off = 0;
  if constexpr (ADD) {
    // based at the workgroup's first query row (64-bit arithmetic), so 32-bit
    // offsets only span its BM rows
    const int64_t slab = (p.kind & K_PER_HEAD) ? bh : (int64_t)b;  // shared, or per head
    const char* abase = (const char*)p.add + (slab * Lq + q0) * (int64_t)Lk * E;
    const int rows = Lq - q0 > BM ? BM : Lq - q0;
    ars = make_rsrc(abase, (uint32_t)((int64_t)rows * Lk * E));
    arow_off = (uint32_t)(qi - q0) * (uint32_t)Lk * E;
  }
  f32x4 am_raw[2];
  // Issue order per step: mask, K, V. LDS holds chunk (c ^ swizzle(row)) of a
  // row at position c; these loads are lane-ordered on the LDS side, so each
  // lane fetches the chunk that belongs at its position.
  auto issue_step = [&](int kb, int buf) {
    if constexpr (ADD) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        am_raw[j] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       ars, arow_off + (uint32_t)(kb + 16 * j + 4 * g) * E, 0, 0));
    }
    char* kl = wlds + buf * 2 * MAT_BYTES;
    char* vl = kl + MAT_BYTES;
#pragma unroll
    for (int it = 0; it < NLD; ++it) {
      const int u = it * 64 + lane;
      const int row = u / CPR, phys = u % CPR;
      const uint32_t goff = (uint32_t)(kb + row) * RB + 16 * (phys ^ (row & KM));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, MHA_LDS_PTR(void, kl + 1024 * it), 16, goff, 0,
                                               0, 0);
    }
#pragma unroll
    for (int it = 0; it < NLD; ++it) {
      const int u = it * 64 + lane;
      const int row = u / CPR, phys = u % CPR;
      const uint32_t goff = (uint32_t)(kb + row) * RB + 16 * (phys ^ (4 * ((row >> 2) & VM)));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, MHA_LDS_PTR(void, vl + 1024 * it), 16, goff, 0,
                                               0, 0);
    }
  };
  const int kend0 = causal ? min(min(q0 + BM, Lq), kpad) : kpad;
  const bool issued0 = ks * BN < kend0;
  if (issued0) issue_step(ks * BN, 0);

  int kend = kpad;  // keys >= kend are masked for every row of the block
  if (causal) kend = min(kend, min(q0 + BM - 1, Lq - 1) + 1);
  const int nsteps = (kend + BNT - 1) / BNT;

  // ---- Q operand (B of S^T = K Q^T): qf[sb] = c * Q[qi][16sb + 4g .. +3] ----
  f32x4 qf[NSB];
  if constexpr (!PRENORM) {
    if (issued0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(MA + 2 * NLD));  // this wave's Q share
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();                                                  // everyone's
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb)
      qf[sb] = *reinterpret_cast<const f32x4*>(qlds + n * RB + 16 * ((4 * sb + g) ^ (n & KM))) * c;
  } else {
    // token statistics over all F = H*D features [LNXA answer step 2]: 16
    // lanes per token, 4 tokens per wave pass, the mean, then the mean squared
    // deviation from it
    const int F = H * D;
    const int nch = F / 4;
    const int l16 = lane & 15;
    for (int r0 = 4 * ks; r0 < BM; r0 += 4 * NK) {
      const int rr = r0 + (lane >> 4);
      const int row = q0 + rr;
      const bool valid = row < Lq;
      const float* xr = (const float*)p.x + ((int64_t)b * Lq + (valid ? row : 0)) * (int64_t)F;
      float s = 0.f;
      if (valid)
        for (int ch = l16; ch < nch; ch += 16) {
          const f32x4 u = *reinterpret_cast<const f32x4*>(xr + 4 * ch);
          s += (u[0] + u[1]) + (u[2] + u[3]);
        }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o, 64);
      const float mean = s / (float)F;
      float v2 = 0.f;
      if (valid)
        for (int ch = l16; ch < nch; ch += 16) {
          const f32x4 u = *reinterpret_cast<const f32x4*>(xr + 4 * ch) - mean;
          v2 += (u[0] * u[0] + u[1] * u[1]) + (u[2] * u[2] + u[3] * u[3]);
        }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) v2 += __shfl_xor(v2, o, 64);
      const float rstd = 1.0f / sqrtf(v2 / (float)F + p.eps);
      if (l16 == 0) stat[rr] = make_float2(mean, rstd);
    }
    __syncthreads();
    const float2 ms = stat[n];
    const int64_t xoff = ((int64_t)b * Lq + (row_ok ? qi : 0)) * (int64_t)F + h * D;
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
      const int f = 16 * sb + 4 * g;
      const f32x4 xv = *reinterpret_cast<const f32x4*>((const float*)p.x + xoff + f);
      const f32x4 gv = *reinterpret_cast<const f32x4*>((const float*)p.gamma + h * D + f);
      const f32x4 bv = *reinterpret_cast<const f32x4*>((const float*)p.beta + h * D + f);
      qf[sb] = ((xv - ms.x) * ms.y * gv + bv) * c;  // rows past Lq: never stored
    }
  }

  // ---- per-lane LDS offsets ----
  // K operand: row n of a 16-key tile, logical chunk 4sb + g
  int koff[NSB];
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) koff[sb] = n * RB + 16 * ((4 * sb + g) ^ (n & KM));
  // V operand for k-slot r: row 4g + r of a 16-key tile, feature 16fb + n
  int voff[NSB];
#pragma unroll
  for (int fb = 0; fb < NSB; ++fb)
    voff[fb] = 4 * g * RB + 16 * (4 * (fb ^ (g & VM)) + (n >> 2)) + 4 * (n & 3);

  f32x4 o[NSB];
#pragma unroll
  for (int fb = 0; fb < NSB; ++fb) o[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  int ncomp = 0;

  for (int t = 0; t < nsteps; ++t) {
    const int buf = t & 1;
    const int kb0 = t * BNT + ks * BN;  // this wave's first key
    bool comp[2] = {kb0 < kend, kb0 + 16 < kend};
    // some key of the wave's range is masked for some row of the block
    const bool edge = (kb0 + BN > kpad) || (causal && kb0 + BN - 1 > q0);

    // additive mask in log2 units, masked entries -inf [MMHA 1: -inf before normalisation]
    float am[2][4];
    if constexpr (ADD) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bool any = false;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kb0 + 16 * j + 4 * g + r;
          // additive: log2 units, -inf stays -inf; keep-mask: 0 masks the key
          float a = (p.kind & K_KEEP) ? (am_raw[j][r] == 0.f ? -INFINITY : 0.f)
                                      : am_raw[j][r] * LOG2E;
          if (!row_ok || (edge && (key >= kpad || (causal && key > qi)))) a = -INFINITY;
          am[j][r] = a;
          any |= a != -INFINITY;
        }
        comp[j] = comp[j] && __ballot(any) != 0;
      }
    }

    // next step's loads for this wave, issued before this step's math
    const bool nxt = t + 1 < nsteps && kb0 + BNT < kend;
    if (nxt) issue_step(kb0 + BNT, buf ^ 1);

    const char* kl = wlds + buf * 2 * MAT_BYTES;
    const char* vl = kl + MAT_BYTES;
    // wait for this step's K (and everything before it), leaving V and the
    // next step in flight; then, before P V, for V
    auto wait_k = [&]() {
      if (nxt) __builtin_amdgcn_s_waitcnt(vmcnt_imm(NLD + MA + 2 * NLD));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(NLD));
    };
    auto wait_v = [&]() {
      if (nxt) __builtin_amdgcn_s_waitcnt(vmcnt_imm(MA + 2 * NLD));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    };

    // NS 16-key tiles starting at tile j0 (NS = 2: both, or the one that has
    // a legal pair); EDGE: some key is masked for some row
    auto tile = [&](auto ns_tag, auto edge_tag, int j0) {
      constexpr int NS = decltype(ns_tag)::value;
      constexpr bool EDGE = decltype(edge_tag)::value;
      // S^T = K Q^T, one accumulator chain per 16-key tile
      wait_k();
      f32x4 kf[NSB][NS];
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int j = 0; j < NS; ++j)
          kf[sb][j] = *reinterpret_cast<const f32x4*>(kl + 16 * (j0 + j) * RB + koff[sb]);
      f32x4 s[NS];
      float va[NS][4][NSB];
#pragma unroll
      for (int j = 0; j < NS; ++j) s[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int j = 0; j < NS; ++j)
            s[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[sb][j][r], qf[sb][r], s[j], 0, 0, 0);
        if (sb == (NSB - 1) / 2) {
          // V operands, read while the remaining MFMAs run (V lands after K)
          wait_v();
#pragma unroll
          for (int j = 0; j < NS; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
              for (int fb = 0; fb < NSB; ++fb)
                va[j][r][fb] =
                    *reinterpret_cast<const float*>(vl + (16 * (j0 + j) + r) * RB + voff[fb]);
        }
      }
      // mask, then the online softmax update [MAX 2.3, 4.2]; scores are in log2 units
      float mt = -INFINITY;
#pragma unroll
      for (int j = 0; j < NS; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float u = s[j][r];
          if constexpr (ADD) {
            u += am[j0 + j][r];
          } else if constexpr (EDGE) {
            const int key = kb0 + 16 * (j0 + j) + 4 * g + r;
            if (key >= kpad || (causal && key > qi)) u = -INFINITY;
          }
          s[j][r] = u;
          mt = fmaxf(mt, u);
        }
      mt = quad_max(mt);
      const float m_new = fmaxf(m_run, mt);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2_fast(m_run - m_use);
      m_run = m_new;
      float rs = 0.f;
#pragma unroll
      for (int j = 0; j < NS; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = exp2_fast(s[j][r] - m_use);  // -inf -> 0
          s[j][r] = e;
          rs += e;
        }
      l_run = l_run * alpha + rs;
      if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
        for (int fb = 0; fb < NSB; ++fb) o[fb] *= alpha;
      }
      // O^T += V^T P^T: k-slot r of lane (g, n) is key 4g + r of the 16-key tile
#pragma unroll
      for (int j = 0; j < NS; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int fb = 0; fb < NSB; ++fb)
            o[fb] = __builtin_amdgcn_mfma_f32_16x16x4f32(va[j][r][fb], s[j][r], o[fb], 0, 0, 0);
    };
    using One = std::integral_constant<int, 1>;
    using Two = std::integral_constant<int, 2>;
    ncomp += (int)comp[0] + (int)comp[1];
    if (comp[0] && comp[1]) {
      if (ADD || edge) tile(Two{}, std::true_type{}, 0);
      else tile(Two{}, std::false_type{}, 0);
    } else if (comp[0] || comp[1]) {
      tile(One{}, std::true_type{}, comp[0] ? 0 : 1);
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load of this wave outlives it

  // ---- debug counters: computed / skipped 16x16 tiles of this wave ----
  if (p.counters && lane == 0) {
    const int nsub = (Lk + 15) / 16;      // 16-key tiles across the key range
    const int npair = (nsub + 1) / 2;     // 32-key wave ranges; this wave owns index % NK == ks
    int mine = npair > ks ? 2 * ((npair - ks + NK - 1) / NK) : 0;
    if ((nsub & 1) && (npair - 1) % NK == ks) mine -= 1;  // the last range has one tile
    atomicAdd(p.counters + 0, (unsigned long long)ncomp);
    atomicAdd(p.counters + 1, (unsigned long long)(mine - ncomp));
  }

  // ---- merge the NK key splits (log-sum-exp); wave w finishes slices w, w+NK, .. ----
  l_run = quad_sum(l_run);
  mml[ks * 64 + lane] = make_float2(m_run, l_run);
#pragma unroll
  for (int fb = 0; fb < NSB; ++fb) mo[(ks * NSB + fb) * 64 + lane] = o[fb];
  __syncthreads();

  constexpr int MINE = (NSB + NK - 1) / NK;  // output slices per wave (some may be empty)
  float2 ml[NK];
  f32x4 po[MINE][NK];
#pragma unroll
  for (int k2 = 0; k2 < NK; ++k2) ml[k2] = mml[k2 * 64 + lane];
#pragma unroll
  for (int i = 0; i < MINE; ++i)
#pragma unroll
    for (int k2 = 0; k2 < NK; ++k2) {
      const int fb = ks + i * NK;
      po[i][k2] = fb < NSB ? mo[(k2 * NSB + fb) * 64 + lane] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  float M = -INFINITY;
#pragma unroll
  for (int k2 = 0; k2 < NK; ++k2) M = fmaxf(M, ml[k2].x);
  float L = 0.f, sk[NK];
#pragma unroll
  for (int k2 = 0; k2 < NK; ++k2) {
    sk[k2] = (M == -INFINITY) ? 0.f : exp2_fast(ml[k2].x - M);
    L += ml[k2].y * sk[k2];
  }
  const float inv = (L != 0.f) ? __builtin_amdgcn_rcpf(L) : 0.f;  // 1 ulp; exact for L = 1

  // ---- epilogue: O / l, pre-LN residual, flags, 16-byte stores ----
  bool nonfinite = false;
  char* orow;
  const char* rrow = nullptr;
  if constexpr (PRENORM) {
    const int64_t off = (((int64_t)b * Lq + (row_ok ? qi : 0)) * (H * D) + h * D) * E;
    orow = (char*)p.out + off;
    if (p.residual) rrow = (const char*)p.residual + off;
  } else {
    orow = (char*)p.out + ((bh * Lq + (row_ok ? qi : 0)) * D) * E;
  }
#pragma unroll
  for (int i = 0; i < MINE; ++i) {
    const int fb = ks + i * NK;
    if (fb >= NSB) break;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k2 = 0; k2 < NK; ++k2) acc += po[i][k2] * sk[k2];
    acc *= inv;
    const int d0 = 16 * fb + 4 * g;
    if constexpr (PRENORM) {
      if (rrow) acc += *reinterpret_cast<const f32x4*>(rrow + d0 * E);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) nonfinite |= !__builtin_isfinite(acc[r]);
    if (row_ok) *reinterpret_cast<f32x4*>(orow + d0 * E) = acc;
  }
  const bool fully = row_ok && !(L != 0.f);
  const unsigned long long fm = __ballot(fully && g == 0 && ks == 0);
  const unsigned long long nf = __ballot(nonfinite && row_ok);
  if (lane == 0) {
    const uint32_t fl = (fm ? F_FULLY_MASKED_ROW : 0u) | (nf ? F_NONFINITE : 0u);
    if (fl) atomicOr(p.flags, fl);
    if (p.counters && fm) atomicAdd(p.counters + 2, (unsigned long long)__popcll(fm));
  }
}

}  // namespace mha
