/*
 * mha.h -- C ABI of libmha: the fused masked multi-head attention forward on
 * AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *   [MMHA]  "masked multi head attention" CUDA implementation notes
 *           (2kiu.com/news/6063113)
 *   [MAX]   "Why attention must compute the max first" (gsyq.cn/news/340375)
 *   [LNXA]  "How to fuse cross-attention and layer-norm into a single CUDA
 *           kernel?" (cms365.cn question page)
 *
 * One call is one kernel launch on the caller's stream (decode: at most two,
 * see mha_decode_fwd; backward: two). Inside it, for every
 * (batch, head, query) row: S = scale * Q K^T, a causal / key-padding /
 * additive mask applied before normalisation, a numerically stable online
 * softmax (running row max, rescaled running sum), and P V accumulated in
 * registers; the S/P tile never reaches device memory.
 *
 * Conventions shared by every entry point
 *   - Tensors are device pointers to contiguous row-major memory owned by the
 *     caller; libmha never frees or retains them. Every tensor pointer must be
 *     16-byte aligned (4-byte for the int32 lengths).
 *   - dtype selects float32, float16 or bfloat16 for every floating tensor of
 *     the call (q, k, v, x, gamma, beta, residual, additive mask, out).
 *     Accumulation is float32 in all cases; the output is rounded to nearest
 *     even.
 *   - stream is a hipStream_t (NULL = the null stream). Calls are
 *     asynchronous: they return once the kernel is enqueued.
 *   - Validation is synchronous and happens before any HIP call: on any
 *     error status nothing is enqueued.
 *   - Conditions found on the device are ORed into one 32-bit flag word per
 *     device (MHA_FLAG_*), read with mha_get_flags.
 *   - out must not alias an input. residual may alias x.
 *   - Thread safety: calls from several host threads are safe; the flag word
 *     and the debug-counter pointer are shared per process/device.
 */
#ifndef MHA_H
#define MHA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MHA_F32 = 0, MHA_F16 = 1, MHA_BF16 = 2 } mha_dtype;

/* Mask kinds (bit flags). [MMHA 1, 3.1]: an upper-triangular (causal) mask,
 * a padding mask, or a custom mask; illegal logits become -inf before the
 * softmax normalisation [MAX 2.4].
 *   CAUSAL    key j is illegal for query i when j > i (top-left aligned, also
 *             when Lq != Lk) [MMHA 4.2 kernel skeleton].
 *   PADDING   mask points to int32 len[B] in device memory; keys j >= len[b]
 *             are illegal for every query of batch entry b. A length outside
 *             [0, Lk] acts clamped and raises MHA_FLAG_BAD_LENGTH.
 *   ADDITIVE  mask points to a [B,1,Lq,Lk] tensor of dtype, shared by all
 *             heads, added to the scaled logits; an entry equal to -inf marks
 *             an illegal key (a large finite negative value is only a bias).
 *   KEEP      mask points to a [B,1,Lq,Lk] tensor of dtype in which an entry
 *             equal to 0 (+0 or -0) marks an illegal key and any other value
 *             keeps it; the values are never added [MMHA 4.2 kernel: a mask
 *             value of 0.0 becomes -inf].
 *   PER_HEAD  with ADDITIVE or KEEP: the tensor is [B,H,Lq,Lk], one slab per
 *             head, instead of being shared by the heads.
 * PADDING, ADDITIVE and KEEP are mutually exclusive (one mask pointer);
 * CAUSAL combines with any of them. mask must be NULL unless one of them is
 * set. */
enum { MHA_MASK_NONE = 0, MHA_MASK_CAUSAL = 1, MHA_MASK_PADDING = 2, MHA_MASK_ADDITIVE = 4,
       MHA_MASK_KEEP = 8, MHA_MASK_PER_HEAD = 16 };

typedef enum {
    MHA_OK = 0,
    MHA_E_NULL = 1,        /* a required pointer is NULL */
    MHA_E_SHAPE = 2,       /* a negative dimension, or H*D beyond the supported width */
    MHA_E_DTYPE = 3,       /* dtype is not one of mha_dtype */
    MHA_E_MASK = 4,        /* unknown bits, more than one of PADDING/ADDITIVE/KEEP, PER_HEAD
                              without a mask tensor, or a mask given where none is used */
    MHA_E_UNSUPPORTED = 5, /* D not in {16, 32, 64, 128} */
    MHA_E_ALIGN = 6,       /* a tensor pointer is not 16-byte aligned (lengths: 4-byte) */
    MHA_E_OVERFLOW = 7,    /* an element count overflows int64, the grid exceeds 2^31-1, one
                              (b, h) head's K or V reaches 4 GiB ((Lk + 256) * D * esize >
                              2^32 - 1), or 32 rows of the additive mask do
                              (32 * (Lk + 256) * esize > 2^32 - 1): the kernels address
                              these through 32-bit buffer offsets */
    MHA_E_NO_DEVICE = 8,   /* no usable HIP device / runtime error while preparing */
    MHA_E_LAUNCH = 9,      /* the kernel launch itself failed */
    MHA_E_ARG = 10,        /* scale or eps not finite, scale < 0, eps < 0 */
    MHA_E_WORKSPACE = 11,  /* the decode workspace is NULL, not 16-byte aligned or smaller
                              than mha_decode_workspace_size reports */
    MHA_E_NOT_INITIALIZED = 12, /* an allocation-free entry point was called on a device
                                   where mha_init has not run */
    MHA_E_SCRATCH = 13     /* an allocation-free call needs more scratch than
                              MHA_NOALLOC_SCRATCH_BYTES */
} mha_status;

/* Size of the static scratch array behind the allocation-free entry points:
 * one copy per GPU the library runs on, held until the process ends. */
#define MHA_NOALLOC_SCRATCH_BYTES (16u << 20)

/* Device flag word bits (ORed by kernels, cleared by mha_get_flags). */
enum {
    MHA_FLAG_FULLY_MASKED_ROW = 1, /* a valid query row had no legal key: its output is 0
                                      (pre-LN: the residual) [LNXA knowledge points: an
                                      error flag is raised when the softmax goes bad] */
    MHA_FLAG_NONFINITE = 2,        /* a stored output value is NaN or infinite */
    MHA_FLAG_BAD_LENGTH = 4        /* a padding length lies outside [0, Lk] */
};

/* Set-up of the current device (no passage: library housekeeping).
 * Allocates (once) and zeroes the device's flag word, and looks up (once) the
 * device address of its copy of the allocation-free entry points' static
 * scratch array. Optional for the allocating entry points, whose first call
 * on a device does the flag word otherwise; required, once per device, before
 * mha_decode_fwd_noalloc. Call it before capturing launches into a HIP graph
 * so that nothing is allocated during capture. */
mha_status mha_init(void);

/* Masked multi-head self/cross attention forward [MMHA 2, 4.2; MAX 2.4].
 *   q    [B,H,Lq,D]   queries
 *   k, v [B,H,Lk,D]   keys and values
 *   mask see the mask kinds above
 *   out  [B,H,Lq,D]   o[b,h,i,:] = sum_j softmax_j(scale*q.k_j (+ mask)) v_j over
 *                     the legal keys j; 0 for a row with no legal key.
 *   scale >= 0, finite (1/sqrt(D) is the usual choice [MAX 5.2]).
 * B, H or Lq equal to 0 is an empty call (MHA_OK, nothing enqueued). Lk may
 * be 0: every row is then fully masked. Other sizes must be >= 0;
 * D must be 16, 32, 64 or 128. */
mha_status mha_fwd(const void* q, const void* k, const void* v, const void* mask,
                   unsigned mask_kind, int B, int H, int Lq, int Lk, int D, float scale,
                   mha_dtype dtype, void* stream, void* out);

/* Pre-LayerNorm cross-attention with the residual added in the epilogue
 * [LNXA answer steps 1-4]: for token (b,i) the features x[b,i,:] (H*D of
 * them) are normalised with their mean and biased variance,
 * y = (x - mean) / sqrt(var + eps) * gamma + beta, and Q for head h is
 * y[h*D:(h+1)*D]; then attention over k, v as in mha_fwd, and
 *   out[b,i,h*D+d] = attention + residual[b,i,h*D+d]   (residual may be NULL).
 *   x, residual, out [B,Lq,H*D];  gamma, beta [H*D];  k, v [B,H,Lk,D].
 *   eps >= 0 and finite. H*D must not exceed 65536.
 * A fully masked row stores the residual (or 0). */
mha_status mha_prenorm_cross_fwd(const void* x, const void* k, const void* v, const void* mask,
                                 unsigned mask_kind, const void* gamma, const void* beta,
                                 float eps, const void* residual, int B, int H, int Lq, int Lk,
                                 int D, float scale, mha_dtype dtype, void* stream, void* out);

/* mha_prenorm_cross_fwd with a caller-owned workspace [LNXA answer steps
 * 1-4; mixed precision per its knowledge points]. Same arguments, results
 * and status codes, plus:
 *   workspace        device memory of at least
 *                    mha_prenorm_cross_workspace_size(B,H,Lq,Lk,D,dtype) bytes,
 *                    16-byte aligned, owned by the caller; its contents need
 *                    no initialisation and are overwritten.
 *   workspace_bytes  its size.
 * For bfloat16 calls without a mask tensor (ADDITIVE or KEEP) and with
 * Lk > 0 the call enqueues three kernels: one writes float16 copies of k and
 * v into the workspace (nearest-even rounding, the values the attention
 * kernel otherwise rewrites tile by tile in LDS), per quarter of each head
 * whether any value exceeds 65504 in magnitude, and each token's LayerNorm
 * mean and 1/sqrt(var + eps); then the attention kernel runs on the copies
 * and those statistics for the heads without such a value, and on k, v and
 * x themselves (as mha_prenorm_cross_fwd) for the others. Every other call ignores the workspace and runs
 * as mha_prenorm_cross_fwd. A missing, misaligned or short workspace where
 * one is needed is MHA_E_WORKSPACE. Calls that overlap in time must not share
 * a workspace. */
mha_status mha_prenorm_cross_fwd_ws(const void* x, const void* k, const void* v, const void* mask,
                                    unsigned mask_kind, const void* gamma, const void* beta,
                                    float eps, const void* residual, int B, int H, int Lq, int Lk,
                                    int D, float scale, mha_dtype dtype, void* workspace,
                                    size_t workspace_bytes, void* stream, void* out);

/* Workspace bytes mha_prenorm_cross_fwd_ws needs for these sizes: 0 unless
 * dtype is bfloat16 and B, H, Lq, Lk > 0; then two float16 copies of a
 * [B,H,Lk,D] tensor, B*H*4 int32 flags and B*Lq float32 pairs, each part
 * rounded up to 256 bytes. Pure host computation; MHA_E_NULL, MHA_E_DTYPE,
 * MHA_E_SHAPE, MHA_E_UNSUPPORTED or MHA_E_OVERFLOW as mha_prenorm_cross_fwd.
 * No passage: the pages' kernels take no workspace. */
mha_status mha_prenorm_cross_workspace_size(int B, int H, int Lq, int Lk, int D, mha_dtype dtype,
                                            size_t* bytes);

/* The device error flag [LNXA knowledge points: a global flag the kernel
 * raises when the softmax goes bad, read back by the host]. Synchronise
 * stream, then copy the current device's flag word to *flags; clear != 0
 * resets it to 0 afterwards. The word is per device, not per stream: launches
 * on other streams that have not finished are not seen. */
mha_status mha_get_flags(void* stream, uint32_t* flags, int clear);

/* Row softmax of a materialised score tensor [MAX 2.1: the row-softmax
 * workload; 2.3, 4.2: the online max/sum and the fused one-pass kernel]:
 *   s, p  [rows, cols] in dtype, contiguous (a row = cols consecutive values)
 *   p[r,j] = exp(scale*s[r,j] - m_r) / sum_k exp(scale*s[r,k] - m_r), with m_r
 *   the row maximum; computed in fp32, rounded to nearest even on the store.
 * An entry equal to -inf is a masked position: its weight is 0 whatever the
 * scale. A row whose entries are all -inf is written as zeros and raises
 * MHA_FLAG_FULLY_MASKED_ROW; a NaN score makes the row's unmasked weights NaN;
 * a non-finite stored weight raises MHA_FLAG_NONFINITE (flags as mha_get_flags).
 * scale >= 0, finite. rows or cols equal to 0 is an empty call. s and p must
 * be aligned to the element size; 16-byte aligned rows of up to 4096
 * (16-bit) or 2048 (float32) values take one read and one write of HBM,
 * others two reads. p may equal s (in place); any other overlap is undefined.
 * Asynchronous on `stream` like mha_fwd; the caller owns both tensors. */
mha_status mha_softmax_rows(const void* s, void* p, int64_t rows, int cols, float scale,
                            mha_dtype dtype, void* stream);

/* Decode: one new query row per (batch, head) against a key/value cache
 * [MMHA 6.1: the kernel called from an inference engine's cache update with
 * one new token per sequence; MAX 2.3-2.4: the online softmax, whose running
 * (maximum, sum, output) states of disjoint key ranges merge exactly].
 *   q     [B,H,D]      the new token's queries
 *   k, v  [B,H,Lk,D]   the caches; Lk is their capacity
 *   lens  int32 [B] in device memory, or NULL: keys j >= lens[b] are illegal
 *         for sequence b (the padding mask of mha_fwd with Lq = 1). A length
 *         outside [0, Lk] acts clamped and raises MHA_FLAG_BAD_LENGTH.
 *   out   [B,H,D]      o[b,h,:] = sum_j softmax_j(scale * q.k_j) v_j over the
 *                      legal keys; 0 (and MHA_FLAG_FULLY_MASKED_ROW) for a
 *                      sequence with no legal key.
 *   lse   float32 [B,H] or NULL: log(sum_j exp(scale * q.k_j)) over the legal
 *         keys (natural log; -inf for a row with no legal key). It is the
 *         normaliser that merges this result with attention over other keys.
 *   workspace, workspace_bytes: device scratch for the per-split partial
 *         results, at least mha_decode_workspace_size(...) bytes, 16-byte
 *         aligned, owned by the caller; NULL is allowed when that size is 0.
 *         Its contents need no initialisation and are meaningless afterwards.
 *         Calls that overlap in time must not share a workspace.
 * The keys of a head are split into chunks processed by separate waves when
 * that fills the GPU better; then a second, small kernel merges the chunks
 * (two launches on `stream`), otherwise one launch writes the result.
 * Validation, errors and flags as mha_fwd; B or H equal to 0 is an empty
 * call; Lk may be 0 (every row fully masked). */
mha_status mha_decode_fwd(const void* q, const void* k, const void* v, const int32_t* lens,
                          int B, int H, int Lk, int D, float scale, mha_dtype dtype,
                          void* workspace, size_t workspace_bytes, void* stream, void* out,
                          float* lse);

/* mha_decode_fwd without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc). Same
 * arguments (minus the workspace), results, validation, flags and launches as
 * mha_decode_fwd; the per-split partial results go to a static device array
 * of MHA_NOALLOC_SCRATCH_BYTES per GPU instead.
 *   - mha_init must have run on the current device first, otherwise
 *     MHA_E_NOT_INITIALIZED (nothing is enqueued).
 *   - A call whose mha_decode_workspace_size exceeds MHA_NOALLOC_SCRATCH_BYTES
 *     fails with MHA_E_SCRATCH before any HIP call.
 *   - No hipMalloc, hipFree or other allocating routine is called.
 *   - Every call on a GPU shares that GPU's one scratch array: calls that
 *     overlap in time on one GPU (other streams, other threads) race and give
 *     undefined results. Calls ordered on one stream are safe; the array keeps
 *     the last call's contents, which no call reads before writing. */
mha_status mha_decode_fwd_noalloc(const void* q, const void* k, const void* v,
                                  const int32_t* lens, int B, int H, int Lk, int D, float scale,
                                  mha_dtype dtype, void* stream, void* out, float* lse);

/* *bytes = MHA_NOALLOC_SCRATCH_BYTES (no passage: the limit of the
 * allocation-free entry points). */
mha_status mha_noalloc_scratch_bytes(size_t* bytes);

/* Workspace bytes mha_decode_fwd needs for these sizes (0 when every head is
 * one split); no passage: the size of the split plan's partial results. Pure
 * host computation: no device is touched. Fails with the same shape/dtype
 * status codes as mha_decode_fwd. */
mha_status mha_decode_workspace_size(int B, int H, int Lk, int D, mha_dtype dtype,
                                     size_t* bytes);

/* Backward of mha_fwd: the gradients of the attention output for an
 * upstream gradient dout [MAX 3.3: the softmax Jacobian dp_j/ds_k =
 * p_j (delta_jk - p_k); the row maximum carries no gradient]:
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(P * dP)),
 *   dQ = scale dS K,  dK = scale dS^T Q,   with P the forward's softmax
 *   weights over the legal keys (rebuilt in the kernels from each row's
 *   log-sum-exp; 0 for masked keys). The forward's output is not needed.
 *   q, dout, dq [B,H,Lq,D];  k, v, dk, dv [B,H,Lk,D]
 *   mask, mask_kind: every mask kind of mha_fwd (causal, padding lengths,
 *         additive or keep tensors, shared or PER_HEAD) with the same rules;
 *         a mask is a constant of the forward and gets no gradient.
 *   dtype: MHA_F32, MHA_F16 or MHA_BF16 (all on MFMA, except float32 at
 *         D = 128, which runs on the vector ALUs, one wave per row); D must be
 *         16, 32, 64 or 128.
 *   workspace: at least mha_bwd_workspace_size(...) bytes, 16-byte aligned,
 *         owned by the caller (each row's log-sum-exp and rowsum(P * dP));
 *         no initialisation needed; overlapping calls must not share it.
 * A fully masked query row has dq = 0 and contributes nothing to dk, dv; it
 * raises MHA_FLAG_FULLY_MASKED_ROW. Two launches on `stream` (dq, then dk and
 * dv). Validation, errors and flags as mha_fwd. */
mha_status mha_bwd(const void* q, const void* k, const void* v, const void* dout,
                   const void* mask, unsigned mask_kind, int B, int H, int Lq, int Lk, int D,
                   float scale, mha_dtype dtype, void* workspace, size_t workspace_bytes,
                   void* stream, void* dq, void* dk, void* dv);

/* Workspace bytes mha_bwd needs: 8 * B * H * Lq (no passage: the size of the
 * row statistics the two backward kernels exchange). Pure host computation. */
mha_status mha_bwd_workspace_size(int B, int H, int Lq, mha_dtype dtype, size_t* bytes);

/* Debug counters [MAX 6: count executions with device atomics]: a device
 * pointer to 3 uint64 values, or NULL to stop counting. While set, every
 * launch adds (tiles computed, tiles skipped, valid rows with no legal key).
 * A tile is mha_tile_config's rows x keys block, aligned at multiples of its
 * size; it is skipped when every pair in it is masked [MMHA 2]. The pointer
 * is process-wide; the caller owns and zeroes the memory. */
mha_status mha_set_debug_counters(uint64_t* dev_counters);

/* Tile of the skip decision for a dtype and D: *rows query rows by *keys keys
 * [MMHA 2: whole tiles of masked positions are skipped; the tile size is this
 * library's, the pages' kernels use 16 x 32]. Pure host computation. */
mha_status mha_tile_config(mha_dtype dtype, int D, unsigned mask_kind, int* rows, int* keys);

/* Human-readable name of a status code (static string). No passage: the
 * pages report launch errors with printf [MMHA 4.3]; here they are codes. */
const char* mha_status_str(mha_status s);

#ifdef __cplusplus
}
#endif

#endif /* MHA_H */
