/*
 * mha_oracle.c -- plain, slow, fp64 CPU reference for the masked multi-head
 * attention forward and its pre-LayerNorm cross-attention variant.
 *
 * TEST INFRASTRUCTURE. Only the test-suite, the package smoke check and the
 * CPU-baseline leg of the benchmark load this library. The GPU library never
 * links it, calls it or shares code with it.
 *
 * Sources (web pages; cited by title and section):
 *   [MMHA]  "masked multi head attention" CUDA implementation notes
 *           (2kiu.com/news/6063113)
 *   [MAX]   "Why attention must compute the max first" -- naive, two-pass,
 *           online and fused-online softmax (gsyq.cn/news/340375)
 *   [LNXA]  "How to fuse cross-attention and layer-norm into a single CUDA
 *           kernel?" (cms365.cn question page)
 *
 * What it computes is the plain definition, written out with no blocking,
 * fusion or reordering:
 *   s_j   = scale * <q_i, k_j>                    [MAX 5.2: divide QK^T by sqrt(d_k)]
 *   mask  : an illegal position gets -inf before normalisation
 *           (causal j > i, key padding j >= len_b, an additive mask whose
 *           -inf entries mark illegal keys, or a keep-mask whose 0 entries
 *           do; a mask tensor is shared by the heads or, PER_HEAD, one per
 *           head)                                 [MMHA 1, 3.1, 4.2; MAX 2.4, 4.1]
 *   p_j   = exp(s_j - max) / sum exp(s - max)    three separate passes, the
 *                                                 naive softmax of [MAX 2.1]
 *   o_i   = sum_j p_j v_j                        [MAX 4.1 fused_attn; LNXA
 *                                                 knowledge points: S, P, O chain]
 * Row softmax over a materialised score tensor (the standalone softmax
 * workload of [MAX 2.1]): p_j = exp(c*s_j - max) / sum exp(c*s - max) per row,
 * the same three passes.
 * Decode (one new token per sequence against its key/value cache, the
 * llama.cpp embedding of [MMHA 6.1]): the same row with Lq = 1 and per-sequence
 * key lengths; the query is the newest position, so every cached key up to the
 * length is legal. It also returns the row's log-sum-exp, m + log(sum exp(s -
 * m)), the normaliser of the online softmax [MAX 2.4].
 * Backward (the gradients of the forward for an upstream gradient dO): the
 * softmax Jacobian dp_j/ds_k = p_j (delta_jk - p_k) of [MAX 3.3], chained
 * through S = scale * Q K^T and O = P V; the row maximum carries no gradient
 * (the weights do not depend on it, [MAX 3.3]).
 * Readings where the pages are silent or garbled (each is listed in the design
 * notes of the repository):
 *   - a row with no legal key produces o = 0 and raises FLAG_FULLY_MASKED_ROW
 *     (the pages raise a global error flag on a bad softmax [LNXA knowledge
 *     points, further thoughts]);
 *   - the additive mask is added after scaling and is not itself scaled; only
 *     an entry equal to -inf counts as a masked decision;
 *   - padding lengths outside [0, Lk] raise FLAG_BAD_LENGTH and act clamped;
 *   - pre-LayerNorm normalises each token over all H*D features with the
 *     biased variance and eps inside the square root, then applies gamma and
 *     beta; Q for head h is that token's slice [h*D, (h+1)*D)
 *     [LNXA answer step 2], held in the call's working precision (rounded
 *     to float16/bfloat16/float32, the FP16/BF16 mixed precision of the LNXA
 *     knowledge points); the residual is added after attention
 *     [LNXA answer step 4].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_CAUSAL = 1, OR_PADDING = 2, OR_ADDITIVE = 4, OR_KEEP = 8, OR_PER_HEAD = 16 };
enum { OR_TENSOR = OR_ADDITIVE | OR_KEEP }; /* kinds that read a mask tensor */
enum { OR_FLAG_FULLY_MASKED_ROW = 1, OR_FLAG_NONFINITE = 2, OR_FLAG_BAD_LENGTH = 4 };

int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* The mask decision for query i, key j of batch entry b.
 * causal: future keys (j > i) are illegal [MMHA 4.2 kernel: row < col is masked].
 * padding: keys at or beyond the sequence length are illegal [MMHA 3.1].
 * additive: an entry of -inf marks an illegal key [MMHA 1: illegal logits are
 * set to negative infinity before softmax normalisation].
 * keep: an entry equal to 0 marks an illegal key, any other value keeps it
 * [MMHA 4.2 kernel: a mask value of 0.0 becomes -inf]; keep values are never
 * added to the logits.
 * `m` is the mask tensor's entry for (i, j) (0 when there is none). */
static int is_masked(unsigned kind, int64_t i, int64_t j, int64_t len_b, double m) {
    if ((kind & OR_CAUSAL) && j > i) return 1;
    if ((kind & OR_PADDING) && j >= len_b) return 1;
    if ((kind & OR_ADDITIVE) && isinf(m) && m < 0) return 1;
    if ((kind & OR_KEEP) && m == 0.0) return 1;
    return 0;
}

/* Row i of the mask tensor for batch entry b and head h: [B,1,Lq,Lk], shared
 * by the heads, or [B,H,Lq,Lk] with PER_HEAD. NULL without a mask tensor. */
static const double* mask_row(const double* mask, unsigned kind, int64_t b, int64_t h, int H,
                              int Lq, int Lk, int64_t i) {
    if (!(kind & OR_TENSOR)) return NULL;
    int64_t slab = (kind & OR_PER_HEAD) ? b * H + h : b;
    return mask + (slab * Lq + i) * Lk;
}

static uint32_t length_flags(unsigned kind, const int32_t* lens, int B, int Lk) {
    uint32_t f = 0;
    if (kind & OR_PADDING)
        for (int b = 0; b < B; ++b)
            if (lens[b] < 0 || lens[b] > Lk) f |= OR_FLAG_BAD_LENGTH;
    return f;
}

/* One attention row: scores, mask, then the naive three-pass softmax of
 * [MAX 2.1] (pass 1 the row max, pass 2 the sum of exp(s - max), pass 3 the
 * normalised weights applied to V). s is caller scratch of length Lk; p, when
 * not NULL, receives the softmax weights (0 for masked keys). */
static uint32_t attention_row(const double* q, const double* K, const double* V,
                              int Lk, int D, double scale, unsigned kind,
                              int64_t i, int64_t len_b, const double* addrow,
                              double* s, double* p, double* o) {
    uint32_t flags = 0;
    /* scores and mask decisions */
    for (int j = 0; j < Lk; ++j) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += q[d] * K[(int64_t)j * D + d];
        double add = (kind & OR_TENSOR) ? addrow[j] : 0.0;
        if (is_masked(kind, i, j, len_b, add)) {
            s[j] = -INFINITY;
        } else {
            s[j] = scale * dot;
            if (kind & OR_ADDITIVE) s[j] += add;
        }
    }
    /* pass 1: maximum over legal keys (a masked key holds -inf) */
    double m = -INFINITY;
    for (int j = 0; j < Lk; ++j)
        if (!(s[j] <= m)) m = s[j]; /* a NaN score propagates */
    if (m == -INFINITY) {
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (p) for (int j = 0; j < Lk; ++j) p[j] = 0.0;
        return OR_FLAG_FULLY_MASKED_ROW;
    }
    /* pass 2: normaliser */
    double z = 0.0;
    for (int j = 0; j < Lk; ++j)
        if (s[j] != -INFINITY) z += exp(s[j] - m);
    /* pass 3: weights and the weighted sum of V over the legal keys */
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    for (int j = 0; j < Lk; ++j) {
        if (s[j] == -INFINITY) {
            if (p) p[j] = 0.0;
            continue;
        }
        double w = exp(s[j] - m) / z;
        if (p) p[j] = w;
        for (int d = 0; d < D; ++d) o[d] += w * V[(int64_t)j * D + d];
    }
    for (int d = 0; d < D; ++d)
        if (!isfinite(o[d])) flags |= OR_FLAG_NONFINITE;
    return flags;
}

/* Full forward: q [B,H,Lq,D], k/v [B,H,Lk,D], out [B,H,Lq,D]; lens [B] (PADDING);
 * add [B,1,Lq,Lk] (ADDITIVE, broadcast over heads). Returns the flag word. */
uint32_t oracle_mha_fwd(const double* q, const double* k, const double* v,
                        const int32_t* lens, const double* add, unsigned kind,
                        int B, int H, int Lq, int Lk, int D, double scale, double* out) {
    uint32_t flags = length_flags(kind, lens, B, Lk);
    int64_t nrows = (int64_t)B * H * Lq;
#pragma omp parallel reduction(| : flags)
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Lk > 0 ? Lk : 1));
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t i = r % Lq, bh = r / Lq, b = bh / H, h = bh % H;
            const double* addrow = mask_row(add, kind, b, h, H, Lq, Lk, i);
            int64_t len_b = (kind & OR_PADDING) ? lens[b] : Lk;
            flags |= attention_row(q + r * D, k + bh * Lk * D, v + bh * Lk * D, Lk, D, scale,
                                   kind, i, len_b, addrow, s, NULL, out + r * D);
        }
        free(s);
    }
    return flags;
}

/* Selected rows only: rows holds n triples (b, h, i); out receives n*D values. */
uint32_t oracle_mha_rows(const double* q, const double* k, const double* v,
                         const int32_t* lens, const double* add, unsigned kind,
                         int B, int H, int Lq, int Lk, int D, double scale,
                         const int64_t* rows, int64_t n, double* out) {
    uint32_t flags = length_flags(kind, lens, B, Lk);
#pragma omp parallel reduction(| : flags)
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Lk > 0 ? Lk : 1));
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < n; ++r) {
            int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
            int64_t bh = b * H + h;
            const double* addrow = mask_row(add, kind, b, h, H, Lq, Lk, i);
            int64_t len_b = (kind & OR_PADDING) ? lens[b] : Lk;
            flags |= attention_row(q + (bh * Lq + i) * D, k + bh * Lk * D, v + bh * Lk * D, Lk,
                                   D, scale, kind, i, len_b, addrow, s, NULL, out + r * D);
        }
        free(s);
    }
    return flags;
}

/* Softmax weights of one row (b, h, i): p receives Lk values. */
uint32_t oracle_probs_row(const double* q, const double* k, const int32_t* lens,
                          const double* add, unsigned kind, int B, int H, int Lq, int Lk,
                          int D, double scale, int b, int h, int i, double* p) {
    double* s = (double*)malloc(sizeof(double) * (size_t)(Lk > 0 ? Lk : 1));
    double* o = (double*)calloc((size_t)D, sizeof(double));
    /* V = 0 keeps the row's weights the only output of interest */
    double* vz = (double*)calloc((size_t)Lk * D + 1, sizeof(double));
    int64_t bh = (int64_t)b * H + h;
    const double* addrow = mask_row(add, kind, b, h, H, Lq, Lk, i);
    int64_t len_b = (kind & OR_PADDING) ? lens[b] : Lk;
    uint32_t f = attention_row(q + (bh * Lq + i) * D, k + bh * Lk * D, vz, Lk, D, scale, kind,
                               i, len_b, addrow, s, p, o);
    free(vz);
    free(o);
    free(s);
    return f | length_flags(kind, lens, B, Lk);
}

/* Pre-LayerNorm of one token of F features [LNXA answer step 2]: mean, biased
 * variance, (x - mean) / sqrt(var + eps), then gamma and beta. */
static void layernorm_token(const double* x, const double* gamma, const double* beta,
                            double eps, int F, double* y) {
    double mean = 0.0;
    for (int f = 0; f < F; ++f) mean += x[f];
    mean /= F;
    double var = 0.0;
    for (int f = 0; f < F; ++f) var += (x[f] - mean) * (x[f] - mean);
    var /= F;
    double inv = 1.0 / sqrt(var + eps);
    for (int f = 0; f < F; ++f) y[f] = (x[f] - mean) * inv * gamma[f] + beta[f];
}

void oracle_layernorm(const double* x, const double* gamma, const double* beta, double eps,
                      int64_t ntok, int F, double* y) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < ntok; ++t)
        layernorm_token(x + t * F, gamma, beta, eps, F, y + t * F);
}

/* Pre-LN cross-attention for selected rows: rows holds n triples (b, i, h);
 * out receives n*D values out[b, i, h*D + d] = attention + residual.
 * x, residual [B,Lq,H*D]; k, v [B,H,Lk,D]; gamma, beta [H*D]. residual may be NULL.
 * The normalised query enters the attention exactly as computed, in fp64: the
 * plain definition has no rounding step between the LayerNorm and the scores
 * [LNXA answer step 2: Q = LN(x) feeds S = Q K^T]. */
uint32_t oracle_prenorm_rows(const double* x, const double* k, const double* v,
                             const int32_t* lens, const double* add, unsigned kind,
                             const double* gamma, const double* beta, double eps,
                             const double* residual, int B, int H, int Lq, int Lk, int D,
                             double scale, const int64_t* rows, int64_t n, double* out) {
    uint32_t flags = length_flags(kind, lens, B, Lk);
    int F = H * D;
#pragma omp parallel reduction(| : flags)
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Lk > 0 ? Lk : 1));
        double* y = (double*)malloc(sizeof(double) * (size_t)F);
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < n; ++r) {
            int64_t b = rows[3 * r], i = rows[3 * r + 1], h = rows[3 * r + 2];
            int64_t tok = b * Lq + i, bh = b * H + h;
            layernorm_token(x + tok * F, gamma, beta, eps, F, y);
            const double* addrow = mask_row(add, kind, b, h, H, Lq, Lk, i);
            int64_t len_b = (kind & OR_PADDING) ? lens[b] : Lk;
            double* o = out + r * D;
            flags |= attention_row(y + h * D, k + bh * Lk * D, v + bh * Lk * D, Lk, D, scale,
                                   kind, i, len_b, addrow, s, NULL, o);
            if (residual)
                for (int d = 0; d < D; ++d) o[d] += residual[tok * F + h * D + d];
            for (int d = 0; d < D; ++d)
                if (!isfinite(o[d])) flags |= OR_FLAG_NONFINITE;
        }
        free(y);
        free(s);
    }
    return flags;
}

/* Full pre-LN cross-attention: out [B,Lq,H*D]. */
uint32_t oracle_prenorm_cross_fwd(const double* x, const double* k, const double* v,
                                  const int32_t* lens, const double* add, unsigned kind,
                                  const double* gamma, const double* beta, double eps,
                                  const double* residual, int B, int H, int Lq, int Lk, int D,
                                  double scale, double* out) {
    int64_t n = (int64_t)B * Lq * H;
    int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * 3 * (size_t)(n > 0 ? n : 1));
    for (int64_t r = 0; r < n; ++r) {
        rows[3 * r] = r / ((int64_t)Lq * H);
        rows[3 * r + 1] = (r / H) % Lq;
        rows[3 * r + 2] = r % H;
    }
    /* row r = ((b*Lq + i)*H + h) lands at out + r*D, i.e. out[b, i, h*D + d] */
    uint32_t f = oracle_prenorm_rows(x, k, v, lens, add, kind, gamma, beta, eps, residual,
                                     B, H, Lq, Lk, D, scale, rows, n, out);
    free(rows);
    return f;
}

/* Mask decisions as bytes: dec [B,Hm,Lq,Lk], 1 = masked, where Hm = H with a
 * per-head mask tensor (PER_HEAD) and 1 otherwise (the heads share it). */
void oracle_mask_decisions(const int32_t* lens, const double* add, unsigned kind, int B, int H,
                           int Lq, int Lk, uint8_t* dec) {
    int Hm = (kind & OR_PER_HEAD) ? H : 1;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < Hm; ++h)
            for (int64_t i = 0; i < Lq; ++i) {
                const double* mrow = mask_row(add, kind, b, h, H, Lq, Lk, i);
                int64_t len_b = (kind & OR_PADDING) ? lens[b] : Lk;
                for (int64_t j = 0; j < Lk; ++j)
                    dec[((b * Hm + h) * Lq + i) * Lk + j] =
                        (uint8_t)is_masked(kind, i, j, len_b, mrow ? mrow[j] : 0.0);
            }
}

/* Number of legal (b, h, i, j) pairs: the work that counts as effective. */
int64_t oracle_unmasked_pairs(const int32_t* lens, const double* add, unsigned kind, int B,
                              int H, int Lq, int Lk) {
    int Hm = (kind & OR_PER_HEAD) ? H : 1;
    int64_t cnt = 0;
#pragma omp parallel for reduction(+ : cnt) schedule(static)
    for (int64_t bhi = 0; bhi < (int64_t)B * Hm * Lq; ++bhi) {
        int64_t i = bhi % Lq, bh = bhi / Lq, b = bh / Hm, h = bh % Hm;
        int64_t len_b = (kind & OR_PADDING) ? lens[b] : Lk;
        const double* mrow = mask_row(add, kind, b, h, H, Lq, Lk, i);
        for (int64_t j = 0; j < Lk; ++j)
            if (!is_masked(kind, i, j, len_b, mrow ? mrow[j] : 0.0)) cnt++;
    }
    return cnt * (H / Hm);
}

/* Tiles of rm query rows by bn keys (aligned at multiples of rm and bn) that
 * hold at least one legal pair ("computed") or none ("skipped"), summed over
 * b and h: the whole-work skipping of [MMHA 2], decided by brute force over
 * the mask decisions. counts[0] = computed, counts[1] = skipped. */
void oracle_tile_counts(const int32_t* lens, const double* add, unsigned kind, int B, int H,
                        int Lq, int Lk, int rm, int bn, int64_t* counts) {
    int Hm = (kind & OR_PER_HEAD) ? H : 1;
    int64_t comp = 0, skip = 0;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < Hm; ++h) {
            int64_t len_b = (kind & OR_PADDING) ? lens[b] : Lk;
            for (int64_t i0 = 0; i0 < Lq; i0 += rm)
                for (int64_t j0 = 0; j0 < Lk; j0 += bn) {
                    int legal = 0;
                    for (int64_t i = i0; i < i0 + rm && i < Lq && !legal; ++i) {
                        const double* mrow = mask_row(add, kind, b, h, H, Lq, Lk, i);
                        for (int64_t j = j0; j < j0 + bn && j < Lk; ++j)
                            if (!is_masked(kind, i, j, len_b, mrow ? mrow[j] : 0.0)) {
                                legal = 1;
                                break;
                            }
                    }
                    if (legal) comp++; else skip++;
                }
        }
    counts[0] = comp * (H / Hm);
    counts[1] = skip * (H / Hm);
}

/* Rows with no legal key, summed over b and h. */
int64_t oracle_fully_masked_rows(const int32_t* lens, const double* add, unsigned kind, int B,
                                 int H, int Lq, int Lk) {
    int Hm = (kind & OR_PER_HEAD) ? H : 1;
    int64_t cnt = 0;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < Hm; ++h) {
            int64_t len_b = (kind & OR_PADDING) ? lens[b] : Lk;
            for (int64_t i = 0; i < Lq; ++i) {
                const double* mrow = mask_row(add, kind, b, h, H, Lq, Lk, i);
                int legal = 0;
                for (int64_t j = 0; j < Lk && !legal; ++j)
                    legal = !is_masked(kind, i, j, len_b, mrow ? mrow[j] : 0.0);
                if (!legal) cnt++;
            }
        }
    return cnt * (H / Hm);
}

/* Row softmax of a materialised score matrix [MAX 2.1: the row-softmax
 * workload; 2.2-2.3 for what the online form must reproduce]: for each of
 * `rows` rows of `cols` scores, p_j = exp(scale*s_j - m) / sum_k exp(scale*s_k - m)
 * with m the row maximum, in three passes (max, normaliser, weights). An
 * entry equal to -inf is a masked position (weight 0, whatever the scale); a
 * row with every entry masked gets zeros and FLAG_FULLY_MASKED_ROW; a
 * non-finite weight raises FLAG_NONFINITE. Returns the flag word. */
uint32_t oracle_softmax_rows(const double* s, int64_t rows, int cols, double scale, double* p) {
    uint32_t flags = 0;
#pragma omp parallel for schedule(static) reduction(| : flags)
    for (int64_t r = 0; r < rows; ++r) {
        const double* x = s + r * cols;
        double* y = p + r * cols;
        /* pass 1: maximum of the scaled legal entries (a NaN propagates) */
        double m = -INFINITY;
        for (int j = 0; j < cols; ++j) {
            if (x[j] == -INFINITY) continue;
            double v = scale * x[j];
            if (!(v <= m)) m = v;
        }
        if (m == -INFINITY) {
            for (int j = 0; j < cols; ++j) y[j] = 0.0;
            flags |= OR_FLAG_FULLY_MASKED_ROW;
            continue;
        }
        /* pass 2: normaliser */
        double z = 0.0;
        for (int j = 0; j < cols; ++j)
            if (x[j] != -INFINITY) z += exp(scale * x[j] - m);
        /* pass 3: weights */
        for (int j = 0; j < cols; ++j) {
            y[j] = (x[j] == -INFINITY) ? 0.0 : exp(scale * x[j] - m) / z;
            if (!isfinite(y[j])) flags |= OR_FLAG_NONFINITE;
        }
    }
    return flags;
}

/* Decode: one query row per (b, h) [MMHA 6.1: the llama.cpp-style call with a
 * single new token; MAX 2.4: the fused online softmax], q [B,H,D],
 * k/v [B,H,Lk,D], optional key lengths lens[B] (keys j >= len are illegal).
 * out [B,H,D] = softmax-weighted sum of V; lse [B,H] = log sum_j exp(s_j) over
 * the legal keys, in natural-log units of the scaled logits (-inf for a row
 * with no legal key, whose output is 0 and raises FLAG_FULLY_MASKED_ROW).
 * The same three passes as attention_row; the log-sum-exp is m + log(z). */
uint32_t oracle_decode(const double* q, const double* k, const double* v, const int32_t* lens,
                       int B, int H, int Lk, int D, double scale, double* out, double* lse) {
    unsigned kind = lens ? OR_PADDING : 0;
    uint32_t flags = length_flags(kind, lens, B, Lk);
#pragma omp parallel reduction(| : flags)
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Lk > 0 ? Lk : 1));
#pragma omp for schedule(dynamic, 4)
        for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
            int64_t b = bh / H;
            int64_t len_b = lens ? lens[b] : Lk;
            /* the query is the last position of its sequence: no causal test */
            flags |= attention_row(q + bh * D, k + bh * Lk * D, v + bh * Lk * D, Lk, D, scale,
                                   kind, 0, len_b, NULL, s, NULL, out + bh * D);
            /* log-sum-exp of the legal scores (attention_row left them in s,
             * -inf where masked): pass 1 max, pass 2 sum */
            double m = -INFINITY;
            for (int j = 0; j < Lk; ++j)
                if (!(s[j] <= m)) m = s[j];
            if (m == -INFINITY) {
                lse[bh] = -INFINITY;
                continue;
            }
            double z = 0.0;
            for (int j = 0; j < Lk; ++j)
                if (s[j] != -INFINITY) z += exp(s[j] - m);
            lse[bh] = m + log(z);
        }
        free(s);
    }
    return flags;
}

/* Backward of oracle_mha_fwd for an upstream gradient dout = dL/dO
 * [MAX 3.3: the softmax Jacobian dp_j/ds_k = p_j (delta_jk - p_k)]. Per row i
 * of head (b, h), with p the forward's weights (the same three passes, 0 at
 * masked keys):
 *   dV_j  += p_ij dO_i
 *   dP_ij  = <dO_i, v_j>
 *   dS_ij  = sum_k dP_ik dp_ik/ds_ij = p_ij (dP_ij - sum_k p_ik dP_ik)
 *   dQ_i   = scale sum_j dS_ij k_j,   dK_j += scale dS_ij q_i
 * Masked keys are skipped (they have no weight and no gradient); a fully
 * masked row contributes nothing and has dQ = 0. The additive mask is a
 * constant of the forward (no gradient). dq [B,H,Lq,D], dk/dv [B,H,Lk,D]. */
uint32_t oracle_mha_bwd(const double* q, const double* k, const double* v, const double* dout,
                        const int32_t* lens, const double* add, unsigned kind, int B, int H,
                        int Lq, int Lk, int D, double scale, double* dq, double* dk,
                        double* dv) {
    uint32_t flags = length_flags(kind, lens, B, Lk);
#pragma omp parallel reduction(| : flags)
    {
        size_t n = (size_t)(Lk > 0 ? Lk : 1);
        double* s = (double*)malloc(sizeof(double) * n);
        double* p = (double*)malloc(sizeof(double) * n);
        double* dp = (double*)malloc(sizeof(double) * n);
        double* o = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
            int64_t b = bh / H, h = bh % H;
            const double* K = k + bh * Lk * D;
            const double* V = v + bh * Lk * D;
            double* dK = dk + bh * Lk * D;
            double* dV = dv + bh * Lk * D;
            for (int64_t e = 0; e < (int64_t)Lk * D; ++e) dK[e] = dV[e] = 0.0;
            int64_t len_b = (kind & OR_PADDING) ? lens[b] : Lk;
            for (int64_t i = 0; i < Lq; ++i) {
                const double* qi = q + (bh * Lq + i) * D;
                const double* gi = dout + (bh * Lq + i) * D;
                double* dqi = dq + (bh * Lq + i) * D;
                const double* addrow = mask_row(add, kind, b, h, H, Lq, Lk, i);
                flags |= attention_row(qi, K, V, Lk, D, scale, kind, i, len_b, addrow, s, p, o);
                for (int d = 0; d < D; ++d) dqi[d] = 0.0;
                /* dP over the legal keys, and sum_k p_k dP_k */
                double c = 0.0;
                for (int j = 0; j < Lk; ++j) {
                    if (s[j] == -INFINITY) continue;
                    double t = 0.0;
                    for (int d = 0; d < D; ++d) t += gi[d] * V[(int64_t)j * D + d];
                    dp[j] = t;
                    c += p[j] * t;
                }
                for (int j = 0; j < Lk; ++j) {
                    if (s[j] == -INFINITY) continue;
                    double ds = p[j] * (dp[j] - c);
                    for (int d = 0; d < D; ++d) {
                        dqi[d] += scale * ds * K[(int64_t)j * D + d];
                        dK[(int64_t)j * D + d] += scale * ds * qi[d];
                        dV[(int64_t)j * D + d] += p[j] * gi[d];
                    }
                }
            }
        }
        free(s);
        free(p);
        free(dp);
        free(o);
    }
    return flags;
}
