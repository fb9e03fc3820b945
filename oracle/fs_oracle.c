/*
 * fs_oracle.c -- CPU oracle for exact categorical sampling fused into an
 * LM head (FlashSampling) and for the standalone Gumbel / exponential-race
 * sampler over materialised logits.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library.  The product path
 * (the HIP library and its Python binding) never calls into it, and the two
 * share no source: this file includes nothing from the HIP tree and the HIP
 * tree includes nothing from here.
 *
 * Everything is plain, slow and in float64.  Every function below names the
 * passage of the source pages it follows:
 *   [FS]  "FlashSampling: fast and memory-efficient exact sampling" (paper
 *         summary page): prerequisites (Gumbel-max trick), method, and the
 *         algorithm-details section (Stage 1 steps (1)-(6), Stage 2).
 *   [MG]  Megatron-LM pull request "fp64 sampling noise": sections
 *         "Problem" (race argmax p/E with E = -log U), "The change" (two
 *         Philox words -> 52-bit midpoint uniform, keyed by request seed,
 *         position and vocabulary index) and "Tests".
 *   [SK]  "Write Triton Sampling Kernel" skill page: "Required reasoning
 *         process" items 3-4 (greedy short-circuit; bias before temperature)
 *         and "Correctness requirements" (smallest-index tie-break).
 *   [PH]  Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
 *         1, 2, 3", SC'11, section 4 (the Philox-4x32 bijection, 10 rounds).
 *   [OFP8] OCP 8-bit Floating Point Specification (OFP8), revision 1.0: the
 *         E4M3 encoding of 8-bit weights (FP8 weights are the future work the
 *         FlashSampling page's limitations section names).
 *   [MX]  OCP Microscaling Formats (MX) specification, version 1.0: MXFP4,
 *         blocks of 32 FP4 E2M1 elements sharing one E8M0 scale (MXFP4
 *         weights are the other low-precision input the FlashSampling page's
 *         limitations section names).
 *   [GTK] Gumbel-top-k: the FlashSampling page's limitations and future-work
 *         sections name the top-k extension (k draws without replacement from
 *         the k largest perturbed scores, proved in its appendix D); the
 *         result is the standard one of Kool, van Hoof and Welling, "Stochastic
 *         Beams and Where to Find Them", ICML 2019, section 3.
 *   [SD]  spec-decode-ops kernel card: the description of its `sample`
 *         pipeline (temperature -> top-k -> top-p -> min-p -> Gumbel-argmax
 *         draw) and its "Semantics" section (the transformers processors'
 *         order and boundaries: top-p keeps the smallest sorted prefix whose
 *         probability reaches top_p, the crossing token included, over the
 *         top-k prefix; min-p keeps p >= min_p * p_max; every filter keeps at
 *         least one token).
 *   [SPV] spec-decode-ops kernel card: its description and usage example of
 *         `verify` (speculative-decoding rejection sampling after Leviathan,
 *         Kalman, Matias, ICML 2023, and Chen et al. 2023: accept the draft
 *         token with probability min(1, p_t / p_d), replace the first
 *         rejection by a draw from max(p_t - p_d, 0) renormalised, append a
 *         bonus draw from the target's last position when all are accepted).
 *
 * Definition computed (per batch row b, logical row id r = row_ids[b] or b):
 *   y_i   = sum_d H[b,d] * W[i,d]           float64, d ascending   [FS (1)]
 *   if t = temp[b] > 0:  yt_i = (y_i + bias[b,i]) / t               [SK 4]
 *   else (greedy):       yt_i =  y_i + bias[b,i],  g_i = 0          [SK 3]
 *   Philox4x32-10, key (seed lo, seed hi),
 *     counter (j, r, offset lo, offset hi), j = i>>2 (fp32 noise) or i>>1
 *     (fp64 noise) -> words x[0..3]                         [PH; MG change]
 *   fp32 noise: k = x[i&3] >> 9          (23 bits), u = (2k+1) / 2^24
 *   fp64 noise: k = top 52 bits of x[2(i&1)] : x[2(i&1)+1], u = (2k+1) / 2^53
 *   E_i = -log(u) (computed as -log1p(u-1) when u >= 1/2), g_i = -log(E_i)
 *                                                       [MG problem; FS (3)]
 *   s_i = yt_i + g_i                                                [FS (4)]
 *   out = smallest i attaining max s_i over the i whose s_i is neither NaN nor
 *         -inf; -1 if there is none.                  [FS (5), Stage 2; SK]
 *   gap = s_(1) - s_(2), the top-2 gap of those scores (+inf if only one).
 *   top-k (k draws without replacement) [GTK]: the indices of the k largest
 *         valid s_i, largest first, equal scores in increasing index order;
 *         -1 in the places past the number of valid scores.
 *   filtered sampling [SD]: the draw above restricted to the kept set of
 *         the filter chain on the row's logits (oracle_filter_kept below);
 *         tokens outside it score -inf.
 *   verification [SPV]: see the block comment above oracle_verify.
 *
 * Parity pins (tests marked "not gpu"): the Philox words against an
 * independent engine (the one PyTorch ships as a header); the uniform, E and
 * g values against 60-digit decimal arithmetic; the logits against exact
 * rational sums; the sampled law against softmax by chi-square, by a
 * Poisson tail count with the closed-form miss probability, and by exact
 * enumeration of the noise grid for two-token rows; greedy against numpy's
 * argmax; masks, NaN and empty rows against the rule above.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* Philox4x32-10 [PH].                                                 */
/* One round multiplies counter words 0 and 2 by the two round          */
/* multipliers, keeps both halves of each 64-bit product, and mixes the */
/* high halves with the other two counter words and the key.  The key   */
/* is bumped by the two Weyl constants between rounds.                  */
/* ------------------------------------------------------------------ */
static void philox4x32_10(const uint32_t ctr[4], uint32_t k0, uint32_t k1,
                          uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Words for counter (j, r, offset), key = seed [MG change: keyed by request
 * seed, absolute position and vocabulary index]. */
static void words_for(uint64_t seed, uint64_t offset, uint32_t r, uint32_t j,
                      uint32_t out[4])
{
    uint32_t ctr[4];
    ctr[0] = j;
    ctr[1] = r;
    ctr[2] = (uint32_t)(offset & 0xFFFFFFFFu);
    ctr[3] = (uint32_t)(offset >> 32);
    philox4x32_10(ctr, (uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32), out);
}

/* Uniform on the midpoint grid for vocabulary index i.
 * fp32 noise: one 32-bit word per index, its top 23 bits k, u = (k + 1/2)/2^23.
 * fp64 noise: two words per index, the top 52 bits k of their 64-bit
 * concatenation, u = (k + 1/2)/2^52 [MG change].  Both are exact in double. */
static double uniform_for(uint64_t seed, uint64_t offset, uint32_t r, int64_t i,
                          int fp64)
{
    uint32_t x[4];
    if (!fp64) {
        words_for(seed, offset, r, (uint32_t)(i >> 2), x);
        uint32_t k = x[i & 3] >> 9;
        return ((double)k + 0.5) / 8388608.0;               /* 2^23 */
    }
    words_for(seed, offset, r, (uint32_t)(i >> 1), x);
    uint64_t a = x[2 * (i & 1)], b = x[2 * (i & 1) + 1];
    uint64_t k = ((a << 32) | b) >> 12;                      /* top 52 bits */
    return ((double)k + 0.5) / 4503599627370496.0;           /* 2^52 */
}

/* E = -log u is a standard exponential; g = -log E is a standard Gumbel
 * [MG problem; FS (3)].  Near u = 1 the log1p form keeps E's relative
 * accuracy, which is what decides the deep tail. */
static double exponential_of(double u)
{
    return (u >= 0.5) ? -log1p(u - 1.0) : -log(u);
}

static double gumbel_of(double u) { return -log(exponential_of(u)); }

/* bf16 bit pattern -> double (exact). */
static double bf16_to_double(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* OCP 8-bit floating point E4M3 bit pattern -> double (exact) [OFP8]: sign
 * bit, 4 exponent bits with bias 7, 3 mantissa bits.  Exponent 0 encodes
 * subnormals m/8 * 2^-6; exponent 15 with mantissa 7 is the only NaN (the
 * format has no infinities, so 0x7E = 448 is the largest value). */
static double e4m3_to_double(uint8_t v)
{
    int sign = v >> 7, e = (v >> 3) & 15, m = v & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m / 8.0, -6);
    else mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* FP4 E2M1 code (low 4 bits) -> double (exact) [MX]: sign bit 3, 2 exponent
 * bits with bias 1, 1 mantissa bit; exponent 0 encodes m/2 (0 or 0.5); no
 * infinities or NaN, so the values are 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their
 * negatives. */
static double e2m1_to_double(uint8_t v)
{
    int sign = (v >> 3) & 1, e = (v >> 1) & 3, m = v & 1;
    double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, e - 1);
    return sign ? -mag : mag;
}

/* E8M0 scale -> double [MX]: 2^(e - 127); e = 255 is NaN. */
static double e8m0_to_double(uint8_t e)
{
    if (e == 255) return NAN;
    return ldexp(1.0, (int)e - 127);
}

/* ------------------------------------------------------------------ */
/* Exported helpers.                                                    */
/* ------------------------------------------------------------------ */

double oracle_e4m3_to_double(uint8_t v) { return e4m3_to_double(v); }
double oracle_e2m1_to_double(uint8_t v) { return e2m1_to_double(v); }
double oracle_e8m0_to_double(uint8_t e) { return e8m0_to_double(e); }

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Philox words for counters j = 0..n_ctr-1 of each row: out[B][n_ctr][4]. */
void oracle_philox_words(uint64_t seed, uint64_t offset, const uint32_t *row_ids,
                         int64_t B, int64_t n_ctr, uint32_t *out)
{
    for (int64_t b = 0; b < B; ++b) {
        uint32_t r = row_ids ? row_ids[b] : (uint32_t)b;
        for (int64_t j = 0; j < n_ctr; ++j)
            words_for(seed, offset, r, (uint32_t)j, out + (b * n_ctr + j) * 4);
    }
}

/* Raw Philox block on an arbitrary counter and key (for the engine pin). */
void oracle_philox_block(const uint32_t ctr[4], uint32_t k0, uint32_t k1,
                         uint32_t out[4])
{
    philox4x32_10(ctr, k0, k1, out);
}

/* u, E and g of vocabulary index i of logical row r. */
void oracle_noise_at(uint64_t seed, uint64_t offset, uint32_t r, int64_t i,
                     int fp64, double *u, double *E, double *g)
{
    double uu = uniform_for(seed, offset, r, i, fp64);
    double ee = exponential_of(uu);
    *u = uu;
    *E = ee;
    *g = -log(ee);
}

/* g_i for i = 0 .. V-1 of logical row r: the Gumbel noise of a whole row
 * [MG change; FS (3)]. */
void oracle_noise_row(uint64_t seed, uint64_t offset, uint32_t r, int64_t V, int fp64,
                      double *g)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < V; ++i) g[i] = gumbel_of(uniform_for(seed, offset, r, i, fp64));
}

/* Noise transforms of a given uniform (for the decimal-arithmetic pin). */
void oracle_noise_of_uniform(double u, double *E, double *g)
{
    *E = exponential_of(u);
    *g = gumbel_of(u);
}

/* E and g for the grid points k0 .. k0+n-1 of the 23-bit (fp64 == 0) or 52-bit
 * midpoint grid, u = (k + 1/2) / 2^bits [MG change; FS (3)]. */
void oracle_noise_grid(int fp64, uint64_t k0, int64_t n, double *E, double *g)
{
    const double scale = fp64 ? 4503599627370496.0 : 8388608.0;   /* 2^52 or 2^23 */
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        double u = ((double)(k0 + (uint64_t)t) + 0.5) / scale;
        double e = exponential_of(u);
        E[t] = e;
        g[t] = -log(e);
    }
}

/* Logits Y[b,i] = sum_d H[b,d] W[i,d], float64, d ascending [FS (1)].
 * H[B,D] and W[V,D] are bf16 bit patterns, row-major. */
void oracle_logits(const uint16_t *H, const uint16_t *W, int64_t B, int64_t D,
                   int64_t V, double *Y)
{
    double *hrow = (double *)malloc((size_t)D * sizeof(double));
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t d = 0; d < D; ++d) hrow[d] = bf16_to_double(H[b * D + d]);
        #pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < V; ++i) {
            const uint16_t *w = W + i * D;
            double acc = 0.0;
            for (int64_t d = 0; d < D; ++d) acc += hrow[d] * bf16_to_double(w[d]);
            Y[b * V + i] = acc;
        }
    }
    free(hrow);
}

/* Logits of an LM head whose weight is stored as 8-bit floats with one scale
 * per vocabulary row (the FP8 weights [FS limitations] names as future work):
 * Y[b,i] = scale[i] * sum_d H[b,d] * e4m3(W8[i,d]), float64, d ascending. */
void oracle_logits_w8(const uint16_t *H, const uint8_t *W8, const float *scale,
                      int64_t B, int64_t D, int64_t V, double *Y)
{
    double *hrow = (double *)malloc((size_t)D * sizeof(double));
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t d = 0; d < D; ++d) hrow[d] = bf16_to_double(H[b * D + d]);
        #pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < V; ++i) {
            const uint8_t *w = W8 + i * D;
            double acc = 0.0;
            for (int64_t d = 0; d < D; ++d) acc += hrow[d] * e4m3_to_double(w[d]);
            Y[b * V + i] = (double)scale[i] * acc;
        }
    }
    free(hrow);
}

/* Logits over MXFP4 weights [MX]: row i of W is stored as D/2 bytes, element
 * d in the low nibble of byte d/2 when d is even and in the high nibble when
 * d is odd, and block j (elements 32j .. 32j+31) shares the E8M0 scale
 * S[i, j] (D/32 bytes per row).  y_i = sum_d H[b,d] * e2m1(W[i,d]) *
 * e8m0(S[i, d/32]), float64, d ascending. */
void oracle_logits_w4(const uint16_t *H, const uint8_t *W4, const uint8_t *S,
                      int64_t B, int64_t D, int64_t V, double *Y)
{
    double *hrow = (double *)malloc((size_t)D * sizeof(double));
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t d = 0; d < D; ++d) hrow[d] = bf16_to_double(H[b * D + d]);
        #pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < V; ++i) {
            const uint8_t *w = W4 + i * (D / 2);
            const uint8_t *sc = S + i * (D / 32);
            double y = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                uint8_t code = (d & 1) ? (uint8_t)(w[d / 2] >> 4) : (uint8_t)(w[d / 2] & 15);
                y += hrow[d] * (e2m1_to_double(code) * e8m0_to_double(sc[d / 32]));
            }
            Y[b * V + i] = y;
        }
    }
    free(hrow);
}

/* Perturbed score of one element [FS (2)-(4); SK 3-4].  y is the logit, beta
 * the additive bias (NULL bias means 0), t the row temperature. */
static double score_of(double y, double beta, double t, uint64_t seed,
                       uint64_t offset, uint32_t r, int64_t i, int fp64)
{
    if (!(t > 0.0)) return y + beta;                 /* greedy: no noise */
    double yt = (y + beta) / t;
    return yt + gumbel_of(uniform_for(seed, offset, r, i, fp64));
}

/* Smallest-index argmax over valid scores plus the top-2 gap [FS (5), Stage 2;
 * SK tie-break].  Valid means neither NaN nor -inf. */
static void select_row(const double *s, int64_t V, int64_t *idx, double *gap,
                       double *best)
{
    int64_t bi = -1;
    double b1 = -INFINITY, b2 = -INFINITY;
    int64_t nvalid = 0;
    for (int64_t i = 0; i < V; ++i) {
        double v = s[i];
        if (isnan(v) || v == -INFINITY) continue;
        ++nvalid;
        if (bi < 0) {                 /* first valid score */
            b1 = v;
            bi = i;
        } else if (v > b1) {          /* strictly larger: new leader */
            b2 = b1;
            b1 = v;
            bi = i;
        } else if (v > b2) {          /* v <= b1; an equal score keeps the
                                         smaller index and makes the gap 0 */
            b2 = v;
        }
    }
    *idx = bi;
    if (bi < 0) {
        *gap = NAN;
        *best = -INFINITY;
    } else {
        *gap = (nvalid == 1) ? INFINITY : b1 - b2;
        *best = b1;
    }
}

/* The k largest valid scores [GTK], largest first, equal scores in
 * increasing index order: idx[0..k) (-1 past the number of valid scores) and
 * their scores top[0..k] with one more place (-inf past the end), so a caller
 * can see the margin between consecutive places.  A plain repeated scan: the
 * j-th place is the best valid score not taken by an earlier place. */
static void select_topk(const double *s, int64_t V, int k, int64_t *idx, double *top)
{
    for (int j = 0; j <= k; ++j) {
        int64_t bi = -1;
        double bv = -INFINITY;
        for (int64_t i = 0; i < V; ++i) {
            double v = s[i];
            if (isnan(v) || v == -INFINITY) continue;
            int taken = 0;
            for (int q = 0; q < j; ++q)
                if (idx[q] == i) taken = 1;
            if (taken) continue;
            if (bi < 0 || v > bv) {    /* equal scores keep the smaller index */
                bi = i;
                bv = v;
            }
        }
        if (j < k) idx[j] = bi;
        top[j] = bv;
        if (bi < 0) {                  /* no valid score left */
            for (int q = j + 1; q < k; ++q) idx[q] = -1;
            for (int q = j + 1; q <= k; ++q) top[q] = -INFINITY;
            break;
        }
    }
}

/* Fused path: logits from H and W, then transform, noise and selection.
 * temp[B]; bias[B,V] or NULL; row_ids[B] or NULL.  Outputs per row: the
 * sampled index, the top-2 perturbed-score gap and the winning score. */
void oracle_sample_fused(const uint16_t *H, const uint16_t *W, int64_t B,
                         int64_t D, int64_t V, const float *temp,
                         const float *bias, uint64_t seed, uint64_t offset,
                         const uint32_t *row_ids, int fp64_noise,
                         int64_t *out_idx, double *out_gap, double *out_best)
{
    double *s = (double *)malloc((size_t)V * sizeof(double));
    double *hrow = (double *)malloc((size_t)D * sizeof(double));
    for (int64_t b = 0; b < B; ++b) {
        uint32_t r = row_ids ? row_ids[b] : (uint32_t)b;
        double t = (double)temp[b];
        for (int64_t d = 0; d < D; ++d) hrow[d] = bf16_to_double(H[b * D + d]);
        #pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < V; ++i) {
            const uint16_t *w = W + i * D;
            double y = 0.0;
            for (int64_t d = 0; d < D; ++d) y += hrow[d] * bf16_to_double(w[d]);
            double beta = bias ? (double)bias[b * V + i] : 0.0;
            s[i] = score_of(y, beta, t, seed, offset, r, i, fp64_noise);
        }
        select_row(s, V, &out_idx[b], &out_gap[b], &out_best[b]);
    }
    free(hrow);
    free(s);
}

/* Fused path over FP8 weights: the logits of oracle_logits_w8, then the same
 * transform, noise and selection as oracle_sample_fused. */
void oracle_sample_fused_w8(const uint16_t *H, const uint8_t *W8, const float *scale,
                            int64_t B, int64_t D, int64_t V, const float *temp,
                            const float *bias, uint64_t seed, uint64_t offset,
                            const uint32_t *row_ids, int fp64_noise,
                            int64_t *out_idx, double *out_gap, double *out_best)
{
    double *s = (double *)malloc((size_t)V * sizeof(double));
    double *hrow = (double *)malloc((size_t)D * sizeof(double));
    for (int64_t b = 0; b < B; ++b) {
        uint32_t r = row_ids ? row_ids[b] : (uint32_t)b;
        double t = (double)temp[b];
        for (int64_t d = 0; d < D; ++d) hrow[d] = bf16_to_double(H[b * D + d]);
        #pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < V; ++i) {
            const uint8_t *w = W8 + i * D;
            double acc = 0.0;
            for (int64_t d = 0; d < D; ++d) acc += hrow[d] * e4m3_to_double(w[d]);
            double y = (double)scale[i] * acc;
            double beta = bias ? (double)bias[b * V + i] : 0.0;
            s[i] = score_of(y, beta, t, seed, offset, r, i, fp64_noise);
        }
        select_row(s, V, &out_idx[b], &out_gap[b], &out_best[b]);
    }
    free(hrow);
    free(s);
}

/* Fused path over MXFP4 weights: the logits of oracle_logits_w4, then the
 * same transform, noise and selection as oracle_sample_fused. */
void oracle_sample_fused_w4(const uint16_t *H, const uint8_t *W4, const uint8_t *S,
                            int64_t B, int64_t D, int64_t V, const float *temp,
                            const float *bias, uint64_t seed, uint64_t offset,
                            const uint32_t *row_ids, int fp64_noise,
                            int64_t *out_idx, double *out_gap, double *out_best)
{
    double *y = (double *)malloc((size_t)V * sizeof(double));
    double *s = (double *)malloc((size_t)V * sizeof(double));
    for (int64_t b = 0; b < B; ++b) {
        uint32_t r = row_ids ? row_ids[b] : (uint32_t)b;
        double t = (double)temp[b];
        oracle_logits_w4(H + b * D, W4, S, 1, D, V, y);
        #pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < V; ++i) {
            double beta = bias ? (double)bias[b * V + i] : 0.0;
            s[i] = score_of(y[i], beta, t, seed, offset, r, i, fp64_noise);
        }
        select_row(s, V, &out_idx[b], &out_gap[b], &out_best[b]);
    }
    free(s);
    free(y);
}

/* Gumbel-top-k over the fused path's scores [GTK]: per row, k places of
 * out_idx[B, k] and k + 1 places of out_top[B, k + 1] (see select_topk). */
void oracle_sample_fused_topk(const uint16_t *H, const uint16_t *W, int64_t B,
                              int64_t D, int64_t V, const float *temp,
                              const float *bias, uint64_t seed, uint64_t offset,
                              const uint32_t *row_ids, int fp64_noise, int k,
                              int64_t *out_idx, double *out_top)
{
    double *s = (double *)malloc((size_t)V * sizeof(double));
    double *hrow = (double *)malloc((size_t)D * sizeof(double));
    for (int64_t b = 0; b < B; ++b) {
        uint32_t r = row_ids ? row_ids[b] : (uint32_t)b;
        double t = (double)temp[b];
        for (int64_t d = 0; d < D; ++d) hrow[d] = bf16_to_double(H[b * D + d]);
        #pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < V; ++i) {
            const uint16_t *w = W + i * D;
            double y = 0.0;
            for (int64_t d = 0; d < D; ++d) y += hrow[d] * bf16_to_double(w[d]);
            double beta = bias ? (double)bias[b * V + i] : 0.0;
            s[i] = score_of(y, beta, t, seed, offset, r, i, fp64_noise);
        }
        select_topk(s, V, k, out_idx + b * k, out_top + b * (k + 1));
    }
    free(hrow);
    free(s);
}

/* Gumbel-top-k over materialised float32 logits[B,V] [GTK; MG problem]. */
void oracle_sample_logits_topk(const float *logits, int64_t B, int64_t V,
                               const float *temp, uint64_t seed, uint64_t offset,
                               const uint32_t *row_ids, int fp64_noise, int k,
                               int64_t *out_idx, double *out_top)
{
    double *s = (double *)malloc((size_t)V * sizeof(double));
    for (int64_t b = 0; b < B; ++b) {
        uint32_t r = row_ids ? row_ids[b] : (uint32_t)b;
        double t = (double)temp[b];
        #pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < V; ++i)
            s[i] = score_of((double)logits[b * V + i], 0.0, t, seed, offset, r, i,
                            fp64_noise);
        select_topk(s, V, k, out_idx + b * k, out_top + b * (k + 1));
    }
    free(s);
}

/* Gumbel-top-k for many logical rows sharing one logits row (law tests);
 * out_idx[n_rows, k]. */
void oracle_topk_repeated_row(const float *logits, int64_t V, float temp,
                              uint64_t seed, uint64_t offset, const uint32_t *row_ids,
                              int64_t n_rows, int fp64_noise, int k, int64_t *out_idx)
{
    #pragma omp parallel
    {
        double *s = (double *)malloc((size_t)V * sizeof(double));
        double *top = (double *)malloc((size_t)(k + 1) * sizeof(double));
        #pragma omp for schedule(static)
        for (int64_t q = 0; q < n_rows; ++q) {
            for (int64_t i = 0; i < V; ++i)
                s[i] = score_of((double)logits[i], 0.0, (double)temp, seed, offset,
                                row_ids[q], i, fp64_noise);
            select_topk(s, V, k, out_idx + q * k, top);
        }
        free(top);
        free(s);
    }
}

/* Standalone sampler over materialised float32 logits[B,V]: the same
 * transform, noise and selection with y_i = logits[b,i] [MG problem;
 * FS prerequisites]. */
void oracle_sample_logits(const float *logits, int64_t B, int64_t V,
                          const float *temp, uint64_t seed, uint64_t offset,
                          const uint32_t *row_ids, int fp64_noise,
                          int64_t *out_idx, double *out_gap, double *out_best)
{
    double *s = (double *)malloc((size_t)V * sizeof(double));
    for (int64_t b = 0; b < B; ++b) {
        uint32_t r = row_ids ? row_ids[b] : (uint32_t)b;
        double t = (double)temp[b];
        #pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < V; ++i)
            s[i] = score_of((double)logits[b * V + i], 0.0, t, seed, offset, r, i,
                            fp64_noise);
        select_row(s, V, &out_idx[b], &out_gap[b], &out_best[b]);
    }
    free(s);
}

/* Many logical rows that share one logits row: row k of the batch has
 * logical id row_ids[k] and the logits of `logits[0..V)`.  This is the same
 * computation as oracle_sample_logits with the row repeated, without
 * materialising the repeats (used by the tail-rate and chi-square tests,
 * whose rows are identical by construction).  out_gap may be NULL. */
void oracle_sample_repeated_row(const float *logits, int64_t V, float temp,
                                uint64_t seed, uint64_t offset,
                                const uint32_t *row_ids, int64_t n_rows,
                                int fp64_noise, int64_t *out_idx, double *out_gap)
{
    #pragma omp parallel
    {
        double *s = (double *)malloc((size_t)V * sizeof(double));
        #pragma omp for schedule(static)
        for (int64_t k = 0; k < n_rows; ++k) {
            double gap, best;
            for (int64_t i = 0; i < V; ++i)
                s[i] = score_of((double)logits[i], 0.0, (double)temp, seed, offset,
                                row_ids[k], i, fp64_noise);
            select_row(s, V, &out_idx[k], &gap, &best);
            if (out_gap) out_gap[k] = gap;
        }
        free(s);
    }
}

/* ------------------------------------------------------------------ */
/* Filtered exact sampling [SD sample pipeline and Semantics].          */
/* ------------------------------------------------------------------ */

/* A logit and its index; sorted by value descending, ties in increasing
 * index order. */
typedef struct {
    double v;
    int64_t i;
} vi_t;
static int cmp_desc(const void *pa, const void *pb)
{
    const vi_t *a = (const vi_t *)pa, *b = (const vi_t *)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    return (a->i > b->i) - (a->i < b->i);
}

/* The kept set of one row of logits y[0..V) under temperature t and the
 * filters top_k (off when k <= 0 or k >= the number of valid tokens), top_p
 * (off when p >= 1 or NaN) and min_p (off when m <= 0 or NaN), applied in
 * that order [SD].  Valid tokens are those whose logit is neither NaN nor
 * -inf; no other token is ever kept.
 *   probabilities: softmax of y/t over the tokens a filter sees, written
 *     through the masses e_i = exp((y_i - M)/t) with M = the row's largest
 *     valid logit (e = 1 on a +inf logit and 0 on the others when M = +inf);
 *   top-k: the tokens whose logit is at least the k-th largest valid logit
 *     (a tie at the k-th value keeps the whole tie class);
 *   top-p: over the top-k survivors, a token is kept when the probability of
 *     the strictly larger survivors is below p (the prefix up to and including
 *     the crossing token; equal logits are kept or dropped together);
 *   min-p: over the top-p survivors, a token is kept when e_i >= m, i.e.
 *     p_i >= m * p_max (renormalising does not change that ratio);
 *   each filter that would keep nothing keeps the largest logit's tie class.
 * Greedy rows (!(t > 0)) keep the largest logit's tie class: their draw is the
 * argmax whatever the filters.  The logits are float64 (float32 rows convert
 * exactly).  Returns the kept mask and two margins, so that a comparison with
 * another implementation can set aside the rows whose kept set rounding may
 * decide:
 *   *margin, the smallest distance of a top-p or min-p decision from its
 *     boundary (relative: |A - pZ| / Z for top-p, |e_i - m| / m for min-p;
 *     +inf when neither decides anything).  The largest logit's class has no
 *     such distance: its mass above is 0 and its mass ratio 1 exactly, and
 *     the filters keep it whatever p and m are;
 *   *vmargin, the logit gap at each cut the top-k and top-p filters make
 *     (the last kept value minus the first dropped value; +inf when neither
 *     cuts): a smaller perturbation of the logits cannot reorder the tokens
 *     on either side of a cut. */
static void filter_row(const double *y, int64_t V, double t, int32_t k, float p,
                       float m, vi_t *order, double *e, uint8_t *kept,
                       double *margin, double *vmargin)
{
    int64_t n = 0;
    for (int64_t i = 0; i < V; ++i) {
        kept[i] = 0;
        if (!isnan(y[i]) && y[i] != -INFINITY) {
            order[n].v = y[i];
            order[n].i = i;
            ++n;
        }
    }
    *margin = INFINITY;
    *vmargin = INFINITY;
    if (n == 0) return;
    qsort(order, (size_t)n, sizeof(vi_t), cmp_desc);
    const double M = (double)order[0].v;
    /* the largest logit's tie class: order[0 .. nmax) */
    int64_t nmax = 1;
    while (nmax < n && order[nmax].v == order[0].v) ++nmax;
    if (!(t > 0.0)) {
        for (int64_t j = 0; j < nmax; ++j) kept[order[j].i] = 1;
        return;
    }
    for (int64_t j = 0; j < n; ++j) {
        double v = (double)order[j].v;
        if (M == INFINITY) e[j] = (v == INFINITY) ? 1.0 : 0.0;
        else e[j] = exp((v - M) / t);
    }
    /* top-k: survivors order[0 .. n1) */
    int64_t n1 = n;
    if (k > 0 && (int64_t)k < n) {
        const double theta = order[k - 1].v;
        n1 = k;
        while (n1 < n && order[n1].v == theta) ++n1;
        if (n1 < n) *vmargin = fmin(*vmargin, order[n1 - 1].v - order[n1].v);
    }
    /* top-p over the top-k survivors: order[0 .. n2) */
    int64_t n2 = n1;
    if (p < 1.0f && !(p > 0.0f)) {        /* keeps nothing: the largest class */
        n2 = nmax;
    } else if (p < 1.0f) {                /* NaN compares false: off */
        double Z = 0.0;
        for (int64_t j = 0; j < n1; ++j) Z += e[j];
        const double target = (double)p * Z;
        double above = 0.0;               /* mass of strictly larger logits */
        n2 = 0;
        int64_t j = 0;
        while (j < n1) {
            int64_t j2 = j + 1;           /* the tie class order[j .. j2) */
            double cls = e[j];
            while (j2 < n1 && order[j2].v == order[j].v) cls += e[j2++];
            if (j > 0) {                  /* the largest class: above = 0 < pZ */
                double d = fabs(above - target) / Z;
                if (d < *margin) *margin = d;
            }
            if (!(above < target)) break;
            n2 = j2;
            above += cls;
            j = j2;
        }
        if (n2 == 0) n2 = nmax;
        if (n2 < n1) *vmargin = fmin(*vmargin, order[n2 - 1].v - order[n2].v);
    }
    /* min-p over the top-p survivors */
    int64_t n3 = 0;
    if (m > 0.0f) {                       /* NaN compares false: off */
        for (int64_t j = 0; j < n2; ++j) {
            double d = fabs(e[j] - (double)m) / (double)m;
            if (j >= nmax && d < *margin) *margin = d;
            if (e[j] >= (double)m) {
                kept[order[j].i] = 1;
                ++n3;
            }
        }
        if (n3 == 0)
            for (int64_t j = 0; j < nmax; ++j) kept[order[j].i] = 1;
    } else {
        for (int64_t j = 0; j < n2; ++j) kept[order[j].i] = 1;
    }
}

/* Kept sets of logits[B,V] (see filter_row): kept[B,V] (1 = kept) and
 * margin[B].  top_k, top_p, min_p are per-row arrays or NULL (off). */
void oracle_filter_kept(const float *logits, int64_t B, int64_t V, const float *temp,
                        const int32_t *top_k, const float *top_p, const float *min_p,
                        uint8_t *kept, double *margin)
{
    #pragma omp parallel
    {
        vi_t *order = (vi_t *)malloc((size_t)(V > 0 ? V : 1) * sizeof(vi_t));
        double *e = (double *)malloc((size_t)(V > 0 ? V : 1) * sizeof(double));
        double *y = (double *)malloc((size_t)(V > 0 ? V : 1) * sizeof(double));
        #pragma omp for schedule(dynamic)
        for (int64_t b = 0; b < B; ++b) {
            double vm;
            for (int64_t i = 0; i < V; ++i) y[i] = (double)logits[b * V + i];
            filter_row(y, V, (double)temp[b], top_k ? top_k[b] : 0,
                       top_p ? top_p[b] : 1.0f, min_p ? min_p[b] : 0.0f, order, e,
                       kept + b * V, &margin[b], &vm);
        }
        free(y);
        free(e);
        free(order);
    }
}

/* Fused filtered exact sampling [SD sample pipeline and Semantics; FS
 * algorithm details step (1)]: per row, the logits y = H W^T in float64 (the
 * sum of oracle_logits), the kept set of filter_row over them, then the draw
 * of oracle_sample_fused (no bias) over the kept tokens only.  Outputs per
 * row: the sampled index (-1 if none), the top-2 gap of the kept perturbed
 * scores, and filter_row's two margins. */
void oracle_sample_fused_filtered(const uint16_t *H, const uint16_t *W, int64_t B, int64_t D,
                                  int64_t V, const float *temp, const int32_t *top_k,
                                  const float *top_p, const float *min_p, uint64_t seed,
                                  uint64_t offset, const uint32_t *row_ids, int fp64_noise,
                                  int64_t *out_idx, double *out_gap, double *out_margin,
                                  double *out_vmargin)
{
    double *y = (double *)malloc((size_t)(V > 0 ? V : 1) * sizeof(double));
    double *s = (double *)malloc((size_t)(V > 0 ? V : 1) * sizeof(double));
    double *e = (double *)malloc((size_t)(V > 0 ? V : 1) * sizeof(double));
    vi_t *order = (vi_t *)malloc((size_t)(V > 0 ? V : 1) * sizeof(vi_t));
    uint8_t *kept = (uint8_t *)malloc((size_t)(V > 0 ? V : 1));
    for (int64_t b = 0; b < B; ++b) {
        const uint32_t r = row_ids ? row_ids[b] : (uint32_t)b;
        const double t = (double)temp[b];
        oracle_logits(H + b * D, W, 1, D, V, y);
        filter_row(y, V, t, top_k ? top_k[b] : 0, top_p ? top_p[b] : 1.0f,
                   min_p ? min_p[b] : 0.0f, order, e, kept, &out_margin[b], &out_vmargin[b]);
        double best;
        #pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < V; ++i)
            s[i] = kept[i] ? score_of(y[i], 0.0, t, seed, offset, r, i, fp64_noise) : -INFINITY;
        select_row(s, V, &out_idx[b], &out_gap[b], &best);
    }
    free(kept);
    free(order);
    free(e);
    free(s);
    free(y);
}

/* Repetition penalty [SD sample pipeline: the penalty comes before the
 * temperature; the transformers processor's rule]: every token that occurs in
 * row b's previous tokens prev[b, 0..L) (entries outside [0, V) are padding)
 * has its logit y replaced by y * penalty when y < 0 and by y / penalty
 * otherwise; the other logits are unchanged.  A row whose penalty is not
 * positive (or NaN) is unchanged.  Computed in float64 and rounded to float32
 * (for a product or a quotient of two float32 values this is the correctly
 * rounded float32 result). */
void oracle_repetition_penalty(const float *logits, int64_t B, int64_t V, const int64_t *prev,
                               int64_t L, const float *penalty, float *out)
{
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t i = 0; i < V; ++i) out[b * V + i] = logits[b * V + i];
        double p = (double)penalty[b];
        if (!(p > 0.0)) continue;
        for (int64_t j = 0; j < L; ++j) {
            int64_t x = prev[b * L + j];
            if (x < 0 || x >= V) continue;
            double y = (double)logits[b * V + x];
            out[b * V + x] = (float)((y < 0.0) ? y * p : y / p);
        }
    }
}

/* The filter chain's output [SD API table: filter_logits]: out[b, i] =
 * logits[b, i] / t on the kept tokens of oracle_filter_kept and -inf
 * elsewhere; greedy rows (!(t > 0)) keep the largest logit's tie class
 * unscaled.  margin[b] as in oracle_filter_kept. */
void oracle_filter_logits(const float *logits, int64_t B, int64_t V, const float *temp,
                          const int32_t *top_k, const float *top_p, const float *min_p,
                          double *out, double *margin)
{
    uint8_t *kept = (uint8_t *)malloc((size_t)(B * V > 0 ? B * V : 1));
    oracle_filter_kept(logits, B, V, temp, top_k, top_p, min_p, kept, margin);
    for (int64_t b = 0; b < B; ++b) {
        double t = (double)temp[b];
        for (int64_t i = 0; i < V; ++i) {
            double y = (double)logits[b * V + i];
            out[b * V + i] = kept[b * V + i] ? ((t > 0.0) ? y / t : y) : -INFINITY;
        }
    }
    free(kept);
}

/* Filtered exact sampling over float32 logits[B,V] [SD; FS prerequisites]:
 * the kept set of oracle_filter_kept, then the standalone sampler's noise,
 * transform and selection over the kept tokens only (the others score -inf).
 * Outputs per row: the sampled index (-1 if none), the top-2 gap of the kept
 * perturbed scores, and the filter margin. */
void oracle_sample_logits_filtered(const float *logits, int64_t B, int64_t V,
                                   const float *temp, const int32_t *top_k,
                                   const float *top_p, const float *min_p,
                                   uint64_t seed, uint64_t offset,
                                   const uint32_t *row_ids, int fp64_noise,
                                   int64_t *out_idx, double *out_gap,
                                   double *out_margin)
{
    uint8_t *kept = (uint8_t *)malloc((size_t)(B * V > 0 ? B * V : 1));
    double *s = (double *)malloc((size_t)(V > 0 ? V : 1) * sizeof(double));
    oracle_filter_kept(logits, B, V, temp, top_k, top_p, min_p, kept, out_margin);
    for (int64_t b = 0; b < B; ++b) {
        uint32_t r = row_ids ? row_ids[b] : (uint32_t)b;
        double t = (double)temp[b], best;
        #pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < V; ++i)
            s[i] = kept[b * V + i]
                       ? score_of((double)logits[b * V + i], 0.0, t, seed, offset, r, i,
                                  fp64_noise)
                       : -INFINITY;
        select_row(s, V, &out_idx[b], &out_gap[b], &best);
    }
    free(s);
    free(kept);
}

/* Filtered draws for many logical rows sharing one logits row (law tests):
 * the kept set once, then one draw per logical row id. */
void oracle_filtered_repeated_row(const float *logits, int64_t V, float temp,
                                  int32_t top_k, float top_p, float min_p,
                                  uint64_t seed, uint64_t offset,
                                  const uint32_t *row_ids, int64_t n_rows,
                                  int fp64_noise, int64_t *out_idx)
{
    uint8_t *kept = (uint8_t *)malloc((size_t)(V > 0 ? V : 1));
    double margin;
    oracle_filter_kept(logits, 1, V, &temp, &top_k, &top_p, &min_p, kept, &margin);
    #pragma omp parallel
    {
        double *s = (double *)malloc((size_t)(V > 0 ? V : 1) * sizeof(double));
        #pragma omp for schedule(static)
        for (int64_t q = 0; q < n_rows; ++q) {
            double gap, best;
            for (int64_t i = 0; i < V; ++i)
                s[i] = kept[i] ? score_of((double)logits[i], 0.0, (double)temp, seed,
                                          offset, row_ids[q], i, fp64_noise)
                               : -INFINITY;
            select_row(s, V, &out_idx[q], &gap, &best);
        }
        free(s);
    }
    free(kept);
}

/* ------------------------------------------------------------------ */
/* Speculative-decoding verification [SPV]: the spec-decode-ops card's  */
/* description of `verify` (rejection sampling after Leviathan et al.   */
/* 2023 and Chen et al. 2023) and its usage example (target logits     */
/* [B, K+1, V], draft logits [B, K, V], draft tokens [B, K]; the tokens */
/* out[b, 0 .. accept_len] are emitted).                                */
/*                                                                      */
/* Per row b (logical id r) and position i < K, with p_t and p_d the    */
/* temperature softmaxes of target row i and draft row i:               */
/*   u_i  = the 52-bit midpoint uniform of Philox counter               */
/*          (2^32 - 1, r, offset + i): words 0 and 1, as the fp64 noise */
/*          takes them.  Vocabulary words never reach that counter      */
/*          value, so u_i is independent of every noise value;          */
/*   accept x_i iff u_i * p_d(x_i) < p_t(x_i), i.e. with probability    */
/*          min(1, p_t(x_i) / p_d(x_i)) (a token outside [0, V) has     */
/*          probability 0 under both and is rejected);                  */
/*   accept_len = the first rejected position, or K.                    */
/* out[j] = x_j for j < accept_len; -1 past accept_len; and out at      */
/* accept_len is                                                         */
/*   a rejected position: a draw from max(p_t - p_d, 0) renormalised,   */
/*          as the Gumbel-max of log r_j with the noise of counter      */
/*          position offset + accept_len (the standalone sampler's      */
/*          stream at that offset); if the residual is all zero (p_t    */
/*          equals p_d), the draw from p_t itself;                      */
/*   K accepted: the bonus draw from target row K, which is the         */
/*          standalone sampler's draw on that row at offset + K.        */
/* Greedy rows (!(t > 0)): p is one-hot on the row's first largest      */
/* valid logit; the draw at a rejected position is the target argmax.   */
/* ------------------------------------------------------------------ */

/* Temperature softmax of one row, p[0..V), over its valid logits (neither
 * NaN nor -inf): e_j = exp((y_j - M)/t) with M the largest valid logit, or,
 * when M = +inf, e_j = 1 on the +inf logits and 0 elsewhere (the limit of
 * softmax); p_j = e_j / sum e.  Greedy rows: one-hot on the first largest
 * valid logit.  No valid logit: p = 0. */
static void row_probs(const float *y, int64_t V, double t, double *p)
{
    int64_t am = -1;
    for (int64_t j = 0; j < V; ++j) {
        p[j] = 0.0;
        if (isnan(y[j]) || y[j] == -INFINITY) continue;
        if (am < 0 || y[j] > y[am]) am = j;
    }
    if (am < 0) return;
    const double M = (double)y[am];
    if (!(t > 0.0)) {
        p[am] = 1.0;
        return;
    }
    double Z = 0.0;
    for (int64_t j = 0; j < V; ++j) {
        if (isnan(y[j]) || y[j] == -INFINITY) continue;
        if (M == INFINITY)
            p[j] = (y[j] == INFINITY) ? 1.0 : 0.0;
        else
            p[j] = exp(((double)y[j] - M) / t);
        Z += p[j];
    }
    for (int64_t j = 0; j < V; ++j) p[j] /= Z;
}

/* The acceptance uniform of position `pos` (= offset + i) of logical row r. */
static double accept_uniform(uint64_t seed, uint64_t pos, uint32_t r)
{
    uint32_t x[4];
    words_for(seed, pos, r, 0xFFFFFFFFu, x);
    uint64_t k = (((uint64_t)x[0] << 32) | (uint64_t)x[1]) >> 12;
    return ((double)k + 0.5) / 4503599627370496.0;           /* 2^52 */
}

double oracle_accept_uniform(uint64_t seed, uint64_t pos, uint32_t r)
{
    return accept_uniform(seed, pos, r);
}

typedef struct {
    double *pt, *pd, *s;
} verify_buf_t;

static int verify_buf_alloc(verify_buf_t *w, int64_t V)
{
    size_t n = (size_t)(V > 0 ? V : 1) * sizeof(double);
    w->pt = (double *)malloc(n);
    w->pd = (double *)malloc(n);
    w->s = (double *)malloc(n);
    return w->pt && w->pd && w->s;
}

static void verify_buf_free(verify_buf_t *w)
{
    free(w->pt);
    free(w->pd);
    free(w->s);
}

/* One row of the verification (see the block comment above).  tg: K+1 rows
 * of V target logits, dr: K rows of draft logits, tok: K draft tokens.
 * Writes *accept_len, out[0..K], and two margins for comparisons with
 * another implementation:
 *   *margin: the smallest relative distance |u q - a| / max(a, q) of an
 *     acceptance decision from its boundary over the decided positions
 *     (0 when a and q are both below 1e-30, where float32 underflow decides);
 *   *gap: the top-2 gap of the perturbed scores of the draw at accept_len
 *     (the bonus or fallback draw's scores, or the residual draw's
 *     log r_j + g_j); +inf on greedy rows. */
static void verify_row(const float *tg, const float *dr, const int64_t *tok, int64_t K,
                       int64_t V, double t, uint64_t seed, uint64_t offset, uint32_t r,
                       int fp64, verify_buf_t *w, int64_t *accept_len, int64_t *out,
                       double *margin, double *gap)
{
    *margin = INFINITY;
    int64_t L = K;
    for (int64_t i = 0; i < K; ++i) {
        row_probs(tg + i * V, V, t, w->pt);
        row_probs(dr + i * V, V, t, w->pd);
        const int64_t x = tok[i];
        double a = 0.0, q = 0.0;
        if (x >= 0 && x < V) {
            a = w->pt[x];
            q = w->pd[x];
        }
        const double u = accept_uniform(seed, offset + (uint64_t)i, r);
        if (a > 0.0 || q > 0.0) {
            double d = (fmax(a, q) < 1e-30) ? 0.0 : fabs(u * q - a) / fmax(a, q);
            if (d < *margin) *margin = d;
        }
        if (!(u * q < a)) {
            L = i;
            break;
        }
    }
    *accept_len = L;
    for (int64_t j = 0; j <= K; ++j) out[j] = (j < L) ? tok[j] : -1;
    const uint64_t pos = offset + (uint64_t)L;
    const float *y = tg + L * V;
    double best;
    if (L == K || !(t > 0.0)) {
        /* the bonus draw, or a greedy row's target argmax */
        for (int64_t j = 0; j < V; ++j)
            w->s[j] = score_of((double)y[j], 0.0, t, seed, pos, r, j, fp64);
        select_row(w->s, V, &out[L], gap, &best);
        if (!(t > 0.0)) *gap = INFINITY;
        return;
    }
    /* residual max(p_t - p_d, 0) of position L (pt, pd hold its rows) */
    int any = 0;
    for (int64_t j = 0; j < V; ++j) {
        double d = w->pt[j] - w->pd[j];
        w->s[j] = d > 0.0 ? d : 0.0;
        any |= d > 0.0;
    }
    if (!any) {
        for (int64_t j = 0; j < V; ++j)
            w->s[j] = score_of((double)y[j], 0.0, t, seed, pos, r, j, fp64);
        select_row(w->s, V, &out[L], gap, &best);
        return;
    }
    for (int64_t j = 0; j < V; ++j) {
        double rr = w->s[j];
        w->s[j] = rr > 0.0 ? log(rr) + gumbel_of(uniform_for(seed, pos, r, j, fp64)) : -INFINITY;
    }
    select_row(w->s, V, &out[L], gap, &best);
}

/* Verification of B rows: target[B, K+1, V], draft[B, K, V], tokens[B, K],
 * temp[B]; accept_len[B], out[B, K+1], margin[B], gap[B]. */
void oracle_verify(const float *target, const float *draft, const int64_t *tokens,
                   int64_t B, int64_t K, int64_t V, const float *temp, uint64_t seed,
                   uint64_t offset, const uint32_t *row_ids, int fp64_noise,
                   int64_t *accept_len, int64_t *out, double *margin, double *gap)
{
    #pragma omp parallel
    {
        verify_buf_t w;
        int ok = verify_buf_alloc(&w, V);
        #pragma omp for schedule(dynamic)
        for (int64_t b = 0; b < B; ++b) {
            if (!ok) continue;
            uint32_t r = row_ids ? row_ids[b] : (uint32_t)b;
            verify_row(target + b * (K + 1) * V, draft + b * K * V, tokens + b * K, K, V,
                       (double)temp[b], seed, offset, r, fp64_noise, &w, &accept_len[b],
                       out + b * (K + 1), &margin[b], &gap[b]);
        }
        verify_buf_free(&w);
    }
}

/* Many logical rows that share one target block [K+1, V] and one draft block
 * [K, V], each with its own draft tokens tokens[q, 0..K) and logical id
 * row_ids[q] (law tests). */
void oracle_verify_repeated(const float *target, const float *draft, const int64_t *tokens,
                            int64_t K, int64_t V, float temp, uint64_t seed, uint64_t offset,
                            const uint32_t *row_ids, int64_t n_rows, int fp64_noise,
                            int64_t *accept_len, int64_t *out)
{
    #pragma omp parallel
    {
        verify_buf_t w;
        int ok = verify_buf_alloc(&w, V);
        #pragma omp for schedule(static)
        for (int64_t q = 0; q < n_rows; ++q) {
            if (!ok) continue;
            double margin, gap;
            verify_row(target, draft, tokens + q * K, K, V, (double)temp, seed, offset,
                       row_ids[q], fp64_noise, &w, &accept_len[q], out + q * (K + 1), &margin,
                       &gap);
        }
        verify_buf_free(&w);
    }
}
