/*
 * fsample.h -- C ABI of libfsample.so: exact categorical sampling fused into an
 * LM-head matmul, and the standalone sampler over materialised logits, for
 * AMD Instinct MI355X (gfx950).
 *
 * Citations name the page and the section that defines each operation:
 *   [FS]  "FlashSampling: fast and memory-efficient exact sampling" (paper
 *         summary page), sections "core method" and "algorithm details"
 *         (Stage 1 steps (1)-(6); Stage 2).
 *   [MG]  Megatron-LM pull request "fp64 sampling noise", sections "Problem"
 *         and "The change".
 *   [SD]  spec-decode-ops kernel card: the description of its sample
 *         pipeline, sections "Usage", "API", "Semantics" (the filter order and
 *         boundaries) and "Measured behavior" (determinism).
 *   [SK]  "Write Triton Sampling Kernel" skill page, "Required reasoning
 *         process" items 3-4 and 10, "Correctness requirements".
 *   [OFP8] OCP 8-bit Floating Point Specification (OFP8), revision 1.0, the
 *         E4M3 format (FP8 weights: the FlashSampling page's "limitations"
 *         section names low-precision weights as future work).
 *   [MX]  OCP Microscaling Formats (MX) specification 1.0: MXFP4, blocks of 32
 *         FP4 E2M1 elements sharing an E8M0 scale (the other low-precision
 *         weight format the FlashSampling page's "limitations" names).
 *   [GTK] Gumbel-top-k: the FlashSampling page's "limitations" and future
 *         work name the top-k extension (k draws without replacement, the k
 *         largest perturbed scores; its appendix D proves it); the standard
 *         statement is Kool, van Hoof and Welling, ICML 2019, section 3.
 *   [SPV] spec-decode-ops kernel card: the description of its `verify`
 *         (speculative-decoding rejection sampling after Leviathan, Kalman and
 *         Matias, ICML 2023, and Chen et al. 2023), its "Speculative
 *         verification" usage example and its "API" table.
 *
 * Conventions shared by every entry point
 *   Pointers.   Arguments documented as "device" are device (HBM) pointers the
 *               caller allocated; arguments documented as "host" are plain host
 *               values.  The library allocates nothing per call and keeps no
 *               pointer after it returns.
 *   Layouts.    All matrices are row-major and dense: a row of n elements is
 *               followed immediately by the next row.  bf16 values are passed
 *               as their 16-bit patterns (fs_bf16).
 *   Streams.    Work is enqueued on `stream` (a hipStream_t; NULL means the
 *               default stream) and the call returns without synchronising.
 *               Outputs are valid once that stream has reached the work.
 *   Errors.     Every call returns an fs_status.  Arguments are checked on the
 *               host before any HIP call, so an invalid call enqueues nothing
 *               and leaves every output untouched.  FS_ERR_HIP reports a launch
 *               failure (the HIP error text is available from fs_last_error()).
 *               No call inspects device data: temperatures, biases and logits
 *               of any value are legal and have the meaning defined below.
 *   Determinism. For fixed inputs, seed, offset, row ids and flags, outputs
 *               are bitwise identical from call to call, independent of the
 *               batch position of a row, of other rows in the batch and of
 *               concurrent work on other streams [MG "Tests"; SD determinism].
 *               The caller advances `offset` every decode step [SK item 10].
 *
 * Sampling rule (both entry points), per batch row b with logical row id
 * r = row_ids ? row_ids[b] : b, temperature t = temp[b]:
 *   if t > 0:   s_i = (y_i + bias_i) / t + g_i              [FS (2)-(4); SK 4]
 *   otherwise (t <= 0 or NaN, greedy): s_i = y_i + bias_i   [SK 3]
 *   out_idx[b] = the smallest i with the largest s_i among the s_i that are
 *   neither NaN nor -inf, or -1 if there is none            [FS (5), Stage 2]
 * where g_i = -log(-log u_i) is Gumbel noise of a midpoint-grid uniform u_i
 * drawn by Philox4x32-10 with key (seed lo, seed hi) and counter
 * (j, r, offset lo, offset hi) [MG "The change"]:
 *   default noise:  j = i >> 2, word i & 3, u = (top 23 bits + 1/2) / 2^23;
 *   FS_FP64_NOISE:  j = i >> 1, words 2(i&1) and 2(i&1)+1, u = (top 52 bits of
 *                   their concatenation + 1/2) / 2^52, and the score is formed
 *                   in float64 (noise in [1.1e-16, 36.7], a tail of about 40
 *                   rather than 20 nats [MG "What does this PR do"]).
 * This is an exact draw from softmax((y + bias) / t) [FS prerequisites].
 */
#ifndef FSAMPLE_H
#define FSAMPLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fs_status {
    FS_OK = 0,
    FS_ERR_INVALID_ARG = 1, /* null required pointer, non-positive size, V >= 2^31 */
    FS_ERR_UNSUPPORTED = 2, /* D not a multiple of 8 (16 FP8, 256 MXFP4), H/W not 16-byte aligned,
                               B > 2^22 or V * D beyond the addressable span (fused) */
    FS_ERR_WORKSPACE = 3,   /* workspace missing or smaller than fs_workspace_bytes() */
    FS_ERR_HIP = 4          /* a HIP launch or runtime call failed */
} fs_status;

typedef uint16_t fs_bf16;   /* bfloat16 bit pattern */
typedef void *fs_stream_t;  /* hipStream_t */

/* flags for fs_sample_fused, fs_sample_fused_w8 and fs_workspace_bytes */
#define FS_FP64_NOISE 0x1u

/*
 * Bytes of device workspace the sampling calls need for a batch of B rows over
 * a vocabulary of V entries (covers fs_sample_fused, fs_sample_fused_w8 and
 * fs_sample_logits; pass FS_FP64_NOISE in flags if any of them will use
 * float64 noise).  The workspace starts with a fixed 256 KiB region of completion counters, which
 * pick, for each batch tile (fused) or row (standalone), the workgroup that
 * runs Stage 2; the per-tile candidates (m, idx) of Stage 1 [FS Stage 1 step
 * (6)] follow it.  The caller allocates the workspace and must zero-fill it
 * once before its first use (hipMemset, torch.zeros); every call returns the
 * counters to zero by the time its work completes, so the workspace can then
 * be reused call after call, for any sizes, on one stream without clearing.
 * It must not be shared between calls that can run concurrently.  Counters
 * that are not zero give wrong or missing out_idx values (never a fault or a
 * hang).  Host only; returns 0 for invalid sizes.
 */
size_t fs_workspace_bytes(int64_t B, int64_t V, uint32_t flags);

/* Most places a Gumbel-top-k call returns per row. */
#define FS_TOPK_MAX 8

/*
 * Workspace bytes for the Gumbel-top-k calls (fs_sample_logits_topk,
 * fs_sample_fused_topk): the same counter region, then FS_TOPK_MAX candidates
 * per (row, tile).  Same zero-fill and reuse contract as fs_workspace_bytes;
 * a workspace of this size also serves every other call.  Host only; 0 for
 * invalid sizes.
 */
size_t fs_workspace_bytes_topk(int64_t B, int64_t V, uint32_t flags);

/*
 * Fused LM-head + exact sampling [FS "core method", "algorithm details"].
 *   H        device, bf16 [B, D]   hidden states of the decode batch
 *   W        device, bf16 [V, D]   LM-head weight (nn.Linear layout)
 *   B, D, V  host sizes: 0 <= B <= 2^22 (0 is a no-op), D >= 8 with
 *            D % 8 == 0, 1 <= V < 2^31
 *   temp     device, float [B]     per-row temperature (see the sampling rule)
 *   bias     device, float [B, V] or NULL: additive logit bias; -inf masks a
 *            token.  Added before the division by temperature [SK item 4].
 *   seed, offset  host: Philox key and the decode-step/position counter words
 *   out_idx  device, int64 [B]     sampled token per row, or -1
 *   row_ids  device, uint32 [B] or NULL (then row b has logical id b): the row
 *            identity the noise is keyed by, so that a row's draw does not depend
 *            on its batch position [MG "The change"]
 *   flags    host: 0 or FS_FP64_NOISE
 *   workspace, workspace_bytes  device scratch of at least
 *            fs_workspace_bytes(B, V, flags) bytes, zero-filled before its
 *            first use (see fs_workspace_bytes)
 *   stream   hipStream_t
 * Computes y = H W^T tile by tile on chip (bf16 inputs, float32 accumulation)
 * and never writes the [B, V] logits: Stage 1 keeps each row's per-tile
 * (max score, index), Stage 2 reduces those to out_idx [FS Stage 1, Stage 2].
 * Both stages run in one kernel launch.  H and W must be 16-byte aligned.
 */
fs_status fs_sample_fused(const fs_bf16 *H, const fs_bf16 *W, int64_t B, int64_t D,
                          int64_t V, const float *temp, const float *bias,
                          uint64_t seed, uint64_t offset, int64_t *out_idx,
                          const uint32_t *row_ids, uint32_t flags, void *workspace,
                          size_t workspace_bytes, fs_stream_t stream);

/*
 * fs_sample_fused for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, rule and results as fs_sample_fused, without the workspace:
 * the per-tile candidates and completion counters live in a scratch array
 * built into the library, one per GPU, of 4 MiB + 4 KiB (held until the
 * process ends), sized for
 *   B <= 1024 rows (FS_ERR_UNSUPPORTED beyond; B = 0 is a no-op).
 * The first call on a device looks up that device's copy of the array and
 * clears its counters with a small kernel on `stream`; no call allocates
 * (no hipMalloc, hipFree or allocating library routine).  Every call on a GPU
 * shares that GPU's array and leaves its counters at zero: calls that can
 * overlap on one GPU (other streams, other threads) race on it and must be
 * serialised by the caller.  bf16 weights, one draw per row.
 */
fs_status fs_sample_fused_noalloc(const fs_bf16 *H, const fs_bf16 *W, int64_t B, int64_t D,
                                  int64_t V, const float *temp, const float *bias,
                                  uint64_t seed, uint64_t offset, int64_t *out_idx,
                                  const uint32_t *row_ids, uint32_t flags, fs_stream_t stream);

/*
 * Fused LM-head + exact sampling with FP8 weights: W8 holds OCP FP8 E4M3 codes
 * [OFP8] (sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinities;
 * 0x7F and 0xFF are NaN) and row i of the weight is w_scale[i] * W8[i, :].
 *   H        device, bf16 [B, D]
 *   W8       device, uint8 [V, D]  E4M3 codes, row-major
 *   w_scale  device, float [V]     one scale per vocabulary row; the caller
 *            keeps it finite and positive (a zero, negative or non-finite
 *            scale gives that row's logits the IEEE meaning of the product)
 *   B, D, V  host sizes: 0 <= B <= 2^22, D >= 16 with D % 16 == 0,
 *            1 <= V < 2^31
 *   the other arguments, the workspace and the sampling rule are those of
 *   fs_sample_fused, with y_i = w_scale[i] * sum_d H[b,d] * e4m3(W8[i,d]).
 * Every E4M3 value is exactly a bf16 value: the kernel widens W8 on chip and
 * runs the same bf16 MFMA contraction (float32 accumulation) as
 * fs_sample_fused, then multiplies each row's sum by its scale.  W crosses
 * HBM at one byte per element, half the bytes of fs_sample_fused.  H and W8
 * must be 16-byte aligned.
 */
fs_status fs_sample_fused_w8(const fs_bf16 *H, const uint8_t *W8, const float *w_scale,
                             int64_t B, int64_t D, int64_t V, const float *temp,
                             const float *bias, uint64_t seed, uint64_t offset,
                             int64_t *out_idx, const uint32_t *row_ids, uint32_t flags,
                             void *workspace, size_t workspace_bytes, fs_stream_t stream);

/*
 * Standalone exact sampler over materialised float32 logits [MG "Problem",
 * "The change"; SD "Usage" sample(logits, temperature, seed, offset)].
 *   logits   device, float [B, V]  y_i of each row (no bias term)
 *   B, V     host sizes: B >= 0 (0 is a no-op), 1 <= V < 2^31
 *   temp     device, float [B]
 *   seed, offset  host
 *   fp64_noise    host: nonzero selects float64 race noise (52-bit uniforms
 *            from two Philox words) [MG "The change"]
 *   out_idx  device, int64 [B]
 *   row_ids  device, uint32 [B] or NULL
 *   workspace, workspace_bytes  as for fs_sample_fused (size it with
 *            FS_FP64_NOISE when fp64_noise is set)
 *   stream   hipStream_t
 * Same rule and the same Philox stream as fs_sample_fused, given the same
 * y + bias: the draw for (row id, vocabulary index) is identical in both.
 */
fs_status fs_sample_logits(const float *logits, int64_t B, int64_t V, const float *temp,
                           uint64_t seed, uint64_t offset, int fp64_noise,
                           int64_t *out_idx, const uint32_t *row_ids, void *workspace,
                           size_t workspace_bytes, fs_stream_t stream);

/*
 * Filtered exact sampling over materialised float32 logits [SD sample
 * pipeline, "Semantics"]: per row, the kept set of the filter chain
 * temperature -> top-k -> top-p -> min-p, then the draw of fs_sample_logits
 * (same transform, noise stream, keys and tie rule) over the kept tokens only.
 *   top_k    device, int32 [B] or NULL: keep the tokens whose logit is at
 *            least the k-th largest valid logit (a tie at that value is kept
 *            whole); off when k <= 0, k >= the row's number of valid logits,
 *            or top_k is NULL
 *   top_p    device, float [B] or NULL: over the top-k survivors with
 *            probabilities softmax(y / t), keep a token when the survivors with
 *            strictly larger logits carry less than p of their mass (the
 *            smallest prefix that reaches p, the crossing token included;
 *            equal logits are kept or dropped together); off when p >= 1, p is
 *            NaN or top_p is NULL; p <= 0 keeps the largest logit's tie class
 *   min_p    device, float [B] or NULL: over the top-p survivors, keep a token
 *            when its probability is at least m times the largest one; off
 *            when m <= 0, m is NaN or min_p is NULL; m >= 1 keeps the largest
 *            logit's tie class
 *   workspace, workspace_bytes  device, 256-byte aligned, at least
 *            fs_workspace_bytes_filtered(B, V) bytes (NULL when that is 0); zero
 *            it once before first use, as for fs_sample_fused: every call
 *            leaves its counters at zero, and calls sharing one workspace are
 *            serialised by their stream
 *   the other arguments as for fs_sample_logits.
 * Valid logits are those neither NaN nor -inf; no other token is ever kept,
 * and a row without one gets -1.  Greedy rows (t <= 0 or NaN) take the argmax
 * whatever the filters (each keeps the largest logit).  A row whose filters
 * are all off draws exactly what fs_sample_logits draws.  The top-p masses are
 * summed in 64-bit fixed point (units of 2^-40 of the largest token's mass),
 * so a call is reproducible bit for bit.
 */
fs_status fs_sample_logits_filtered(const float *logits, int64_t B, int64_t V,
                                    const float *temp, const int32_t *top_k,
                                    const float *top_p, const float *min_p, uint64_t seed,
                                    uint64_t offset, int fp64_noise, int64_t *out_idx,
                                    const uint32_t *row_ids, void *workspace,
                                    size_t workspace_bytes, fs_stream_t stream);

/*
 * Filtered exact sampling fused into the LM head [SD sample pipeline,
 * "Semantics"; FS "core method", "algorithm details"]: per row, exactly the
 * draw fs_sample_logits_filtered makes over the float32 logits y = H W^T that
 * the fused kernels form (fs_debug_logits), without writing those logits:
 *   H, W, B, D, V  as for fs_sample_fused (bf16, no bias), B <= 65535
 *   temp, top_k, top_p, min_p, seed, offset, out_idx, row_ids  as for
 *            fs_sample_logits_filtered (each filter array may be NULL: off)
 *   flags    host: 0 or FS_FP64_NOISE
 *   workspace, workspace_bytes  device, 256-byte aligned, at least
 *            fs_workspace_bytes_fused_filtered(B, V) bytes, zeroed once before
 *            first use (every call leaves its counters and flags at zero;
 *            calls sharing one workspace are serialised by their stream)
 * Stage 1 keeps, per row and vocabulary tile, the tile's 8 largest logits,
 * its best perturbed score, its mass sum exp((y - m) / t) relative to its
 * largest logit m and its count of valid logits [FS Stage 1; the grouped
 * form's per-group masses, "technical novelty"].  Stage 2 walks the tiles'
 * sorted lists in descending order to place the top-k, top-p and min-p cuts
 * and draws over the kept tokens.  A row whose cuts or draw reach below what
 * the lists hold (kept sets wider than the tiles' lists, e.g. top-p alone
 * over a flat row) is resolved exactly by a fallback in the same call: the
 * filtered sampler over that row's logits in the workspace.  Stage 1 writes
 * them there as it goes for sampled rows with top-p or min-p but no top-k
 * (the rows whose cuts usually lie below the lists); any other such row gets
 * them from a second pass of the fused matmul that stores only its logits.  Rows with top-k resolve with the
 * filtered sampler's fixed-point masses, so they draw what it draws bit for
 * bit; rows with top-p but no top-k take the total mass from the tiles'
 * float64 sums (a decision within about 1e-6 relative of its boundary may
 * differ).  Four launches on `stream`.
 */
size_t fs_workspace_bytes_fused_filtered(int64_t B, int64_t V);
fs_status fs_sample_fused_filtered(const fs_bf16 *H, const fs_bf16 *W, int64_t B, int64_t D,
                                   int64_t V, const float *temp, const int32_t *top_k,
                                   const float *top_p, const float *min_p, uint64_t seed,
                                   uint64_t offset, int64_t *out_idx, const uint32_t *row_ids,
                                   uint32_t flags, void *workspace, size_t workspace_bytes,
                                   fs_stream_t stream);

/*
 * Repetition penalty [SD sample pipeline and Semantics: the penalty comes
 * before the temperature]: out_logits = logits, except that every token
 * occurring in row b's previous tokens has its logit y replaced by
 * y * penalty[b] when y < 0 and by y / penalty[b] otherwise (float32,
 * correctly rounded; a token occurring several times is penalised once).
 * Rows whose penalty is not positive (or NaN) are copied unchanged.
 *   logits       device, float [B, V], 4-byte aligned
 *   prev_tokens  device, int64 [B, L]; entries outside [0, V) are padding
 *                (NULL when L = 0)
 *   penalty      device, float [B]
 *   out_logits   device, float [B, V]; may be logits itself (in place)
 *   B, V, L      host: 0 <= B <= 65535, 1 <= V < 2^31, L >= 0
 * Followed by fs_sample_logits_filtered at the row temperatures, this is the
 * card's sample pipeline (penalty, temperature, top-k, top-p, min-p, draw).
 */
fs_status fs_repetition_penalty(const float *logits, int64_t B, int64_t V,
                                const int64_t *prev_tokens, int64_t L, const float *penalty,
                                float *out_logits, fs_stream_t stream);

/*
 * The filter chain's output [SD API table, filter_logits; Semantics]: the
 * logits scaled by 1/t on fs_sample_logits_filtered's kept set, -inf off it,
 *   out_logits[b, i] = logits[b, i] * (1 / t)   for the kept tokens,
 *                      -inf                      elsewhere (NaN included);
 * greedy rows (t <= 0 or NaN) keep the largest valid logit's tie class,
 * unscaled.  With the same filters applied to a target's and a draft's
 * logits, fs_verify at temperature 1 on the two outputs verifies against the
 * filtered distributions (the card's filtered speculative decoding).
 *   out_logits  device, float [B, V], 4-byte aligned (may not alias logits)
 *   the other arguments as for fs_sample_logits_filtered; no workspace, one
 *   workgroup per row.
 */
fs_status fs_filter_logits(const float *logits, int64_t B, int64_t V, const float *temp,
                           const int32_t *top_k, const float *top_p, const float *min_p,
                           float *out_logits, fs_stream_t stream);

/*
 * Workspace bytes fs_sample_logits_filtered needs for (B, V): 0 when it runs
 * one workgroup per row (no workspace; NULL is accepted), otherwise the
 * library's fixed completion-counter region (the same leading 256 KiB every
 * entry point keeps its counters in, so one workspace can serve them all)
 * followed by each row's chunk headers and candidate lists (small batches
 * split each row over several workgroups).  0 for invalid sizes.
 */
size_t fs_workspace_bytes_filtered(int64_t B, int64_t V);

/*
 * Speculative-decoding verification over materialised float32 logits [SPV].
 * Per sequence b (logical row id r = row_ids[b], or b) and position i < K,
 * with p_t and p_d the temperature softmaxes of target row i and draft row i
 * (over the valid logits, those neither NaN nor -inf; a +inf maximum shares
 * the mass among the +inf logits; greedy rows, t <= 0 or NaN, are one-hot on
 * the first largest valid logit):
 *   the draft token x_i is accepted iff u_i * p_d(x_i) < p_t(x_i), i.e. with
 *   probability min(1, p_t(x_i) / p_d(x_i)); u_i = (k + 1/2) / 2^52 with k the
 *   top 52 bits of words 0 and 1 of Philox counter (2^32 - 1, r,
 *   offset + i) under the seed key (no noise value uses that counter); a
 *   token outside [0, V) has probability 0 under both and is rejected;
 *   accept_len[b] = the first rejected position, or K;
 *   out[b, j] = x_j for j < accept_len[b], -1 for j > accept_len[b], and at
 *   j = accept_len[b]:
 *     after a rejection, a draw from max(p_t - p_d, 0) renormalised (the
 *     Gumbel-max of log max(p_t - p_d, 0) with the noise fs_sample_logits
 *     uses at offset + j and row id r); if that residual is all zero, the
 *     draw fs_sample_logits makes from target row j at offset + j; on greedy
 *     rows, the target argmax;
 *     after K acceptances, the bonus draw: exactly fs_sample_logits on target
 *     row K at offset + K.
 * The tokens out[b, 0 .. accept_len[b]] are then distributed as the target
 * model's own draws.  Position i's noise and uniform use offset + i, the
 * absolute position: advance offset by at least the tokens emitted.
 *   target    device, float [B, K+1, V], 4-byte aligned (16-byte aligned
 *             rows with V % 4 == 0 take vector loads)
 *   draft     device, float [B, K, V]
 *   tokens    device, int64 [B, K] draft tokens
 *   B, K, V   host: 0 <= B <= 65536, 0 <= K <= FS_VERIFY_MAX_K, 1 <= V < 2^31
 *             (K = 0 is a plain draw from target row 0)
 *   temp      device, float [B]
 *   seed, offset, fp64_noise, row_ids   as for fs_sample_logits (fp64_noise
 *             selects the float64 noise of the residual and bonus draws; the
 *             acceptance uniforms are always 52-bit)
 *   accept_len  device, int64 [B];  out  device, int64 [B, K+1]
 *   workspace, workspace_bytes  device, 256-byte aligned, at least
 *             fs_workspace_bytes_verify(B, K, V) bytes, zeroed once before
 *             first use (every call leaves its counters at zero; calls sharing
 *             one workspace are serialised by their stream)
 * The softmax normalisers are float32 sums of float32 exponentials merged in
 * float64; the acceptance test runs in float64; the residual is formed in
 * float32.  Two launches on `stream`; deterministic for fixed arguments.
 */
#define FS_VERIFY_MAX_K 32
fs_status fs_verify(const float *target, const float *draft, const int64_t *tokens,
                    int64_t B, int64_t K, int64_t V, const float *temp, uint64_t seed,
                    uint64_t offset, int fp64_noise, int64_t *accept_len, int64_t *out,
                    const uint32_t *row_ids, void *workspace, size_t workspace_bytes,
                    fs_stream_t stream);

/*
 * Workspace bytes fs_verify needs for (B, K, V); 0 for invalid sizes.
 */
size_t fs_workspace_bytes_verify(int64_t B, int64_t K, int64_t V);

/*
 * Gumbel-top-k over materialised float32 logits [GTK]: k draws without
 * replacement per row, the places of the k largest perturbed scores s_i of
 * the sampling rule above (same transform, noise stream and keys as
 * fs_sample_logits), largest first; equal scores in increasing index order;
 * scores that are NaN or -inf never take a place.
 *   k        host, 1 <= k <= FS_TOPK_MAX
 *   out_idx  device, int64 [B, k] row-major: place j of row b at b * k + j,
 *            -1 for places past the row's number of valid scores
 *   workspace, workspace_bytes  at least fs_workspace_bytes_topk(B, V, flags)
 *            bytes (flags = FS_FP64_NOISE when fp64_noise is set)
 *   the other arguments as for fs_sample_logits.
 * Place 0 is the draw fs_sample_logits makes for the same arguments; the
 * places in order are a draw of k distinct tokens without replacement from
 * softmax(y / t) (Plackett-Luce); greedy rows (t <= 0 or NaN) get the k
 * largest y_i.
 */
fs_status fs_sample_logits_topk(const float *logits, int64_t B, int64_t V, const float *temp,
                                uint64_t seed, uint64_t offset, int fp64_noise, int k,
                                int64_t *out_idx, const uint32_t *row_ids, void *workspace,
                                size_t workspace_bytes, fs_stream_t stream);

/*
 * Fused LM-head + exact sampling with MXFP4 weights [MX]: row i of the weight
 * is D FP4 E2M1 elements (sign, 2 exponent bits with bias 1, 1 mantissa bit:
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6 and negatives) in blocks of 32 along D, block j
 * scaled by the E8M0 value 2^(e - 127) of w4_scale[i, j] (e = 255 is NaN).
 *   W4        device, uint8 [V, D/2]  element d of row i in byte i*D/2 + d/2,
 *             the low nibble for even d, the high nibble for odd d; 16-byte
 *             aligned
 *   w4_scale  device, uint8 [V, D/32] E8M0 block scales, 8-byte aligned
 *   B, D, V   host sizes: 0 <= B <= 2^22, D >= 256 with D % 256 == 0,
 *             1 <= V < 2^31
 *   the other arguments, the workspace and the sampling rule are those of
 *   fs_sample_fused, with y_i = sum_d H[b,d] * e2m1(W4[i,d]) * 2^(e(i,d/32)-127).
 * The kernel widens each element times its block scale to bf16 on chip
 * (exact while the scaled values stay in bf16's normal range: the caller
 * keeps 2^(e - 127) * 6 below 2^128 and 2^(e - 127) * 0.5 at least 2^-126)
 * and runs the bf16 MFMA contraction with float32 accumulation.  W crosses
 * HBM at half a byte per element plus one byte of scale per 32 elements.
 */
fs_status fs_sample_fused_mxfp4(const fs_bf16 *H, const uint8_t *W4, const uint8_t *w4_scale,
                                int64_t B, int64_t D, int64_t V, const float *temp,
                                const float *bias, uint64_t seed, uint64_t offset,
                                int64_t *out_idx, const uint32_t *row_ids, uint32_t flags,
                                void *workspace, size_t workspace_bytes, fs_stream_t stream);

/*
 * Gumbel-top-k fused into the LM head [GTK; FS "algorithm details"]: the
 * places of the k largest perturbed scores of fs_sample_fused's rule (same
 * logits, transform, noise stream and keys), largest first; equal scores in
 * increasing index order; NaN and -inf never take a place.
 *   k        host, 1 <= k <= FS_TOPK_MAX
 *   out_idx  device, int64 [B, k] row-major, -1 past a row's valid scores
 *   workspace, workspace_bytes  at least fs_workspace_bytes_topk(B, V, flags)
 *   the other arguments as for fs_sample_fused (bf16 W), with B <= 2^20.
 * Stage 1 keeps each row's FS_TOPK_MAX best places per vocabulary tile,
 * Stage 2 picks the row's k places from them; the [B, V] logits are never
 * written.  The noise is added after each pass's contraction (as with
 * FS_FP64_NOISE), so place 0 equals fs_sample_fused's draw wherever that
 * draw is not a near-tie in float32.
 */
fs_status fs_sample_fused_topk(const fs_bf16 *H, const fs_bf16 *W, int64_t B, int64_t D,
                               int64_t V, const float *temp, const float *bias,
                               uint64_t seed, uint64_t offset, int k, int64_t *out_idx,
                               const uint32_t *row_ids, uint32_t flags, void *workspace,
                               size_t workspace_bytes, fs_stream_t stream);

/*
 * Kernel timing.  Between fs_profile_begin() and fs_profile_end(), every
 * fs_sample_fused, fs_sample_fused_w8, fs_sample_fused_mxfp4 and
 * fs_sample_logits call (and their top-k forms) also records
 * HIP events on its stream around its one launch (Stage 1 with Stage 2 in its
 * last workgroups; the FlashSampling page, "reproduction", times kernels the
 * same way: device timestamps per kernel).  fs_profile_end() waits for those
 * events, writes the summed kernel duration in milliseconds and the number of
 * timed calls (either pointer may be NULL; host memory), and stops recording.
 * At most 4096 calls are timed per begin/end pair; later calls run untimed.
 * Enabling adds two event records per call and nothing else.  Process-wide;
 * host only.
 */
fs_status fs_profile_begin(void);
fs_status fs_profile_end(double *kernel_ms, int64_t *calls);

/*
 * fs_profile_end with the per-call figures as well (host memory, NULL to
 * skip): launch_ms[c] = call c's kernel duration (its two events) for
 * c < min(calls, cap); start_to_start_ms[c] = the time from call c's first
 * event to call c + 1's first event for c < min(calls - 1, cap - 1) -- with
 * calls issued back to back on one stream, the per-call step time.
 */
fs_status fs_profile_end_detail(double *kernel_ms, int64_t *calls, float *launch_ms,
                                float *start_to_start_ms, int64_t cap);

/* Weight formats for fs_fused_tiles. */
#define FS_WEIGHT_BF16 0
#define FS_WEIGHT_FP8 1
#define FS_WEIGHT_MXFP4 2

/*
 * Vocabulary tiles (workgroups along the vocabulary, one per CU) the fused
 * calls split V into for B rows of D-dimensional hidden states on the
 * current device: the count of per-tile candidates each row publishes
 * [FS Stage 1 step (6)], which a caller needs to price a call's candidate
 * traffic.  Host only (queries the device's CU count once); -1 on invalid
 * arguments (fs_last_error() says why).
 */
int fs_fused_tiles(int64_t B, int64_t D, int64_t V, int weight_format);

/*
 * Measurement hook: reads `bytes` of device memory at `buf` once with a
 * plain streaming kernel (16-byte loads, every workgroup a contiguous slice)
 * and xors what it read into *out (device uint64, not cleared).  Its duration
 * prices the read rate an HBM-bound kernel can practically reach on the
 * device; it is timed by fs_profile_begin/end like the sampling calls.
 * buf 16-byte aligned, bytes a multiple of 16.
 */
fs_status fs_debug_stream_read(const void *buf, size_t bytes, uint64_t *out, fs_stream_t stream);

/* Static description of a status code. */
const char *fs_status_string(fs_status status);

/* Detail of the last failure on the calling thread ("" if none). */
const char *fs_last_error(void);

/*
 * Test hook: the Philox4x32-10 words the samplers draw from.  For row b
 * (logical id row_ids[b], or b if row_ids is NULL) and counter j in
 * [0, n_ctr), out[(b * n_ctr + j) * 4 + w] is word w of counter
 * (j, id, offset lo, offset hi) under key (seed lo, seed hi).
 *   row_ids  device uint32 [B] or NULL;  out  device uint32 [B, n_ctr, 4]
 *   B >= 0, n_ctr >= 0, B * n_ctr < 2^31.
 */
fs_status fs_debug_philox_words(uint64_t seed, uint64_t offset, const uint32_t *row_ids,
                                int64_t B, int64_t n_ctr, uint32_t *out,
                                fs_stream_t stream);

/*
 * Test hook: the noise transforms the samplers apply to Philox words.
 * Default noise (fp64 == 0): for t < n, E[t] and g[t] are the exponential and
 * Gumbel variates the kernels derive from the single word words[t].
 * Float64 noise (fp64 != 0): from the word pair (words[2t], words[2t+1]).
 *   words device uint32 [n] or [2n];  E, g device float64 [n];  0 <= n < 2^31.
 */
fs_status fs_debug_noise(const uint32_t *words, int64_t n, int fp64, double *E, double *g,
                         fs_stream_t stream);

/*
 * Test hook: the logits y = H W^T of the fused path, written to Y (device,
 * float [B, V]).  Runs the same matmul code as fs_sample_fused (same tiling and
 * accumulation order) with a store in place of the sampling epilogue.
 * Same size and alignment rules as fs_sample_fused.
 */
fs_status fs_debug_logits(const fs_bf16 *H, const fs_bf16 *W, int64_t B, int64_t D,
                          int64_t V, float *Y, fs_stream_t stream);

/*
 * Test hook: the logits y = w_scale[i] * H e4m3(W8)^T of the FP8 path, written
 * to Y (device, float [B, V]); the twin of fs_debug_logits for
 * fs_sample_fused_w8, with its size and alignment rules.
 */
fs_status fs_debug_logits_w8(const fs_bf16 *H, const uint8_t *W8, const float *w_scale,
                             int64_t B, int64_t D, int64_t V, float *Y, fs_stream_t stream);

/*
 * Test hook: the logits of the MXFP4 path, written to Y (device, float
 * [B, V]); the twin of fs_debug_logits for fs_sample_fused_mxfp4, with its
 * size and alignment rules.
 */
fs_status fs_debug_logits_mxfp4(const fs_bf16 *H, const uint8_t *W4, const uint8_t *w4_scale,
                                int64_t B, int64_t D, int64_t V, float *Y, fs_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FSAMPLE_H */
