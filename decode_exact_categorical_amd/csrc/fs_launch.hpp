// fs_launch.hpp -- host-side launch entry points of the gfx950 kernels (internal;
// the public C ABI is include/fsample.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fs_device.hpp"

namespace fs {

// Kernel timing events of the library call being launched on this thread
// (set by the entry point while its calls are being timed, else null).  The
// first launch of a call carries the start event and every launch the stop
// event, both through the launch packet itself (hipExtLaunchKernelGGL), so
// timing adds no packet of its own between kernels.
struct LaunchTiming {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
LaunchTiming& launch_timing();

template <typename F, typename... Args>
inline void launch(F kernel, const dim3& grid, const dim3& block, uint32_t shmem,
                   hipStream_t stream, Args... args) {
  LaunchTiming& t = launch_timing();
  if (t.start != nullptr || t.stop != nullptr) {
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, t.start, t.stop, 0u, args...);
    t.start = nullptr;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, args...);
  }
}

// Fused sampling kernel (Stage 1: matmul + transform + noise + per-tile argmax;
// Stage 2 in the last workgroup of each batch tile) and its logits-store twin.
struct FusedArgs {
  const uint16_t* H;  // [B, D] bf16
  const uint16_t* W;  // [V, D] bf16, or null when W8 is given
  const uint8_t* W8;       // [V, D] OCP FP8 E4M3, or null
  const float* w_scale;    // [V] scale per vocabulary row (with W8)
  const uint8_t* W4;       // [V, D/2] MXFP4 E2M1 codes (element 2j low nibble), or null
  const uint8_t* w4_scale; // [V, D/32] E8M0 block scales (with W4)
  int64_t B, D, V;
  const float* temp;       // [B]
  const float* bias;       // [B, V] or null
  const uint32_t* row_ids;  // [B] or null
  NoiseKey key;
  void* cand;  // [B, nT] candidates
  int nT;      // vocabulary tiles = workgroups along x
  uint32_t* counters;  // [ceil(B / 64)] completion counters, zero between calls
  int64_t* out;        // [B] sampled indices
  float* Y;    // [B, V] (store epilogue only)
  int bias_vec4;  // bias rows are 16-byte aligned
  int k;          // Gumbel-top-k: places per row (out is [B, k]; cand is [B, nT, kTopKMax])
  // Filtered sampling (kEpiFilt32/64): per-row filters (each may be null:
  // off), cand is [B, nT] FiltRec records; Stage 1 also writes to Y the
  // logits of the rows filt_store_row picks.  Rows Stage 2 cannot resolve
  // from the records get row_flags[b] = 2 when their logits are in Y, else 1
  // (counted on *flag_count); the store epilogue then writes only the rows
  // flagged 1 (skipping the whole launch when *flag_count is 0).
  const int32_t* top_k;
  const float* top_p;
  const float* min_p;
  uint32_t* row_flags;   // [B], zero between calls
  uint32_t* flag_count;  // one word, zero between calls
};

enum FusedEpilogue {
  kEpiSample32 = 0,  // one draw per row, float32 noise
  kEpiSample64 = 1,  // one draw per row, float64 noise
  kEpiStore = 2,     // logits to Y (test hook)
  kEpiTopK32 = 3,    // Gumbel-top-k, float32 noise
  kEpiTopK64 = 4,    // Gumbel-top-k, float64 noise
  kEpiFilt32 = 5,    // filtered sampling, float32 noise
  kEpiFilt64 = 6     // filtered sampling, float64 noise
};

// What the filtered epilogue keeps of one (row, vocabulary tile) for Stage 2:
// the tile's kFiltList largest valid logits (larger first, equal logits in
// increasing index order; -inf / kNoIndex past the tile's valid tokens), its
// best perturbed score over all its valid tokens with that token's index and
// logit, its largest valid logit mm with zz = sum of exp((y - mm) / t) over
// its valid tokens, and its number of valid tokens.
constexpr int kFiltList = 8;
template <typename T>
struct FiltRec {
  float ly[kFiltList];
  int32_t li[kFiltList];
  T bs;
  float by;
  int32_t bi;
  float mm;
  uint32_t nv;
  double zz;
};
constexpr int kFiltRecBytes = 128;  // record stride in the workspace
static_assert(sizeof(FiltRec<double>) <= kFiltRecBytes, "a record fits its stride");
// Fused filtered sampling: Stage 1 with the filtered epilogue, Stage 2 (one
// wave per row), then the exact fallback for the rows Stage 2 flags: the same
// matmul storing those rows' logits to Y, and the filtered sampler over them
// (`fa` carries its arguments; its X is Y).
hipError_t launch_fused_filtered(const FusedArgs& a, bool fp64, const struct FilterArgs& fa,
                                 hipStream_t stream);
// Column blocks the filtered epilogue runs with for a batch of B rows.
int fused_filtered_column_blocks(int64_t B, bool fp64);

// Number of vocabulary tiles (workgroups along x) the fused kernel uses: one
// per CU, at most kMaxFusedTiles (Stage 2 reads a row's candidates in
// kMaxFusedTiles / 64 loads per lane).
constexpr int kMaxFusedTiles = 256;
static_assert(kMaxFusedTiles % 64 == 0, "whole waves of candidates");
// row_bytes (bytes of one W row; 0: unknown) lets it avoid splits whose
// workgroup ranges all start on 16 MiB boundaries.
int fused_num_tiles(int64_t V, int num_cus, int64_t row_bytes = 0);
// MFMA column blocks of 16 per batch tile: up to 4 (64 columns) for B <= 64
// or FP8 / MXFP4 weights, else 8 (tiles of 128 columns).
int fused_column_blocks(int64_t B, bool fp8_weights, bool fp64_noise);
// Largest byte span of W rows one wave addresses through 32-bit offsets.
int64_t fused_wave_span_bytes(int64_t V, int64_t D, int nT, int elem_bytes);
hipError_t launch_fused_stage1(const FusedArgs& a, int epilogue, hipStream_t stream);
// The wide-batch kernel (fs_wide.hip): bf16 weights, more than 64 rows,
// D % 32 == 0, one draw per row (float32 or float64 noise) or the logits.
bool fused_wide_applies(const FusedArgs& a, int epilogue);
bool fused_wide_shape(int64_t B, int64_t D, bool bf16_weights);
// Vocabulary tiles of the wide kernel (its batch tiles of 128 columns share
// the chip).
int fused_wide_tiles(int64_t B, int64_t V, int num_cus);
// Vocabulary tiles of a fused sampling or logits call of this shape.
int fused_call_tiles(int64_t B, int64_t D, int64_t V, bool bf16_weights, int num_cus, int64_t row_bytes);
hipError_t launch_fused_wide(const FusedArgs& a, int epilogue, hipStream_t stream);

// Standalone sampler over float32 logits (Stage 1, Stage 2 in the last
// workgroup of each row).
constexpr int kLogitsChunk = 2048;      // fewest logits per workgroup (sizes the workspace)
constexpr int kLogitsChunkMax = 131072;  // most logits per workgroup
int logits_chunk(int64_t B, int64_t V);         // logits per workgroup, top-k launches
int logits_sample_chunk(int64_t B, int64_t V);  // logits per workgroup, one-draw launches
struct LogitsArgs {
  const float* X;  // [B, V]
  int64_t B, V;
  const float* temp;
  const uint32_t* row_ids;  // [B] or null: then row b has id rid_base + b
  uint32_t rid_base;
  NoiseKey key;
  void* cand;  // [B, nT]
  int chunk;   // logits per workgroup: kLogitsChunk * 2^k <= kLogitsChunkMax
  int nT;      // ceil(V / chunk)
  uint32_t* counters;  // [B] completion counters (B <= 65536), zero between calls
  int64_t* out;        // [B] sampled indices
  int vec4;    // rows 16-byte aligned
  int k;       // Gumbel-top-k only: places per row (out is [B, k]); cand is [B, nT, kTopKMax]
};
hipError_t launch_logits_stage1(const LogitsArgs& a, bool fp64, hipStream_t stream);
hipError_t launch_logits_topk(const LogitsArgs& a, bool fp64, hipStream_t stream);

// Filtered sampling over materialised logits: one workgroup per row.
struct FilterArgs {
  const float* X;  // [B, V]
  int64_t B, V;
  const float* temp;
  const uint32_t* row_ids;  // [B] or null: then row b has id b
  const int32_t* top_k;     // [B] or null
  const float* top_p;       // [B] or null
  const float* min_p;       // [B] or null
  NoiseKey key;
  int64_t* out;  // [B]
  int vec4;      // rows 16-byte aligned
  // Split rows (small batches): per-row completion counters (zero between
  // calls) and filtered_split_words(B, V) 64-bit words of chunk headers and
  // candidate lists; null selects one workgroup per row.
  uint32_t* counters;
  uint64_t* split;
  // Filtered logits (launch_filter_logits): [B, V] out; vec4 then also
  // covers this buffer.
  float* Y;
  // Only the rows with row_flags[b] != 0 (null: every row), each clearing its
  // flag when done; workgroup 0 clears *flag_count.  One workgroup per row.
  uint32_t* row_flags;
  uint32_t* flag_count;
};
// Split rows up to this many run chunks and merge in one launch (the merge in
// each row's last workgroup): at B <= 8 that saves the second launch's gap;
// from B = 16 two launches win (40.1 against 44.5 us at B = 16, 40.5 against
// 55 at B = 24; V = 151936, top-k 50 + top-p 0.95).
constexpr int kSplitMaxRows = 8;
// Up to this many rows the chunks and the merges run as two launches (chunk
// workgroups two a CU, every row's merge at once); beyond it, one workgroup
// per row (measured at V = 151936, top-k 50 + top-p 0.95: 46.5 against 73.1 us
// at B = 32, 57.8 against 78.3 at B = 64, even at 128, behind from 256).
constexpr int kSplitTwoLaunchMaxRows = 96;
constexpr int kSplitMaxChunks = 32;   // chunks of a split row (V <= 262144)
int filtered_split_chunks(int64_t B, int64_t V);  // 0: one workgroup per row
size_t filtered_split_words(int64_t B, int64_t V);
hipError_t launch_logits_filtered(const FilterArgs& a, bool fp64, hipStream_t stream);
// The filter chain's output instead of a draw: a.Y[b, i] = y / t on the kept
// tokens, -inf elsewhere (one workgroup per row).
hipError_t launch_filter_logits(const FilterArgs& a, hipStream_t stream);

// Speculative-decoding verification over materialised target logits
// [B, K+1, V] and draft logits [B, K, V]: a statistics launch over every row,
// then a decision and draw launch.
constexpr int kVerifyMaxK = 32;          // draft tokens per sequence
constexpr int kVerifyChunk = 2048;       // fewest logits per workgroup (sizes the workspace)
constexpr int kVerifyChunkMax = 8192;    // most logits per workgroup
struct VerifyArgs {
  const float* target;     // [B, K+1, V]
  const float* draft;      // [B, K, V]
  const int64_t* tokens;   // [B, K]
  int64_t B, K, V;
  const float* temp;       // [B]
  const uint32_t* row_ids; // [B] or null: then row b has id b
  uint64_t seed, offset;   // position i's noise and uniform use offset + i
  int chunk, nC;           // statistics launch: logits per workgroup, chunks per row
  int chunk2, nC2;         // draw launch: the same
  void* stats;             // [B, 2K, nC] softmax partials (verify_stat_bytes each)
  void* bonus;             // [B, nC] candidates of the target's row K
  void* resid;             // [B, nC2] residual candidates
  uint32_t* counters;      // [B] completion counters, zero between calls
  int64_t* accept_len;     // [B]
  int64_t* out;            // [B, K+1]
  int vec4;                // rows 16-byte aligned
};
size_t verify_stat_bytes();
void verify_chunks(int64_t B, int64_t K, int64_t V, int* chunk, int* nC, int* chunk2, int* nC2);
hipError_t launch_verify(const VerifyArgs& a, bool fp64, hipStream_t stream);

// Repetition penalty over materialised logits: Y = X with the previous
// tokens' logits penalised (Y may be X).  One workgroup per chunk of a row.
constexpr int kPenaltyChunk = 8192;
struct PenaltyArgs {
  const float* X;          // [B, V]
  float* Y;                // [B, V]
  int64_t B, V;
  const int64_t* prev;     // [B, L]; entries outside [0, V) are padding
  int64_t L;
  const float* penalty;    // [B]
  int vec4;                // X and Y rows 16-byte aligned
};
hipError_t launch_repetition_penalty(const PenaltyArgs& a, hipStream_t stream);

// Measurement hook: one plain read of `bytes` (16-byte loads, a multiple of
// 16), xor-folded into *out so no load is dead (out is not cleared first).
hipError_t launch_stream_read(const void* buf, size_t bytes, int cus, uint64_t* out,
                              hipStream_t stream);

// Test hook: the noise transforms applied to given words.
hipError_t launch_noise(const uint32_t* words, int64_t n, bool fp64, double* E, double* g,
                        hipStream_t stream);

// Test hook: Philox words.
hipError_t launch_philox_words(NoiseKey key, const uint32_t* row_ids, int64_t B,
                               int64_t n_ctr, uint32_t* out, hipStream_t stream);

}  // namespace fs
