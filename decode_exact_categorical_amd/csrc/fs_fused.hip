// fs_fused.hip -- fused LM-head matmul + exact sampling for gfx950.
//
// Follows the FlashSampling page ("algorithm details", Stage 1 steps (1)-(6)
// and Stage 2): for a (batch tile x vocabulary tile) the logits Y = H W^T are
// formed on chip, transformed (bias, temperature), perturbed with Gumbel
// noise, and only the per-row tile maximum and its vocabulary index are
// written out.  The [B, V] logits never reach HBM.  Stage 2 runs in the same
// launch: the last workgroup to finish a batch tile reduces its candidates.
//
// Design for MI355X (the page's Triton kernel was written for NVIDIA parts):
//  * One workgroup per CU streams a contiguous slice of W exactly once.  Its
//    8 waves (two per SIMD) each own a contiguous run of vocabulary rows,
//    assigned in 8-row units so every wave of the chip ends within 8 rows of
//    the others.  A wave walks its rows in passes of up to 5 MFMA row blocks
//    (80 rows; 3 blocks, 48 rows, with more than 32 batch columns).
//  * W goes straight from HBM into VGPRs in the bf16 MFMA A-operand layout
//    (lane l holds 16 bytes of row l % 16; the four lanes of a row read 64
//    contiguous bytes).  Loads go in k-step pairs, the two halves of each
//    row's 128-byte segment back to back, with two pairs in flight.
//  * H is the MFMA B operand (batch as the N dimension, 16 to 64 columns).  It
//    is staged through LDS in chunks of 256 k, double-buffered and padded so
//    the fragment reads are bank-conflict free, and shared by the 8 waves: H
//    crosses L2 once per pass of the workgroup rather than once per wave.
//  * v_mfma_f32_16x16x32_bf16 accumulates in fp32, in one fixed k order per
//    vocabulary tile (its 256-k chunks from a per-tile starting chunk on,
//    wrapping around; ascending inside a chunk), so every logit's
//    accumulation order depends neither on B nor on the row's batch position.
//    The per-tile rotation keeps the chip's concurrent W requests spread over
//    the HBM channels; without it the stream rate depends markedly on where W
//    sits in physical memory.
//  * Float32 noise is not left for the end: the Gumbel noise of one output
//    fragment (4 vocabulary rows x 1 batch column per lane, one Philox4x32-10
//    call) is computed inside the memory-bound k-loop and folded into that
//    fragment's accumulator as bias + t * g, at a k-step fixed by the
//    fragment's row block and column block.  After the k-loop the score is
//    acc / t, i.e. (y + bias) / t + g up to fp32 rounding, and the epilogue
//    is a multiply and a compare.  Greedy columns (t <= 0 or NaN) fold in the
//    bias only.  Columns with an infinite (or beyond 2^60) temperature fold in
//    the bias and add g after the division, which keeps (y + bias) / t + g.
//  * Float64 noise keeps the score in float64: y + bias and the noise are
//    combined after the k-loop, with two Philox calls per fragment.
//  * FP8 weights (OCP E4M3 codes, a float32 scale per vocabulary row) stream
//    at one byte per element: a lane's 16-byte load holds two MFMA k-steps of
//    its row, widened on chip to bf16 (exact for every E4M3 value) before the
//    same bf16 MFMAs; the row scale multiplies the finished sum in float32,
//    and the noise is added after the k-loop.
//  * Scores feed a per-lane running argmax (larger score, then smaller index);
//    xor-shuffles and LDS reduce it to one candidate per batch row per
//    workgroup.
//  * Stage 2 needs no second launch: the workgroup that counts last on its
//    batch tile's counter reduces the tile's candidates (finish_last and
//    row_winner, fs_device.hpp), saving the launch and the gap between two
//    kernels, several microseconds against a ~220 us step.  Candidates are
//    published with device-coherent atomic stores, not an L2 write-back.
#include <type_traits>

#include "fs_launch.hpp"

namespace fs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kHPad = 8;          // bf16 padding per LDS column row (16 bytes)
constexpr float kInfTemp = 0x1p60f;  // at or above this, t * g is not kept in the accumulator

enum ColMode { kGreedy = 0, kSample = 1, kInfT = 2, kModeMask = 3, kFiltMass = 4, kFiltStore = 8 };

// Filtered sampling: rows whose cuts the tiles' lists are likely not to hold
// (top-p or min-p without top-k, a sampled row) get their logits written by
// Stage 1 itself, so that a row Stage 2 cannot settle needs no second matmul.
// Stage 1 and Stage 2 both decide with this function, on the same parameters.
__device__ __forceinline__ bool filt_store_row(float t, int32_t k, float p, float m) {
  return (t > 0.0f) && !(k > 0) && ((p < 1.0f) || (m > 0.0f));
}

// Weight formats: bf16, OCP FP8 E4M3 with a float32 scale per row, MXFP4
// (E2M1 elements, an E8M0 scale per block of 32 along k).  MXFP4 kernels
// stage each wave's rows of block scales in LDS for a pass while a row's
// scales fit the LDS row (D <= kS4MaxD); kWFp4Wide, for larger D, reads them
// from memory with each load-step pair's W.
enum WeightFormat { kWBf16 = 0, kWFp8 = 1, kWFp4 = 2, kWFp4Wide = 3 };
constexpr int kS4MaxD = 4096;
constexpr int kS4Row = kS4MaxD / 32 + 8;  // LDS bytes of a row's scales (8 of padding)
static_assert(kS4MaxD / 256 <= 16, "a row's scales in LDS are at most 16 pieces of 8 bytes");

template <int EPI>
struct ScoreType {
  typedef float type;
};
template <>
struct ScoreType<kEpiSample64> {
  typedef double type;
};
template <>
struct ScoreType<kEpiTopK64> {
  typedef double type;
};
template <>
struct ScoreType<kEpiFilt64> {
  typedef double type;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Fragments travel as raw 32-bit words and become bf16 only at the MFMA: a
// select between a loaded bf16 vector and a constant makes the compiler
// repack the vector as soon as it lands, i.e. wait for every load in flight.
__device__ __forceinline__ u32x4 load_frag(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 load_frag(const uint8_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Sixteen OCP FP8 E4M3 values (16 bytes, k ascending) as two bf16x8 MFMA
// operands: bytes 0..7 and bytes 8..15.  Every E4M3 value is a bf16 value, so
// the conversion (v_cvt_scalef32_pk_bf16_fp8, scale 1) is exact.
__device__ __forceinline__ void e4m3x16_to_bf16(u32x4 v, u32x4& lo, u32x4& hi) {
#define FS_CVT(W, HIGH) __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((W), 1.0f, HIGH))
  lo = u32x4{FS_CVT(v[0], false), FS_CVT(v[0], true), FS_CVT(v[1], false), FS_CVT(v[1], true)};
  hi = u32x4{FS_CVT(v[2], false), FS_CVT(v[2], true), FS_CVT(v[3], false), FS_CVT(v[3], true)};
#undef FS_CVT
}

__device__ __forceinline__ bf16x8 as_bf16(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Bias of 4 consecutive vocabulary rows i0..i0+3 of batch row b (0 past V).
__device__ __forceinline__ void load_bias4(const FusedArgs& a, int64_t b, int64_t i0, float beta[4]) {
  beta[0] = beta[1] = beta[2] = beta[3] = 0.f;
  if (!a.bias) return;
  const float* bp = a.bias + b * a.V + i0;
  if (a.bias_vec4 && i0 + 3 < a.V) {
    const float4 v = *reinterpret_cast<const float4*>(bp);
    beta[0] = v.x;
    beta[1] = v.y;
    beta[2] = v.z;
    beta[3] = v.w;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (i0 + j < a.V) beta[j] = bp[j];
  }
}

// How W flows through a wave, per batch width and epilogue (a wave has 256
// VGPRs at two waves per SIMD):
//  * up to 32 columns: 5 MFMA row blocks (80 rows) per pass, two k-step pairs
//    of W in flight, each row block reloaded as soon as its MFMAs issue;
//  * 48 and 64 columns: 5 row blocks with one pair in flight, each row block
//    reloaded as soon as its MFMAs issue ("ring of one"): a wave covers its
//    ~74 rows in one pass, where two pairs in flight would need passes of 3
//    row blocks, i.e. two passes, each restaging H and refilling the pipe.
//    Where the two k-steps' H fragments do not fit at once, they are read one
//    after the other (half_h);
//  * 64 columns with a bias or float64 noise: 3 row blocks, two pairs in
//    flight, each pair reloaded after all its MFMAs (no room for more).
// Passes of 4 row blocks (64 rows) stream W markedly slower than 3 or 5.
// FP8 weights (W8) and MXFP4 weights up to 32 columns: two pairs in flight,
// 5 row blocks, each pair reloaded after its MFMAs; at 48 and 64 columns the
// ring of one (5 row blocks, one pass), except 64 columns with a bias or
// float64 noise: 3 row blocks and two pairs in flight.  (The ring of one took
// FP8 at 48 / 64 columns from 137 / 160 to 122 / 149 us at the Qwen head and
// MXFP4 from 122 / 136 to 105 / 116.)
// Batch tiles wider than 64 columns (8 column blocks: the large-batch end,
// where the contraction approaches the MFMA roofline) use every W fragment
// for 8 MFMAs: 2 row blocks a pass (64 accumulators a lane), two pairs in
// flight, and H chunks of 128 k.  There the fragment slots that receive the
// noise are one per (row block, column block).
template <int NB, int EPI, bool HAS_BIAS, int WF>
struct Pipeline {
  static constexpr bool narrow = WF != kWBf16;  // FP8 or MXFP4 weights
  // Noise added after the k-loop (float64 noise, filtered sampling): the same
  // register budget as float64 noise.  (Gumbel-top-k with float32 noise folds
  // it, as the single draw does.)
  static constexpr bool late_noise = EPI == kEpiSample64 || EPI == kEpiTopK64 ||
                                     EPI == kEpiFilt32 || EPI == kEpiFilt64;
  static constexpr bool wide = NB > 4;
  static constexpr bool wide_extra = NB == 4 && (HAS_BIAS || (late_noise && EPI != kEpiFilt32));
  static constexpr bool ring1 = !wide && NB >= 3 && !wide_extra;
  static constexpr int row_blocks = wide ? 2 : ((NB <= 2 || ring1) ? 5 : 3);
  static constexpr bool half_h = ring1 && !narrow && (NB == 4 || HAS_BIAS || late_noise);
  static constexpr bool interleave = !narrow && !wide && !wide_extra;
  // k per H chunk in LDS.  MXFP4 at 16 and 32 columns takes chunks of two
  // load-step pairs (512 k), as FP8's 256-k chunks are: one barrier per four
  // 16-byte loads of a row (measured 5 us faster there; with 3-row-block
  // passes, and at 32 columns with a bias or float64 noise, whose registers
  // it overflows, 256-k chunks of one pair each are faster).
  static constexpr bool w4_long =
      (WF == kWFp4 || WF == kWFp4Wide) && (NB == 1 || (NB == 2 && !HAS_BIAS && !late_noise));
  static constexpr int chunk_k = wide ? 128 : (w4_long ? 512 : 256);
  // Fragment (rb, cb) gets its noise at k-step noise_slots * rb + cb.
  static constexpr int noise_slots = wide ? NB : 4;
  static_assert(!(wide && narrow), "FP8 and MXFP4 weights use batch tiles of at most 64 columns");
};

// Whether the noise is folded into the accumulators inside the k-loop: float32
// noise is over bf16 and MXFP4 weights (MXFP4's block scales are applied as
// the elements are widened, so its accumulator holds the logit itself), and
// over FP8 weights at 16 and 48 columns: FP8's row scale multiplies the
// finished sum, so its fold adds (bias + t g) / scale and keeps the scales
// live through the k-loop, which the 32- and 64-column FP8 kernels have no
// registers for (measured: they spill and run slower; they add the noise
// after the k-loop, as float64 noise does everywhere).  Rows whose scale is
// zero or not finite fold nothing and are scored from their sums after the
// k-loop.
template <int NB, int EPI, bool HAS_BIAS, int WF>
struct FoldNoise {
  static constexpr bool value =
      (EPI == kEpiSample32 || EPI == kEpiTopK32) && (WF != kWFp8 || (NB & 1) != 0);
};

// An FP8 row scale the fold can divide by: nonzero and finite.
__device__ __forceinline__ bool fold_scale_ok(float s) {
  return s != 0.0f && __builtin_fabsf(s) < __builtin_inff();
}

// BV4: the bias rows are 16-byte aligned (V % 4 == 0), so a fragment's four
// biases come in one load.
// ---------------------------------------------------------------------------
// Gumbel-top-k Stage 2 of one row, by one wave.  Lane l reads the sorted
// lists of tiles l, l + 64, l + 128, l + 192 (clamped addresses).  Among any k
// candidates the k-th best bounds the row's k-th place from below, so with
// theta the k-th best of the tile maxima (place 0 of each list), only
// candidates at or above theta can take a place: a prefix of each list, about
// k tiles' worth.  So the maxima come first, then only the lists whose maximum
// is at or above theta; the survivors go to the wave's LDS list and the places
// are picked from it, two candidates a lane.  A row with more survivors (rows
// with fewer than k valid scores) picks them from the lists themselves.
// ---------------------------------------------------------------------------
constexpr int kS2TilesPerLane = kMaxFusedTiles / 64;
constexpr int kS2SurvPerLane = 2;
constexpr int kS2SurvPerWave = 64 * kS2SurvPerLane;
constexpr int64_t kStage2InKernelRows = 16;  // widest tile whose Stage 2 runs in the fused kernel

template <typename T>
__device__ __forceinline__ void topk_load_maxima(const FusedArgs& a, int64_t b, int lane,
                                                 Cand<T> (&mx)[kS2TilesPerLane]) {
  const Cand<T>* rc = reinterpret_cast<const Cand<T>*>(a.cand) + b * a.nT * kTopKMax;
#pragma unroll
  for (int j = 0; j < kS2TilesPerLane; ++j) {
    const int t = lane + 64 * j;
    mx[j] = load_cand(rc + (t < a.nT ? t * kTopKMax : 0));
    if (t >= a.nT) mx[j] = Cand<T>{neg_inf<T>(), kNoIndex};
  }
}

template <typename T>
__device__ __forceinline__ void topk_row_places(const FusedArgs& a, int64_t b, int lane,
                                                const Cand<T> (&mx)[kS2TilesPerLane],
                                                Cand<T>* surv) {
  constexpr int kPer = kS2TilesPerLane * kTopKMax;
  const Cand<T>* rc = reinterpret_cast<const Cand<T>*>(a.cand) + b * a.nT * kTopKMax;
  // theta is the k-th place among the tile maxima.
  Cand<T> th = Cand<T>{neg_inf<T>(), kNoIndex};
#pragma unroll 1
  for (int r = 0; r < a.k; ++r) th = next_place(mx, r == 0, th.m, th.idx);
  // Then the rest of the lists whose maximum is at or above theta (the others
  // cannot hold a survivor).
  Cand<T> c[kPer];
#pragma unroll
  for (int j = 0; j < kS2TilesPerLane; ++j) {
    const int t = lane + 64 * j;
    const bool live = t < a.nT && !after(mx[j].m, mx[j].idx, th.m, th.idx);
    c[j * kTopKMax] = mx[j];
#pragma unroll
    for (int p = 1; p < kTopKMax; ++p) {
      c[j * kTopKMax + p] = Cand<T>{neg_inf<T>(), kNoIndex};
      if (live) c[j * kTopKMax + p] = load_cand(rc + t * kTopKMax + p);
    }
  }
  // The survivors (at or above theta) and this lane's offset among them.
  uint32_t cnt = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) cnt += after(c[q].m, c[q].idx, th.m, th.idx) ? 0u : 1u;
  uint32_t off = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t v = __shfl_up(off, o);
    if (lane >= o) off += v;
  }
  const uint32_t total = __shfl(off, 63);
  off -= cnt;
  Cand<T> pl = Cand<T>{neg_inf<T>(), kNoIndex};
  if (total <= (uint32_t)kS2SurvPerWave) {
#pragma unroll
    for (int q = 0; q < kPer; ++q)
      if (!after(c[q].m, c[q].idx, th.m, th.idx)) surv[off++] = c[q];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    Cand<T> c2[kS2SurvPerLane];
#pragma unroll
    for (int q = 0; q < kS2SurvPerLane; ++q)
      c2[q] = (uint32_t)(lane + 64 * q) < total ? surv[lane + 64 * q] : Cand<T>{neg_inf<T>(), kNoIndex};
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll 1
    for (int r = 0; r < a.k; ++r) {
      pl = next_place(c2, r == 0, pl.m, pl.idx);
      if (lane == 0) a.out[b * a.k + r] = pl.m == neg_inf<T>() ? (int64_t)-1 : (int64_t)pl.idx;
    }
  } else {
#pragma unroll 1
    for (int r = 0; r < a.k; ++r) {
      pl = next_place(c, r == 0, pl.m, pl.idx);
      if (lane == 0) a.out[b * a.k + r] = pl.m == neg_inf<T>() ? (int64_t)-1 : (int64_t)pl.idx;
    }
  }
}

// Stage 2 as its own launch: one wave per row, four rows a workgroup.
template <typename T>
__global__ __launch_bounds__(256) void topk_stage2_kernel(FusedArgs a) {
  __shared__ Cand<T> surv[4][kS2SurvPerWave];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t b = (int64_t)blockIdx.x * 4 + wave;
  if (b >= a.B) return;  // whole waves; nothing below waits on another wave
  Cand<T> mx[kS2TilesPerLane];
  topk_load_maxima(a, b, lane, mx);
  topk_row_places(a, b, lane, mx, surv[wave]);
}

template <int NB, int EPI, bool HAS_BIAS, int WF, bool BV4 = false>
__global__ __launch_bounds__(kThreads, 1) void fused_stage1_kernel(FusedArgs a) {
  typedef typename ScoreType<EPI>::type T;
  constexpr bool W8 = WF == kWFp8, W4 = WF == kWFp4 || WF == kWFp4Wide;
  constexpr bool kS4L = WF == kWFp4;  // MXFP4 scales staged in LDS
  constexpr bool kFold = FoldNoise<NB, EPI, HAS_BIAS, WF>::value;
  constexpr bool kTopK = EPI == kEpiTopK32 || EPI == kEpiTopK64;
  constexpr bool kFilt = EPI == kEpiFilt32 || EPI == kEpiFilt64;
  typedef Pipeline<NB, EPI, HAS_BIAS, WF> Pipe;
  // The fallback store of the filtered sampler: nothing to do when Stage 2
  // resolved every row.
  if (EPI == kEpiStore && a.flag_count != nullptr && *a.flag_count == 0u) return;
  // W element bytes, and k per 16-byte lane load (one MFMA k-step of bf16,
  // two of FP8).
  // A lane's 16-byte load holds 8 bf16, 16 FP8 or 32 FP4 values of its row;
  // the four lanes of a row cover kKPerLoad k (one load step).  W is
  // addressed in units of one element (bf16, FP8) or one byte (MXFP4).
  constexpr int kKPerLoad = W4 ? 128 : (W8 ? 64 : 32);
  constexpr int kKPerUnit = W4 ? 2 : 1;
  constexpr int kLaneUnits = WF == kWBf16 ? 8 : 16;
  constexpr int kKC = Pipe::chunk_k;
  constexpr int kStepsPerChunk = kKC / 32;
  constexpr int kHRow = kKC + kHPad;
  constexpr int kTile = 16 * NB;  // batch columns of the workgroup
  constexpr int kNoiseSlots = Pipe::noise_slots;
  constexpr int kLoadsPerChunk = kKC / kKPerLoad;
  typedef typename std::conditional<WF != kWBf16, uint8_t, uint16_t>::type WElem;
  const WElem* const wbase = W4   ? reinterpret_cast<const WElem*>(a.W4)
                             : W8 ? reinterpret_cast<const WElem*>(a.W8)
                                  : reinterpret_cast<const WElem*>(a.W);
  constexpr int kRB = Pipe::row_blocks;
  constexpr bool kRing1 = Pipe::ring1;
  constexpr bool kInterleave = Pipe::interleave;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // The wave index is wave-uniform; saying so keeps every quantity derived
  // from it (row range, row-block count) in scalar registers, so branches on
  // them are scalar and do not force the compiler to drain loads in flight.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane >> 4;  // operand k-group; output row group
  const int col = lane & 15;  // A row / B column / output column in a block

  const int64_t B = a.B, D = a.D, V = a.V;
  // Which (vocabulary tile, batch tile) this workgroup takes.  Workgroups go
  // to the 8 XCDs round-robin in launch order, so with several batch tiles the
  // linear id is remapped to put every batch tile of a vocabulary tile on one
  // XCD, launched together: they stream the same W rows at the same time and
  // all but one read them from that XCD's L2.
  const int nT = (int)gridDim.x, nbt = (int)gridDim.y;
  int tile = (int)blockIdx.x, btile = (int)blockIdx.y;
  if (nbt > 1 && nT % 8 == 0) {
    const int lin = (int)blockIdx.y * nT + (int)blockIdx.x;
    tile = (lin / (8 * nbt)) * 8 + lin % 8;
    btile = (lin / 8) % nbt;
  }
  const int64_t bt0 = (int64_t)btile * kTile;

  // Rows of this workgroup and of this wave, in 8-row units.
  const int64_t nunits = (V + 7) >> 3;
  const int64_t g0 = nunits * (int64_t)tile / nT;
  const int64_t g1 = nunits * (int64_t)(tile + 1) / nT;
  const int64_t nu = g1 - g0;
  const int64_t r0 = (g0 + nu * wave / kWaves) * 8;
  int64_t r1 = (g0 + nu * (wave + 1) / kWaves) * 8;
  if (r1 > V) r1 = V;
  const int nrb_wave = r1 > r0 ? (int)((r1 - r0 + 15) >> 4) : 0;
  // Passes are uniform across the workgroup (its waves meet at every H chunk).
  const int max_rb = (int)((((nu + kWaves - 1) / kWaves) * 8 + 15) >> 4);
  const int npass = (max_rb + kRB - 1) / kRB;

  const int KLS = (int)((D + kKPerLoad - 1) / kKPerLoad);  // load steps
  const int NC = (KLS + kLoadsPerChunk - 1) / kLoadsPerChunk;
  // The k-loop of a workgroup visits the H chunks from chunk `rot` on,
  // wrapping around (a rotation fixed per vocabulary tile).  Workgroups then
  // read different k ranges of their rows at the same moment, which spreads
  // the chip's concurrent W requests over more of the HBM channels than rows
  // read in lockstep at one k offset do.
  const int rot = tile % NC;
  // Logical chunk -> the chunk of k it holds.  (Chunks past the last one,
  // which only MXFP4's two-chunk loop reaches, stay past it: their H is zero.)
  auto phys_chunk = [&](int c) -> int { return c >= NC ? c : (c + rot < NC ? c + rot : c + rot - NC); };

  // Per-column sampling constants live in LDS (16 bytes a column), read when a
  // fragment is folded or scored; registers hold only each column's running
  // best (score, index).
  struct ColInfo {
    float t;
    float inv_t;
    uint32_t rid;
    int mode;
  };
  __shared__ ColInfo cols[16 * NB];
  if (tid < 16 * NB) {
    const int64_t b = bt0 + tid;
    const int64_t bc = b < B ? b : 0;
    float t = 1.0f;
    if (EPI != kEpiStore) t = a.temp[bc];
    ColInfo ci;
    ci.mode = !(t > 0.0f) ? kGreedy : (t < kInfTemp ? kSample : kInfT);
    ci.t = t;
    ci.inv_t = ci.mode == kGreedy ? 1.0f : 1.0f / t;
    ci.rid = a.row_ids ? a.row_ids[bc] : (uint32_t)bc;
    if constexpr (kFilt) {
      // Filtered sampling: the tile mass serves only a row whose top-p is on
      // without top-k (kFiltMass); others skip its exponentials.
      const float p = a.top_p ? a.top_p[bc] : 1.0f;
      const int32_t k = a.top_k ? a.top_k[bc] : 0;
      const float m = a.min_p ? a.min_p[bc] : 0.0f;
      if (p < 1.0f && p > 0.0f && !(k > 0)) ci.mode |= kFiltMass;
      if (a.Y != nullptr && filt_store_row(t, k, p, m)) ci.mode |= kFiltStore;
    }
    cols[tid] = ci;
  }
  bool col_ok[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) col_ok[cb] = bt0 + 16 * cb + col < B;

  // Running best (score, index) of each batch column of this wave across its
  // passes, in a wave-private LDS slot: registers hold one pass's bests, and
  // only after that pass's k-loop.
  __shared__ Cand<T> wrun[kWaves][16 * NB];
  if (EPI != kEpiStore && grp == 0) {
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) wrun[wave][16 * cb + col] = Cand<T>{neg_inf<T>(), kNoIndex};
  }
  // Gumbel-top-k: the running kTopKMax places of each batch column of this
  // wave across its passes (a wave-private LDS slot per column).
  constexpr int kTKW = kTopK ? kWaves : 1, kTKC = kTopK ? 16 * NB : 1, kTKK = kTopK ? kTopKMax : 1;
  __shared__ Cand<T> tkc[kTKW][kTKC][kTKK];
  if constexpr (kTopK) {
    if (grp == 0) {
#pragma unroll
      for (int cb = 0; cb < NB; ++cb)
#pragma unroll
        for (int j = 0; j < kTopKMax; ++j) tkc[wave][16 * cb + col][j] = Cand<T>{neg_inf<T>(), kNoIndex};
    }
  }

  // Filtered sampling: each batch column's running top-kFiltList logits and
  // its running best score, mass and count, per wave across its passes.
  struct FiltAux {
    T bs;
    float by;
    int32_t bi;
    float mm;
    uint32_t nv;
    double zz;
  };
  constexpr int kFLW = kFilt ? kWaves : 1, kFLC = kFilt ? 16 * NB : 1, kFLK = kFilt ? kFiltList : 1;
  __shared__ Cand<float> flc[kFLW][kFLC][kFLK];
  __shared__ FiltAux fla[kFLW][kFLC];
  if constexpr (kFilt) {
    if (grp == 0) {
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
#pragma unroll
        for (int j = 0; j < kFiltList; ++j) flc[wave][16 * cb + col][j] = Cand<float>{neg_inf<float>(), kNoIndex};
        fla[wave][16 * cb + col] = FiltAux{neg_inf<T>(), neg_inf<float>(), kNoIndex, neg_inf<float>(), 0u, 0.0};
      }
    }
  }

  __shared__ __attribute__((aligned(16))) uint16_t hs[2][16 * NB][kHRow];
  // MXFP4 block scales of each wave's rows in the current pass (kS4L).
  __shared__ __attribute__((aligned(8))) uint8_t s4l[kS4L ? kWaves : 1][kS4L ? 16 * kRB : 1][kS4L ? kS4Row : 8];

  // H chunk staging.  A chunk is 16*NB columns x kKC k = 16*NB*kKC/8 pieces of
  // 16 bytes; thread t stages pieces t + 512*q, q < kHQ, so every thread
  // issues the same kHQ loads and LDS stores (no branch around either).  Loads
  // use a clamped, always valid address; pieces past D or past B are stored as
  // zero.
  constexpr int kPPC = kKC / 8;                        // pieces per column
  constexpr int kHQ = 16 * NB * kPPC / kThreads;        // pieces per thread
  static_assert(16 * NB * kPPC % kThreads == 0, "whole pieces per thread");
  u32x4 hstage[kHQ];
  bool hvalid[kHQ];
  // Half QH of the pieces (the first (NB+1)/2 or the rest), so only half the
  // staging registers are live at a time.
  constexpr int kQSplit = (kHQ + 1) / 2;
  auto h_load = [&](int c, auto QH) {
    constexpr int q0 = decltype(QH)::value == 0 ? 0 : kQSplit;
    constexpr int q1 = decltype(QH)::value == 0 ? kQSplit : kHQ;
#pragma unroll
    for (int q = q0; q < q1; ++q) {
      const int piece = tid + kThreads * q;
      const int hc = piece / kPPC;               // column within the tile
      const int64_t k = (int64_t)phys_chunk(c) * kKC + (piece % kPPC) * 8;
      const int64_t b = bt0 + hc;
      hvalid[q] = b < B && k < D;
      hstage[q] = load_frag(a.H + (hvalid[q] ? b * D + k : 0));
    }
  };
  auto h_store = [&](int buf, auto QH) {
    constexpr int q0 = decltype(QH)::value == 0 ? 0 : kQSplit;
    constexpr int q1 = decltype(QH)::value == 0 ? kQSplit : kHQ;
#pragma unroll
    for (int q = q0; q < q1; ++q) {
      const int piece = tid + kThreads * q;
      const u32x4 z = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(&hs[buf][piece / kPPC][(piece % kPPC) * 8]) = hvalid[q] ? hstage[q] : z;
    }
  };

  for (int p = 0; p < npass; ++p) {
    const int rb_first = p * kRB;
    int nrb = nrb_wave - rb_first;
    nrb = nrb < 0 ? 0 : (nrb > kRB ? kRB : nrb);

    // Every k-step issues the same kRB loads and kRB x NB MFMAs, whatever the
    // wave's row count: a load or MFMA under a branch leaves the compiler unsure
    // how many loads are in flight, and it then drains them all before using
    // any.  Lanes past the wave's last row, and row blocks past nrb, re-read the
    // wave's last row (same cache lines, no extra HBM traffic); their results
    // are never scored.
    // Addresses: a wave-uniform base (scalar registers) plus a 32-bit element
    // offset per row block and lane (the host checks that a wave's rows span
    // less than 2^31 bytes).  A wave without rows reads row 0.  A lane's 16
    // bytes start 16 * grp bytes into each load step, in both formats.
    const int64_t rbase = nrb_wave > 0 ? r0 : 0;
    const int64_t rlast = nrb_wave > 0 ? r1 - 1 : 0;
    const int64_t row_units = D / kKPerUnit;
    const WElem* wwave = wbase + rbase * row_units;
    uint32_t woff[kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      int64_t row = r0 + 16 * (rb_first + rb) + col;
      if (row > rlast) row = rlast;
      woff[rb] = (uint32_t)((row - rbase) * row_units + kLaneUnits * grp);
    }
    // MXFP4: each lane's row's E8M0 scales, D/32 bytes a row; a lane reads the
    // 4 bytes of a load step's 4 blocks (one per lane of the row) with each
    // load-step pair.  With kS4L the wave's rows of scales for the pass are
    // first copied to its own LDS area (8-byte pieces, rows past the wave's
    // last repeat it) and read from there: read from memory a pair at a
    // time, a row's 128-byte line of scales is fetched again from HBM most
    // of the times it is used (the W stream evicts it from L2 in between),
    // about half as many bytes again as the weights.
    const uint8_t* swave = W4 ? a.w4_scale + rbase * (D / 32) : nullptr;
    uint32_t soff[kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      int64_t row = r0 + 16 * (rb_first + rb) + col;
      if (row > rlast) row = rlast;
      soff[rb] = W4 ? (uint32_t)((row - rbase) * (D / 32)) : 0u;
    }
    // A lane copies 8-byte piece lane % 16 of rows lane / 16 + 4 j: its loads
    // go out here, all of them before the first store waits (a load, a wait
    // and a store per piece in turn would start every pass with some twenty
    // HBM round trips one after the other), and the stores come after the
    // first W loads of the pass have been issued, so that the two round trips
    // overlap.  Lanes past a row's D / 256 pieces repeat its last one.
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    u32x2 sv[kS4L ? 4 * kRB : 1];
    int s4o = 0, s4r = 0;  // the lane's piece offset and first row
    if constexpr (kS4L) {
      const int ppr = (int)(D / 256);  // 8-byte pieces of a row: 1 .. kS4MaxD / 256
      // (An opaque copy of the lane index: computed from it, the addresses
      // are not hoisted out of the pass loop to occupy registers through the
      // k-loop.)
      int ln = lane;
      asm volatile("" : "+v"(ln));
      s4o = (ln % 16 < ppr ? ln % 16 : ppr - 1) * 8;
      s4r = ln / 16;
#pragma unroll
      for (int j = 0; j < 4 * kRB; ++j) {
        int64_t row = r0 + 16 * rb_first + s4r + 4 * j;
        if (row > rlast) row = rlast;
        sv[j] = *reinterpret_cast<const u32x2*>(swave + (row - rbase) * (D / 32) + s4o);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    f32x4 acc[kRB][NB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // FP8 weights: the scales of the lane's 4 output rows in each row block
    // (clamped, always valid addresses), for the finished sums; loaded here
    // when the fold needs them inside the k-loop, else after it.
    float wsc[kRB][4];
    auto load_scales = [&]() {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        const int64_t i0 = r0 + 16 * (rb_first + rb) + 4 * grp;
#pragma unroll
        for (int j = 0; j < 4; ++j) wsc[rb][j] = a.w_scale[i0 + j < V ? i0 + j : V - 1];
      }
    };
    if constexpr (W8 && kFold) load_scales();

    // Float32 noise of fragment slot f = 4*rb + cb (rb < kRB): bias + t * g of
    // the lane's 4 rows, or the bias alone for greedy and infinite-temperature
    // columns; the caller folds it into acc[rb][cb] (FS_FOLD_SLOT).  The bias
    // arrives from bias_slot_load, issued four k-steps earlier, so this issues no
    // memory operation.
    struct Fold {
      float v[4];
      bool any;
    };
    auto slot_noise = [&](int f, const f32x4& beta) -> Fold {
      Fold out = {{0.f, 0.f, 0.f, 0.f}, false};
      if (!kFold || f >= kRB * kNoiseSlots) return out;
      const int rb = f / kNoiseSlots, cb = f - rb * kNoiseSlots;
      if (rb >= nrb || cb >= NB) return out;
      out.any = true;
      const ColInfo ci = cols[16 * cb + col];
      const int m = ci.mode;
      const float t = ci.t;
      const uint32_t r = ci.rid;
      const bool ok = bt0 + 16 * cb + col < B;
      const int64_t i0 = r0 + 16 * (rb_first + rb) + 4 * grp;
      if (ok && i0 < r1) {
        if (HAS_BIAS) {
          out.v[0] = beta[0];
          out.v[1] = beta[1];
          out.v[2] = beta[2];
          out.v[3] = beta[3];
        }
        if (m == kSample) {
          const Words w = noise_words(a.key, (uint32_t)(i0 >> 2), r);
          out.v[0] += t * gumbel_f32(w.w0);
          out.v[1] += t * gumbel_f32(w.w1);
          out.v[2] += t * gumbel_f32(w.w2);
          out.v[3] += t * gumbel_f32(w.w3);
        }
      }
      return out;
    };
    // Bias of fragment slot f: four scalar loads from clamped, valid addresses
    // (the slot's values where they exist, something harmless elsewhere).
    auto bias_slot_load = [&](f32x4& dst, int f) {
      if (!HAS_BIAS || !kFold) return;
      const int ff = f < kRB * kNoiseSlots ? f : 0;
      const int rb = ff / kNoiseSlots, cb = ff - rb * kNoiseSlots;
      int64_t b = bt0 + 16 * cb + col;
      if (b > B - 1) b = B - 1;
      const int64_t i0 = r0 + 16 * (rb_first + rb) + 4 * grp;
      if constexpr (BV4) {
        // With V % 4 == 0 a fragment's rows are wholly inside or past V.
        int64_t i = i0 > V - 4 ? V - 4 : i0;
        if (i < 0) i = 0;
        dst = *reinterpret_cast<const f32x4*>(a.bias + b * V + i);
        return;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int64_t i = i0 + j;
        if (i > V - 1) i = V - 1;
        if (i < 0) i = 0;
        dst[j] = a.bias[b * V + i];
      }
    };
    // What a fold adds to row j of row block rb: the value itself, or over FP8
    // weights the value divided by the row's scale (nothing for a scale the
    // fold cannot divide by).
    auto fold_value = [&](float v, int rb, int j) -> float {
      if constexpr (W8) return fold_scale_ok(wsc[rb][j]) ? v / wsc[rb][j] : 0.0f;
      return v;
    };
#define FS_FOLD_SLOT(F, BETA)                                            \
  do {                                                                   \
    const int f_ = (F);                                                  \
    const Fold n_ = slot_noise(f_, (BETA));                              \
    if (n_.any) {                                                        \
      _Pragma("unroll") for (int rb2 = 0; rb2 < kRB; ++rb2)              \
        _Pragma("unroll") for (int cb2 = 0; cb2 < NB; ++cb2)             \
          if (rb2 * kNoiseSlots + cb2 == f_) {                           \
            acc[rb2][cb2][0] += fold_value(n_.v[0], rb2, 0);             \
            acc[rb2][cb2][1] += fold_value(n_.v[1], rb2, 1);             \
            acc[rb2][cb2][2] += fold_value(n_.v[2], rb2, 2);             \
            acc[rb2][cb2][3] += fold_value(n_.v[3], rb2, 3);             \
          }                                                              \
    }                                                                    \
  } while (0)

    // W of the load-step pair (2q, 2q + 1), row block by row block, so the
    // two 64-byte halves of each row's 128-byte segment are requested back to
    // back: HBM streams markedly faster so than when a whole step of row blocks
    // is requested at a time.  A load step is one k-step of 32 bf16 or two of
    // 64 FP8 values; a step past the last one re-reads the last one.  In a
    // final step that runs past D the lanes past D read k = 0 instead; H is
    // zero there, so their products vanish for finite W.
    // Logical step (loop order; past the end: the last one) -> load step.
    auto phys_step = [&](int ls) -> int {
      if (ls > NC * kLoadsPerChunk - 1) ls = NC * kLoadsPerChunk - 1;
      ls = phys_chunk(ls / kLoadsPerChunk) * kLoadsPerChunk + ls % kLoadsPerChunk;
      return ls > KLS - 1 ? KLS - 1 : ls;
    };
    auto step_base = [&](int ls) -> const WElem* {
      ls = phys_step(ls);
      const int64_t k = (int64_t)ls * kKPerLoad;
      const int kg = (kKPerLoad / 4) * grp;  // the lane's first k
      int64_t kl = 0;
      if (k + kKPerLoad > D) kl = (k + kg < D) ? 0 : -k - kg;
      return wwave + (k + kl) / kKPerUnit;
    };
    // MXFP4: the W fragments of load steps (2q, 2q + 1) and their scale words,
    // one 8-byte load for the pair (a pair's 256 k are 8 blocks of a row; D is
    // a multiple of 256, so a pair inside D starts at an even step, and a pair
    // past D re-reads the last pair's scales, against zero H).
    auto scale_words = [&](uint32_t (&sw)[2][kRB], int q) {
      const uint8_t* sp = swave + 4 * (phys_step(2 * q) & ~1);
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        const u32x2 v = kS4L ? *reinterpret_cast<const u32x2*>(&s4l[wave][16 * rb + col][sp - swave])
                             : *reinterpret_cast<const u32x2*>(sp + soff[rb]);
        sw[0][rb] = v[0];
        sw[1][rb] = v[1];
      }
    };
    auto load_pair4 = [&](u32x4 (&dst)[2][kRB], uint32_t (&sw)[2][kRB], int q) {
      const WElem* w0 = step_base(2 * q);
      const WElem* w1 = step_base(2 * q + 1);
      const uint8_t* sp = swave + 4 * (phys_step(2 * q) & ~1);
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        dst[0][rb] = load_frag(w0 + woff[rb]);
        dst[1][rb] = load_frag(w1 + woff[rb]);
        const u32x2 v = kS4L ? *reinterpret_cast<const u32x2*>(&s4l[wave][16 * rb + col][sp - swave])
                             : *reinterpret_cast<const u32x2*>(sp + soff[rb]);
        sw[0][rb] = v[0];
        sw[1][rb] = v[1];
      }
    };
    auto load_pair = [&](u32x4 (&dst)[2][kRB], int q) {
      const WElem* w0 = step_base(2 * q);
      const WElem* w1 = step_base(2 * q + 1);
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        dst[0][rb] = load_frag(w0 + woff[rb]);
        dst[1][rb] = load_frag(w1 + woff[rb]);
      }
    };
    // The MFMAs of one k-step pair, row block by row block, each row block's
    // W registers reloaded (pair q) as soon as its MFMAs have issued, so the
    // first loads of the next pair leave one row block after the data
    // arrived rather than a whole phase later.
    auto mma_reload = [&](u32x4 (&w)[2][kRB], int buf, int kk, int q) {
      const WElem* w0 = step_base(2 * q);
      const WElem* w1 = step_base(2 * q + 1);
      if constexpr (Pipe::half_h) {
        // The first k-step's MFMAs over every row block, then the second
        // k-step's with the reloads: one k-step of H fragments live at a time.
        {
          bf16x8 h0[NB];
#pragma unroll
          for (int cb = 0; cb < NB; ++cb)
            h0[cb] = *reinterpret_cast<const bf16x8*>(&hs[buf][16 * cb + col][kk + 8 * grp]);
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
            for (int cb = 0; cb < NB; ++cb)
              acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(w[0][rb]), h0[cb], acc[rb][cb], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 h1[NB];
#pragma unroll
        for (int cb = 0; cb < NB; ++cb)
          h1[cb] = *reinterpret_cast<const bf16x8*>(&hs[buf][16 * cb + col][kk + 32 + 8 * grp]);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
#pragma unroll
          for (int cb = 0; cb < NB; ++cb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(w[1][rb]), h1[cb], acc[rb][cb], 0, 0, 0);
          w[0][rb] = load_frag(w0 + woff[rb]);
          w[1][rb] = load_frag(w1 + woff[rb]);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        bf16x8 h0[NB], h1[NB];
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
          h0[cb] = *reinterpret_cast<const bf16x8*>(&hs[buf][16 * cb + col][kk + 8 * grp]);
          h1[cb] = *reinterpret_cast<const bf16x8*>(&hs[buf][16 * cb + col][kk + 32 + 8 * grp]);
        }
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
#pragma unroll
          for (int cb = 0; cb < NB; ++cb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(w[0][rb]), h0[cb], acc[rb][cb], 0, 0, 0);
#pragma unroll
          for (int cb = 0; cb < NB; ++cb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(w[1][rb]), h1[cb], acc[rb][cb], 0, 0, 0);
          w[0][rb] = load_frag(w0 + woff[rb]);
          w[1][rb] = load_frag(w1 + woff[rb]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    auto mma = [&](const u32x4 (&w)[kRB], int buf, int kk) {
      if constexpr (Pipe::wide) {
        // One H fragment at a time, used by every row block.
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
          const bf16x8 hf = *reinterpret_cast<const bf16x8*>(&hs[buf][16 * cb + col][kk + 8 * grp]);
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(w[rb]), hf, acc[rb][cb], 0, 0, 0);
        }
        return;
      }
      bf16x8 hf[NB];
#pragma unroll
      for (int cb = 0; cb < NB; ++cb)
        hf[cb] = *reinterpret_cast<const bf16x8*>(&hs[buf][16 * cb + col][kk + 8 * grp]);
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int cb = 0; cb < NB; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(w[rb]), hf[cb], acc[rb][cb], 0, 0, 0);
    };
    // MXFP4: the eight MFMA k-steps of one load-step pair (256 k from chunk
    // offset kk in buffer buf).  Load step ls of lane group g holds block
    // 4 ls + g, k in [kk + 128 ls + 32 g, +32); its dword i meets H at
    // k = kk + 128 ls + 32 g + 8 i.
    // v_cvt_scalef32_pk_bf16_fp4 widens two E2M1 values times the block's
    // scale (a power of two) to bf16: exact while the products stay in bf16's
    // normal range.
    auto mma4 = [&](const u32x4 (&w)[2][kRB], const uint32_t (&sw)[2][kRB], int buf, int kk) {
#pragma unroll
      for (int ls = 0; ls < 2; ++ls)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bf16x8 hf[NB];
#pragma unroll
          for (int cb = 0; cb < NB; ++cb)
            hf[cb] = *reinterpret_cast<const bf16x8*>(&hs[buf][16 * cb + col][kk + 128 * ls + 32 * grp + 8 * i]);
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb) {
            const uint32_t e = (sw[ls][rb] >> (8 * grp)) & 255u;
            const float sc = __builtin_bit_cast(
                float, e == 0u ? 0x00400000u : (e == 255u ? 0x7fc00000u : e << 23));
            const uint32_t d = w[ls][rb][i];
            const u32x4 v = u32x4{
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 0)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 1)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 2)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 3))};
#pragma unroll
            for (int cb = 0; cb < NB; ++cb)
              acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(v), hf[cb], acc[rb][cb], 0, 0, 0);
          }
        }
    };
    // FP8: the four MFMA k-steps of one load-step pair starting at chunk
    // offset kk.  Load step ls of lane group g holds k in [64 ls + 16 g, +16):
    // its first 8 values meet H at k = kk + 64 ls + 16 g, the next 8 at +8.
    // The order of k inside an MFMA's sum is the hardware's either way; which
    // k a lane carries is a choice the A and B operands make together.
    auto mma8 = [&](const u32x4 (&w)[2][kRB], int buf, int kk) {
#pragma unroll
      for (int ls = 0; ls < 2; ++ls) {
        bf16x8 h0[NB], h1[NB];
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
          h0[cb] = *reinterpret_cast<const bf16x8*>(&hs[buf][16 * cb + col][kk + 64 * ls + 16 * grp]);
          h1[cb] = *reinterpret_cast<const bf16x8*>(&hs[buf][16 * cb + col][kk + 64 * ls + 16 * grp + 8]);
        }
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          u32x4 lo, hi;
          e4m3x16_to_bf16(w[ls][rb], lo, hi);
#pragma unroll
          for (int cb = 0; cb < NB; ++cb) {
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(lo), h0[cb], acc[rb][cb], 0, 0, 0);
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(hi), h1[cb], acc[rb][cb], 0, 0, 0);
          }
        }
      }
    };

    // FP8 and MXFP4 with one load-step pair in flight (48 and 64 columns):
    // the pair's MFMAs load step by load step over every row block, and in
    // the last one each row block's W (and MXFP4 scale words) is reloaded
    // with pair q as soon as its MFMAs have issued.
    auto mma8_reload = [&](u32x4 (&w)[2][kRB], int buf, int kk, int q) {
      const WElem* w0 = step_base(2 * q);
      const WElem* w1 = step_base(2 * q + 1);
      // Per load step, the first 8 values of every row block, then the next
      // 8 (each accumulator still takes its MFMAs in mma8's order), so one
      // H fragment per column block is live at a time.
#pragma unroll
      for (int ls = 0; ls < 2; ++ls)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          bf16x8 hf[NB];
#pragma unroll
          for (int cb = 0; cb < NB; ++cb)
            hf[cb] = *reinterpret_cast<const bf16x8*>(&hs[buf][16 * cb + col][kk + 64 * ls + 16 * grp + 8 * h]);
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb) {
            u32x4 lo, hi;
            e4m3x16_to_bf16(w[ls][rb], lo, hi);
#pragma unroll
            for (int cb = 0; cb < NB; ++cb)
              acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(h == 0 ? lo : hi), hf[cb], acc[rb][cb],
                                                                    0, 0, 0);
            if (ls == 1 && h == 1) {
              w[0][rb] = load_frag(w0 + woff[rb]);
              w[1][rb] = load_frag(w1 + woff[rb]);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto mma4_reload = [&](u32x4 (&w)[2][kRB], uint32_t (&sw)[2][kRB], int buf, int kk, int q) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const WElem* w0 = step_base(2 * q);
      const WElem* w1 = step_base(2 * q + 1);
      const uint8_t* sp = swave + 4 * (phys_step(2 * q) & ~1);
#pragma unroll
      for (int ls = 0; ls < 2; ++ls)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bf16x8 hf[NB];
#pragma unroll
          for (int cb = 0; cb < NB; ++cb)
            hf[cb] = *reinterpret_cast<const bf16x8*>(&hs[buf][16 * cb + col][kk + 128 * ls + 32 * grp + 8 * i]);
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb) {
            const uint32_t e = (sw[ls][rb] >> (8 * grp)) & 255u;
            const float sc = __builtin_bit_cast(
                float, e == 0u ? 0x00400000u : (e == 255u ? 0x7fc00000u : e << 23));
            const uint32_t d = w[ls][rb][i];
            const u32x4 v = u32x4{
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 0)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 1)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 2)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 3))};
#pragma unroll
            for (int cb = 0; cb < NB; ++cb)
              acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(v), hf[cb], acc[rb][cb], 0, 0, 0);
            if (ls == 1 && i == 3) {
              w[0][rb] = load_frag(w0 + woff[rb]);
              w[1][rb] = load_frag(w1 + woff[rb]);
              const u32x2 sv = kS4L ? *reinterpret_cast<const u32x2*>(&s4l[wave][16 * rb + col][sp - swave])
                                    : *reinterpret_cast<const u32x2*>(sp + soff[rb]);
              sw[0][rb] = sv[0];
              sw[1][rb] = sv[1];
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          if (ls == 1 && i == 3) __builtin_amdgcn_sched_barrier(0);
        }
    };

    // The k-loop is straight-line: every k-step pair issues the same loads in
    // the same order (2 x kRB W fragments, then the biases of the slots folded
    // four steps later), every chunk the same NB H loads, and every pass runs
    // NC * 8 k-steps (steps past the last real one re-read it against zero H).
    // The compiler can then count loads in flight exactly and waits only for
    // the ones it needs, keeping two k-step pairs of W in flight across the
    // barriers.
    typedef std::integral_constant<int, 0> Half0;
    typedef std::integral_constant<int, 1> Half1;
    // The first H chunk's loads go out first and its LDS stores come after the
    // first W loads, so the W stream starts one H round trip earlier (loads
    // complete in order: waiting for H then waits for nothing issued later).
    h_load(0, Half0{});
    h_load(0, Half1{});

    u32x4 pa[2][kRB], pb[2][kRB];
    uint32_t sa[2][kRB], sb[2][kRB];  // MXFP4 scale words of pa, pb
    const f32x4 z4 = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 ba0 = z4, ba1 = z4, bb0 = z4, bb1 = z4;
    // The prologue issues pair 0 before pair 1, as the loop does: were the
    // scheduler to swap them, the first pass through the loop head would see
    // pair 0 as the newest loads, and the compiler would wait for nearly all
    // loads there on every pass.
    // With the MXFP4 scales in LDS, the first pairs' scale words are read once
    // the staged scales are stored (after the pairs' W loads).
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (W4 && !kS4L)
      load_pair4(pa, sa, 0);
    else
      load_pair(pa, 0);
    bias_slot_load(ba0, 0);
    bias_slot_load(ba1, 1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (W4 && !kS4L && !kRing1)
      load_pair4(pb, sb, 1);
    else if constexpr (!kRing1)
      load_pair(pb, 1);
    bias_slot_load(bb0, 2);
    bias_slot_load(bb1, 3);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kS4L) {
#pragma unroll
      for (int j = 0; j < 4 * kRB; ++j) *reinterpret_cast<u32x2*>(&s4l[wave][s4r + 4 * j][s4o]) = sv[j];
      // (The area is the wave's own: its LDS operations complete in order.)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      scale_words(sa, 0);
      if constexpr (!kRing1) scale_words(sb, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    h_store(0, Half0{});
    h_store(0, Half1{});
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    static_assert(kStepsPerChunk % 4 == 0, "a chunk holds whole pairs of pairs");
    // One H chunk per iteration, not unrolled: an unrolled or peeled copy
    // enters the loop with its loads in another order, and the compiler then
    // waits for nearly all loads in flight at the loop head.
    if constexpr (W4 && !Pipe::w4_long) {
      // MXFP4 in 256-k chunks: a chunk is one load-step pair; two chunks per
      // iteration (pa in buffer 0, pb in buffer 1) keep two pairs in flight.
      // An odd chunk count gets one empty chunk (zero H) at the end.  Noise
      // slots 2c and 2c + 1 are folded after chunk c, their biases loaded a
      // chunk ahead.
      const int NCe = NC + (NC & 1);
#pragma unroll 1
      for (int c = 0; c < NCe; c += 2) {
        h_load(c + 1, Half0{});
        h_load(c + 1, Half1{});
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kRing1) {
          // One pair in flight (48 and 64 columns): both chunks' pairs run
          // through pa, each reloaded with the next chunk's as it is used.
          mma4_reload(pa, sa, 0, 0, c + 1);
          FS_FOLD_SLOT(2 * c, ba0);
          FS_FOLD_SLOT(2 * c + 1, ba1);
          __builtin_amdgcn_sched_barrier(0);
          bias_slot_load(ba0, 2 * c + 4);
          bias_slot_load(ba1, 2 * c + 5);
          __builtin_amdgcn_sched_barrier(0);
          h_store(1, Half0{});
          h_store(1, Half1{});
          __syncthreads();
          h_load(c + 2, Half0{});
          h_load(c + 2, Half1{});
          __builtin_amdgcn_sched_barrier(0);
          mma4_reload(pa, sa, 1, 0, c + 2);
          FS_FOLD_SLOT(2 * c + 2, bb0);
          FS_FOLD_SLOT(2 * c + 3, bb1);
          __builtin_amdgcn_sched_barrier(0);
          bias_slot_load(bb0, 2 * c + 6);
          bias_slot_load(bb1, 2 * c + 7);
          __builtin_amdgcn_sched_barrier(0);
          h_store(0, Half0{});
          h_store(0, Half1{});
          __syncthreads();
          continue;
        }
        mma4(pa, sa, 0, 0);
        FS_FOLD_SLOT(2 * c, ba0);
        FS_FOLD_SLOT(2 * c + 1, ba1);
        __builtin_amdgcn_sched_barrier(0);
        load_pair4(pa, sa, c + 2);
        bias_slot_load(ba0, 2 * c + 4);
        bias_slot_load(ba1, 2 * c + 5);
        __builtin_amdgcn_sched_barrier(0);
        h_store(1, Half0{});
        h_store(1, Half1{});
        __syncthreads();
        h_load(c + 2, Half0{});
        h_load(c + 2, Half1{});
        __builtin_amdgcn_sched_barrier(0);
        mma4(pb, sb, 1, 0);
        FS_FOLD_SLOT(2 * c + 2, bb0);
        FS_FOLD_SLOT(2 * c + 3, bb1);
        __builtin_amdgcn_sched_barrier(0);
        load_pair4(pb, sb, c + 3);
        bias_slot_load(bb0, 2 * c + 6);
        bias_slot_load(bb1, 2 * c + 7);
        __builtin_amdgcn_sched_barrier(0);
        h_store(0, Half0{});
        h_store(0, Half1{});
        __syncthreads();
      }
    }
#pragma unroll 1
    for (int c = 0; c < ((W4 && !Pipe::w4_long) ? 0 : NC); ++c) {
      const int buf = c & 1;
      const int cn = c + 1 < NC ? c + 1 : c;
      h_load(cn, Half0{});
      if constexpr (Pipe::wide) h_load(cn, Half1{});
      if constexpr (W8) {
        // FP8: a chunk of 256 k is two load-step pairs, 2c (pa) and 2c + 1 (pb).
        // The next chunk's H is loaded first and stored last: waiting for it
        // earlier would also wait for every W load issued before it (loads
        // complete in order), draining the pipe to one pair.
        // Noise slots 4c + j are folded two per pair, their biases loaded a
        // chunk ahead.
        h_load(cn, Half1{});
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kRing1) {
          // One pair in flight: the chunk's two pairs both run through pa.
          mma8_reload(pa, buf, 0, 2 * c + 1);
          FS_FOLD_SLOT(4 * c, ba0);
          FS_FOLD_SLOT(4 * c + 1, ba1);
          __builtin_amdgcn_sched_barrier(0);
          bias_slot_load(ba0, 4 * c + 4);
          bias_slot_load(ba1, 4 * c + 5);
          __builtin_amdgcn_sched_barrier(0);
          mma8_reload(pa, buf, 128, 2 * c + 2);
          FS_FOLD_SLOT(4 * c + 2, bb0);
          FS_FOLD_SLOT(4 * c + 3, bb1);
          __builtin_amdgcn_sched_barrier(0);
          bias_slot_load(bb0, 4 * c + 6);
          bias_slot_load(bb1, 4 * c + 7);
          __builtin_amdgcn_sched_barrier(0);
          h_store(buf ^ 1, Half0{});
          h_store(buf ^ 1, Half1{});
          __syncthreads();
          continue;
        }
        mma8(pa, buf, 0);
        FS_FOLD_SLOT(4 * c, ba0);
        FS_FOLD_SLOT(4 * c + 1, ba1);
        __builtin_amdgcn_sched_barrier(0);
        load_pair(pa, 2 * c + 2);
        bias_slot_load(ba0, 4 * c + 4);
        bias_slot_load(ba1, 4 * c + 5);
        __builtin_amdgcn_sched_barrier(0);
        mma8(pb, buf, 128);
        FS_FOLD_SLOT(4 * c + 2, bb0);
        FS_FOLD_SLOT(4 * c + 3, bb1);
        __builtin_amdgcn_sched_barrier(0);
        load_pair(pb, 2 * c + 3);
        bias_slot_load(bb0, 4 * c + 6);
        bias_slot_load(bb1, 4 * c + 7);
        __builtin_amdgcn_sched_barrier(0);
        h_store(buf ^ 1, Half0{});
        h_store(buf ^ 1, Half1{});
        __syncthreads();
        continue;
      }
      if constexpr (W4) {
        // MXFP4 in 512-k chunks: a chunk is two load-step pairs, 2c (pa) and 2c + 1
        // (pb), with H loaded and stored as for FP8.  Noise slots 4c + j are
        // folded two per pair, their biases loaded a chunk ahead.  When D is
        // an odd multiple of 256 the last chunk's second pair lies past D: it
        // re-reads the last load step against zero H.
        h_load(cn, Half1{});
        __builtin_amdgcn_sched_barrier(0);
        mma4(pa, sa, buf, 0);
        FS_FOLD_SLOT(4 * c, ba0);
        FS_FOLD_SLOT(4 * c + 1, ba1);
        __builtin_amdgcn_sched_barrier(0);
        load_pair4(pa, sa, 2 * c + 2);
        bias_slot_load(ba0, 4 * c + 4);
        bias_slot_load(ba1, 4 * c + 5);
        __builtin_amdgcn_sched_barrier(0);
        mma4(pb, sb, buf, 256);
        FS_FOLD_SLOT(4 * c + 2, bb0);
        FS_FOLD_SLOT(4 * c + 3, bb1);
        __builtin_amdgcn_sched_barrier(0);
        load_pair4(pb, sb, 2 * c + 3);
        bias_slot_load(bb0, 4 * c + 6);
        bias_slot_load(bb1, 4 * c + 7);
        __builtin_amdgcn_sched_barrier(0);
        h_store(buf ^ 1, Half0{});
        h_store(buf ^ 1, Half1{});
        __syncthreads();
        continue;
      }
#pragma unroll
      for (int j = 0; j < kStepsPerChunk; j += 4) {
        const int ks = c * kStepsPerChunk + j;
        const int q = ks >> 1;
        // sched_barrier keeps each phase where it is written, so the compiler
        // does not move the loads of a pair next to their use.
        if constexpr (kRing1) {
          mma_reload(pa, buf, j * 32, q + 1);
          FS_FOLD_SLOT(ks, ba0);
          FS_FOLD_SLOT(ks + 1, ba1);
        } else if constexpr (kInterleave) {
          mma_reload(pa, buf, j * 32, q + 2);
          FS_FOLD_SLOT(ks, ba0);
          FS_FOLD_SLOT(ks + 1, ba1);
        } else {
          mma(pa[0], buf, j * 32);
          FS_FOLD_SLOT(ks, ba0);
          mma(pa[1], buf, (j + 1) * 32);
          FS_FOLD_SLOT(ks + 1, ba1);
          __builtin_amdgcn_sched_barrier(0);
          load_pair(pa, q + 2);
        }
        __builtin_amdgcn_sched_barrier(0);
        bias_slot_load(ba0, ks + 4);
        bias_slot_load(ba1, ks + 5);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kRing1) {
          mma_reload(pa, buf, (j + 2) * 32, q + 2);
          FS_FOLD_SLOT(ks + 2, bb0);
          FS_FOLD_SLOT(ks + 3, bb1);
        } else if constexpr (kInterleave) {
          mma_reload(pb, buf, (j + 2) * 32, q + 3);
          FS_FOLD_SLOT(ks + 2, bb0);
          FS_FOLD_SLOT(ks + 3, bb1);
        } else {
          mma(pb[0], buf, (j + 2) * 32);
          FS_FOLD_SLOT(ks + 2, bb0);
          mma(pb[1], buf, (j + 3) * 32);
          FS_FOLD_SLOT(ks + 3, bb1);
          __builtin_amdgcn_sched_barrier(0);
          load_pair(pb, q + 3);
        }
        __builtin_amdgcn_sched_barrier(0);
        bias_slot_load(bb0, ks + 6);
        bias_slot_load(bb1, ks + 7);
        __builtin_amdgcn_sched_barrier(0);
        // The other buffer was last read in the previous chunk, before the
        // barrier that ended it, so the next chunk can land there at once.
        // Wide tiles (one j step a chunk) store the whole next chunk here,
        // loaded at the chunk's start: only W loads issued after it are in
        // flight behind it.
        if constexpr (Pipe::wide) {
          h_store(buf ^ 1, Half0{});
          h_store(buf ^ 1, Half1{});
        } else if (j == 0) {
          h_store(buf ^ 1, Half0{});
          h_load(cn, Half1{});
        } else {
          h_store(buf ^ 1, Half1{});
        }
      }
      __syncthreads();
    }
    // Short contractions (fewer k-steps, or MXFP4 chunks, than slots): the
    // remaining slots.
    for (int f = W8 ? 4 * NC : (!W4 ? NC * kStepsPerChunk : (Pipe::w4_long ? 4 * NC : 2 * (NC + (NC & 1))));
         f < kRB * kNoiseSlots; ++f) {
      f32x4 bt = f32x4{0.f, 0.f, 0.f, 0.f};
      bias_slot_load(bt, f);
      FS_FOLD_SLOT(f, bt);
    }
#undef FS_FOLD_SLOT

    if constexpr (W8 && !kFold) load_scales();

    // End of pass: scores of this wave's fragments.
    T bm[NB];
    int32_t bi[NB];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      bm[cb] = neg_inf<T>();
      bi[cb] = kNoIndex;
    }
    if constexpr (kTopK) {
      // Column block by column block: the lane's scores of the pass, in
      // increasing index order, into a sorted list in registers; then that
      // list, the column's other three row groups' lists and the column's
      // running places (LDS) merge into the new running places.
#pragma unroll 1
      for (int cb = 0; cb < NB; ++cb) {
        T lm[kTopKMax];
        int32_t li[kTopKMax];
#pragma unroll
        for (int j = 0; j < kTopKMax; ++j) {
          lm[j] = neg_inf<T>();
          li[j] = kNoIndex;
        }
        const ColInfo ci = cols[16 * cb + col];
        const bool greedy = ci.mode == kGreedy;
        const T it = greedy ? T(1) : T(1) / T(ci.t);
        const int64_t bcol = bt0 + 16 * cb + col < B ? bt0 + 16 * cb + col : B - 1;
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          if (rb >= nrb) break;
          f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c2 = 0; c2 < NB; ++c2)
            if (c2 == cb) y = acc[rb][c2];
          const int64_t i0 = r0 + 16 * (rb_first + rb) + 4 * grp;
          T s[4];
          if constexpr (kFold) {
            // The noise and the bias are in the sums already: acc / t (greedy
            // columns carry 1 / t = 1), infinite temperatures add g after it.
#pragma unroll
            for (int j = 0; j < 4; ++j) s[j] = T(y[j] * ci.inv_t);
            if (__builtin_amdgcn_ballot_w64(ci.mode == kInfT) != 0ull && ci.mode == kInfT) {
              const Words w = noise_words(a.key, (uint32_t)(i0 >> 2), ci.rid);
              s[0] += gumbel_f32(w.w0);
              s[1] += gumbel_f32(w.w1);
              s[2] += gumbel_f32(w.w2);
              s[3] += gumbel_f32(w.w3);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
              topk_insert(lm, li, i0 + j < r1 ? s[j] : neg_inf<T>(), (int32_t)(i0 + j));
            continue;
          }
          float beta[4];
          load_bias4(a, bcol, i0, beta);
          if (greedy) {
#pragma unroll
            for (int j = 0; j < 4; ++j) s[j] = T(y[j]) + T(beta[j]);
          } else if constexpr (EPI == kEpiTopK32) {
            const Words w = noise_words(a.key, (uint32_t)(i0 >> 2), ci.rid);
            s[0] = (y[0] + beta[0]) * it + gumbel_f32(w.w0);
            s[1] = (y[1] + beta[1]) * it + gumbel_f32(w.w1);
            s[2] = (y[2] + beta[2]) * it + gumbel_f32(w.w2);
            s[3] = (y[3] + beta[3]) * it + gumbel_f32(w.w3);
          } else {
            const Words w0 = noise_words(a.key, (uint32_t)(i0 >> 1), ci.rid);
            const Words w1 = noise_words(a.key, (uint32_t)(i0 >> 1) + 1u, ci.rid);
            s[0] = (T(y[0]) + T(beta[0])) * it + T(gumbel_f64(w0.w0, w0.w1));
            s[1] = (T(y[1]) + T(beta[1])) * it + T(gumbel_f64(w0.w2, w0.w3));
            s[2] = (T(y[2]) + T(beta[2])) * it + T(gumbel_f64(w1.w0, w1.w1));
            s[3] = (T(y[3]) + T(beta[3])) * it + T(gumbel_f64(w1.w2, w1.w3));
          }
          // Rows past the wave's last one enter as -inf, which never takes a
          // place (no branch around the insert).
#pragma unroll
          for (int j = 0; j < 4; ++j)
            topk_insert(lm, li, i0 + j < r1 ? s[j] : neg_inf<T>(), (int32_t)(i0 + j));
        }
        // The column's running places (held by its row-group-0 lane), then
        // the other row groups' lists (lanes 16 and 32 apart), merged in:
        // bitonic merges of sorted lists with float32 scores; with float64
        // scores (whose exchanged lists would need more registers than the
        // 64-column kernel has) place by place.
        if constexpr (EPI == kEpiTopK64) {
          Cand<T> c[2 * kTopKMax];
#pragma unroll
          for (int j = 0; j < kTopKMax; ++j) {
            c[j] = Cand<T>{lm[j], li[j]};
            c[kTopKMax + j] = grp == 0 ? tkc[wave][16 * cb + col][j] : Cand<T>{neg_inf<T>(), kNoIndex};
          }
          Cand<T> pl = Cand<T>{neg_inf<T>(), kNoIndex};
#pragma unroll 1
          for (int r = 0; r < kTopKMax; ++r) {
            pl = next_place(c, r == 0, pl.m, pl.idx, 4);
            if (grp == 0) tkc[wave][16 * cb + col][r] = pl;
          }
        } else {
          T om[kTopKMax];
          int32_t oi[kTopKMax];
#pragma unroll
          for (int j = 0; j < kTopKMax; ++j) {
            const Cand<T> o = grp == 0 ? tkc[wave][16 * cb + col][j] : Cand<T>{neg_inf<T>(), kNoIndex};
            om[j] = o.m;
            oi[j] = o.idx;
          }
          merge_top(lm, li, om, oi);
#pragma unroll
          for (int x = 16; x <= 32; x <<= 1) {
#pragma unroll
            for (int j = 0; j < kTopKMax; ++j) {
              om[j] = __shfl_xor(lm[j], x, 64);
              oi[j] = __shfl_xor(li[j], x, 64);
            }
            merge_top(lm, li, om, oi);
          }
          if (grp == 0) {
#pragma unroll
            for (int j = 0; j < kTopKMax; ++j) tkc[wave][16 * cb + col][j] = Cand<T>{lm[j], li[j]};
          }
        }
      }
    } else if constexpr (kFilt) {
      // Filtered sampling, column block by column block: each lane's rows of
      // the pass (in increasing index order) update its sorted list of the
      // kFiltList largest valid logits, its best perturbed score (the
      // unfiltered sampler's arithmetic: y / t + g, greedy y), its running
      // mass exp((y - mm) / t) relative to its largest logit mm, and its count
      // of valid logits; then the column's four row groups (lanes 16 apart)
      // and the column's running state (LDS) merge into the new running state.
#pragma unroll 1
      for (int cb = 0; cb < NB; ++cb) {
        float lm[kFiltList];
        int32_t li[kFiltList];
#pragma unroll
        for (int j = 0; j < kFiltList; ++j) {
          lm[j] = neg_inf<float>();
          li[j] = kNoIndex;
        }
        T bs = neg_inf<T>();
        int32_t bi = kNoIndex;
        float by = neg_inf<float>();
        float mm = neg_inf<float>(), mz = 0.0f;
        uint32_t nv = 0u;
        const ColInfo ci = cols[16 * cb + col];
        const bool greedy = (ci.mode & kModeMask) == kGreedy;
        const float inv_tf = greedy ? 1.0f : 1.0f / ci.t;
        const T inv_t = greedy ? T(1) : T(1) / T(ci.t);
        // whether any column of the wave needs the tile mass (wave-uniform)
        const bool any_mass = __builtin_amdgcn_ballot_w64((ci.mode & kFiltMass) != 0) != 0ull;
        // mass of logit y relative to a larger-or-equal logit m
        auto rel_mass = [&](float y, float m) -> float {
          if (m == __builtin_inff()) return y == m ? 1.0f : 0.0f;
          return expf((y - m) * inv_tf);
        };
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          if (rb >= nrb) break;
          f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c2 = 0; c2 < NB; ++c2)
            if (c2 == cb) y = acc[rb][c2];
          const int64_t i0 = r0 + 16 * (rb_first + rb) + 4 * grp;
          if ((ci.mode & kFiltStore) != 0 && bt0 + 16 * cb + col < B) {
            float* yr = a.Y + (bt0 + 16 * cb + col) * V;
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (i0 + j < r1) yr[i0 + j] = y[j];
          }
          bool ok[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) ok[j] = (i0 + j < r1) & (y[j] == y[j]) & (y[j] != neg_inf<float>());
          T sc[4];
          if (greedy) {
#pragma unroll
            for (int j = 0; j < 4; ++j) sc[j] = T(y[j]);
          } else if constexpr (EPI == kEpiFilt32) {
            const Words w = noise_words(a.key, (uint32_t)(i0 >> 2), ci.rid);
            sc[0] = T(y[0] * inv_tf) + T(gumbel_f32(w.w0));
            sc[1] = T(y[1] * inv_tf) + T(gumbel_f32(w.w1));
            sc[2] = T(y[2] * inv_tf) + T(gumbel_f32(w.w2));
            sc[3] = T(y[3] * inv_tf) + T(gumbel_f32(w.w3));
          } else {
            const Words w0 = noise_words(a.key, (uint32_t)(i0 >> 1), ci.rid);
            const Words w1 = noise_words(a.key, (uint32_t)(i0 >> 1) + 1u, ci.rid);
            sc[0] = T(y[0]) * inv_t + T(gumbel_f64(w0.w0, w0.w1));
            sc[1] = T(y[1]) * inv_t + T(gumbel_f64(w0.w2, w0.w3));
            sc[2] = T(y[2]) * inv_t + T(gumbel_f64(w1.w0, w1.w1));
            sc[3] = T(y[3]) * inv_t + T(gumbel_f64(w1.w2, w1.w3));
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int32_t i = (int32_t)(i0 + j);
            // rows past the wave's last one and invalid logits enter as -inf,
            // which never takes a place (no branch around the insert)
            topk_insert(lm, li, ok[j] ? y[j] : neg_inf<float>(), i);
            if (ok[j]) {
              ++nv;
              if (y[j] > mm) {
                if (any_mass) mz = mm == neg_inf<float>() ? 1.0f : mz * rel_mass(mm, y[j]) + 1.0f;
                mm = y[j];
              } else if (any_mass) {
                mz += rel_mass(y[j], mm);
              }
              if (sc[j] > bs) {  // increasing index order: ties keep the smaller
                bs = sc[j];
                bi = i;
                by = y[j];
              }
            }
          }
        }
        double zz = (double)mz;
        // the column's running state (row group 0 only), then the other row
        // groups' (lanes 16 and 32 apart)
        auto merge_aux = [&](T os, int32_t oi, float oy, float om, double oz, uint32_t on) {
          if (beats(os, oi, bs, bi)) {
            bs = os;
            bi = oi;
            by = oy;
          }
          if (om > mm) {
            zz = (mm == neg_inf<float>() ? 0.0 : zz * (double)rel_mass(mm, om)) + oz;
            mm = om;
          } else if (om != neg_inf<float>()) {
            zz += oz * (double)rel_mass(om, mm);
          }
          nv += on;
        };
        {
          float om[kFiltList];
          int32_t oi[kFiltList];
#pragma unroll
          for (int j = 0; j < kFiltList; ++j) {
            const Cand<float> o = grp == 0 ? flc[wave][16 * cb + col][j] : Cand<float>{neg_inf<float>(), kNoIndex};
            om[j] = o.m;
            oi[j] = o.idx;
          }
          merge_top(lm, li, om, oi);
          if (grp == 0) {
            const FiltAux o = fla[wave][16 * cb + col];
            merge_aux(o.bs, o.bi, o.by, o.mm, o.zz, o.nv);
          }
#pragma unroll
          for (int x = 16; x <= 32; x <<= 1) {
#pragma unroll
            for (int j = 0; j < kFiltList; ++j) {
              om[j] = __shfl_xor(lm[j], x, 64);
              oi[j] = __shfl_xor(li[j], x, 64);
            }
            merge_top(lm, li, om, oi);
            const T os = __shfl_xor(bs, x, 64);
            const int32_t obi = __shfl_xor(bi, x, 64);
            const float oy = __shfl_xor(by, x, 64);
            const float omm = __shfl_xor(mm, x, 64);
            const double oz = __shfl_xor(zz, x, 64);
            const uint32_t on = (uint32_t)__shfl_xor((int)nv, x, 64);
            merge_aux(os, obi, oy, omm, oz, on);
          }
        }
        if (grp == 0) {
#pragma unroll
          for (int j = 0; j < kFiltList; ++j) flc[wave][16 * cb + col][j] = Cand<float>{lm[j], li[j]};
          fla[wave][16 * cb + col] = FiltAux{bs, by, bi, mm, nv, zz};
        }
      }
    } else if (EPI == kEpiStore || kFold) {
      const int32_t r1s = (int32_t)r1;  // V < 2^31
      // Per column: 1 / t (1 for greedy) and whether any column of the wave
      // has an infinite temperature (a wave-uniform test, so the rare noise
      // path stays a branch rather than being computed for every fragment).
      float inv_t[NB];
      bool inf_any[NB];
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const ColInfo ci = cols[16 * cb + col];
        inv_t[cb] = ci.inv_t;
        inf_any[cb] = EPI != kEpiStore && __builtin_amdgcn_ballot_w64(ci.mode == kInfT) != 0;
      }
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        if (rb >= nrb) continue;
        const int64_t i0 = r0 + 16 * (rb_first + rb) + 4 * grp;
        const int32_t i0s = (int32_t)i0;
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
          const f32x4 y = acc[rb][cb];
          if (EPI == kEpiStore) {
            if (!col_ok[cb]) continue;
            const int64_t b = bt0 + 16 * cb + col;
            if (a.row_flags != nullptr && a.row_flags[b] != 1u) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (i0 + j < r1) a.Y[b * V + i0 + j] = W8 ? y[j] * wsc[rb][j] : y[j];
            continue;
          }
          // Greedy columns carry inv_t = 1, so one multiply scores both folded
          // modes; infinite temperatures add their noise after it.  Columns
          // past B are scored too and never published.
          float s[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) s[j] = (W8 ? y[j] * wsc[rb][j] : y[j]) * inv_t[cb];
          if constexpr (W8) {
            // Rows whose scale the fold could not divide by (zero or not
            // finite) carry their bare sums: score them here (a wave-uniform
            // branch, taken only when some lane has such a row).
            bool bad = false;
#pragma unroll
            for (int j = 0; j < 4; ++j) bad |= !fold_scale_ok(wsc[rb][j]);
            if (__builtin_amdgcn_ballot_w64(bad) != 0) {
              const ColInfo ci = cols[16 * cb + col];
              const int64_t bcol = bt0 + 16 * cb + col < B ? bt0 + 16 * cb + col : B - 1;
              float beta[4];
              load_bias4(a, bcol, i0, beta);
              const Words w = noise_words(a.key, (uint32_t)(i0 >> 2), ci.rid);
              const float g[4] = {gumbel_f32(w.w0), gumbel_f32(w.w1), gumbel_f32(w.w2),
                                  gumbel_f32(w.w3)};
#pragma unroll
              for (int j = 0; j < 4; ++j)
                if (!fold_scale_ok(wsc[rb][j]))
                  s[j] = (y[j] * wsc[rb][j] + beta[j]) * ci.inv_t + (ci.mode == kGreedy ? 0.0f : g[j]);
            }
          }
          if (inf_any[cb]) {
            const ColInfo ci = cols[16 * cb + col];
            if (ci.mode == kInfT) {
              const Words w = noise_words(a.key, (uint32_t)(i0 >> 2), ci.rid);
              s[0] += gumbel_f32(w.w0);
              s[1] += gumbel_f32(w.w1);
              s[2] += gumbel_f32(w.w2);
              s[3] += gumbel_f32(w.w3);
            }
          }
          // A lane meets the rows of one column in increasing index order,
          // so only a strictly larger score takes over (a tie keeps the
          // smaller index; NaN never takes over).
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool take = (i0s + j < r1s) & (T(s[j]) > bm[cb]);
            bm[cb] = take ? T(s[j]) : bm[cb];
            bi[cb] = take ? i0s + j : bi[cb];
          }
        }
      }
    } else {
      // Noise added after the k-loop: float64 noise (the score is formed in
      // float64), and float32 noise over FP8 weights (after the row scale).
      // The per-fragment work (one or two Philox calls, four transforms) is
      // large, so the loop stays rolled and the fragment is picked out of the
      // accumulators by uniform branches.
#pragma unroll 1
      for (int f = 0; f < kRB * NB; ++f) {
        const int rb = f / NB, cb = f - rb * NB;
        if (rb >= nrb) break;
        f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
        T lbm = neg_inf<T>();
        int32_t lbi = kNoIndex;
#pragma unroll
        for (int rb2 = 0; rb2 < kRB; ++rb2)
#pragma unroll
          for (int cb2 = 0; cb2 < NB; ++cb2)
            if (rb2 == rb && cb2 == cb) y = acc[rb2][cb2];
#pragma unroll
        for (int c = 0; c < NB; ++c)
          if (c == cb) {
            lbm = bm[c];
            lbi = bi[c];
          }
        const ColInfo ci = cols[16 * cb + col];
        const int m = ci.mode;
        const T it = m == kGreedy ? T(1) : T(1) / T(ci.t);
        const uint32_t r = ci.rid;
        if (bt0 + 16 * cb + col >= B) continue;
        const int64_t i0 = r0 + 16 * (rb_first + rb) + 4 * grp;
        float beta[4];
        load_bias4(a, bt0 + 16 * cb + col, i0, beta);
        // FP8 weights: the row scale applies in float32, as in the logits the
        // store epilogue writes.
        if constexpr (W8) {
#pragma unroll
          for (int rb2 = 0; rb2 < kRB; ++rb2)
            if (rb2 == rb) {
#pragma unroll
              for (int j = 0; j < 4; ++j) y[j] *= wsc[rb2][j];
            }
        }
        T yv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) yv[j] = T(y[j]);
        T s[4];
        if (m == kGreedy) {
#pragma unroll
          for (int j = 0; j < 4; ++j) s[j] = yv[j] + T(beta[j]);
        } else if constexpr (EPI == kEpiSample32) {
          // Float32 noise that is not folded into the k-loop (FP8 weights,
          // whose row scale only applies after it).
          const Words w = noise_words(a.key, (uint32_t)(i0 >> 2), r);
          s[0] = (yv[0] + beta[0]) * it + gumbel_f32(w.w0);
          s[1] = (yv[1] + beta[1]) * it + gumbel_f32(w.w1);
          s[2] = (yv[2] + beta[2]) * it + gumbel_f32(w.w2);
          s[3] = (yv[3] + beta[3]) * it + gumbel_f32(w.w3);
        } else {
          const Words w0 = noise_words(a.key, (uint32_t)(i0 >> 1), r);
          const Words w1 = noise_words(a.key, (uint32_t)(i0 >> 1) + 1u, r);
          s[0] = (yv[0] + T(beta[0])) * it + T(gumbel_f64(w0.w0, w0.w1));
          s[1] = (yv[1] + T(beta[1])) * it + T(gumbel_f64(w0.w2, w0.w3));
          s[2] = (yv[2] + T(beta[2])) * it + T(gumbel_f64(w1.w0, w1.w1));
          s[3] = (yv[3] + T(beta[3])) * it + T(gumbel_f64(w1.w2, w1.w3));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int32_t i = (int32_t)(i0 + j);
          if (i0 + j < r1 && beats(s[j], i, lbm, lbi)) {
            lbm = s[j];
            lbi = i;
          }
        }
#pragma unroll
        for (int c = 0; c < NB; ++c)
          if (c == cb) {
            bm[c] = lbm;
            bi[c] = lbi;
          }
      }
    }
    if (EPI != kEpiStore && !kTopK && !kFilt) {
      // Lanes that share a column (the 4 row groups) -> one value per column,
      // merged into the wave's running best.
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        wave_argmax_xor(bm[cb], bi[cb], 4);
        if (grp == 0) {
          const Cand<T> o = wrun[wave][16 * cb + col];
          if (beats(bm[cb], bi[cb], o.m, o.idx)) wrun[wave][16 * cb + col] = Cand<T>{bm[cb], bi[cb]};
        }
      }
    }
  }

  if (EPI == kEpiStore) return;

  if constexpr (kFilt) {
    // Per column, its record: the kFiltList places among the 8 waves' lists
    // (one candidate a lane: lane l holds place l % 8 of wave l / 8), lane r
    // keeping place r; the waves' best scores, masses and counts merged by
    // lanes 0-7.  Stage 2 is a launch of its own.
    __syncthreads();
    static_assert(kWaves * kFiltList == 64, "one candidate per lane");
#pragma unroll 1
    for (int c = wave; c < 16 * NB; c += kWaves) {
      const int64_t b = bt0 + c;
      Cand<float> it[1];
      it[0] = flc[lane / kFiltList][c][lane % kFiltList];
      Cand<float> pl = Cand<float>{neg_inf<float>(), kNoIndex};
      float my = neg_inf<float>();
      int32_t mi = kNoIndex;
#pragma unroll 1
      for (int r = 0; r < kFiltList; ++r) {
        pl = next_place(it, r == 0, pl.m, pl.idx);
        if (lane == r) {
          my = pl.m;
          mi = pl.idx;
        }
      }
      const ColInfo ci = cols[c];
      const float inv_tf = (ci.mode & kModeMask) == kGreedy ? 1.0f : 1.0f / ci.t;
      auto rel_mass = [&](float y, float m) -> float {
        if (m == __builtin_inff()) return y == m ? 1.0f : 0.0f;
        return expf((y - m) * inv_tf);
      };
      FiltAux x = lane < kWaves ? fla[lane][c]
                                : FiltAux{neg_inf<T>(), neg_inf<float>(), kNoIndex, neg_inf<float>(), 0u, 0.0};
#pragma unroll
      for (int o = 1; o < kWaves; o <<= 1) {
        const T os = __shfl_xor(x.bs, o, 64);
        const int32_t obi = __shfl_xor(x.bi, o, 64);
        const float oy = __shfl_xor(x.by, o, 64);
        const float om = __shfl_xor(x.mm, o, 64);
        const double oz = __shfl_xor(x.zz, o, 64);
        const uint32_t on = (uint32_t)__shfl_xor((int)x.nv, o, 64);
        if (beats(os, obi, x.bs, x.bi)) {
          x.bs = os;
          x.bi = obi;
          x.by = oy;
        }
        if (om > x.mm) {
          x.zz = (x.mm == neg_inf<float>() ? 0.0 : x.zz * (double)rel_mass(x.mm, om)) + oz;
          x.mm = om;
        } else if (om != neg_inf<float>()) {
          x.zz += oz * (double)rel_mass(om, x.mm);
        }
        x.nv += on;
      }
      if (b < B) {
        FiltRec<T>* rec = reinterpret_cast<FiltRec<T>*>(static_cast<char*>(a.cand) +
                                                        (b * a.nT + tile) * (int64_t)kFiltRecBytes);
        if (lane < kFiltList) {
          rec->ly[lane] = my;
          rec->li[lane] = mi;
        }
        if (lane == 0) {
          rec->bs = x.bs;
          rec->by = x.by;
          rec->bi = x.bi;
          rec->mm = x.mm;
          rec->nv = x.nv;
          rec->zz = (ci.mode & kFiltMass) != 0 ? x.zz : -1.0;  // -1: not summed
        }
      }
    }
    return;
  }

  if constexpr (kTopK) {
    // Per column, its kTopKMax places among the 8 waves' running places
    // (each sorted best first): wave w takes columns w, w + 8, ..., one group
    // of 8 lanes a column, whose lane l holds wave l's list; three
    // xor-exchanges and bitonic merges of sorted lists leave the column's
    // places in every lane of the group, and lane l stores place l.
    __syncthreads();
    static_assert(kWaves == kTopKMax && kWaves * kWaves == 64, "a group of 8 lanes per column");
    {
      const int src = lane % kWaves;
      const int c = wave + kWaves * (lane / kWaves);
      const bool cv = c < 16 * NB;
      T lm[kTopKMax];
      int32_t li[kTopKMax];
#pragma unroll
      for (int j = 0; j < kTopKMax; ++j) {
        const Cand<T> o = tkc[src][cv ? c : 0][j];
        lm[j] = cv ? o.m : neg_inf<T>();
        li[j] = cv ? o.idx : kNoIndex;
      }
#pragma unroll
      for (int x = 1; x < kWaves; x <<= 1) {
        T om[kTopKMax];
        int32_t oi[kTopKMax];
#pragma unroll
        for (int j = 0; j < kTopKMax; ++j) {
          om[j] = __shfl_xor(lm[j], x, 64);
          oi[j] = __shfl_xor(li[j], x, 64);
        }
        merge_top(lm, li, om, oi);
      }
      Cand<T> mine = Cand<T>{lm[0], li[0]};
#pragma unroll
      for (int j = 1; j < kTopKMax; ++j)
        if (src == j) mine = Cand<T>{lm[j], li[j]};
      const int64_t b = bt0 + c;
      if (cv && b < B) store_cand(reinterpret_cast<Cand<T>*>(a.cand) + (b * a.nT + tile) * kTopKMax + src, mine);
    }
    wait_stores_complete();

    // Stage 2 (topk_row_places above), here for tiles of at most
    // kStage2InKernelRows rows: wave w takes rows w, w + 8, ... of the tile,
    // each row's maxima requested with the previous row's list loads.  Wider
    // tiles leave it to a launch of one wave per row (topk_stage2_kernel, made
    // by launch_fused_stage1), since here a tile's rows would queue 8 to a wave.
    if constexpr (16 * NB > kStage2InKernelRows) {
      return;
    } else {
      if (!finish_last(a.counters + btile, (uint32_t)nT)) return;
      static_assert(kWaves * kS2SurvPerWave * sizeof(Cand<T>) <= sizeof(hs),
                    "the survivors of every wave fit in the H staging buffer");
      Cand<T>* const surv = reinterpret_cast<Cand<T>*>(&hs[0][0][0]) + wave * kS2SurvPerWave;
      Cand<T> mxn[kS2TilesPerLane];
      if (bt0 + wave < B) topk_load_maxima(a, bt0 + wave, lane, mxn);
#pragma unroll 1
      for (int i = wave; i < kTile; i += kWaves) {
        const int64_t b = bt0 + i;
        if (b >= B) break;
        Cand<T> mx[kS2TilesPerLane];
#pragma unroll
        for (int j = 0; j < kS2TilesPerLane; ++j) mx[j] = mxn[j];
        if (i + kWaves < kTile && b + kWaves < B) topk_load_maxima(a, b + kWaves, lane, mxn);
        topk_row_places(a, b, lane, mx, surv);
      }
      if (tid == 0) clear_counter(a.counters + btile);
      return;
    }
  }

  // Across the waves, in wave order, through LDS.
  __syncthreads();
  if (tid < NB * 16) {
    Cand<T> best = wrun[0][tid];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      const Cand<T> o = wrun[w][tid];
      if (beats(o.m, o.idx, best.m, best.idx)) best = o;
    }
    const int64_t b = bt0 + tid;
    if (b < B) {
      store_cand(reinterpret_cast<Cand<T>*>(a.cand) + b * a.nT + tile, best);
      wait_stores_complete();
    }
  }

  // Stage 2 of this batch tile, in the workgroup that finishes it last.  Row r
  // of the tile goes to kTPR consecutive threads (8 to 32, so a row's threads
  // share a wave), thread q of them taking the row's candidates q, q + kTPR,
  // ...: every thread issues all its candidate loads (clamped, always valid
  // addresses) before it compares any, and the rows reduce side by side, so
  // the tail costs one round trip to the coherence point and a few lane
  // exchanges.  (A wave per row in turn, each across its 64 lanes, cost about
  // 4 us more at 64 rows.)
  if (!finish_last(a.counters + btile, (uint32_t)nT)) return;
  {
    constexpr int kTPR = kTile <= 16 ? 32 : (kTile <= 32 ? 16 : 8);
    constexpr int kPerThread = kMaxFusedTiles / kTPR;
    static_assert(64 % kTPR == 0, "a row's threads lie in one wave");
    const Cand<T>* cand = reinterpret_cast<const Cand<T>*>(a.cand);
    const int q = tid % kTPR;
    // (Tiles of 128 rows: two rows a group of threads, one after the other.)
#pragma unroll 1
    for (int r = tid / kTPR; r < kTile; r += kThreads / kTPR) {
      const int64_t b = bt0 + r;
      if (b >= B) break;
      Cand<T> c[kPerThread];
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) {
        const int t = q + kTPR * j < a.nT ? q + kTPR * j : a.nT - 1;
        c[j] = load_cand(cand + b * a.nT + t);
      }
      // Four independent chains (candidate j in chain j % 4), then the four.
      T cm[4];
      int32_t ci[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        cm[k] = neg_inf<T>();
        ci[k] = kNoIndex;
      }
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) {
        const bool take = q + kTPR * j < a.nT && beats_nb(c[j].m, c[j].idx, cm[j % 4], ci[j % 4]);
        cm[j % 4] = take ? c[j].m : cm[j % 4];
        ci[j % 4] = take ? c[j].idx : ci[j % 4];
      }
      T bm = cm[0];
      int32_t bi = ci[0];
#pragma unroll
      for (int k = 1; k < 4; ++k) {
        const bool take = beats_nb(cm[k], ci[k], bm, bi);
        bm = take ? cm[k] : bm;
        bi = take ? ci[k] : bi;
      }
      group_argmax<kTPR>(bm, bi);
      if (q == 0) a.out[b] = bm == neg_inf<T>() ? (int64_t)-1 : (int64_t)bi;
    }
  }
  if (tid == 0) clear_counter(a.counters + btile);
}

// ---------------------------------------------------------------------------
// Filtered sampling, Stage 2: one wave per row resolves the row's kept set
// from its tiles' records, with the filtered sampler's rules and arithmetic
// over the same float32 logits (fs_filter.hip: top-k by value, top-p by
// 64-bit fixed-point masses exp((y - M) / t) in units of 2^-40, min-p by
// exp((y - M) / t) >= m, each cut keeping whole classes of equal logits),
// then draws over the kept tokens.
//
// The lists hold every token above C (the largest last-listed logit among
// tiles with more valid tokens than their list), so any count or mass over
// "the tokens above x" is exact for x >= C.  Each lane holds its tiles' list
// entries as order-preserving keys.  The k-th largest key is found bit by bit
// from the top (the largest x with at least k keys >= x: a count per step),
// and the top-p cut likewise (the largest x whose strictly larger survivors
// carry at least p of the mass: a 64-bit mass sum per step; the lowest kept
// class is the smallest survivor key above it).  A row is resolved when each
// cut it needs lies above C, and every tile either lists all its kept tokens
// (its last listed logit is not kept, or it has no more tokens) or has its
// best-scoring token kept (then that token is its best kept one).  Other rows
// are flagged for the exact fallback.  Top-p without top-k takes the total
// mass from the tiles' float64 sums instead of the filtered sampler's sum of
// per-token fixed-point masses.
// ---------------------------------------------------------------------------
constexpr int kFiltRowsPerBlock = 4;

__device__ __forceinline__ uint32_t filt_order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Sums over a whole wave64 by DPP exchanges inside each row of 16 lanes
// (xor 1, xor 2, then the half-row and row mirrors, each pairing groups that
// already hold their sums) and the four rows' sums read back with readlane:
// no LDS round trip.  The result is wave-uniform.
template <int kCtrl>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v) {
  return (unsigned long long)dpp_u32<kCtrl>((uint32_t)v) |
         ((unsigned long long)dpp_u32<kCtrl>((uint32_t)(v >> 32)) << 32);
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += dpp_u32<0xb1>(v);
  v += dpp_u32<0x4e>(v);
  v += dpp_u32<0x141>(v);
  v += dpp_u32<0x140>(v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0) + (uint32_t)__builtin_amdgcn_readlane((int)v, 16) +
         (uint32_t)__builtin_amdgcn_readlane((int)v, 32) + (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
}
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
  v += dpp_u64<0xb1>(v);
  v += dpp_u64<0x4e>(v);
  v += dpp_u64<0x141>(v);
  v += dpp_u64<0x140>(v);
  unsigned long long r = 0ull;
#pragma unroll
  for (int row = 0; row < 4; ++row)
    r += (unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 16 * row) |
         ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * row) << 32);
  return r;
}

// Wave-wide max / min by the same DPP pattern (float max, int32 min).
__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, dpp_val<0xb1>(v));
  v = fmaxf(v, dpp_val<0x4e>(v));
  v = fmaxf(v, dpp_val<0x141>(v));
  v = fmaxf(v, dpp_val<0x140>(v));
  return fmaxf(fmaxf(lane_val(v, 0), lane_val(v, 16)), fmaxf(lane_val(v, 32), lane_val(v, 48)));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<0xb1>(v));
  v = min(v, dpp_u32<0x4e>(v));
  v = min(v, dpp_u32<0x141>(v));
  v = min(v, dpp_u32<0x140>(v));
  return min(min((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             min((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}
__device__ __forceinline__ int32_t wave_min_i32(int32_t v) {
  v = min(v, (int32_t)dpp_u32<0xb1>((uint32_t)v));
  v = min(v, (int32_t)dpp_u32<0x4e>((uint32_t)v));
  v = min(v, (int32_t)dpp_u32<0x141>((uint32_t)v));
  v = min(v, (int32_t)dpp_u32<0x140>((uint32_t)v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// The first bit at which keys in [lo, hi] can differ, and their common
// prefix above it: the descents below need only decide the bits from there.
__device__ __forceinline__ int filt_top_bit(uint32_t lo, uint32_t hi, uint32_t* prefix) {
  const uint32_t d = lo ^ hi;
  if (d == 0u) {
    *prefix = hi;
    return -1;
  }
  const int top = 31 - __builtin_clz(d);
  *prefix = top == 31 ? 0u : (hi & ~((2u << top) - 1u));
  return top;
}

// The largest x with at least k of the wave's keys >= x, found bit by bit
// from the top with ballot counts, knowing that it lies in [lo, hi] (lo: the
// smallest, hi: the largest valid key; at least k valid keys).
template <int N>
__device__ __forceinline__ uint32_t filt_kth_key(const uint32_t (&k_)[N], uint32_t k, uint32_t lo,
                                                 uint32_t hi) {
  uint32_t x;
#pragma unroll 1
  for (int bit = filt_top_bit(lo, hi, &x); bit >= 0; --bit) {
    const uint32_t tx = x | (1u << bit);
    uint32_t c = 0u;  // wave-uniform
#pragma unroll
    for (int e = 0; e < N; ++e)
      c += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(k_[e] >= tx));
    if (c >= k) x = tx;
  }
  return x;
}

// The largest x whose strictly larger keys of the wave carry a mass sum that
// is not below target (as float64), found bit by bit from the top, knowing
// that it lies in [lo, hi] (the caller checks the sum above lo first).
template <int N>
__device__ __forceinline__ uint32_t filt_mass_cut(const uint32_t (&k_)[N],
                                                  const unsigned long long (&m_)[N],
                                                  double target, uint32_t lo, uint32_t hi) {
  uint32_t x;
#pragma unroll 1
  for (int bit = filt_top_bit(lo, hi, &x); bit >= 0; --bit) {
    const uint32_t tx = x | (1u << bit);
    unsigned long long g = 0ull;
#pragma unroll
    for (int e = 0; e < N; ++e) g += k_[e] > tx ? m_[e] : 0ull;
    if (!((double)wave_sum_u64(g) < target)) x = tx;
  }
  return x;
}

// The smallest and largest of the wave's nonzero keys (0xffffffff, 0 when none).
template <int N>
__device__ __forceinline__ void filt_key_range(const uint32_t (&k_)[N], uint32_t* lo, uint32_t* hi) {
  uint32_t l = 0xffffffffu, h = 0u;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    l = (k_[e] != 0u && k_[e] < l) ? k_[e] : l;
    h = k_[e] > h ? k_[e] : h;
  }
  *lo = wave_min_u32(l);
  *hi = ~wave_min_u32(~h);
}

template <typename T>
__global__ __launch_bounds__(64 * kFiltRowsPerBlock) void filt_stage2_kernel(FusedArgs a) {
  constexpr int kQ = kMaxFusedTiles / 64;  // tiles per lane
  constexpr int kCand = 512;               // candidate slots of a row (kCL a lane)
  constexpr int kCL = kCand / 64;
  // The row's lists (tile t's entries at [t][e]), its candidates and the
  // listed tokens its draw scores, per wave.  The loops over them stay rolled:
  // one wave works a row alone, so its instruction stream must stay in cache.
  __shared__ float sly[kFiltRowsPerBlock][kMaxFusedTiles][kFiltList];
  __shared__ int32_t sli[kFiltRowsPerBlock][kMaxFusedTiles][kFiltList];
  __shared__ uint32_t cks[kFiltRowsPerBlock][kCand];
  __shared__ float cys[kFiltRowsPerBlock][kCand];
  __shared__ int32_t cis[kFiltRowsPerBlock][kCand];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t b = (int64_t)blockIdx.x * kFiltRowsPerBlock + wave;
  if (b >= a.B) return;  // whole waves; nothing below waits on another wave
  const int nT = a.nT;
  const char* rbase = static_cast<const char*>(a.cand) + b * nT * (int64_t)kFiltRecBytes;
  // the row's parameters, requested with the records (one round trip)
  const float t = a.temp[b];
  const uint32_t rid = a.row_ids ? a.row_ids[b] : (uint32_t)b;
  const int32_t top_k = a.top_k ? a.top_k[b] : 0;
  const float top_p = a.top_p ? a.top_p[b] : 1.0f;
  const float min_p = a.min_p ? a.min_p[b] : 0.0f;

  // This lane's tiles t = lane + 64 q: the record fields in registers, the
  // lists in LDS.  Tiles past nT hold nothing (-inf entries).
  float tm[kQ], tby[kQ], tl7[kQ];
  uint32_t tn[kQ];
  double tz[kQ];
  T tbs[kQ];
  int32_t tbi[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const int tt = lane + 64 * q;
    const bool live = tt < nT;
    const FiltRec<T>* r =
        reinterpret_cast<const FiltRec<T>*>(rbase + (int64_t)(live ? tt : 0) * kFiltRecBytes);
    float4 y0 = *reinterpret_cast<const float4*>(&r->ly[0]);
    float4 y1 = *reinterpret_cast<const float4*>(&r->ly[4]);
    const int4 i0 = *reinterpret_cast<const int4*>(&r->li[0]);
    const int4 i1 = *reinterpret_cast<const int4*>(&r->li[4]);
    const float ninf = neg_inf<float>();
    if (!live) y0 = y1 = make_float4(ninf, ninf, ninf, ninf);
    *reinterpret_cast<float4*>(&sly[wave][tt][0]) = y0;
    *reinterpret_cast<float4*>(&sly[wave][tt][4]) = y1;
    *reinterpret_cast<int4*>(&sli[wave][tt][0]) = i0;
    *reinterpret_cast<int4*>(&sli[wave][tt][4]) = i1;
    tl7[q] = y1.w;
    tm[q] = live ? r->mm : ninf;
    tn[q] = live ? r->nv : 0u;
    tz[q] = live ? r->zz : 0.0;
    tbs[q] = live ? r->bs : neg_inf<T>();
    tby[q] = live ? r->by : ninf;
    tbi[q] = live ? r->bi : kNoIndex;
  }

  // The row's largest valid logit, its number of valid logits, and C.
  float M = neg_inf<float>(), C = neg_inf<float>();
  uint32_t n_valid = 0u;
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    M = fmaxf(M, tm[q]);
    n_valid += tn[q];
    if (tn[q] > (uint32_t)kFiltList) C = fmaxf(C, tl7[q]);
  }
  M = wave_max_f32(M);
  C = wave_max_f32(C);
  n_valid = wave_sum_u32(n_valid);
  if (n_valid == 0u) {
    if (lane == 0) a.out[b] = -1;
    return;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (!(t > 0.0f)) {
    // greedy: the smallest index among the tiles whose largest logit is M
    // (each list holds its tile's smallest such index first)
    int32_t bi = kNoIndex;
#pragma unroll
    for (int q = 0; q < kQ; ++q)
      if (tm[q] == M && tn[q] > 0u) bi = min(bi, sli[wave][lane + 64 * q][0]);
    bi = wave_min_i32(bi);
    if (lane == 0) a.out[b] = (int64_t)bi;
    return;
  }
  const T inv_t = T(1) / T(t);
  const float inv_tf = 1.0f / t;
  // NaN parameters compare false: their filters are off.
  const bool use_k = top_k > 0 && (int64_t)top_k < (int64_t)n_valid;
  const bool use_p = top_p < 1.0f;
  bool use_m = min_p > 0.0f;
  auto mass_of = [&](float y) -> float {
    if (M == __builtin_inff()) return y == M ? 1.0f : 0.0f;
    return expf((y - M) * inv_tf);
  };
  auto key_of = [&](float y) -> uint32_t {  // 0 for invalid logits
    return (y == y) & (y != neg_inf<float>()) ? filt_order_key(y) : 0u;
  };
  const uint32_t keyC = C == neg_inf<float>() ? 0u : filt_order_key(C);

  bool unresolved = false;
  uint32_t key_k = 0u, key_p = 0u;
  if (use_k || (use_p && top_p > 0.0f)) {
    // Candidates: the entries the cuts can involve.  With top-k, every entry
    // at or above the k-th largest tile maximum (at least k tokens reach it,
    // so the k-th largest logit does); without it, every entry above C (a
    // top-p cut at or below C is not resolved here).  More than kCand
    // candidates: the fallback.
    uint32_t lo = keyC + 1u;
    if (use_k) {
      uint32_t tk[kQ];
      uint32_t nmax = 0u;
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        tk[q] = tn[q] > 0u ? filt_order_key(tm[q]) : 0u;
        nmax += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(tk[q] != 0u));
      }
      lo = 0u;  // fewer than k tiles with a valid logit: every entry
      if (nmax >= (uint32_t)top_k) {
        uint32_t l, h;
        filt_key_range(tk, &l, &h);
        lo = filt_kth_key(tk, (uint32_t)top_k, l, h);
      }
      lo = lo < 1u ? 1u : lo;
    }
    uint32_t count = 0u;
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll 1
    for (int q = 0; q < kQ; ++q) {
      const int tt = lane + 64 * q;
      const float4 v0 = *reinterpret_cast<const float4*>(&sly[wave][tt][0]);
      const float4 v1 = *reinterpret_cast<const float4*>(&sly[wave][tt][4]);
      const float yv[kFiltList] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int e = 0; e < kFiltList; ++e) {
        const uint32_t k = key_of(yv[e]);
        const bool c = k >= lo;
        const unsigned long long bal = __builtin_amdgcn_ballot_w64(c);
        const uint32_t pos = count + (uint32_t)__builtin_popcountll(bal & below);
        if (c && pos < (uint32_t)kCand) {
          cks[wave][pos] = k;
          cys[wave][pos] = yv[e];
        }
        count += (uint32_t)__builtin_popcountll(bal);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (count > (uint32_t)kCand) {
      unresolved = true;
    } else if (count <= 64u) {
      // Few candidates (the common case with top-k): one a lane, sorted by
      // key, largest first (bitonic; equal keys end up adjacent); the k-th
      // key is then lane k - 1's, and top-p is a prefix sum of the masses.
      uint32_t sk = (uint32_t)lane < count ? cks[wave][lane] : 0u;
      float sy = (uint32_t)lane < count ? cys[wave][lane] : neg_inf<float>();
#pragma unroll
      for (int kk = 2; kk <= 64; kk <<= 1)
#pragma unroll
        for (int jj = kk >> 1; jj > 0; jj >>= 1) {
          const uint32_t ok = (uint32_t)__shfl_xor((int)sk, jj, 64);
          const float oy = __shfl_xor(sy, jj, 64);
          // descending blocks keep the larger key in the lower lane
          const bool larger = ((lane & kk) == 0) == ((lane & jj) == 0);
          const bool take = larger ? (ok > sk) : (ok < sk);
          sk = take ? ok : sk;
          sy = take ? oy : sy;
        }
      if (use_k) {
        if ((uint32_t)top_k <= count) key_k = (uint32_t)__builtin_amdgcn_readlane((int)sk, top_k - 1);
        if (key_k <= keyC) unresolved = true;  // also when fewer than k keys are listed
      }
      if (use_p && !unresolved) {
        if (!(top_p > 0.0f)) {
          key_p = filt_order_key(M);
        } else {
          const bool sv = sk != 0u && sk >= key_k;
          const unsigned long long m = sv ? (unsigned long long)(mass_of(sy) * 0x1p40f) : 0ull;
          unsigned long long incl = m;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const unsigned long long u = (unsigned long long)__shfl_up((long long)incl, o, 64);
            incl += lane >= o ? u : 0ull;
          }
          const unsigned long long total =
              (unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)incl, 63) |
              ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(incl >> 32), 63) << 32);
          double target;
          if (use_k) {
            target = (double)top_p * (double)total;
          } else {
            // (a tile mass of -1 was not summed: this row's top-k is set but
            // not below its count of valid logits; the fallback decides it)
            double zt = 0.0;
            bool missing = false;
#pragma unroll
            for (int q = 0; q < kQ; ++q)
              if (tn[q] > 0u) {
                zt += tz[q] * (double)mass_of(tm[q]);
                missing |= tz[q] < 0.0;
              }
            zt += dpp_val<0xb1>(zt);
            zt += dpp_val<0x4e>(zt);
            zt += dpp_val<0x141>(zt);
            zt += dpp_val<0x140>(zt);
            zt = (lane_val(zt, 0) + lane_val(zt, 16)) + (lane_val(zt, 32) + lane_val(zt, 48));
            target = (double)top_p * (zt * 0x1p40);
            if (__builtin_amdgcn_ballot_w64(missing) != 0ull) target = __builtin_inf();
          }
          if ((double)total < target) {
            unresolved = true;  // the cut lies at or below C
          } else {
            // a class's mass above is the prefix before its first member; the
            // kept classes are those whose mass above is below the target
            const uint32_t prev = (uint32_t)__shfl_up((int)sk, 1, 64);
            const bool start = sv && (lane == 0 || prev != sk);
            const unsigned long long kb = __builtin_amdgcn_ballot_w64(start && (double)(incl - m) < target);
            key_p = (uint32_t)__builtin_amdgcn_readlane((int)sk, 63 - __builtin_clzll(kb));
          }
        }
      }
    } else {
      uint32_t ck[kCL];
      unsigned long long cm[kCL];
#pragma unroll
      for (int j = 0; j < kCL; ++j) {
        const uint32_t slot = (uint32_t)(lane + 64 * j);
        ck[j] = slot < count ? cks[wave][slot] : 0u;
      }
      if (use_k) {
        uint32_t nk = 0u;
#pragma unroll
        for (int j = 0; j < kCL; ++j)
          nk += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(ck[j] != 0u));
        if (nk >= (uint32_t)top_k) {
          uint32_t l, h;
          filt_key_range(ck, &l, &h);
          key_k = filt_kth_key(ck, (uint32_t)top_k, l, h);
        }
        if (key_k <= keyC) unresolved = true;  // also when fewer than k keys are listed
      }
      if (use_p && !unresolved) {
        if (!(top_p > 0.0f)) {
          key_p = filt_order_key(M);
        } else {
          // survivors: the candidates at or above key_k (every candidate
          // without top-k), with their fixed-point masses; the others get key
          // 0 and mass 0
          unsigned long long zs = 0ull;
#pragma unroll 1
          for (int j = 0; j < kCL; ++j) {
            const bool sv = ck[j] != 0u && ck[j] >= key_k;
            const uint32_t slot = (uint32_t)(lane + 64 * j);
            const float y = sv ? cys[wave][slot] : M;
            cm[j] = sv ? (unsigned long long)(mass_of(y) * 0x1p40f) : 0ull;
            ck[j] = sv ? ck[j] : 0u;
            zs += cm[j];
          }
          double target;
          if (use_k) {
            target = (double)top_p * (double)wave_sum_u64(zs);
          } else {
            double zt = 0.0;
            bool missing = false;
#pragma unroll
            for (int q = 0; q < kQ; ++q)
              if (tn[q] > 0u) {
                zt += tz[q] * (double)mass_of(tm[q]);
                missing |= tz[q] < 0.0;
              }
            zt += dpp_val<0xb1>(zt);
            zt += dpp_val<0x4e>(zt);
            zt += dpp_val<0x141>(zt);
            zt += dpp_val<0x140>(zt);
            zt = (lane_val(zt, 0) + lane_val(zt, 16)) + (lane_val(zt, 32) + lane_val(zt, 48));
            target = (double)top_p * (zt * 0x1p40);
            if (__builtin_amdgcn_ballot_w64(missing) != 0ull) target = __builtin_inf();
          }
          // The largest x whose strictly larger survivors carry at least the
          // target; the lowest kept class is the smallest survivor key above
          // it.  Below the smallest survivor key l the sum is every
          // survivor's mass: when that is short of the target (possible only
          // without top-k: the survivors held are the tokens above C) the cut
          // lies at or below C and is not resolved here; otherwise x lies in
          // [l - 1, the largest key].
          if ((double)wave_sum_u64(zs) < target) {
            unresolved = true;
          } else {
            uint32_t l, h;
            filt_key_range(ck, &l, &h);
            const uint32_t x = filt_mass_cut(ck, cm, target, l - 1u, h);
            uint32_t kp = 0xffffffffu;
#pragma unroll
            for (int j = 0; j < kCL; ++j)
              if (ck[j] != 0u) kp = (ck[j] > x && ck[j] < kp) ? ck[j] : kp;
            key_p = wave_min_u32(kp);
          }
        }
      }
    }
  }
  uint32_t kappa = key_k > key_p ? key_k : key_p;
  if (use_m && !(min_p < 1.0f)) {
    const uint32_t km = filt_order_key(M);
    kappa = kappa > km ? kappa : km;
    use_m = false;
  }

  // The draw over the kept tokens: valid, key >= kappa, and the min-p test.
  T bm = neg_inf<T>();
  int32_t bi = kNoIndex;
  if (!unresolved) {
    auto kept = [&](float y) -> bool {
      const uint32_t k = key_of(y);
      return k != 0u && k >= kappa && (!use_m || mass_of(y) >= min_p);
    };
    // Per tile: its best-scoring token when that token is kept (it is then
    // the tile's best kept token, no noise to compute), else the kept tokens
    // of its list when the list holds all of them, else the row is lost.
    // The listed tokens to score are gathered first, so that the lanes
    // compute their noise side by side rather than one tile at a time.
    bool lost = false;
    uint32_t lmask = 0u;  // bit q: tile q's kept tokens come from its list
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      if (tn[q] == 0u) continue;
      if (kept(tby[q])) {
        if (beats(tbs[q], tbi[q], bm, bi)) {
          bm = tbs[q];
          bi = tbi[q];
        }
      } else if (tn[q] <= (uint32_t)kFiltList || !kept(tl7[q])) {
        lmask |= 1u << q;
      } else {
        lost = true;
      }
    }
    uint32_t nd = 0u;
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll 1
    for (int q = 0; q < kQ; ++q) {
      // (a wave-uniform skip when no lane takes this tile slot from its list)
      if (__builtin_amdgcn_ballot_w64(((lmask >> q) & 1u) != 0u) == 0ull) continue;
      const int tt = lane + 64 * q;
      const float4 v0 = *reinterpret_cast<const float4*>(&sly[wave][tt][0]);
      const float4 v1 = *reinterpret_cast<const float4*>(&sly[wave][tt][4]);
      const int4 j0 = *reinterpret_cast<const int4*>(&sli[wave][tt][0]);
      const int4 j1 = *reinterpret_cast<const int4*>(&sli[wave][tt][4]);
      const float yv[kFiltList] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      const int32_t iv[kFiltList] = {j0.x, j0.y, j0.z, j0.w, j1.x, j1.y, j1.z, j1.w};
#pragma unroll
      for (int e = 0; e < kFiltList; ++e) {
        const bool d = ((lmask >> q) & 1u) != 0u && kept(yv[e]);
        const unsigned long long bal = __builtin_amdgcn_ballot_w64(d);
        const uint32_t pos = nd + (uint32_t)__builtin_popcountll(bal & below);
        if (d && pos < (uint32_t)kCand) {
          cys[wave][pos] = yv[e];
          cis[wave][pos] = iv[e];
        }
        nd += (uint32_t)__builtin_popcountll(bal);
      }
    }
    if (nd > (uint32_t)kCand) lost = true;  // (more listed kept tokens than slots: the fallback)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll 1
    for (uint32_t slot = (uint32_t)lane; slot < nd && slot < (uint32_t)kCand; slot += 64u) {
      const float y = cys[wave][slot];
      const int32_t i = cis[wave][slot];
      T sv;
      if constexpr (std::is_same<T, float>::value) {
        const Words w = noise_words(a.key, (uint32_t)i >> 2, rid);
        const uint32_t qq = (uint32_t)i & 3u;
        const uint32_t word = qq == 0 ? w.w0 : (qq == 1 ? w.w1 : (qq == 2 ? w.w2 : w.w3));
        sv = T(y * inv_tf) + T(gumbel_f32(word));
      } else {
        const Words w = noise_words(a.key, (uint32_t)i >> 1, rid);
        sv = (i & 1) ? T(y) * inv_t + T(gumbel_f64(w.w2, w.w3))
                     : T(y) * inv_t + T(gumbel_f64(w.w0, w.w1));
      }
      if (beats(sv, i, bm, bi)) {
        bm = sv;
        bi = i;
      }
    }
    unresolved = __builtin_amdgcn_ballot_w64(lost) != 0;
    wave_argmax_xor(bm, bi, 0);
  }
  if (lane == 0) {
    if (unresolved && filt_store_row(t, top_k, top_p, min_p)) {
      a.row_flags[b] = 2u;  // its logits are in Y already (Stage 1 wrote them)
    } else if (unresolved) {
      a.row_flags[b] = 1u;  // the store launch writes its logits
      __hip_atomic_fetch_add(a.flag_count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      a.out[b] = bm == neg_inf<T>() ? (int64_t)-1 : (int64_t)bi;
    }
  }
}

// Kernels that fold the float32 noise fold the bias with it (a bias
// template); the others read the bias after the k-loop.
template <int NB, int WF>
hipError_t launch_nb(const FusedArgs& a, int epi, dim3 grid, hipStream_t stream) {
  constexpr bool BF = WF == kWBf16;
  constexpr bool FB = FoldNoise<NB, kEpiSample32, false, WF>::value;
  switch (epi) {
    case kEpiSample32:
      if (a.bias && FB && a.bias_vec4)
        launch((fused_stage1_kernel<NB, kEpiSample32, FB, WF, FB>), grid, dim3(kThreads),
                           0, stream, a);
      else if (a.bias && FB)
        launch((fused_stage1_kernel<NB, kEpiSample32, FB, WF>), grid, dim3(kThreads), 0,
                           stream, a);
      else
        launch((fused_stage1_kernel<NB, kEpiSample32, false, WF>), grid, dim3(kThreads),
                           0, stream, a);
      break;
    case kEpiSample64:
      launch((fused_stage1_kernel<NB, kEpiSample64, false, WF>), grid, dim3(kThreads), 0,
                         stream, a);
      break;
    case kEpiTopK32:
      // Gumbel-top-k: tiles of at most 64 columns, bf16 weights; the float32
      // noise and the bias are folded as for one draw.
      if constexpr (NB <= 4 && BF) {
        constexpr bool FT = FoldNoise<NB, kEpiTopK32, false, kWBf16>::value;
        if (a.bias && FT && a.bias_vec4)
          launch((fused_stage1_kernel<NB, kEpiTopK32, FT, kWBf16, FT>), grid, dim3(kThreads), 0,
                 stream, a);
        else if (a.bias && FT)
          launch((fused_stage1_kernel<NB, kEpiTopK32, FT, kWBf16>), grid, dim3(kThreads), 0,
                 stream, a);
        else
          launch((fused_stage1_kernel<NB, kEpiTopK32, false, kWBf16>), grid, dim3(kThreads), 0,
                 stream, a);
      } else {
        return hipErrorInvalidValue;
      }
      break;
    case kEpiTopK64:
      // Float64 scores: tiles of 16 or 64 columns (the 32- and 48-column
      // layouts run out of registers).
      if constexpr ((NB == 1 || NB == 4) && BF)
        launch((fused_stage1_kernel<NB, kEpiTopK64, false, kWBf16>), grid,
                           dim3(kThreads), 0, stream, a);
      else
        return hipErrorInvalidValue;
      break;
    case kEpiFilt32:
      // Filtered sampling: tiles of at most 64 columns, bf16 weights.
      if constexpr (NB <= 4 && BF)
        launch((fused_stage1_kernel<NB, kEpiFilt32, false, kWBf16>), grid, dim3(kThreads), 0,
               stream, a);
      else
        return hipErrorInvalidValue;
      break;
    case kEpiFilt64:
      if constexpr ((NB == 1 || NB == 4) && BF)
        launch((fused_stage1_kernel<NB, kEpiFilt64, false, kWBf16>), grid, dim3(kThreads), 0,
               stream, a);
      else
        return hipErrorInvalidValue;
      break;
    default:
      launch((fused_stage1_kernel<NB, kEpiStore, false, WF>), grid, dim3(kThreads), 0,
                         stream, a);
      break;
  }
  return hipGetLastError();
}

template <int WF>
hipError_t launch_w(const FusedArgs& a, int epi, dim3 grid, int nb, hipStream_t stream) {
  switch (nb) {
    case 1: return launch_nb<1, WF>(a, epi, grid, stream);
    case 2: return launch_nb<2, WF>(a, epi, grid, stream);
    case 3: return launch_nb<3, WF>(a, epi, grid, stream);
    default: return launch_nb<4, WF>(a, epi, grid, stream);
  }
}

// Wide batch tiles (128 columns): bf16 weights only.
hipError_t launch_wide(const FusedArgs& a, int epi, dim3 grid, hipStream_t stream) {
  return launch_nb<8, kWBf16>(a, epi, grid, stream);
}

}  // namespace

int fused_num_tiles(int64_t V, int num_cus, int64_t row_bytes) {
  const int64_t nunits = (V + 7) >> 3;
  int64_t g = num_cus < kMaxFusedTiles ? num_cus : kMaxFusedTiles;  // one workgroup per CU
  // Workgroup W ranges that all start on 16 MiB boundaries stream markedly
  // slower (D = 8192, V = 262144, B = 1: 980 us with 256 tiles, 731 with 255,
  // 792 with 252; the neighbouring shapes stream at 5.3-6.1 TB/s), so such a
  // split gives up one CU to move the range starts off those boundaries.
  if (row_bytes > 0 && g > 8) {
    const int64_t stride = (nunits + g - 1) / g * 8 * row_bytes;
    if (stride % ((int64_t)16 << 20) == 0) g -= 1;
  }
  if (g > nunits) g = nunits;
  if (g < 1) g = 1;
  return (int)g;
}

int fused_column_blocks(int64_t B, bool fp8_weights, bool fp64_noise) {
  if (B <= 64 || fp8_weights) {
    const int64_t cols = B >= 64 ? 64 : B;
    return cols < 1 ? 1 : (int)((cols + 15) / 16);
  }
  // Beyond 64 columns: tiles of 128 columns.  Wider tiles would need more
  // than the 256 registers a lane has at two waves per SIMD.
  (void)fp64_noise;
  return 8;
}

hipError_t launch_fused_stage1(const FusedArgs& a, int epi, hipStream_t stream) {
  if (epi == kEpiTopK32 || epi == kEpiTopK64) {
    int nb = fused_column_blocks(a.B, true, false);  // tiles of at most 64 columns
    if (epi == kEpiTopK64 && nb > 1) nb = 4;
    const dim3 grid((unsigned)a.nT, (unsigned)((a.B + 16 * nb - 1) / (16 * nb)));
    hipError_t e = launch_w<kWBf16>(a, epi, grid, nb, stream);
    // Tiles wider than kStage2InKernelRows rows: Stage 2 in a launch of its own.
    if (e != hipSuccess || 16 * nb <= kStage2InKernelRows) return e;
    const dim3 g2((unsigned)((a.B + 3) / 4));
    if (epi == kEpiTopK64)
      launch(topk_stage2_kernel<double>, g2, dim3(256), 0, stream, a);
    else
      launch(topk_stage2_kernel<float>, g2, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  if (fused_wide_applies(a, epi)) return launch_fused_wide(a, epi, stream);
  const bool narrow = a.W8 != nullptr || a.W4 != nullptr;
  const int nb = fused_column_blocks(a.B, narrow, epi == kEpiSample64);
  const int64_t tile = 16 * nb;
  const int64_t nbt = (a.B + tile - 1) / tile;
  const dim3 grid((unsigned)a.nT, (unsigned)nbt);
  // Each column's logits come from its own MFMA column, so the tile width
  // does not change any row's arithmetic.
  if (a.W4)
    return a.D <= kS4MaxD ? launch_w<kWFp4>(a, epi, grid, nb, stream) : launch_w<kWFp4Wide>(a, epi, grid, nb, stream);
  if (a.W8) return launch_w<kWFp8>(a, epi, grid, nb, stream);
  if (nb > 4) return launch_wide(a, epi, grid, stream);
  return launch_w<kWBf16>(a, epi, grid, nb, stream);
}

int fused_filtered_column_blocks(int64_t B, bool fp64) {
  int nb = fused_column_blocks(B, true, false);  // tiles of at most 64 columns
  if (fp64 && nb > 1) nb = 4;                    // float64 scores: 16 or 64 columns
  return nb;
}

hipError_t launch_fused_filtered(const FusedArgs& a, bool fp64, const FilterArgs& fa,
                                 hipStream_t stream) {
  const int nb = fused_filtered_column_blocks(a.B, fp64);
  const dim3 grid((unsigned)a.nT, (unsigned)((a.B + 16 * nb - 1) / (16 * nb)));
  // Stage 1 writes the logits of the rows filt_store_row picks into the
  // fallback's buffer as it goes.
  FusedArgs s1 = a;
  s1.Y = fa.X == nullptr ? nullptr : const_cast<float*>(fa.X);
  hipError_t e = launch_w<kWBf16>(s1, fp64 ? kEpiFilt64 : kEpiFilt32, grid, nb, stream);
  if (e != hipSuccess) return e;
  const dim3 g2((unsigned)((a.B + kFiltRowsPerBlock - 1) / kFiltRowsPerBlock));
  if (fp64)
    launch(filt_stage2_kernel<double>, g2, dim3(64 * kFiltRowsPerBlock), 0, stream, a);
  else
    launch(filt_stage2_kernel<float>, g2, dim3(64 * kFiltRowsPerBlock), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // The fallback: the same tiles' logits of the flagged rows whose logits
  // Stage 1 did not write (flag 1; the store epilogue returns at once when
  // there is none), then the filtered sampler over every flagged row (one
  // workgroup per row, the others return at once).
  FusedArgs s = a;
  s.Y = fa.X == nullptr ? nullptr : const_cast<float*>(fa.X);
  e = launch_w<kWBf16>(s, kEpiStore, grid, nb, stream);
  if (e != hipSuccess) return e;
  return launch_logits_filtered(fa, fp64, stream);
}

int64_t fused_wave_span_bytes(int64_t V, int64_t D, int nT, int elem_bytes) {
  // Most 8-row units of one workgroup, then of one of its waves.
  const int64_t nunits = (V + 7) >> 3;
  const int64_t nu = (nunits + nT - 1) / nT;
  const int64_t rows = ((nu + kWaves - 1) / kWaves) * 8;
  return rows * D * elem_bytes;
}

}  // namespace fs
