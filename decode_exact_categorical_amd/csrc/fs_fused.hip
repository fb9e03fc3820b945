// fs_fused.hip -- fused LM-head matmul + exact sampling, Stage 1, for gfx950.
//
// Follows the FlashSampling page ("algorithm details", Stage 1 steps (1)-(6)):
// for a (batch tile x vocabulary tile) the logits Y = H W^T are formed on chip,
// transformed (bias, temperature), perturbed with Gumbel noise, and only the
// per-row tile maximum and its vocabulary index are written out.  The [B, V]
// logits never reach HBM.
//
// Design for MI355X (differs from the page's Triton kernel, written for NVIDIA):
//  * W streams from HBM exactly once.  A workgroup owns a contiguous range of
//    16-row vocabulary blocks (about nblk / grid blocks each, so the 256 CUs
//    finish within one 16-row block of each other) and walks it in passes of
//    64 rows.
//  * The 4 waves of a workgroup split the contraction dimension D into four
//    contiguous quarters.  Each wave streams its quarter of the pass's 64 W
//    rows straight into VGPRs in the bf16 MFMA A-operand layout (lane l reads
//    16 bytes of row l%16; the 4 lanes of a row cover 64 contiguous bytes per
//    instruction) and the matching H fragments (B operand, batch as the MFMA
//    N dimension), one or two k-slices per pipeline stage, double-buffered.
//    v_mfma_f32_16x16x32_bf16 accumulates in fp32.
//  * The four partial sums meet in LDS and are added in a fixed order (wave 0,
//    1, 2, 3), so every logit has one accumulation order that depends neither
//    on B nor on the row's batch position.
//  * Epilogue: wave w takes row block w of the pass.  In the MFMA output
//    layout a lane holds 4 consecutive vocabulary rows of one batch column, so
//    one Philox4x32-10 call gives the noise of all four (two calls for float64
//    noise).  Scores feed a per-lane running argmax; at the end, xor-shuffles
//    and LDS reduce it to one candidate per batch row for the workgroup.
#include <type_traits>

#include "fs_launch.hpp"

namespace fs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;                // K-split across the waves of a workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kRB = 4;                   // 16-row blocks per pass
constexpr int kBatchTile = 64;           // batch columns per workgroup (<= 4 MFMA blocks)

template <int EPI>
struct ScoreType {
  typedef float type;
};
template <>
struct ScoreType<kEpiSample64> {
  typedef double type;
};

__device__ __forceinline__ bf16x8 load_frag(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x8 zero_frag() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.0f;
  return z;
}

// 32-wide k-slices per pipeline stage: two while the register file allows it
// (at two waves per SIMD a wave has 256 VGPRs), one for three or four column
// blocks, whose accumulators and H fragments need the room.
template <int NB>
struct Stage {
  static constexpr int kS = NB <= 2 ? 2 : 1;
};

template <int NB, int EPI>
__global__ __launch_bounds__(kThreads, 2) void fused_stage1_kernel(FusedArgs a) {
  typedef typename ScoreType<EPI>::type T;
  constexpr int kS = Stage<NB>::kS;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane >> 4;  // k-group of the operands, row group of the output
  const int col = lane & 15;  // A row / B column / output column within a block

  const int64_t B = a.B, D = a.D, V = a.V;
  const int64_t bt0 = (int64_t)blockIdx.y * kBatchTile;

  // This workgroup's 16-row vocabulary blocks [blk0, blk1).
  const int64_t nblk = (V + 15) >> 4;
  const int64_t blk0 = nblk * (int64_t)blockIdx.x / gridDim.x;
  const int64_t blk1 = nblk * (int64_t)(blockIdx.x + 1) / gridDim.x;

  // This wave's 32-wide k-steps [ks0, ks1).
  const int KS = (int)((D + 31) >> 5);
  const int ks0 = KS * wave / kWaves;
  const int ks1 = KS * (wave + 1) / kWaves;

  // H fragment pointers, one per 16-column batch block (rows past B are
  // clamped to B-1; their results are discarded by the epilogue).
  const uint16_t* hp[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    int64_t b = bt0 + 16 * cb + col;
    if (b > B - 1) b = B - 1;
    hp[cb] = a.H + b * D + 8 * grp;
  }

  // Per-column sampling constants.
  bool col_ok[NB], greedy[NB];
  T inv_t[NB];
  uint32_t rid[NB];
  T bm[NB];
  int32_t bi[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    const int64_t b = bt0 + 16 * cb + col;
    col_ok[cb] = b < B;
    const int64_t bc = col_ok[cb] ? b : 0;
    float t = 1.0f;
    if (EPI != kEpiStore) t = a.temp[bc];
    greedy[cb] = !(t > 0.0f);
    inv_t[cb] = greedy[cb] ? T(1) : T(1) / T(t);
    rid[cb] = a.row_ids ? a.row_ids[bc] : (uint32_t)bc;
    bm[cb] = neg_inf<T>();
    bi[cb] = kNoIndex;
  }

  __shared__ f32x4 red[kWaves][kRB][NB][64];

  for (int64_t pb = blk0; pb < blk1; pb += kRB) {
    const int nrb = (int)((blk1 - pb) < kRB ? (blk1 - pb) : kRB);

    const uint16_t* wp[kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      int64_t row = (pb + rb) * 16 + col;
      if (row > V - 1) row = V - 1;
      wp[rb] = a.W + row * D + 8 * grp;
    }

    f32x4 acc[kRB][NB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

    bf16x8 wb[2][kS][kRB];
    bf16x8 hb[2][kS][NB];

    // Loads of one pipeline stage (kS k-steps) into buffer BUF.  A k-step that
    // runs past D (D % 32 != 0) zero-fills the lanes whose 8 elements lie past D.
    auto load_stage = [&](auto BUFC, int ksb) {
      constexpr int BUF = decltype(BUFC)::value;
#pragma unroll
      for (int s = 0; s < kS; ++s) {
        const int ks = ksb + s;
        if (ks < ks1) {
          const int64_t k = (int64_t)ks * 32;
          if (k + 32 <= D) {
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb)
              if (rb < nrb) wb[BUF][s][rb] = load_frag(wp[rb] + k);
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) hb[BUF][s][cb] = load_frag(hp[cb] + k);
          } else {
            const bool in = k + 8 * grp < D;
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb)
              if (rb < nrb) wb[BUF][s][rb] = in ? load_frag(wp[rb] + k) : zero_frag();
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) hb[BUF][s][cb] = in ? load_frag(hp[cb] + k) : zero_frag();
          }
        }
      }
    };
    auto compute_stage = [&](auto BUFC, int ksb) {
      constexpr int BUF = decltype(BUFC)::value;
#pragma unroll
      for (int s = 0; s < kS; ++s) {
        if (ksb + s < ks1) {
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb)
            if (rb < nrb)
#pragma unroll
              for (int cb = 0; cb < NB; ++cb)
                acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    wb[BUF][s][rb], hb[BUF][s][cb], acc[rb][cb], 0, 0, 0);
        }
      }
    };

    typedef std::integral_constant<int, 0> Buf0;
    typedef std::integral_constant<int, 1> Buf1;
    load_stage(Buf0{}, ks0);
    for (int ks = ks0; ks < ks1; ks += 2 * kS) {
      load_stage(Buf1{}, ks + kS);
      compute_stage(Buf0{}, ks);
      load_stage(Buf0{}, ks + 2 * kS);
      compute_stage(Buf1{}, ks + kS);
    }

    // Partial sums of the four K quarters meet in LDS.
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) red[wave][rb][cb][lane] = acc[rb][cb];
    __syncthreads();

    if (wave < nrb) {
      const int rb = wave;
      const int64_t i0 = (pb + rb) * 16 + 4 * grp;  // first of this lane's 4 rows
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        f32x4 y = red[0][rb][cb][lane];
        y += red[1][rb][cb][lane];
        y += red[2][rb][cb][lane];
        y += red[3][rb][cb][lane];
        if (!col_ok[cb]) continue;
        const int64_t b = bt0 + 16 * cb + col;
        if (EPI == kEpiStore) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (i0 + j < V) a.Y[b * V + i0 + j] = y[j];
          continue;
        }
        float beta[4] = {0.f, 0.f, 0.f, 0.f};
        if (a.bias) {
          const float* bp = a.bias + b * V + i0;
          if (a.bias_vec4 && i0 + 3 < V) {
            const float4 v = *reinterpret_cast<const float4*>(bp);
            beta[0] = v.x; beta[1] = v.y; beta[2] = v.z; beta[3] = v.w;
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (i0 + j < V) beta[j] = bp[j];
          }
        }
        T s[4];
        if (greedy[cb]) {
#pragma unroll
          for (int j = 0; j < 4; ++j) s[j] = T(y[j]) + T(beta[j]);
        } else if (EPI == kEpiSample32) {
          const Words w = noise_words(a.key, (uint32_t)(i0 >> 2), rid[cb]);
          s[0] = T((y[0] + beta[0]) * inv_t[cb]) + T(gumbel_f32(w.w0));
          s[1] = T((y[1] + beta[1]) * inv_t[cb]) + T(gumbel_f32(w.w1));
          s[2] = T((y[2] + beta[2]) * inv_t[cb]) + T(gumbel_f32(w.w2));
          s[3] = T((y[3] + beta[3]) * inv_t[cb]) + T(gumbel_f32(w.w3));
        } else {
          const Words w0 = noise_words(a.key, (uint32_t)(i0 >> 1), rid[cb]);
          const Words w1 = noise_words(a.key, (uint32_t)(i0 >> 1) + 1u, rid[cb]);
          s[0] = (T(y[0]) + T(beta[0])) * inv_t[cb] + T(gumbel_f64(w0.w0, w0.w1));
          s[1] = (T(y[1]) + T(beta[1])) * inv_t[cb] + T(gumbel_f64(w0.w2, w0.w3));
          s[2] = (T(y[2]) + T(beta[2])) * inv_t[cb] + T(gumbel_f64(w1.w0, w1.w1));
          s[3] = (T(y[3]) + T(beta[3])) * inv_t[cb] + T(gumbel_f64(w1.w2, w1.w3));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int32_t i = (int32_t)(i0 + j);
          if (i0 + j < V && beats(s[j], i, bm[cb], bi[cb])) {
            bm[cb] = s[j];
            bi[cb] = i;
          }
        }
      }
    }
    __syncthreads();
  }

  if (EPI == kEpiStore) return;

  // Lanes that share a column (the 4 row groups) -> one value per column.
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) wave_argmax_xor(bm[cb], bi[cb], 4);

  // Across the 4 waves, in wave order, through LDS (the reduction buffer is free).
  Cand<T>* wbest = reinterpret_cast<Cand<T>*>(&red[0][0][0][0]);
  if (grp == 0) {
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) wbest[wave * (NB * 16) + cb * 16 + col] = Cand<T>{bm[cb], bi[cb]};
  }
  __syncthreads();
  if (threadIdx.x < NB * 16) {
    const int c = threadIdx.x;
    Cand<T> best = wbest[c];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      const Cand<T> o = wbest[w * (NB * 16) + c];
      if (beats(o.m, o.idx, best.m, best.idx)) best = o;
    }
    const int64_t b = bt0 + c;
    if (b < B) reinterpret_cast<Cand<T>*>(a.cand)[b * a.nT + blockIdx.x] = best;
  }
}

template <int NB>
hipError_t launch_nb(const FusedArgs& a, int epi, dim3 grid, hipStream_t stream) {
  switch (epi) {
    case kEpiSample32:
      hipLaunchKernelGGL((fused_stage1_kernel<NB, kEpiSample32>), grid, dim3(kThreads), 0, stream, a);
      break;
    case kEpiSample64:
      hipLaunchKernelGGL((fused_stage1_kernel<NB, kEpiSample64>), grid, dim3(kThreads), 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL((fused_stage1_kernel<NB, kEpiStore>), grid, dim3(kThreads), 0, stream, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace

int fused_num_tiles(int64_t V, int num_cus) {
  const int64_t nblk = (V + 15) >> 4;
  int64_t g = 2 * (int64_t)num_cus;  // two workgroups per CU
  if (g > nblk) g = nblk;
  if (g < 1) g = 1;
  return (int)g;
}

hipError_t launch_fused_stage1(const FusedArgs& a, int epi, hipStream_t stream) {
  const int64_t nbt = (a.B + kBatchTile - 1) / kBatchTile;
  const dim3 grid((unsigned)a.nT, (unsigned)nbt);
  // 16-wide column blocks per batch tile: enough for the widest tile.  Each
  // column's logits come from its own MFMA column, so this does not change
  // any row's arithmetic.
  const int64_t cols = a.B >= kBatchTile ? kBatchTile : a.B;
  const int nb = (int)((cols + 15) / 16);
  switch (nb) {
    case 1: return launch_nb<1>(a, epi, grid, stream);
    case 2: return launch_nb<2>(a, epi, grid, stream);
    case 3: return launch_nb<3>(a, epi, grid, stream);
    default: return launch_nb<4>(a, epi, grid, stream);
  }
}

}  // namespace fs
