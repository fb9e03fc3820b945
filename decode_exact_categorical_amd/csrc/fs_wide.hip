// fs_wide.hip -- the fused LM-head + exact sampling kernel for wide batches
// (more than 64 rows) on gfx950.
//
// Follows the FlashSampling page ("algorithm details", Stage 1 steps (1)-(6)
// and Stage 2) like the narrow kernel (fs_fused.hip): the logits of a
// (vocabulary tile x batch tile) are formed on chip, transformed, perturbed
// and reduced to one candidate per batch row, and never reach HBM.
//
// Past 64 batch columns the contraction nears the MFMA roofline (the page's
// "limitations" note that the LM head turns compute bound at large batch), so
// the tiling is chosen for operand reuse as well as for the W stream:
//  * One workgroup per CU owns a contiguous slice of the vocabulary and all
//    the batch columns of its batch tile (up to 256), so W crosses HBM once.
//    Its 4 waves (one per SIMD, up to 512 registers a lane) each hold a
//    64 x 128 block of float32 accumulators (4 MFMA row blocks x 8 column
//    blocks, 128 registers a lane): with 128 columns the 4 waves take 4 row
//    groups, with 256 columns 2 row groups x 2 column halves, whose two waves
//    read the same W rows at the same time (the second read is served by the
//    CU's cache).  At two waves per SIMD (256 registers) this tile spills.
//  * W goes straight from HBM into VGPRs in the bf16 MFMA A-operand layout,
//    three to four k-steps ahead (each pass requests its own first k-steps).
//    Each W fragment feeds 8 MFMAs.
//  * H is the B operand, staged through LDS in double-buffered chunks of 128 k
//    for all the workgroup's columns; each H fragment read from LDS feeds the
//    wave's 4 row blocks.
//  * v_mfma_f32_16x16x32_bf16 accumulates in float32 in one fixed k order per
//    vocabulary tile (128-k chunks from a per-tile starting chunk on, wrapping
//    around), independent of the row's batch position.
//  * Float32 noise (bias + t * g of one 4-row x 1-column fragment, one
//    Philox4x32-10 call) is folded into the accumulators inside the k-loop:
//    the k-loop runs in iterations of 8 k-steps, and in 4 of them, spread
//    evenly over the contraction, k-step j folds the noise of column block j
//    of one row block.  After the k-loop the score is acc / t.  Float64 noise
//    is added after the k-loop, the score formed in float64.
//  * Stage 2 (the row's best candidate over the vocabulary tiles) is a small
//    second launch of one wave per row.
#include <type_traits>
#include <utility>

#include "fs_launch.hpp"

namespace fs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#ifndef FS_WIDE_RB
#define FS_WIDE_RB 4
#endif
constexpr int kXRB = FS_WIDE_RB;           // row blocks of a wave pass
constexpr int kXKC = 128;                  // k per H chunk (four k-steps)
constexpr int kXCS = kXKC / 32;            // k-steps per chunk
constexpr int kXCP = kXKC / 8;             // 16-byte pieces of one column's chunk
constexpr int kXRow = kXKC + 8;            // padded LDS row of one column (bf16)
constexpr int kXAhead = 4;                 // k-steps of W (and biases) in flight
constexpr int kXBody = 8;                  // k-steps per iteration: one fold per column block
static_assert(kXBody % (2 * kXCS) == 0, "an iteration holds whole chunk pairs");
constexpr float kXInfTemp = 0x1p60f;       // at or above this, t * g is not folded

enum XColMode { kXGreedy = 0, kXSample = 1, kXInfT = 2 };

// f(integral_constant<int, J>) for J = 0 .. N-1, each call with J a constant.
template <typename Fn, int... J>
__device__ __forceinline__ void static_for_impl(Fn&& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>()), ...);
}
template <int N, typename Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>());
}

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ bf16x8 as_bf(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// A raw buffer resource (gfx9 family descriptor word 3): 32-bit byte offsets
// from a wave-uniform base; loads at offsets at or past num_records return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_records) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_records, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
constexpr uint32_t kXOob = 0x80000000u;  // an offset past every resource used here

// NW waves of NBW column blocks each; CG: the tile's columns in units of 128
// (1 or 2).  Sizes fit 32 bits (the host checks D < 2^22 and V < 2^31);
// per-lane indices stay 32-bit.
template <int NW, int NBW, int CG, int EPI, bool HAS_BIAS, bool BV4>
__global__ __launch_bounds__(64 * NW) void fused_wide_kernel(FusedArgs a) {
  constexpr int kXThreads = 64 * NW;
  constexpr int kXNB = NBW;
  constexpr int kWC = 16 * NBW;  // columns of a wave
  typedef typename std::conditional<EPI == kEpiSample64, double, float>::type T;
  constexpr bool kFold = EPI == kEpiSample32;
  constexpr bool kLoadBias = kFold && HAS_BIAS;
  constexpr int kTC = 128 * CG;              // columns of the workgroup
  constexpr int RG = NW / (kTC / kWC);       // row groups
  static_assert(kTC % kWC == 0 && NW % (kTC / kWC) == 0, "whole column groups");
  constexpr int kPieces = kTC * (kXKC / 8);  // 16-byte pieces of an H chunk
  constexpr int kHQ = kPieces / kXThreads;   // pieces a thread stages
  static_assert(kPieces % kXThreads == 0, "whole pieces per thread");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave % RG, cg = wave / RG;
  const int grp = lane >> 4;  // operand k-group; output row group
  const int col = lane & 15;  // A row / B column / output column in a block
  const int B = (int)a.B, D = (int)a.D, V = (int)a.V;

  // (vocabulary tile, batch tile): the batch tiles of a vocabulary tile run
  // on one XCD together (workgroups go to the 8 XCDs round-robin), so all
  // but one of them read their W rows from that XCD's L2.
  const int nT = (int)gridDim.x, nbt = (int)gridDim.y;
  int tile = (int)blockIdx.x, btile = (int)blockIdx.y;
  if (nbt > 1 && nT % 8 == 0) {
    const int lin = (int)blockIdx.y * nT + (int)blockIdx.x;
    tile = (lin / (8 * nbt)) * 8 + lin % 8;
    btile = (lin / 8) % nbt;
  }
  const int bt0 = btile * kTC;
  const int ncol = B - bt0 < kTC ? B - bt0 : kTC;  // valid columns of the tile
  const int wcol0 = kWC * cg;                      // the wave's first column in the tile

  // The workgroup's rows (8-row units) split evenly over its row groups; a
  // row group walks its rows in passes of 64, the same number of passes for
  // every wave (the barriers of the H staging are shared).
  const int nunits = (int)(((int64_t)V + 7) >> 3);
  const int g0 = (int)((int64_t)nunits * tile / nT);
  const int g1 = (int)((int64_t)nunits * (tile + 1) / nT);
  const int nu = g1 - g0;
  const int r0 = (g0 + nu * rg / RG) * 8;
  int r1 = (g0 + nu * (rg + 1) / RG) * 8;
  if (r1 > V) r1 = V;
  const int max_rows = ((nu + RG - 1) / RG) * 8;
  const int npass = (max_rows + 16 * kXRB - 1) / (16 * kXRB);

  // The contraction in k-steps of 32, padded to whole iterations, at least 4
  // (one per folded row block); steps past D meet zero H.
  const int KS = D / 32;
  int NI = (KS + kXBody - 1) / kXBody;
  if (NI < kXRB) NI = kXRB;
  const int KSP = NI * kXBody;
  const int NCP = KSP / kXCS;              // chunks of the padded contraction
  const int NC = (KS + kXCS - 1) / kXCS;   // chunks that hold part of D
  const int rot = tile % NC;
  auto phys_chunk = [&](int c) -> int { return c >= NC ? c : (c + rot < NC ? c + rot : c + rot - NC); };
  auto phys_step = [&](int s) -> int {
    const int c = s / kXCS;
    const int ps = (c >= NC ? KS : phys_chunk(c) * kXCS) + s % kXCS;
    return ps < KS ? ps : 0;
  };

  // Per-column sampling constants.
  struct ColInfo {
    float t;
    float inv_t;
    uint32_t rid;
    int mode;
  };
  __shared__ ColInfo cols[kTC];
  for (int c = tid; c < kTC; c += kXThreads) {
    const int bc = c < ncol ? bt0 + c : 0;
    float t = 1.0f;
    if (EPI != kEpiStore) t = a.temp[bc];
    ColInfo ci;
    ci.mode = !(t > 0.0f) ? kXGreedy : (t < kXInfTemp ? kXSample : kXInfT);
    ci.t = t;
    ci.inv_t = ci.mode == kXGreedy ? 1.0f : 1.0f / t;
    ci.rid = a.row_ids ? a.row_ids[bc] : (uint32_t)bc;
    cols[c] = ci;
  }
  // Each wave's running best per column across its passes.
  __shared__ Cand<T> wrun[NW][kWC];
  if (EPI != kEpiStore)
    for (int c = lane; c < kWC; c += 64) wrun[wave][c] = Cand<T>{neg_inf<T>(), kNoIndex};
  __shared__ __attribute__((aligned(16))) uint16_t hs[2][kTC][kXRow];

  // H chunk staging through VGPRs: thread t stages pieces t + 256 q (column
  // piece / 8, k offset 8 (piece % 8)) from a resource over the tile's valid
  // columns; columns past B and k past D read as zero.
  const __amdgpu_buffer_rsrc_t hrsrc = make_rsrc(a.H + (int64_t)bt0 * D, (uint32_t)ncol * (uint32_t)D * 2u);
  uint32_t hv[kHQ];
  int hk[kHQ];
#pragma unroll
  for (int q = 0; q < kHQ; ++q) {
    const int piece = tid + kXThreads * q;
    const int hc = piece / kXCP;
    hk[q] = (piece % kXCP) * 8;
    hv[q] = hc < ncol ? ((uint32_t)hc * (uint32_t)D + (uint32_t)hk[q]) * 2u : kXOob;
  }
  u32x4 hst[kHQ];
  auto h_load = [&](int c) {
    const int pc = phys_chunk(c);
#pragma unroll
    for (int q = 0; q < kHQ; ++q)
      hst[q] = bload16(hrsrc, pc * kXKC + hk[q] < D ? hv[q] : kXOob, (uint32_t)pc * (kXKC * 2));
  };
  auto h_store = [&](int buf) {
#pragma unroll
    for (int q = 0; q < kHQ; ++q) {
      const int piece = tid + kXThreads * q;
      *reinterpret_cast<u32x4*>(&hs[buf][piece / kXCP][(piece % kXCP) * 8]) = hst[q];
    }
  };

  // W: a resource based at the row group's first row, a 32-bit byte offset
  // per row block and lane (a row group spans at most twice the rows of the
  // narrow kernel's waves, whose span the host bounds by 2^31 bytes) and the
  // k-step's offset as the uniform soffset.  Rows past the row group's last
  // re-read it (never scored).
  const int rbase = r1 > r0 ? r0 : 0;
  const int rlast = r1 > r0 ? r1 - 1 : 0;
  const __amdgpu_buffer_rsrc_t wrsrc = make_rsrc(a.W + (int64_t)rbase * D, 0xffffffffu);
  auto row_offsets = [&](int p, uint32_t (&o)[kXRB]) {
#pragma unroll
    for (int rb = 0; rb < kXRB; ++rb) {
      int row = r0 + p * 16 * kXRB + 16 * rb + col;
      if (row > rlast) row = rlast;
      o[rb] = ((uint32_t)(row - rbase) * (uint32_t)D + 8u * grp) * 2u;
    }
  };
  auto w_load = [&](u32x4 (&dst)[kXRB], const uint32_t (&o)[kXRB], int s) {
    const uint32_t soff = (uint32_t)phys_step(s) * 64u;
#pragma unroll
    for (int rb = 0; rb < kXRB; ++rb) dst[rb] = bload16(wrsrc, o[rb], soff);
  };
  // k-steps s (even) and s + 1, row block by row block.
  auto w_load_pair = [&](u32x4 (&d0)[kXRB], u32x4 (&d1)[kXRB], const uint32_t (&o)[kXRB], int s) {
    const uint32_t s0 = (uint32_t)phys_step(s) * 64u, s1 = (uint32_t)phys_step(s + 1) * 64u;
#pragma unroll
    for (int rb = 0; rb < kXRB; ++rb) {
      d0[rb] = bload16(wrsrc, o[rb], s0);
      d1[rb] = bload16(wrsrc, o[rb], s1);
    }
  };
  // The bias of fold slot (pass p, row block rb, column block cb): the lane's
  // 4 rows of one column.
  const float* bias_tile = a.bias + (int64_t)bt0 * V;
  auto bias_load = [&](f32x4& dst, int p, int rb, int cb) {
    if constexpr (!kLoadBias) return;
    int c = wcol0 + 16 * cb + col;
    if (c > ncol - 1) c = ncol - 1;
    const float* bp = bias_tile + (int64_t)c * V;
    const int i0 = r0 + p * 16 * kXRB + 16 * rb + 4 * grp;
    if constexpr (BV4) {
      dst = *reinterpret_cast<const f32x4*>(bp + (i0 > V - 4 ? V - 4 : i0));
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[j] = bp[i0 + j < V ? i0 + j : V - 1];
    }
  };

  // One H fragment (16 columns x 32 k) of k-step kk of the chunk in buffer buf.
  auto h_frag = [&](int buf, int cb, int kk) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(&hs[buf][wcol0 + 16 * cb + col][kk * 32 + 8 * grp]);
  };
  bf16x8 hf[2][kXNB];
  f32x4 acc[kXRB][kXNB];
  u32x4 wb[kXAhead][kXRB];
  f32x4 bring[kXAhead];
  uint32_t wo[kXRB];

  // Prologue: H chunk 0 (each pass's last chunk stages the next pass's
  // first).
  h_load(0);
  __syncthreads();  // cols
  h_store(0);
  __syncthreads();

  for (int p = 0; p < npass; ++p) {
    // The pass's first k-steps of W and the biases of its first fold slots.
    row_offsets(p, wo);
#pragma unroll
    for (int s = 0; s < kXAhead; s += 2) w_load_pair(wb[s], wb[s + 1], wo, s);
#pragma unroll
    for (int s = 0; s < kXAhead; ++s) {
      bring[s] = f32x4{0.f, 0.f, 0.f, 0.f};
      bias_load(bring[s], p, 0, s);
    }
    const int pr0 = r0 + p * 16 * kXRB;
#pragma unroll
    for (int rb = 0; rb < kXRB; ++rb)
#pragma unroll
      for (int cb = 0; cb < kXNB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One iteration: 8 k-steps (2 H chunks).  In the 4 fold iterations that
    // open a pass (float32 noise), k-step j also folds the noise of fragment
    // (row block it, column block j).
    // FI: the fold iteration (its row block), or -1 for a plain iteration.
    auto body = [&](auto fold_tag, int it) {
      constexpr int FI = decltype(fold_tag)::value;
      constexpr bool F = FI >= 0;
      static_for<kXBody>([&](auto jtag) {
        constexpr int j = decltype(jtag)::value;
        const int buf = (j / kXCS) & 1;
        if (j % kXCS == 0) {
          // the next chunk (after the last: the next pass's first)
          const int c1 = it * (kXBody / kXCS) + j / kXCS + 1;
          h_load(c1 < NCP ? c1 : 0);
        }
        // H fragments: a chunk's first k-step reads its own after the
        // barrier; every other k-step's were read during the previous one.
        if constexpr (j % kXCS == 0) {
#pragma unroll
          for (int cb = 0; cb < kXNB; ++cb) hf[j & 1][cb] = h_frag(buf, cb, j % kXCS);
        }
        constexpr bool kFoldStep = F && j < kXNB;
        // Fold slot j (fold iterations): the noise of fragment (row block FI,
        // column block j), bias + t * g, computed in the MFMAs' scheduling
        // region so its VALU work interleaves with them; its bias was loaded
        // four k-steps ago.
        f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (kFoldStep) {
          const f32x4 beta = bring[j % kXAhead];
          if constexpr (kLoadBias) {
            constexpr int g4 = (F ? FI : 0) * kXBody + j + kXAhead;  // the slot four k-steps on
            if constexpr (g4 / kXBody < kXRB && g4 % kXBody < kXNB)
              bias_load(bring[j % kXAhead], p, g4 / kXBody, g4 % kXBody);
          }
          __builtin_amdgcn_sched_barrier(0);
          const ColInfo ci = cols[wcol0 + 16 * j + col];
          const bool ok = wcol0 + 16 * j + col < ncol;
          const int i0 = pr0 + 16 * FI + 4 * grp;
          // (branch-free: every lane computes the noise, selects apply it)
          const Words w = noise_words(a.key, (uint32_t)i0 >> 2, ci.rid);
          const bool use = ok && i0 < r1;
          const float tn = use && ci.mode == kXSample ? ci.t : 0.0f;
          const float g[4] = {gumbel_f32(w.w0), gumbel_f32(w.w1), gumbel_f32(w.w2), gumbel_f32(w.w3)};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float b = HAS_BIAS && use ? beta[e] : 0.0f;
            v[e] = tn == 0.0f ? b : b + tn * g[e];
          }
        } else {
          __builtin_amdgcn_sched_barrier(0);
        }
        // The MFMAs of k-step j: each H fragment meets the wave's 4 row blocks,
        // while the next k-step's fragments (same chunk) are read.
#pragma unroll
        for (int cb = 0; cb < kXNB; ++cb) {
          if constexpr (j % kXCS != kXCS - 1) hf[(j + 1) & 1][cb] = h_frag(buf, cb, (j + 1) % kXCS);
#pragma unroll
          for (int rb = 0; rb < kXRB; ++rb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(wb[j % kXAhead][rb]), hf[j & 1][cb],
                                                                  acc[rb][cb], 0, 0, 0);
        }
        if constexpr (kFoldStep) {
          // one MFMA, then up to three VALU instructions of the noise
#pragma unroll
          for (int q = 0; q < kXRB * kXNB; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kFoldStep) acc[F ? FI : 0][j < kXNB ? j : 0] += v;
        // Refill the ring: after every second k-step, the two slots just used
        // take k-steps j + 3 and j + 4, the two 64-byte halves of each row's
        // 128-byte segment requested back to back (HBM streams markedly
        // faster so).  Past the pass's end: step 0 against zero H, never used.
        if constexpr (j % 2 == 1)
          w_load_pair(wb[(j - 1) % kXAhead], wb[j % kXAhead], wo, it * kXBody + j - 1 + kXAhead);
        if (j % kXCS == kXCS - 1) {
          __builtin_amdgcn_sched_barrier(0);
          h_store(buf ^ 1);
          __syncthreads();
        }
      });
    };
    // (Each fold iteration is its own copy: it folds into fixed registers.)
    if constexpr (kFold) {
      static_for<kXRB>([&](auto ftag) { body(ftag, decltype(ftag)::value); });
    }
#pragma unroll 1
    for (int it = kFold ? kXRB : 0; it < NI; ++it) body(std::integral_constant<int, -1>(), it);

    if constexpr (EPI == kEpiStore) {
#pragma unroll
      for (int cb = 0; cb < kXNB; ++cb) {
        const int c = wcol0 + 16 * cb + col;
        if (c >= ncol) continue;
        float* yp = a.Y + (int64_t)(bt0 + c) * V;
#pragma unroll
        for (int rb = 0; rb < kXRB; ++rb) {
          const int i0 = pr0 + 16 * rb + 4 * grp;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (i0 + j < r1) yp[i0 + j] = acc[rb][cb][j];
        }
      }
    } else if constexpr (kFold) {
      // Scores: acc / t (+ g after the division for infinite temperatures);
      // per column the lane's 16 rows in increasing index order (only a
      // strictly larger score takes over: ties keep the smaller index, NaN
      // never takes over), then the column's 4 row groups (lanes 16 apart),
      // merged into the wave's running best.
#pragma unroll
      for (int cb = 0; cb < kXNB; ++cb) {
        const ColInfo ci = cols[wcol0 + 16 * cb + col];
        const bool inf_any = __builtin_amdgcn_ballot_w64(ci.mode == kXInfT) != 0ull;
        float bm = neg_inf<float>();
        int32_t bi = kNoIndex;
#pragma unroll
        for (int rb = 0; rb < kXRB; ++rb) {
          const int i0 = pr0 + 16 * rb + 4 * grp;
          float s[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) s[j] = acc[rb][cb][j] * ci.inv_t;
          if (inf_any && ci.mode == kXInfT) {
            const Words w = noise_words(a.key, (uint32_t)i0 >> 2, ci.rid);
            s[0] += gumbel_f32(w.w0);
            s[1] += gumbel_f32(w.w1);
            s[2] += gumbel_f32(w.w2);
            s[3] += gumbel_f32(w.w3);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool take = (i0 + j < r1) & (s[j] > bm);
            bm = take ? s[j] : bm;
            bi = take ? i0 + j : bi;
          }
        }
        wave_argmax_xor(bm, bi, 4);
        if (grp == 0) {
          const Cand<float> o = wrun[wave][16 * cb + col];
          if (beats(bm, bi, o.m, o.idx)) wrun[wave][16 * cb + col] = Cand<float>{bm, bi};
        }
      }
    } else {
      // Float64 noise: the score (y + bias) / t + g formed in float64 after
      // the k-loop.  The work per fragment (two Philox calls, four
      // transforms) is large, so the column blocks run in a rolled loop that
      // picks its 4 fragments out of the accumulators.
#pragma unroll 1
      for (int cb = 0; cb < kXNB; ++cb) {
        f32x4 y[kXRB];
#pragma unroll
        for (int rb = 0; rb < kXRB; ++rb) {
          y[rb] = acc[rb][0];
#pragma unroll
          for (int c2 = 1; c2 < kXNB; ++c2)
            if (c2 == cb) y[rb] = acc[rb][c2];
        }
        const ColInfo ci = cols[wcol0 + 16 * cb + col];
        int c = wcol0 + 16 * cb + col;
        if (c > ncol - 1) c = ncol - 1;
        const float* bp = HAS_BIAS ? bias_tile + (int64_t)c * V : nullptr;
        const T it = ci.mode == kXGreedy ? T(1) : T(1) / T(ci.t);
        T bm = neg_inf<T>();
        int32_t bi = kNoIndex;
#pragma unroll
        for (int rb = 0; rb < kXRB; ++rb) {
          const int i0 = pr0 + 16 * rb + 4 * grp;
          float beta[4] = {0.f, 0.f, 0.f, 0.f};
          if (HAS_BIAS) {
#pragma unroll
            for (int j = 0; j < 4; ++j) beta[j] = bp[i0 + j < V ? i0 + j : V - 1];
          }
          T s[4];
          if (ci.mode == kXGreedy) {
#pragma unroll
            for (int j = 0; j < 4; ++j) s[j] = T(y[rb][j]) + T(beta[j]);
          } else {
            const Words w0 = noise_words(a.key, (uint32_t)i0 >> 1, ci.rid);
            const Words w1 = noise_words(a.key, ((uint32_t)i0 >> 1) + 1u, ci.rid);
            s[0] = (T(y[rb][0]) + T(beta[0])) * it + T(gumbel_f64(w0.w0, w0.w1));
            s[1] = (T(y[rb][1]) + T(beta[1])) * it + T(gumbel_f64(w0.w2, w0.w3));
            s[2] = (T(y[rb][2]) + T(beta[2])) * it + T(gumbel_f64(w1.w0, w1.w1));
            s[3] = (T(y[rb][3]) + T(beta[3])) * it + T(gumbel_f64(w1.w2, w1.w3));
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool take = (i0 + j < r1) & (s[j] > bm);
            bm = take ? s[j] : bm;
            bi = take ? i0 + j : bi;
          }
        }
        wave_argmax_xor(bm, bi, 4);
        if (grp == 0) {
          const Cand<T> o = wrun[wave][16 * cb + col];
          if (beats(bm, bi, o.m, o.idx)) wrun[wave][16 * cb + col] = Cand<T>{bm, bi};
        }
      }
    }
  }
  if constexpr (EPI != kEpiStore) {
    // Across the row groups; one candidate per (row, vocabulary tile).
    __syncthreads();
    for (int c = tid; c < ncol; c += kXThreads) {
      const int h = c / kWC, cc = c % kWC;
      Cand<T> best = wrun[h * RG][cc];
#pragma unroll
      for (int g = 1; g < RG; ++g) {
        const Cand<T> o = wrun[h * RG + g][cc];
        if (beats(o.m, o.idx, best.m, best.idx)) best = o;
      }
      reinterpret_cast<Cand<T>*>(a.cand)[(int64_t)(bt0 + c) * a.nT + tile] = best;
    }
  }
}

// Stage 2 of the wide kernel: one wave per row, the best of its nT
// candidates (a launch of its own, after Stage 1's plain stores).
template <typename T>
__global__ __launch_bounds__(256) void wide_stage2_kernel(FusedArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t b = (int64_t)blockIdx.x * 4 + wave;
  if (b >= a.B) return;
  const Cand<T>* c = reinterpret_cast<const Cand<T>*>(a.cand) + b * a.nT;
  T bm = neg_inf<T>();
  int32_t bi = kNoIndex;
  for (int t = lane; t < a.nT; t += 64) {
    const Cand<T> o = c[t];
    if (beats(o.m, o.idx, bm, bi)) {
      bm = o.m;
      bi = o.idx;
    }
  }
  wave_argmax_xor(bm, bi, 0);
  if (lane == 0) a.out[b] = bm == neg_inf<T>() ? (int64_t)-1 : (int64_t)bi;
}

template <int NW, int NBW, int CG>
hipError_t launch_wide_cfg(const FusedArgs& a, int epi, hipStream_t stream) {
  const dim3 grid((unsigned)a.nT, (unsigned)((a.B + 128 * CG - 1) / (128 * CG)));
  const dim3 block(64 * NW);
  if (epi == kEpiStore) {
    launch((fused_wide_kernel<NW, NBW, CG, kEpiStore, false, false>), grid, block, 0, stream, a);
    return hipGetLastError();
  }
  if (epi == kEpiSample64) {
    if (a.bias)
      launch((fused_wide_kernel<NW, NBW, CG, kEpiSample64, true, false>), grid, block, 0, stream, a);
    else
      launch((fused_wide_kernel<NW, NBW, CG, kEpiSample64, false, false>), grid, block, 0, stream, a);
  } else {
    if (a.bias && a.bias_vec4)
      launch((fused_wide_kernel<NW, NBW, CG, kEpiSample32, true, true>), grid, block, 0, stream, a);
    else if (a.bias)
      launch((fused_wide_kernel<NW, NBW, CG, kEpiSample32, true, false>), grid, block, 0, stream, a);
    else
      launch((fused_wide_kernel<NW, NBW, CG, kEpiSample32, false, false>), grid, block, 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g2((unsigned)((a.B + 3) / 4));
  if (epi == kEpiSample64)
    launch(wide_stage2_kernel<double>, g2, dim3(256), 0, stream, a);
  else
    launch(wide_stage2_kernel<float>, g2, dim3(256), 0, stream, a);
  return hipGetLastError();
}

#ifndef FS_WIDE_NW
#define FS_WIDE_NW 4
#endif
constexpr int kWideWaves = FS_WIDE_NW;
constexpr int kWideBlocks = kWideWaves == 4 ? 8 : 4;

}  // namespace

bool fused_wide_shape(int64_t B, int64_t D, bool bf16_weights) {
  return bf16_weights && B > 64 && D % 32 == 0 && D < ((int64_t)1 << 22);
}

bool fused_wide_applies(const FusedArgs& a, int epi) {
  if (!fused_wide_shape(a.B, a.D, a.W != nullptr && a.W8 == nullptr && a.W4 == nullptr)) return false;
  if (epi == kEpiStore) return a.row_flags == nullptr;
  return epi == kEpiSample32 || epi == kEpiSample64;
}

int fused_call_tiles(int64_t B, int64_t D, int64_t V, bool bf16_weights, int num_cus, int64_t row_bytes) {
  if (fused_wide_shape(B, D, bf16_weights)) return fused_wide_tiles(B, V, num_cus);
  return fused_num_tiles(V, num_cus, B <= 64 ? row_bytes : 0);
}

hipError_t launch_fused_wide(const FusedArgs& a, int epi, hipStream_t stream) {
  // Batch tiles of 128 columns; with several, the vocabulary is split into
  // fewer tiles (fused_wide_tiles), so all the workgroups run at once.
  return launch_wide_cfg<kWideWaves, kWideBlocks, 1>(a, epi, stream);
}

int fused_wide_tiles(int64_t B, int64_t V, int num_cus) {
  const int64_t nbt = (B + 127) / 128;
  int64_t t = fused_num_tiles(V, num_cus) / nbt;
  t -= t % 8;  // whole XCD rounds, so a vocabulary tile's batch tiles share one XCD
  if (t < 8) t = 8;
  const int64_t nunits = (V + 7) >> 3;
  if (t > nunits) t = nunits;
  return (int)t;
}

}  // namespace fs
