// fs_logits.hip -- standalone exact sampler over materialised float32 logits,
// Stage 1, for gfx950.
//
// The Megatron-LM "fp64 sampling noise" page ("Cost") notes that its sampler
// materialises the noise and the ratio p/E in HBM, and that one program per
// row is latency-bound at small batch.  Here the noise is generated in
// registers and each row is split over ceil(V / chunk) workgroups, each
// reducing `chunk` logits to one (score, index) candidate; the last of them
// to finish runs Stage 2, picking the row's winner (finish_last, row_winner
// in fs_device.hpp).  The chunk (2048 to 32768 logits) is the largest that
// still gives the launch a few thousand workgroups, so small batches spread a
// row over many CUs and large ones amortise each workgroup's fixed cost.  Same transform, noise stream and tie rule as the fused
// path, so equal y + bias gives equal draws.
#include <type_traits>

#include "fs_launch.hpp"

namespace fs {
namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 4;  // float4 loads in flight per thread

// (y * inv_t + g) scores of 4 consecutive logits starting at i0 (i0 % 4 == 0),
// folded into the running best (bm, bi); entries at or past `hi` are skipped.
template <typename T>
__device__ __forceinline__ void score4(const LogitsArgs& a, bool greedy, T inv_t, uint32_t rid,
                                       int64_t i0, int64_t hi, float y0, float y1, float y2,
                                       float y3, T& bm, int32_t& bi) {
  T s[4];
  if (greedy) {
    s[0] = T(y0);
    s[1] = T(y1);
    s[2] = T(y2);
    s[3] = T(y3);
  } else if (sizeof(T) == 4) {
    const Words w = noise_words(a.key, (uint32_t)(i0 >> 2), rid);
    s[0] = T(y0 * (float)inv_t) + T(gumbel_f32(w.w0));
    s[1] = T(y1 * (float)inv_t) + T(gumbel_f32(w.w1));
    s[2] = T(y2 * (float)inv_t) + T(gumbel_f32(w.w2));
    s[3] = T(y3 * (float)inv_t) + T(gumbel_f32(w.w3));
  } else {
    const Words w0 = noise_words(a.key, (uint32_t)(i0 >> 1), rid);
    const Words w1 = noise_words(a.key, (uint32_t)(i0 >> 1) + 1u, rid);
    s[0] = T(y0) * inv_t + T(gumbel_f64(w0.w0, w0.w1));
    s[1] = T(y1) * inv_t + T(gumbel_f64(w0.w2, w0.w3));
    s[2] = T(y2) * inv_t + T(gumbel_f64(w1.w0, w1.w1));
    s[3] = T(y3) * inv_t + T(gumbel_f64(w1.w2, w1.w3));
  }
  // A thread meets its logits in increasing index order, so a strictly larger
  // score is the only way to beat the running best: on equal scores the
  // earlier (smaller) index stays, as the candidate order requires.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (i0 + j < hi && s[j] > bm) {
      bm = s[j];
      bi = (int32_t)(i0 + j);
    }
  }
}

template <bool FP64>
__global__ __launch_bounds__(kThreads) void logits_stage1_kernel(LogitsArgs a) {
  typedef typename std::conditional<FP64, double, float>::type T;
  const int64_t b = (int64_t)blockIdx.x / a.nT;
  const int tile = (int)((int64_t)blockIdx.x - b * a.nT);
  const int64_t V = a.V;
  const float t = a.temp[b];
  const bool greedy = !(t > 0.0f);  // uniform across the workgroup
  const T inv_t = greedy ? T(1) : T(1) / T(t);
  const uint32_t rid = a.row_ids ? a.row_ids[b] : a.rid_base + (uint32_t)b;
  const float* x = a.X + b * V;
  const int64_t lo = (int64_t)tile * a.chunk;
  const int64_t hi = lo + a.chunk < V ? lo + a.chunk : V;

  T bm = neg_inf<T>();
  int32_t bi = kNoIndex;
  // Thread t takes the float4 groups t, t + 256, ... of the tile; kInFlight of
  // them are loaded before any is scored.
  constexpr int64_t kStride = 4 * kThreads;
  int64_t i0 = lo + 4 * (int64_t)threadIdx.x;
  if (a.vec4) {
    for (; i0 + kStride * (kInFlight - 1) < hi; i0 += kStride * kInFlight) {
      float4 v[kInFlight];
#pragma unroll
      for (int u = 0; u < kInFlight; ++u) v[u] = *reinterpret_cast<const float4*>(x + i0 + kStride * u);
#pragma unroll
      for (int u = 0; u < kInFlight; ++u)
        score4(a, greedy, inv_t, rid, i0 + kStride * u, hi, v[u].x, v[u].y, v[u].z, v[u].w, bm, bi);
    }
  }
  for (; i0 < hi; i0 += kStride) {
    float y[4];
    if (a.vec4) {  // hi is a multiple of 4 here
      const float4 v = *reinterpret_cast<const float4*>(x + i0);
      y[0] = v.x;
      y[1] = v.y;
      y[2] = v.z;
      y[3] = v.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = (i0 + j < hi) ? x[i0 + j] : neg_inf<float>();
    }
    score4(a, greedy, inv_t, rid, i0, hi, y[0], y[1], y[2], y[3], bm, bi);
  }

  wave_argmax_xor(bm, bi, 0);
  __shared__ Cand<T> wbest[kThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) wbest[wave] = Cand<T>{bm, bi};
  __syncthreads();
  if (threadIdx.x == 0) {
    Cand<T> best = wbest[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w)
      if (beats(wbest[w].m, wbest[w].idx, best.m, best.idx)) best = wbest[w];
    store_cand(reinterpret_cast<Cand<T>*>(a.cand) + b * a.nT + tile, best);
    wait_stores_complete();
  }

  // Stage 2 of this row, in the workgroup that finishes it last.
  if (!finish_last(a.counters + b, (uint32_t)a.nT)) return;
  if (wave == 0) {
    const int64_t o = row_winner(reinterpret_cast<const Cand<T>*>(a.cand) + b * a.nT, a.nT, lane);
    if (lane == 0) a.out[b] = o;
  }
  if (threadIdx.x == 0) clear_counter(a.counters + b);
}

}  // namespace

int logits_chunk(int64_t B, int64_t V) {
  constexpr int64_t kTargetWorkgroups = 2048;  // 8 per CU
  int64_t chunk = kLogitsChunk;
  while (chunk < kLogitsChunkMax && B * ((V + 2 * chunk - 1) / (2 * chunk)) >= kTargetWorkgroups)
    chunk *= 2;
  return (int)chunk;
}

hipError_t launch_logits_stage1(const LogitsArgs& a, bool fp64, hipStream_t stream) {
  const dim3 grid((unsigned)(a.B * a.nT));
  if (fp64)
    launch(logits_stage1_kernel<true>, grid, dim3(kThreads), 0, stream, a);
  else
    launch(logits_stage1_kernel<false>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fs
