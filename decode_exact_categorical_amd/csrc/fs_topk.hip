// fs_topk.hip -- Gumbel-top-k over materialised float32 logits for gfx950:
// k draws without replacement per row, the k largest perturbed scores
// (FlashSampling page, "limitations" and future work, which names the top-k
// extension; the noise, transform and tie rule are the single sampler's).
//
// Same split as the single sampler (fs_logits.hip): each workgroup reduces a
// chunk of a row to its kTopKMax best (score, index) places and the last to
// finish runs Stage 2 over the row's chunks.
//  * Every thread keeps its own sorted list of kTopKMax places in registers
//    (its logits arrive in increasing index order, so a strict compare keeps
//    the smaller index first on equal scores).
//  * The workgroup's lists go through LDS to one wave, which picks the
//    chunk's places one after the other: each lane offers its best candidate
//    after the previous place, the wave takes the best offer.
//  * Stage 2 does the same over the row's chunks, reading the published
//    candidates a slice at a time.
#include <type_traits>

#include "fs_launch.hpp"

namespace fs {
namespace {

constexpr int kThreads = 256;
constexpr int kK = kTopKMax;

template <bool FP64>
__global__ __launch_bounds__(kThreads) void logits_topk_kernel(LogitsArgs a) {
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

  T lm[kK];
  int32_t li[kK];
#pragma unroll
  for (int j = 0; j < kK; ++j) {
    lm[j] = neg_inf<T>();
    li[j] = kNoIndex;
  }
  // Thread t takes the 4-logit groups t, t + 256, ... of the chunk.
  constexpr int64_t kStride = 4 * kThreads;
  for (int64_t i0 = lo + 4 * (int64_t)threadIdx.x; i0 < hi; i0 += kStride) {
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
    T s[4];
    if (greedy) {
#pragma unroll
      for (int j = 0; j < 4; ++j) s[j] = T(y[j]);
    } else if constexpr (!FP64) {
      const Words w = noise_words(a.key, (uint32_t)(i0 >> 2), rid);
      s[0] = T(y[0] * (float)inv_t) + T(gumbel_f32(w.w0));
      s[1] = T(y[1] * (float)inv_t) + T(gumbel_f32(w.w1));
      s[2] = T(y[2] * (float)inv_t) + T(gumbel_f32(w.w2));
      s[3] = T(y[3] * (float)inv_t) + T(gumbel_f32(w.w3));
    } else {
      const Words w0 = noise_words(a.key, (uint32_t)(i0 >> 1), rid);
      const Words w1 = noise_words(a.key, (uint32_t)(i0 >> 1) + 1u, rid);
      s[0] = T(y[0]) * inv_t + T(gumbel_f64(w0.w0, w0.w1));
      s[1] = T(y[1]) * inv_t + T(gumbel_f64(w0.w2, w0.w3));
      s[2] = T(y[2]) * inv_t + T(gumbel_f64(w1.w0, w1.w1));
      s[3] = T(y[3]) * inv_t + T(gumbel_f64(w1.w2, w1.w3));
    }
    // Entries past the chunk enter as -inf, which never takes a place.
#pragma unroll
    for (int j = 0; j < 4; ++j)
      topk_insert(lm, li, i0 + j < hi ? s[j] : neg_inf<T>(), (int32_t)(i0 + j));
  }

  // The chunk's places: every thread's list through LDS to wave 0.
  __shared__ Cand<T> lists[kK][kThreads];
#pragma unroll
  for (int j = 0; j < kK; ++j) lists[j][threadIdx.x] = Cand<T>{lm[j], li[j]};
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  Cand<T>* out_c = reinterpret_cast<Cand<T>*>(a.cand) + (b * a.nT + tile) * kK;
  if (wave == 0) {
    Cand<T> c[kK * kThreads / 64];
#pragma unroll
    for (int q = 0; q < kThreads / 64; ++q)
#pragma unroll
      for (int j = 0; j < kK; ++j) c[q * kK + j] = lists[j][lane + 64 * q];
    Cand<T> p = Cand<T>{neg_inf<T>(), kNoIndex};
#pragma unroll 1
    for (int r = 0; r < kK; ++r) {
      p = next_place(c, r == 0, p.m, p.idx);
      if (lane == 0) store_cand(out_c + r, p);
    }
    if (lane == 0) wait_stores_complete();
  }

  // Stage 2 of this row, in the workgroup that finishes it last: wave 0 picks
  // the row's k places among its nT * kTopKMax candidates, 64 per lane at a
  // time per round.
  if (!finish_last(a.counters + b, (uint32_t)a.nT)) return;
  if (wave == 0) {
    const Cand<T>* rc = reinterpret_cast<const Cand<T>*>(a.cand) + b * a.nT * kK;
    const int n = a.nT * kK;
    T pm = neg_inf<T>();
    int32_t pi = kNoIndex;
#pragma unroll 1
    for (int r = 0; r < a.k; ++r) {
      T bm = neg_inf<T>();
      int32_t bi = kNoIndex;
#pragma unroll 1
      for (int base = 0; base < n; base += 64 * 8) {
        Cand<T> c[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int e = base + lane + 64 * q;
          c[q] = load_cand(rc + (e < n ? e : n - 1));
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const bool take = (base + lane + 64 * q < n) & ((r == 0) | after(c[q].m, c[q].idx, pm, pi)) &
                            beats_nb(c[q].m, c[q].idx, bm, bi);
          bm = take ? c[q].m : bm;
          bi = take ? c[q].idx : bi;
        }
      }
      wave_argmax_xor(bm, bi, 0);
      if (lane == 0) a.out[b * a.k + r] = bm == neg_inf<T>() ? (int64_t)-1 : (int64_t)bi;
      pm = bm;
      pi = bi;
    }
  }
  if (threadIdx.x == 0) clear_counter(a.counters + b);
}

}  // namespace

hipError_t launch_logits_topk(const LogitsArgs& a, bool fp64, hipStream_t stream) {
  const dim3 grid((unsigned)(a.B * a.nT));
  if (fp64)
    launch(logits_topk_kernel<true>, grid, dim3(kThreads), 0, stream, a);
  else
    launch(logits_topk_kernel<false>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fs
