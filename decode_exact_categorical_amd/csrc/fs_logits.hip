// fs_logits.hip -- standalone exact sampler over materialised float32 logits,
// Stage 1, for gfx950.
//
// The Megatron-LM "fp64 sampling noise" page ("Cost") notes that its sampler
// materialises the noise and the ratio p/E in HBM, and that one program per
// row is latency-bound at small batch.  Here the noise is generated in
// registers and each row is split over ceil(V / chunk) workgroups, each
// reducing `chunk` logits to one (score, index) candidate; the last of them
// to finish runs Stage 2, picking the row's winner (finish_last, row_winner
// in fs_device.hpp).  The chunk (2048 to 131072 logits) is the largest that
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

// Upper bound of the Gumbel noise of every uniform whose word (float32 noise)
// or high word (float64 noise) has top 8 bits b: g = -log(-log u) increases
// with u, so every u of the bin lies at or below the bin's largest grid point
// u_b, and g(u_b) plus a margin far above the transforms' pinned error (a few
// 1e-7 relative) bounds the g the kernel computes there.  Rounded up to float.
template <bool FP64>
__device__ float gumbel_bin_bound(int b) {
  // fp32: k = top 23 bits, bin b holds k in [b 2^15, (b + 1) 2^15), u = (2k + 1) / 2^24;
  // fp64: k = top 52 bits, bin b holds k in [b 2^44, (b + 1) 2^44), u = (2k + 1) / 2^53.
  const double top = FP64 ? ((double)(b + 1) * 0x1p44 - 1.0) : ((double)(b + 1) * 0x1p15 - 1.0);
  const double umax = (2.0 * top + 1.0) * (FP64 ? 0x1p-53 : 0x1p-24);
  const double g = -log(-log(umax));
  const double m = g + 1e-5 * fmax(1.0, fabs(g));
  float f = (float)m;
  if ((double)f < m) f = nextafterf(f, __builtin_inff());
  return f;
}

// Bound-then-refine: a logit whose score cannot reach the best score already
// found in this workgroup's wave (y / t plus its noise bound falls strictly
// below it) is skipped; one whose bound reaches it goes to a per-wave queue in
// LDS, and 64 queued logits at a time (one a lane, the wave fully busy) get
// their exact noise and are scored.  Skipping needs a score at least as large
// as one the chunk holds, so the chunk's best (score, index) is the one the
// exhaustive scan finds; the queue's order does not matter (the candidate
// order is total).  Groups of 4 logits whose bound with the largest noise of
// all falls below it skip the Philox call too.
template <bool FP64>
struct RefineQueue {
  typedef typename std::conditional<FP64, double, float>::type T;
  static constexpr int kCap = 128;
  int32_t idx[kThreads / 64][kCap];
  T base[kThreads / 64][kCap];
  uint32_t w0[kThreads / 64][kCap];
  uint32_t w1[kThreads / 64][FP64 ? kCap : 1];
};

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
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  T bm = neg_inf<T>();
  int32_t bi = kNoIndex;
  // Thread t takes the float4 groups t, t + 256, ... of the tile; kInFlight of
  // them are loaded before any is scored.
  constexpr int64_t kStride = 4 * kThreads;
  int64_t i0 = lo + 4 * (int64_t)threadIdx.x;
  if (greedy) {
    if (a.vec4) {
      for (; i0 + kStride * (kInFlight - 1) < hi; i0 += kStride * kInFlight) {
        float4 v[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) v[u] = *reinterpret_cast<const float4*>(x + i0 + kStride * u);
#pragma unroll
        for (int u = 0; u < kInFlight; ++u)
          score4(a, true, inv_t, rid, i0 + kStride * u, hi, v[u].x, v[u].y, v[u].z, v[u].w, bm, bi);
      }
    }
    for (; i0 < hi; i0 += kStride) {
      float y[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = (i0 + j < hi) ? x[i0 + j] : neg_inf<float>();
      score4(a, true, inv_t, rid, i0, hi, y[0], y[1], y[2], y[3], bm, bi);
    }
  } else {
    __shared__ float gup[256];
    __shared__ RefineQueue<FP64> q;
    gup[threadIdx.x] = gumbel_bin_bound<FP64>((int)threadIdx.x);
    __syncthreads();
    const T gmax = T(gup[255]);
    T thr = neg_inf<T>();  // the best score this wave has found
    int count = 0;          // queued logits of this wave (uniform)
    // Score the queue's first n entries (n <= 64), one a lane, and move the
    // rest to its front; then share the wave's best.
    auto flush = [&](int n) {
      if (lane < n) {
        const T base = q.base[wave][lane];
        const int32_t i = q.idx[wave][lane];
        T g;
        if constexpr (FP64)
          g = T(gumbel_f64(q.w0[wave][lane], q.w1[wave][lane]));
        else
          g = T(gumbel_f32(q.w0[wave][lane]));
        const T sc = base + g;
        if (sc > neg_inf<T>() && beats(sc, i, bm, bi)) {
          bm = sc;
          bi = i;
        }
      }
      const int rest = count - n;
      if (lane < rest) {
        const int32_t i = q.idx[wave][n + lane];
        const T base = q.base[wave][n + lane];
        const uint32_t u0 = q.w0[wave][n + lane];
        uint32_t u1 = 0;
        if constexpr (FP64) u1 = q.w1[wave][n + lane];
        q.idx[wave][lane] = i;
        q.base[wave][lane] = base;
        q.w0[wave][lane] = u0;
        if constexpr (FP64) q.w1[wave][lane] = u1;
      }
      count = rest;
      T m = bm;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const T om = __shfl_xor(m, o);
        m = om > m ? om : m;
      }
      thr = m;
    };
    // Queue logit i0 + j of this lane when `want`.
    auto push = [&](bool want, int32_t i, T base, uint32_t u0, uint32_t u1) {
      const uint64_t mask = __builtin_amdgcn_ballot_w64(want);
      if (mask == 0) return;
      if (want) {
        const int pos = count + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
        q.idx[wave][pos] = i;
        q.base[wave][pos] = base;
        q.w0[wave][pos] = u0;
        if constexpr (FP64) q.w1[wave][pos] = u1;
      }
      count += __builtin_popcountll(mask);
      if (count >= 64) flush(64);
    };
    auto group = [&](int64_t g0, float y0, float y1, float y2, float y3) {
      const float yv[4] = {y0, y1, y2, y3};
      T base[4];
      bool any = false;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        base[j] = FP64 ? T(yv[j]) * inv_t : T(yv[j] * (float)inv_t);
        // (NaN bases compare false and are queued: they are scored, never kept)
        any |= (g0 + j < hi) & !(base[j] + gmax < thr);
      }
      if (__builtin_amdgcn_ballot_w64(any) == 0) return;
      uint32_t u0[4], u1[4];
      if constexpr (FP64) {
        const Words wa = noise_words(a.key, (uint32_t)(g0 >> 1), rid);
        const Words wb = noise_words(a.key, (uint32_t)(g0 >> 1) + 1u, rid);
        u0[0] = wa.w0; u1[0] = wa.w1; u0[1] = wa.w2; u1[1] = wa.w3;
        u0[2] = wb.w0; u1[2] = wb.w1; u0[3] = wb.w2; u1[3] = wb.w3;
      } else {
        const Words w = noise_words(a.key, (uint32_t)(g0 >> 2), rid);
        u0[0] = w.w0; u0[1] = w.w1; u0[2] = w.w2; u0[3] = w.w3;
#pragma unroll
        for (int j = 0; j < 4; ++j) u1[j] = 0;
      }
      bool want[4];
      bool some = false;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        want[j] = (g0 + j < hi) & any & !(base[j] + T(gup[u0[j] >> 24]) < thr);
        some |= want[j];
      }
      if (__builtin_amdgcn_ballot_w64(some) == 0) return;
#pragma unroll
      for (int j = 0; j < 4; ++j) push(want[j], (int32_t)(g0 + j), base[j], u0[j], u1[j]);
    };
    // Every lane of a wave runs the same iterations (the queue is per wave):
    // the loops run on the wave's first group, w0, and end on its last lane.
    int64_t w0 = lo + 4 * (int64_t)(64 * wave);
    if (a.vec4) {
      for (; w0 + 4 * 63 + 3 + kStride * (kInFlight - 1) < hi; w0 += kStride * kInFlight) {
        const int64_t g0 = w0 + 4 * lane;
        float4 v[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) v[u] = *reinterpret_cast<const float4*>(x + g0 + kStride * u);
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) group(g0 + kStride * u, v[u].x, v[u].y, v[u].z, v[u].w);
      }
    }
    // The tail, element by element: lanes past hi take no part (group masks
    // them).
    for (; w0 < hi; w0 += kStride) {
      const int64_t g0 = w0 + 4 * lane;
      float y[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = (g0 + j < hi) ? x[g0 + j] : neg_inf<float>();
      group(g0, y[0], y[1], y[2], y[3]);
    }
    if (count > 0) flush(count);
  }

  wave_argmax_xor(bm, bi, 0);
  __shared__ Cand<T> wbest[kThreads / 64];
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

namespace {
// The largest chunk (kLogitsChunk 2^k <= kLogitsChunkMax) that leaves at least
// `target` workgroups.
int64_t largest_chunk(int64_t B, int64_t V, int64_t target) {
  int64_t chunk = kLogitsChunk;
  while (chunk < kLogitsChunkMax && B * ((V + 2 * chunk - 1) / (2 * chunk)) >= target) chunk *= 2;
  return chunk;
}
}  // namespace

int logits_chunk(int64_t B, int64_t V) {
  return (int)largest_chunk(B, V, 2048);  // 8 workgroups per CU
}

int logits_sample_chunk(int64_t B, int64_t V) {
  // Longer chunks let a wave's running best skip more transforms (bound then
  // refine); more workgroups hide more latency.  Measured at V = 131072: the
  // largest chunk that leaves 1024 workgroups (4 a CU), unless that chunk is
  // under 32768 logits (B < 256), where the largest that leaves 512 is
  // faster (float32 noise, us: B = 64 29 -> 21, B = 128 38 -> 33, B = 256 71
  // -> 50, B = 512 -> 75, B = 4096 unchanged).
  int64_t chunk = largest_chunk(B, V, 1024);
  if (chunk < 32768) chunk = largest_chunk(B, V, 512);
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
