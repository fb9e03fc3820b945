// fs_filter.hip -- filtered exact sampling over materialised float32 logits
// for gfx950: the filter chain temperature -> top-k -> top-p -> min-p, then
// the Gumbel-argmax draw over the kept tokens (spec-decode-ops kernel card:
// its sample pipeline and "Semantics"; FlashSampling page, prerequisites).
//
// Every filter keeps a set {i : y_i >= threshold} (equal logits are kept or
// dropped together), so a row's kept set is one threshold on its logits plus
// the min-p test, and the draw needs no sort:
//  * one workgroup per row, which re-reads its row (from L2) once a pass;
//  * top-k: the k-th largest valid logit, by radix select over an
//    order-preserving 32-bit key of the float, 8 bits a pass, with the counts
//    in an LDS histogram;
//  * top-p: the same descent weighted by the probability masses
//    e_i = exp((y_i - M) * (1/t)) of the top-k survivors (M the row's largest
//    valid logit), held as 64-bit fixed-point integers in units of 2^-40, so
//    every sum is exact whatever order the threads add in, and the threshold
//    is the lowest logit whose strictly larger survivors carry less than
//    p times the survivors' total mass;
//  * min-p: e_i >= min_p, tested token by token in the draw;
//  * the draw: the unfiltered sampler's scores, noise stream and tie rule,
//    over the kept tokens only, so a row with every filter off draws exactly
//    what the unfiltered sampler draws.
#include <type_traits>

#include "fs_launch.hpp"

namespace fs {
namespace {

constexpr int kFThreads = 512;
constexpr int kFWaves = kFThreads / 64;
constexpr float kMassUnit = 0x1p40f;  // fixed-point scale of the masses

// Larger floats have larger keys (NaN is never keyed: it is never kept).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ bool valid_logit(float y) { return y == y && y != neg_inf<float>(); }

// Probability mass of a valid logit relative to the row's largest valid logit
// M (unnormalised): exp((y - M) * inv_t); with M = +inf, 1 on the +inf logits
// and 0 on the others.  Every pass computes it with these same instructions.
__device__ __forceinline__ float mass_of(float y, float M, float inv_t) {
  if (M == __builtin_inff()) return y == M ? 1.0f : 0.0f;
  return expf((y - M) * inv_t);
}

__device__ __forceinline__ unsigned long long mass_fixed(float e) {
  return (unsigned long long)(e * kMassUnit);
}

// The row's logits, 4 at a time in increasing index order per thread:
// f(i0, y[4]) with entries at or past V set to -inf (never valid).
template <typename F>
__device__ __forceinline__ void for_row(const float* x, int64_t V, bool vec4, F&& f) {
  constexpr int64_t kStride = 4 * kFThreads;
  int64_t i0 = 4 * (int64_t)threadIdx.x;
  if (vec4) {  // V % 4 == 0, rows 16-byte aligned
    for (; i0 + kStride < V; i0 += 2 * kStride) {
      const float4 u = *reinterpret_cast<const float4*>(x + i0);
      const float4 v = *reinterpret_cast<const float4*>(x + i0 + kStride);
      const float yu[4] = {u.x, u.y, u.z, u.w};
      const float yv[4] = {v.x, v.y, v.z, v.w};
      f(i0, yu);
      f(i0 + kStride, yv);
    }
  }
  for (; i0 < V; i0 += kStride) {
    float y[4];
    if (vec4) {
      const float4 u = *reinterpret_cast<const float4*>(x + i0);
      y[0] = u.x;
      y[1] = u.y;
      y[2] = u.z;
      y[3] = u.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = i0 + j < V ? x[i0 + j] : neg_inf<float>();
    }
    f(i0, y);
  }
}

template <typename U>
__device__ __forceinline__ U wave_sum(U v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Exclusive prefix sum over the lanes of a wave (lane order).
template <typename U>
__device__ __forceinline__ U wave_exclusive_scan(U v, int lane) {
  U inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const U n = __shfl_up(inc, o);
    if (lane >= o) inc += n;
  }
  return inc - v;
}

template <bool FP64>
__global__ __launch_bounds__(kFThreads) void logits_filtered_kernel(FilterArgs a) {
  typedef typename std::conditional<FP64, double, float>::type T;
  const int64_t b = blockIdx.x;
  const int64_t V = a.V;
  const float* x = a.X + b * V;
  const bool vec4 = a.vec4 != 0;
  const float t = a.temp[b];
  const bool greedy = !(t > 0.0f);  // uniform across the workgroup
  const T inv_t = greedy ? T(1) : T(1) / T(t);
  const float inv_tf = greedy ? 1.0f : 1.0f / t;
  const uint32_t rid = a.row_ids ? a.row_ids[b] : (uint32_t)b;
  const int32_t top_k = a.top_k ? a.top_k[b] : 0;
  const float top_p = a.top_p ? a.top_p[b] : 1.0f;
  const float min_p = a.min_p ? a.min_p[b] : 0.0f;
  // NaN parameters compare false: their filters are off.
  bool use_k = !greedy && top_k > 0;
  bool use_p = !greedy && top_p < 1.0f;
  bool use_m = !greedy && min_p > 0.0f;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  __shared__ uint32_t hcount[256];
  __shared__ unsigned long long hmass[256];
  __shared__ float red_f[kFWaves];
  __shared__ uint32_t red_u[kFWaves];
  __shared__ uint32_t sel_digit, sel_rest;
  __shared__ unsigned long long sel_above;

  uint32_t kappa = 0u;  // kept tokens: valid, key >= kappa (and the min-p test)
  float M = neg_inf<float>();
  if (use_k || use_p || use_m) {
    // The largest valid logit and the number of valid logits.
    float lm = neg_inf<float>();
    uint32_t nv = 0;
    for_row(x, V, vec4, [&](int64_t, const float (&y)[4]) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (valid_logit(y[j])) {
          lm = fmaxf(lm, y[j]);
          ++nv;
        }
    });
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) lm = fmaxf(lm, __shfl_xor(lm, o));
    nv = wave_sum(nv);
    if (lane == 0) {
      red_f[wave] = lm;
      red_u[wave] = nv;
    }
    __syncthreads();
    uint32_t n_valid = 0;
#pragma unroll
    for (int w = 0; w < kFWaves; ++w) {
      M = fmaxf(M, red_f[w]);
      n_valid += red_u[w];
    }
    if (n_valid == 0) use_k = use_p = use_m = false;  // nothing to keep
    if ((int64_t)top_k >= (int64_t)n_valid) use_k = false;

    // Top-k: the key of the k-th largest valid logit, 8 bits a pass.
    uint32_t key_k = 0u;
    if (use_k) {
      uint32_t prefix = 0u, mask = 0u, rest = (uint32_t)top_k;
      for (int shift = 24; shift >= 0; shift -= 8) {
        if (tid < 256) hcount[tid] = 0u;
        __syncthreads();
        for_row(x, V, vec4, [&](int64_t, const float (&y)[4]) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t key = order_key(y[j]);
            if (valid_logit(y[j]) && (key & mask) == prefix)
              atomicAdd(&hcount[(key >> shift) & 255u], 1u);
          }
        });
        __syncthreads();
        if (wave == 0) {
          // Lane l holds digits 255 - 4l - j, j < 4: lane order is descending.
          uint32_t c[4], s = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            c[j] = hcount[255 - 4 * lane - j];
            s += c[j];
          }
          uint32_t before = wave_exclusive_scan(s, lane);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (before < rest && rest <= before + c[j]) {
              sel_digit = (uint32_t)(255 - 4 * lane - j);
              sel_rest = rest - before;
            }
            before += c[j];
          }
        }
        __syncthreads();
        prefix |= sel_digit << shift;
        mask |= 255u << shift;
        rest = sel_rest;
      }
      key_k = prefix;
    }

    // Top-p over the top-k survivors: the key of the lowest kept logit.
    uint32_t key_p = 0u;
    if (use_p) {
      if (!(top_p > 0.0f)) {
        key_p = order_key(M);  // keeps nothing: the largest logit's tie class
      } else {
        uint32_t prefix = 0u, mask = 0u;
        unsigned long long above = 0ull;  // mass of the survivors above the bucket
        double target = 0.0;
        for (int shift = 24; shift >= 0; shift -= 8) {
          if (tid < 256) {
            hcount[tid] = 0u;
            hmass[tid] = 0ull;
          }
          __syncthreads();
          for_row(x, V, vec4, [&](int64_t, const float (&y)[4]) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint32_t key = order_key(y[j]);
              if (valid_logit(y[j]) && key >= key_k && (key & mask) == prefix) {
                const uint32_t d = (key >> shift) & 255u;
                atomicAdd(&hcount[d], 1u);
                atomicAdd(&hmass[d], mass_fixed(mass_of(y[j], M, inv_tf)));
              }
            }
          });
          __syncthreads();
          if (wave == 0) {
            uint32_t c[4];
            unsigned long long w[4], s = 0ull;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              c[j] = hcount[255 - 4 * lane - j];
              w[j] = hmass[255 - 4 * lane - j];
              s += w[j];
            }
            // The first pass sees every survivor: its total is the mass Z.
            if (shift == 24) target = (double)top_p * (double)wave_sum(s);
            unsigned long long run = above + wave_exclusive_scan(s, lane);
            // The kept buckets are the non-empty ones whose mass above is
            // below the target; it grows downwards, so they form a prefix and
            // the last of them holds the threshold.
            int pos = -1;
            unsigned long long at = 0ull;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              if (c[j] > 0u && (double)run < target) {
                pos = 4 * lane + j;
                at = run;
              }
              run += w[j];
            }
            int best = pos;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) best = max(best, __shfl_xor(best, o));
            if (pos == best && pos >= 0) {
              sel_digit = (uint32_t)(255 - pos);
              sel_above = at;
            }
          }
          __syncthreads();
          prefix |= sel_digit << shift;
          mask |= 255u << shift;
          above = sel_above;
        }
        key_p = prefix;
      }
    }
    kappa = key_k > key_p ? key_k : key_p;
    // min-p at or above 1 keeps the largest logit's tie class only.
    if (use_m && !(min_p < 1.0f)) {
      const uint32_t km = order_key(M);
      kappa = kappa > km ? kappa : km;
      use_m = false;
    }
  }

  // The draw over the kept tokens: the unfiltered sampler's scores.
  T bm = neg_inf<T>();
  int32_t bi = kNoIndex;
  for_row(x, V, vec4, [&](int64_t i0, const float (&y)[4]) {
    bool keep[4];
    bool any = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      keep[j] = valid_logit(y[j]) && order_key(y[j]) >= kappa &&
                (!use_m || mass_of(y[j], M, inv_tf) >= min_p);
      any |= keep[j];
    }
    if (!any) return;
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
    // Increasing index order per thread: only a strictly larger score takes
    // over (equal scores keep the smaller index; NaN never takes over).
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (keep[j] && s[j] > bm) {
        bm = s[j];
        bi = (int32_t)(i0 + j);
      }
  });
  wave_argmax_xor(bm, bi, 0);
  __shared__ Cand<T> wbest[kFWaves];
  if (lane == 0) wbest[wave] = Cand<T>{bm, bi};
  __syncthreads();
  if (tid == 0) {
    Cand<T> best = wbest[0];
#pragma unroll
    for (int w = 1; w < kFWaves; ++w)
      if (beats(wbest[w].m, wbest[w].idx, best.m, best.idx)) best = wbest[w];
    a.out[b] = best.m == neg_inf<T>() ? (int64_t)-1 : (int64_t)best.idx;
  }
}

}  // namespace

hipError_t launch_logits_filtered(const FilterArgs& a, bool fp64, hipStream_t stream) {
  const dim3 grid((unsigned)a.B);
  if (fp64)
    hipLaunchKernelGGL(logits_filtered_kernel<true>, grid, dim3(kFThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(logits_filtered_kernel<false>, grid, dim3(kFThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fs
