// fs_filter.hip -- filtered exact sampling over materialised float32 logits
// for gfx950: the filter chain temperature -> top-k -> top-p -> min-p, then
// the Gumbel-argmax draw over the kept tokens (spec-decode-ops kernel card:
// its sample pipeline and "Semantics"; FlashSampling page, prerequisites).
//
// Every filter keeps a set {i : y_i >= threshold} (equal logits are kept or
// dropped together), so a row's kept set is one threshold on its logits plus
// the min-p test, and the draw needs no sort.  One workgroup per row:
//  1. the row's largest valid logit M;
//  2. a histogram of the valid logits in bins of 1/8 nat below M (by
//     z = (M - y) / t), with counts and probability masses; the masses
//     e = exp((y - M) / t) are 64-bit fixed-point integers in units of 2^-40,
//     so every sum is exact whatever order the threads add in.  From the bins
//     alone, each active filter bounds the bins its kept tokens can lie in;
//  3. if those bins hold at most kCap tokens, they are copied to LDS and
//     everything else happens there: the k-th largest logit (radix select
//     over an order-preserving 32-bit key, 8 bits a round), the top-p
//     threshold (the same descent weighted by the masses: the lowest logit
//     whose strictly larger top-k survivors carry less than p of their mass),
//     the min-p test (e >= min_p) and the draw;
//  4. otherwise (flat rows: more than kCap tokens within the bound) the same
//     selections run over the row itself, one pass per 8-bit round, and the
//     draw is one more pass.
// The draw uses the unfiltered sampler's scores, noise stream and tie rule,
// over the kept tokens only, so a row with every filter off draws exactly
// what the unfiltered sampler draws.
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

constexpr int kCap = 8192;               // candidate tokens a workgroup holds in LDS
constexpr float kBinsPerNat = 8.0f;      // z-histogram resolution
constexpr float kZTop = 255.0f / kBinsPerNat;  // bins 0..254 hold z < kZTop, bin 255 the rest

// The z-histogram bin of a valid logit: z = (M - y) * inv_t, bin floor(8 z)
// up to 254, 255 beyond (with M = +inf: 0 for the +inf logits, 255 for the
// others).  Non-decreasing as y decreases, so "bin <= b" is a set of the form
// {y >= threshold}.
__device__ __forceinline__ int z_bin(float y, float M, float inv_t) {
  if (M == __builtin_inff()) return y == M ? 0 : 255;
  const float z = (M - y) * inv_t;
  return z < kZTop ? (int)(z * kBinsPerNat) : 255;
}

// The key of the rest-th largest element (rest >= 1) of those `visit`
// enumerates: radix select, 8 bits a round, counts in an LDS histogram.
// visit(f) calls f(key, y) for every element; every thread calls this.
template <typename Visit>
__device__ uint32_t kth_largest_key(Visit&& visit, uint32_t rest, uint32_t* hcount,
                                    uint32_t* sel) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t prefix = 0u, mask = 0u;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hcount[tid] = 0u;
    __syncthreads();
    visit([&](uint32_t key, float) {
      if ((key & mask) == prefix) atomicAdd(&hcount[(key >> shift) & 255u], 1u);
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
          sel[0] = (uint32_t)(255 - 4 * lane - j);
          sel[1] = rest - before;
        }
        before += c[j];
      }
    }
    __syncthreads();
    prefix |= sel[0] << shift;
    mask |= 255u << shift;
    rest = sel[1];
  }
  return prefix;
}

// The key of the lowest class top-p keeps among the elements `visit`
// enumerates (the top-k survivors, or a set of the form {y >= threshold}
// holding them all): the lowest key whose strictly larger elements carry less
// than p * Z of mass.  Z is z_total, or, when z_total is 0, the mass of every
// element visited.  0 < p < 1.
template <typename Visit>
__device__ uint32_t top_p_key(Visit&& visit, float M, float inv_t, float p,
                              unsigned long long z_total, uint32_t* hcount,
                              unsigned long long* hmass, uint32_t* sel,
                              unsigned long long* sel_above) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t prefix = 0u, mask = 0u;
  unsigned long long above = 0ull;  // mass of the elements above the bucket
  double target = (double)p * (double)z_total;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) {
      hcount[tid] = 0u;
      hmass[tid] = 0ull;
    }
    __syncthreads();
    visit([&](uint32_t key, float y) {
      if ((key & mask) == prefix) {
        const uint32_t d = (key >> shift) & 255u;
        atomicAdd(&hcount[d], 1u);
        atomicAdd(&hmass[d], mass_fixed(mass_of(y, M, inv_t)));
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
      if (shift == 24 && z_total == 0ull) target = (double)p * (double)wave_sum(s);
      unsigned long long run = above + wave_exclusive_scan(s, lane);
      // The kept buckets are the non-empty ones whose mass above is below the
      // target; it grows downwards, so they form a prefix and the last of
      // them holds the threshold.
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
        sel[0] = (uint32_t)(255 - pos);
        *sel_above = at;
      }
    }
    __syncthreads();
    prefix |= sel[0] << shift;
    mask |= 255u << shift;
    above = *sel_above;
  }
  return prefix;
}

template <typename T>
__device__ __forceinline__ void wave_then_block_best(T& bm, int32_t& bi, Cand<T>* wbest) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  wave_argmax_xor(bm, bi, 0);
  if (lane == 0) wbest[wave] = Cand<T>{bm, bi};
  __syncthreads();
  Cand<T> best = wbest[0];
#pragma unroll
  for (int w = 1; w < kFWaves; ++w)
    if (beats(wbest[w].m, wbest[w].idx, best.m, best.idx)) best = wbest[w];
  bm = best.m;
  bi = best.idx;
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
  __shared__ uint32_t sel[2];
  __shared__ unsigned long long sel_above, z_all;
  __shared__ int bin_cut, bin_k;
  __shared__ uint32_t n_cut, n_cand;
  __shared__ float cval[kCap];
  __shared__ int32_t cidx[kCap];
  __shared__ Cand<T> wbest[kFWaves];

  T bm = neg_inf<T>();
  int32_t bi = kNoIndex;
  // The score of logit y at index i: the unfiltered sampler's arithmetic.
  auto score1 = [&](float y, int64_t i) -> T {
    if (greedy) return T(y);
    if constexpr (!FP64) {
      const Words w = noise_words(a.key, (uint32_t)(i >> 2), rid);
      const uint32_t q = i & 3;
      const uint32_t word = q == 0 ? w.w0 : (q == 1 ? w.w1 : (q == 2 ? w.w2 : w.w3));
      return T(y * (float)inv_t) + T(gumbel_f32(word));
    } else {
      const Words w = noise_words(a.key, (uint32_t)(i >> 1), rid);
      return (i & 1) ? T(y) * inv_t + T(gumbel_f64(w.w2, w.w3))
                     : T(y) * inv_t + T(gumbel_f64(w.w0, w.w1));
    }
  };

  uint32_t kappa = 0u;  // kept tokens: valid, key >= kappa, and the min-p test
  float M = neg_inf<float>();
  bool done = false;    // the draw was made over the LDS candidates
  if (use_k || use_p || use_m) {
    // 1. The largest valid logit and the number of valid logits.
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
  }
  if (use_k || use_p || use_m) {
    // 2. The z-histogram: counts and fixed-point masses per bin.
    if (tid < 256) {
      hcount[tid] = 0u;
      hmass[tid] = 0ull;
    }
    __syncthreads();
    for_row(x, V, vec4, [&](int64_t, const float (&y)[4]) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (valid_logit(y[j])) {
          const int bin = z_bin(y[j], M, inv_tf);
          atomicAdd(&hcount[bin], 1u);
          atomicAdd(&hmass[bin], mass_fixed(mass_of(y[j], M, inv_tf)));
        }
    });
    __syncthreads();
    if (wave == 0) {
      // Lane l holds bins 4l .. 4l + 3 (ascending z: descending logits).
      uint32_t c[4], cs = 0;
      unsigned long long w[4], ws = 0ull;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hcount[4 * lane + j];
        w[j] = hmass[4 * lane + j];
        cs += c[j];
        ws += w[j];
      }
      const uint32_t c0 = wave_exclusive_scan(cs, lane);
      const unsigned long long w0 = wave_exclusive_scan(ws, lane);
      const unsigned long long z_total = wave_sum(ws);
      // Top-k: the bin of the k-th largest logit, and the mass of the bins
      // above it and including it (bounds of the top-k survivors' mass).
      int bk = 255;
      unsigned long long zk_hi = z_total;
      if (use_k) {
        uint32_t cc = c0;
        unsigned long long ww = w0;
        int mine = 256;
        unsigned long long hi = 0ull;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          cc += c[j];
          ww += w[j];
          if (mine == 256 && cc >= (uint32_t)top_k) {
            mine = 4 * lane + j;
            hi = ww;
          }
        }
        int first = mine;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) first = min(first, __shfl_xor(first, o));
        bk = first;
        // the lane holding bin bk supplies the mass up to and including it
        const int src = bk >> 2;
        zk_hi = __shfl(hi, src);
      }
      // Top-p: no kept token lies below the first bin whose cumulative mass
      // reaches p times the largest the survivors' mass can be.
      int bp = 255;
      if (use_p) {
        if (!(top_p > 0.0f)) {
          bp = 0;
        } else {
          const double target = (double)top_p * (double)zk_hi;
          unsigned long long ww = w0;
          int mine = 256;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            ww += w[j];
            if (mine == 256 && (double)ww >= target) mine = 4 * lane + j;
          }
          int first = mine;
#pragma unroll
          for (int o = 32; o >= 1; o >>= 1) first = min(first, __shfl_xor(first, o));
          bp = first > 255 ? 255 : first;
        }
      }
      // Min-p: e >= m needs z <= -ln m (with a margin for the float32 exp).
      int bmn = 255;
      if (use_m) {
        if (!(min_p < 1.0f)) {
          bmn = 0;
        } else {
          const double zmax = -log((double)min_p) * (1.0 + 1e-5) + 1e-5;
          bmn = zmax < (double)kZTop ? (int)(zmax * kBinsPerNat) : 255;
        }
      }
      // Every kept token lies in bins 0 .. min(bk, bp, bmn).  The candidates
      // are those bins, and with top-k and top-p both on every bin up to bk:
      // top-p then needs the survivors' exact mass, so the k-th largest logit
      // exactly.  (Without top-p a cut above bk leaves top-k nothing to do.)
      int cut = bk < bp ? bk : bp;
      cut = cut < bmn ? cut : bmn;
      if (use_k && use_p) cut = bk;
      // tokens in bins 0 .. cut
      uint32_t cc = c0, mine = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        cc += c[j];
        if (4 * lane + j == cut) mine = cc;
      }
      const uint32_t ncut = __shfl(mine, cut >> 2);
      if (lane == 0) {
        bin_cut = cut;
        bin_k = bk;
        n_cut = ncut;
        z_all = z_total;
        n_cand = 0u;
      }
    }
    __syncthreads();
    const int cut = bin_cut;
    const unsigned long long z_total = z_all;
    if (n_cut <= (uint32_t)kCap) {
      // 3. The candidates (every token that can be kept) into LDS.
      for_row(x, V, vec4, [&](int64_t i0, const float (&y)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (valid_logit(y[j]) && z_bin(y[j], M, inv_tf) <= cut) {
            const uint32_t q = atomicAdd(&n_cand, 1u);
            if (q < (uint32_t)kCap) {
              cval[q] = y[j];
              cidx[q] = (int32_t)(i0 + j);
            }
          }
      });
      __syncthreads();
      const int n = (int)(n_cand < (uint32_t)kCap ? n_cand : (uint32_t)kCap);
      auto visit_all = [&](auto&& f) {
        for (int q = tid; q < n; q += kFThreads) f(order_key(cval[q]), cval[q]);
      };
      // Top-k binds only when the candidates reach its bin; then they hold
      // every logit down to the k-th largest.
      uint32_t key_k = 0u, key_p = 0u;
      if (use_k && cut == bin_k)
        key_k = kth_largest_key(visit_all, (uint32_t)top_k, hcount, sel);
      if (use_p) {
        if (!(top_p > 0.0f)) {
          key_p = order_key(M);
        } else {
          auto visit_s1 = [&](auto&& f) {
            for (int q = tid; q < n; q += kFThreads) {
              const uint32_t key = order_key(cval[q]);
              if (key >= key_k) f(key, cval[q]);
            }
          };
          // Without top-k the survivors are every valid token: their mass is
          // the histogram's total; with it they are all among the candidates.
          key_p = top_p_key(visit_s1, M, inv_tf, top_p, use_k ? 0ull : z_total, hcount, hmass,
                            sel, &sel_above);
        }
      }
      kappa = key_k > key_p ? key_k : key_p;
      if (use_m && !(min_p < 1.0f)) {
        const uint32_t km = order_key(M);
        kappa = kappa > km ? kappa : km;
        use_m = false;
      }
      // The draw over the kept candidates.
      for (int q = tid; q < n; q += kFThreads) {
        const float y = cval[q];
        if (order_key(y) < kappa || (use_m && !(mass_of(y, M, inv_tf) >= min_p))) continue;
        const int32_t i = cidx[q];
        const T s = score1(y, i);
        if (beats(s, i, bm, bi)) {
          bm = s;
          bi = i;
        }
      }
      done = true;
    } else {
      // 4. Too many candidates: the same selections over the row.
      auto visit_row = [&](auto&& f) {
        for_row(x, V, vec4, [&](int64_t, const float (&y)[4]) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (valid_logit(y[j])) f(order_key(y[j]), y[j]);
        });
      };
      uint32_t key_k = 0u, key_p = 0u;
      if (use_k) key_k = kth_largest_key(visit_row, (uint32_t)top_k, hcount, sel);
      if (use_p) {
        if (!(top_p > 0.0f)) {
          key_p = order_key(M);
        } else {
          auto visit_s1 = [&](auto&& f) {
            for_row(x, V, vec4, [&](int64_t, const float (&y)[4]) {
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const uint32_t key = order_key(y[j]);
                if (valid_logit(y[j]) && key >= key_k) f(key, y[j]);
              }
            });
          };
          key_p = top_p_key(visit_s1, M, inv_tf, top_p, use_k ? 0ull : z_total, hcount, hmass,
                            sel, &sel_above);
        }
      }
      kappa = key_k > key_p ? key_k : key_p;
      if (use_m && !(min_p < 1.0f)) {
        const uint32_t km = order_key(M);
        kappa = kappa > km ? kappa : km;
        use_m = false;
      }
    }
  }

  if (!done) {
    // The draw over the row: every valid token with key >= kappa that passes
    // the min-p test (every valid token when no filter is on).
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
  }
  wave_then_block_best(bm, bi, wbest);
  if (tid == 0) a.out[b] = bm == neg_inf<T>() ? (int64_t)-1 : (int64_t)bi;
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
