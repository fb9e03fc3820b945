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

// Threads of a workgroup (the most; arrays are sized for it).  The split
// kernel always runs 16 waves.  The one-row-per-workgroup kernels run 16 waves
// while the rows do not fill the chip: a row's passes are VALU-bound on its one
// CU (exp2 for the masses, Philox and the Gumbel transform for the draw), and
// four waves a SIMD hide the transcendental latency that two do not (measured
// 97.6 -> 76.3 us at B = 64, V = 151936, top-k 50 + top-p 0.95).  With more
// rows than CUs they run 8 waves, two rows a CU, whose serial phases then
// overlap each other's streaming (953 against 1140 us at 4096 x 131072).
// The row helpers below take the thread count from blockDim.
constexpr int kFThreads = 1024;
constexpr int kFWaves = kFThreads / 64;
constexpr int kRowThreadsWide = 512;  // one-row kernels when B exceeds kRowsNarrow
constexpr int64_t kRowsNarrow = 256;  // rows up to about one per CU
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
// f(i0, y[4]) with entries at or past V set to -inf (never valid).  One
// workgroup streams a whole row, so each thread keeps kRowInFlight 16-byte
// loads in flight (a pass is bound by load latency, not bandwidth).
constexpr int kRowInFlight = 8;
template <typename F>
__device__ __forceinline__ void for_row(const float* x, int64_t V, bool vec4, F&& f) {
  const int64_t kStride = 4 * (int64_t)blockDim.x;
  int64_t i0 = 4 * (int64_t)threadIdx.x;
  if (vec4) {  // V % 4 == 0, rows 16-byte aligned
    for (; i0 + (kRowInFlight - 1) * kStride < V; i0 += kRowInFlight * kStride) {
      float4 v[kRowInFlight];
#pragma unroll
      for (int u = 0; u < kRowInFlight; ++u) v[u] = *reinterpret_cast<const float4*>(x + i0 + u * kStride);
#pragma unroll
      for (int u = 0; u < kRowInFlight; ++u) {
        const float y[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        f(i0 + u * kStride, y);
      }
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

constexpr int kCap = 8192;               // candidates of the one-workgroup-per-row kernel
constexpr int kSplitCap = 16384;         // candidates of the split kernel's merge
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

// Where a radix descent over the keys `visit` enumerates starts.  Over the
// whole key range (narrow = false), or (narrow = true, one more visit: meant
// for LDS lists) below the bits that the smallest and the largest key share:
// then the first 8-bit digit already separates the elements (logits near the
// top of a row share their sign and exponent bits, and a first digit made of
// those puts every element in one or two bins, whose LDS atomics serialise).
struct RadixStart {
  uint32_t prefix, mask;
  int shift;
};
template <typename Visit>
__device__ __forceinline__ RadixStart radix_start(Visit&& visit, bool narrow, uint32_t* red) {
  if (!narrow) return RadixStart{0u, 0u, 24};
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t lo = 0xffffffffu, hi = 0u;
  visit([&](uint32_t key, float) {
    lo = key < lo ? key : lo;
    hi = key > hi ? key : hi;
  });
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo = min(lo, __shfl_xor(lo, o));
    hi = max(hi, __shfl_xor(hi, o));
  }
  __syncthreads();
  if (lane == 0) {
    red[2 * wave] = lo;
    red[2 * wave + 1] = hi;
  }
  __syncthreads();
  lo = 0xffffffffu;
  hi = 0u;
#pragma unroll
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
    lo = min(lo, red[2 * w]);
    hi = max(hi, red[2 * w + 1]);
  }
  __syncthreads();
  const uint32_t diff = hi ^ lo;
  if (diff == 0u) return RadixStart{hi, 0xffffffffu, -1};  // one key: nothing to select
  const int top = 31 - __builtin_clz(diff);                // highest bit that differs
  const uint32_t above = top == 31 ? 0u : ~((2u << top) - 1u);
  return RadixStart{hi & above, above, top >= 7 ? top - 7 : 0};
}

// The key of the rest-th largest element (rest >= 1) of those `visit`
// enumerates: radix select, 8 bits a round, counts in an LDS histogram.
// visit(f) calls f(key, y) for every element; every thread calls this.
// (A last round may overlap bits already fixed: those match the prefix.)
template <typename Visit>
__device__ __forceinline__ uint32_t kth_largest_key(Visit&& visit, uint32_t rest, uint32_t* hcount,
                                                    uint32_t* sel, bool narrow) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const RadixStart st = radix_start(visit, narrow, hcount);
  uint32_t prefix = st.prefix, mask = st.mask;
  for (int shift = st.shift; shift >= 0; shift = shift >= 8 ? shift - 8 : (shift > 0 ? 0 : -1)) {
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
  __syncthreads();
  return prefix;
}

// The key of the lowest class top-p keeps among the elements `visit`
// enumerates (the top-k survivors, or a set of the form {y >= threshold}
// holding them all): the lowest key whose strictly larger elements carry less
// than p * Z of mass.  Z is z_total (in units of the fixed-point masses), or,
// when z_total is 0, the mass of every element visited.  0 < p < 1.
template <typename Visit>
__device__ __forceinline__ uint32_t top_p_key(Visit&& visit, float M, float inv_t, float p,
                                              double z_total, uint32_t* hcount,
                                              unsigned long long* hmass, uint32_t* sel,
                                              unsigned long long* sel_above, bool narrow) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const RadixStart st = radix_start(visit, narrow, hcount);
  uint32_t prefix = st.prefix, mask = st.mask;
  unsigned long long above = 0ull;  // mass of the elements above the bucket
  double target = (double)p * z_total;
  if (st.shift < 0) return prefix;  // one class: the largest, which is kept
  const int first = st.shift;
  for (int shift = st.shift; shift >= 0; shift = shift >= 8 ? shift - 8 : (shift > 0 ? 0 : -1)) {
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
      if (shift == first && z_total == 0.0) target = (double)p * (double)wave_sum(s);
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
  __syncthreads();
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
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w)
    if (beats(wbest[w].m, wbest[w].idx, best.m, best.idx)) best = wbest[w];
  bm = best.m;
  bi = best.idx;
}

// LDS of a filtering workgroup holding up to Cap candidates.
template <typename T, int Cap>
struct FilterShared {
  uint32_t hcount[256];
  unsigned long long hmass[256];
  float red_f[kFWaves];
  uint32_t red_u[kFWaves];
  uint32_t sel[2];
  unsigned long long sel_above, z_all;
  int bin_cut, bin_k;
  uint32_t n_cut, n_cand;
  float cval[Cap];
  int32_t cidx[Cap];
  Cand<T> wbest[kFWaves];
};

// Row b filtered and drawn by one workgroup (steps 1-4 above): the sampled
// index, or -1, in every thread.  STORE: instead of the draw, the row's
// filtered logits go to a.Y: y / t on the kept tokens, -inf elsewhere (greedy
// rows keep the largest logit's tie class, unscaled); returns 0.
template <bool FP64, int Cap, bool STORE = false>
__device__ __forceinline__ int64_t filter_row_single(
    const FilterArgs& a, int64_t b,
    FilterShared<typename std::conditional<FP64, double, float>::type, Cap>& sh) {
  typedef typename std::conditional<FP64, double, float>::type T;
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

  uint32_t* const hcount = sh.hcount;
  unsigned long long* const hmass = sh.hmass;
  float* const red_f = sh.red_f;
  uint32_t* const red_u = sh.red_u;
  uint32_t* const sel = sh.sel;
  unsigned long long& sel_above = sh.sel_above;
  unsigned long long& z_all = sh.z_all;
  int& bin_cut = sh.bin_cut;
  int& bin_k = sh.bin_k;
  uint32_t& n_cut = sh.n_cut;
  uint32_t& n_cand = sh.n_cand;
  float* const cval = sh.cval;
  int32_t* const cidx = sh.cidx;
  // Every caller reaches here together; LDS from earlier use is free again.
  __syncthreads();

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
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
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
    if (n_cut <= (uint32_t)Cap) {
      // 3. The candidates (every token that can be kept) into LDS.
      for_row(x, V, vec4, [&](int64_t i0, const float (&y)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (valid_logit(y[j]) && z_bin(y[j], M, inv_tf) <= cut) {
            const uint32_t q = atomicAdd(&n_cand, 1u);
            if (q < (uint32_t)Cap) {
              cval[q] = y[j];
              cidx[q] = (int32_t)(i0 + j);
            }
          }
      });
      __syncthreads();
      const int n = (int)(n_cand < (uint32_t)Cap ? n_cand : (uint32_t)Cap);
      auto visit_all = [&](auto&& f) {
        for (int q = tid; q < n; q += (int)blockDim.x) f(order_key(cval[q]), cval[q]);
      };
      // Top-k binds only when the candidates reach its bin; then they hold
      // every logit down to the k-th largest.
      uint32_t key_k = 0u, key_p = 0u;
      if (use_k && cut == bin_k)
        key_k = kth_largest_key(visit_all, (uint32_t)top_k, hcount, sel, true);
      if (use_p) {
        if (!(top_p > 0.0f)) {
          key_p = order_key(M);
        } else {
          auto visit_s1 = [&](auto&& f) {
            for (int q = tid; q < n; q += (int)blockDim.x) {
              const uint32_t key = order_key(cval[q]);
              if (key >= key_k) f(key, cval[q]);
            }
          };
          // Without top-k the survivors are every valid token: their mass is
          // the histogram's total; with it they are all among the candidates.
          key_p = top_p_key(visit_s1, M, inv_tf, top_p, use_k ? 0.0 : (double)z_total, hcount, hmass,
                            sel, &sel_above, true);
        }
      }
      kappa = key_k > key_p ? key_k : key_p;
      if (use_m && !(min_p < 1.0f)) {
        const uint32_t km = order_key(M);
        kappa = kappa > km ? kappa : km;
        use_m = false;
      }
      // The draw over the kept candidates (the store variant writes the
      // whole row below).
      if constexpr (!STORE) {
        for (int q = tid; q < n; q += (int)blockDim.x) {
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
      }
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
      if (use_k) key_k = kth_largest_key(visit_row, (uint32_t)top_k, hcount, sel, false);
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
          key_p = top_p_key(visit_s1, M, inv_tf, top_p, use_k ? 0.0 : (double)z_total, hcount, hmass,
                            sel, &sel_above, false);
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

  if constexpr (STORE) {
    // The filtered logits: every valid token with key >= kappa that passes the
    // min-p test, scaled by 1/t; greedy rows keep the largest logit's class.
    if (greedy) {
      float lm = neg_inf<float>();
      for_row(x, V, vec4, [&](int64_t, const float (&y)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (valid_logit(y[j])) lm = fmaxf(lm, y[j]);
      });
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) lm = fmaxf(lm, __shfl_xor(lm, o));
      if (lane == 0) red_f[wave] = lm;
      __syncthreads();
      M = neg_inf<float>();
#pragma unroll
      for (int w = 0; w < (int)(blockDim.x >> 6); ++w) M = fmaxf(M, red_f[w]);
      kappa = valid_logit(M) ? order_key(M) : 0xFFFFFFFFu;
    }
    float* const yo = a.Y + b * V;
    for_row(x, V, vec4, [&](int64_t i0, const float (&y)[4]) {
      float o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool keep = valid_logit(y[j]) && order_key(y[j]) >= kappa &&
                          (!use_m || mass_of(y[j], M, inv_tf) >= min_p);
        o[j] = keep ? y[j] * inv_tf : neg_inf<float>();
      }
      if (vec4) {
        *reinterpret_cast<float4*>(yo + i0) = make_float4(o[0], o[1], o[2], o[3]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (i0 + j < V) yo[i0 + j] = o[j];
      }
    });
    return 0;
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
  wave_then_block_best(bm, bi, sh.wbest);
  return bm == neg_inf<T>() ? (int64_t)-1 : (int64_t)bi;
}

template <bool FP64>
__global__ __launch_bounds__(kFThreads) void logits_filtered_kernel(FilterArgs a) {
  typedef typename std::conditional<FP64, double, float>::type T;
  __shared__ FilterShared<T, kCap> sh;
  if (a.row_flags) {
    // Only the flagged rows (the fused filtered sampler's fallback): the
    // previous launches have read the flag count, so it is cleared here.
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.flag_count = 0u;
    if (a.row_flags[blockIdx.x] == 0u) return;
  }
  const int64_t o = filter_row_single<FP64, kCap>(a, (int64_t)blockIdx.x, sh);
  if (threadIdx.x == 0) {
    a.out[blockIdx.x] = o;
    if (a.row_flags) a.row_flags[blockIdx.x] = 0u;
  }
}

// ---------------------------------------------------------------------------
// Split rows (small batches): a row is cut into chunks of kChunk logits, one
// workgroup each, so a decode-sized batch fills the chip.  Each chunk's
// workgroup publishes (in the workspace) its largest valid logit, its count,
// its fixed-point mass relative to its own largest logit, and either its
// unfiltered best (s, index) -- rows with no filter on -- or a list of at most
// kListCap candidates: every logit of the chunk at or above a key tau_g (the
// chunk's z-histogram bins that fit).  The workgroup that finishes a row last
// merges the lists in LDS.  Their union holds every logit at or above
// tau = max_g tau_g; when the kept set provably lies above tau (the top-k or
// top-p threshold does, or min-p rejects the largest logit below it) the
// selections and the draw run on the union, and otherwise the merging
// workgroup runs the one-workgroup path over the row.
// ---------------------------------------------------------------------------
constexpr int kChunk = 8192;            // logits per workgroup (all held in LDS)
constexpr int kListCap = 512;           // candidates a chunk publishes
static_assert(kChunk <= kSplitCap && kSplitMaxChunks * kListCap <= kSplitCap,
              "the LDS holds a chunk and a union");
constexpr int kHdrWords = 8;            // 64-bit words of a chunk's header

__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// MODE kSplitOne: chunks and merge in one launch (the merge in the row's last
// workgroup).  kSplitChunks / kSplitMerge: the same two halves as two
// launches, so that the chunk workgroups hold only their chunk in LDS (two a
// CU) and every row's merge starts at once (batches past kSplitMaxRows).
enum SplitMode { kSplitOne = 0, kSplitChunks = 1, kSplitMerge = 2 };

template <bool FP64, int MODE>
__global__ __launch_bounds__(kFThreads) void logits_filtered_split_kernel(FilterArgs a) {
  typedef typename std::conditional<FP64, double, float>::type T;
  __shared__ FilterShared<T, MODE == kSplitChunks ? kChunk : kSplitCap> sh;
  __shared__ float gM[kSplitMaxChunks];
  __shared__ unsigned long long gZ[kSplitMaxChunks];
  __shared__ uint32_t gN[kSplitMaxChunks], gTau[kSplitMaxChunks], gList[kSplitMaxChunks],
      gBase[kSplitMaxChunks + 1];
  __shared__ Cand<T> gBest[kSplitMaxChunks];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t b = blockIdx.y;
  const int64_t V = a.V;
  const int g = blockIdx.x;
  const int G = MODE == kSplitMerge ? (int)((V + kChunk - 1) / kChunk) : (int)gridDim.x;
  const float* x = a.X + b * V;
  const float t = a.temp[b];
  const bool greedy = !(t > 0.0f);
  const T inv_t = greedy ? T(1) : T(1) / T(t);
  const float inv_tf = greedy ? 1.0f : 1.0f / t;
  const uint32_t rid = a.row_ids ? a.row_ids[b] : (uint32_t)b;
  const int32_t top_k = a.top_k ? a.top_k[b] : 0;
  const float top_p = a.top_p ? a.top_p[b] : 1.0f;
  const float min_p = a.min_p ? a.min_p[b] : 0.0f;
  bool use_k = !greedy && top_k > 0;
  bool use_p = !greedy && top_p < 1.0f;
  bool use_m = !greedy && min_p > 0.0f;
  const bool filtered = use_k || use_p || use_m;  // the same in every chunk of the row
  const int64_t c0 = (int64_t)g * kChunk;
  const int n = (int)((V - c0) < kChunk ? (V - c0) : kChunk);
  uint64_t* const hdr = a.split + ((b * G + g) * (kHdrWords + kListCap));
  uint64_t* const lst = hdr + kHdrWords;

  if constexpr (MODE != kSplitMerge) {
    // 1. The chunk into LDS; its largest valid logit and count.
    if (a.vec4) {  // V % 4 == 0 and kChunk % 4 == 0: n % 4 == 0, aligned
      for (int q = 4 * tid; q < n; q += 4 * kFThreads) {
        const float4 v = *reinterpret_cast<const float4*>(x + c0 + q);
        sh.cval[q] = v.x;
        sh.cval[q + 1] = v.y;
        sh.cval[q + 2] = v.z;
        sh.cval[q + 3] = v.w;
      }
    } else {
      for (int q = tid; q < n; q += kFThreads) sh.cval[q] = x[c0 + q];
    }
    __syncthreads();
    float lm = neg_inf<float>();
    uint32_t nv = 0;
    for (int q = tid; q < n; q += kFThreads)
      if (valid_logit(sh.cval[q])) {
        lm = fmaxf(lm, sh.cval[q]);
        ++nv;
      }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) lm = fmaxf(lm, __shfl_xor(lm, o));
    nv = wave_sum(nv);
    if (lane == 0) {
      sh.red_f[wave] = lm;
      sh.red_u[wave] = nv;
    }
    __syncthreads();
    float Mg = neg_inf<float>();
    uint32_t nvg = 0;
#pragma unroll
    for (int w = 0; w < kFWaves; ++w) {
      Mg = fmaxf(Mg, sh.red_f[w]);
      nvg += sh.red_u[w];
    }

    if (!filtered) {
      // 2a. The chunk's unfiltered best: groups of 4 in increasing index order
      // per thread, the unfiltered sampler's scores.
      T bm = neg_inf<T>();
      int32_t bi = kNoIndex;
      for (int q = 4 * tid; q < n; q += 4 * kFThreads) {
        const int64_t i0 = c0 + q;
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = q + j < n ? sh.cval[q + j] : neg_inf<float>();
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
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (valid_logit(y[j]) && s[j] > bm) {
            bm = s[j];
            bi = (int32_t)(i0 + j);
          }
      }
      wave_then_block_best(bm, bi, sh.wbest);
      if (tid == 0) {
        cand_store_u64(hdr + 3, FP64 ? (uint64_t)__double_as_longlong((double)bm)
                                     : (uint64_t)__float_as_uint((float)bm));
        cand_store_u64(hdr + 4, (uint64_t)(uint32_t)bi);
        cand_store_u64(hdr + 2, 0ull);
        cand_store_u64(hdr + 1, 0ull);
      }
    } else {
      // 2b. The chunk's z-histogram relative to its own largest logit.
      if (tid < 256) {
        sh.hcount[tid] = 0u;
        sh.hmass[tid] = 0ull;
      }
      __syncthreads();
      for (int q = tid; q < n; q += kFThreads) {
        const float y = sh.cval[q];
        if (valid_logit(y)) {
          const int bin = z_bin(y, Mg, inv_tf);
          atomicAdd(&sh.hcount[bin], 1u);
          atomicAdd(&sh.hmass[bin], mass_fixed(mass_of(y, Mg, inv_tf)));
        }
      }
      __syncthreads();
      if (wave == 0) {
        // The listed bins 0 .. cut: the longest prefix holding at most kListCap
        // logits (cut = -1 when bin 0 alone holds more), and no further than the
        // chunk's own bounds: with top-k on, the bin of its k-th largest logit
        // (the row's top-k lie within the chunks' top-k, and top-p then needs
        // only those); with min-p on, the bins whose mass relative to the
        // chunk's largest logit can reach min_p (the row's largest is larger).
        uint32_t c[4], cs = 0;
        unsigned long long ws = 0ull;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c[j] = sh.hcount[4 * lane + j];
          cs += c[j];
          ws += sh.hmass[4 * lane + j];
        }
        uint32_t cc = wave_exclusive_scan(cs, lane);
        int mine = -1, kbin = 256;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          cc += c[j];
          if (cc <= (uint32_t)kListCap) mine = 4 * lane + j;
          if (kbin == 256 && use_k && cc >= (uint32_t)top_k) kbin = 4 * lane + j;
        }
        int cut = mine;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
          cut = max(cut, __shfl_xor(cut, o));
          kbin = min(kbin, __shfl_xor(kbin, o));
        }
        if (use_k && kbin < cut) cut = kbin;
        if (use_m) {
          int mbin = 0;
          if (min_p < 1.0f) {
            const double zmax = -log((double)min_p) * (1.0 + 1e-5) + 1e-5;
            mbin = zmax < (double)kZTop ? (int)(zmax * kBinsPerNat) : 255;
          }
          if (mbin < cut) cut = mbin;
        }
        const unsigned long long zg = wave_sum(ws);
        if (lane == 0) {
          sh.bin_cut = cut;
          sh.z_all = zg;
          sh.n_cand = 0u;
        }
      }
      __syncthreads();
      const int cut = sh.bin_cut;
      // 3. The listed logits out; the largest unlisted key gives tau_g.
      uint32_t unl = 0u;
      bool any_unl = false;
      for (int q = tid; q < n; q += kFThreads) {
        const float y = sh.cval[q];
        if (!valid_logit(y)) continue;
        if (z_bin(y, Mg, inv_tf) <= cut) {
          const uint32_t slot = atomicAdd(&sh.n_cand, 1u);
          cand_store_u64(lst + slot,
                         (uint64_t)__float_as_uint(y) | ((uint64_t)(uint32_t)(c0 + q) << 32));
        } else {
          const uint32_t k = order_key(y);
          unl = any_unl ? (unl > k ? unl : k) : k;
          any_unl = true;
        }
      }
      // tau_g = largest unlisted key + 1 (0 when every valid logit is listed);
      // keys of valid logits are below 0xff800001, so the sum cannot wrap.
      uint32_t tg = any_unl ? unl + 1u : 0u;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) tg = max(tg, __shfl_xor(tg, o));
      if (lane == 0) sh.red_u[wave] = tg;
      __syncthreads();
      if (tid == 0) {
        uint32_t tau = 0u;
#pragma unroll
        for (int w = 0; w < kFWaves; ++w) tau = tau > sh.red_u[w] ? tau : sh.red_u[w];
        cand_store_u64(hdr + 1, sh.z_all);
        cand_store_u64(hdr + 2, (uint64_t)tau | ((uint64_t)sh.n_cand << 32));
      }
    }
    if (tid == 0) cand_store_u64(hdr + 0, (uint64_t)__float_as_uint(Mg) | ((uint64_t)nvg << 32));
    wait_stores_complete();
  }

  // 4. The row's last workgroup merges (or the merge launch's workgroup).
  if constexpr (MODE == kSplitChunks) {
    return;
  } else {
    if constexpr (MODE == kSplitOne) {
      if (!finish_last(a.counters + b, (uint32_t)G)) return;
    }
    if (tid < G) {
      const uint64_t* h = a.split + ((b * G + tid) * (kHdrWords + kListCap));
      const uint64_t h0 = cand_load_u64(h + 0);
      gM[tid] = __uint_as_float((uint32_t)h0);
      gN[tid] = (uint32_t)(h0 >> 32);
      gZ[tid] = cand_load_u64(h + 1);
      const uint64_t h2 = cand_load_u64(h + 2);
      gTau[tid] = (uint32_t)h2;
      gList[tid] = (uint32_t)(h2 >> 32);
      if (!filtered) {
        const uint64_t m = cand_load_u64(h + 3);
        gBest[tid] = Cand<T>{FP64 ? T(__longlong_as_double((long long)m)) : T(__uint_as_float((uint32_t)m)),
                             (int32_t)(uint32_t)cand_load_u64(h + 4)};
      }
    }
    __syncthreads();
    int64_t out = -1;
    if (!filtered) {
      if (tid == 0) {
        Cand<T> best = Cand<T>{neg_inf<T>(), kNoIndex};
        for (int q = 0; q < G; ++q)
          if (beats(gBest[q].m, gBest[q].idx, best.m, best.idx)) best = gBest[q];
        a.out[b] = best.m == neg_inf<T>() ? (int64_t)-1 : (int64_t)best.idx;
        clear_counter(a.counters + b);
      }
      return;
    }
    float M = neg_inf<float>();
    uint32_t n_valid = 0u, tau = 0u;
    for (int q = 0; q < G; ++q) {
      M = fmaxf(M, gM[q]);
      n_valid += gN[q];
      tau = tau > gTau[q] ? tau : gTau[q];
    }
    if (tid == 0) {
      uint32_t base = 0u;
      for (int q = 0; q < G; ++q) {
        gBase[q] = base;
        base += gList[q];
      }
      gBase[G] = base;
    }
    __syncthreads();
    bool covered = n_valid > 0u;
    if ((int64_t)top_k >= (int64_t)n_valid) use_k = false;
    if (!(use_k || use_p || use_m)) covered = false;  // nothing filters: the full row is kept
    // The survivors' total mass without top-k: every chunk's fixed-point mass
    // rescaled to the row's largest logit (float64; the units stay 2^-40).
    double z_total = 0.0;
    for (int q = 0; q < G; ++q) {
      if (gN[q] == 0u) continue;
      if (M == __builtin_inff())
        z_total += gM[q] == M ? (double)gZ[q] : 0.0;
      else
        z_total += (double)gZ[q] * exp((double)(gM[q] - M) * (double)inv_tf);
    }
    // The union of the lists into LDS: each thread takes union entries
    // tid, tid + kFThreads, ... (chunk q holds entries gBase[q] .. gBase[q+1]),
    // so all of its loads are in flight together.
    const int nu = (int)gBase[G];
    {
      constexpr int kPer = kSplitCap / kFThreads;
      uint64_t v[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int e = tid + u * kFThreads;
        if (e >= nu) break;
        int q = 0;
        while (q + 1 < G && (int)gBase[q + 1] <= e) ++q;
        v[u] = cand_load_u64(a.split + ((b * G + q) * (kHdrWords + kListCap)) + kHdrWords +
                             (e - (int)gBase[q]));
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int e = tid + u * kFThreads;
        if (e >= nu) break;
        sh.cval[e] = __uint_as_float((uint32_t)v[u]);
        sh.cidx[e] = (int32_t)(uint32_t)(v[u] >> 32);
      }
    }
    __syncthreads();
    auto visit_u = [&](auto&& f) {
      for (int q = tid; q < nu; q += kFThreads) f(order_key(sh.cval[q]), sh.cval[q]);
    };
    uint32_t key_k = 0u, key_p = 0u;
    if (covered && use_k) {
      // the union's top top_k are the row's when it holds that many above tau
      uint32_t ca = 0u;
      for (int q = tid; q < nu; q += kFThreads) ca += order_key(sh.cval[q]) >= tau ? 1u : 0u;
      ca = wave_sum(ca);
      if (lane == 0) sh.red_u[wave] = ca;
      __syncthreads();
      uint32_t above = 0u;
#pragma unroll
      for (int w = 0; w < kFWaves; ++w) above += sh.red_u[w];
      __syncthreads();
      if (above >= (uint32_t)top_k)
        key_k = kth_largest_key(visit_u, (uint32_t)top_k, sh.hcount, sh.sel, true);
      else
        covered = false;
    }
    if (covered && use_p) {
      if (!(top_p > 0.0f)) {
        key_p = order_key(M);
      } else {
        auto visit_s1 = [&](auto&& f) {
          for (int q = tid; q < nu; q += kFThreads) {
            const uint32_t key = order_key(sh.cval[q]);
            if (key >= key_k) f(key, sh.cval[q]);
          }
        };
        key_p = top_p_key(visit_s1, M, inv_tf, top_p, use_k ? 0.0 : z_total, sh.hcount, sh.hmass,
                          sh.sel, &sh.sel_above, true);
        if (key_p < tau) covered = false;  // the crossing may lie among unlisted logits
      }
    }
    uint32_t kappa = key_k > key_p ? key_k : key_p;
    if (use_m && !(min_p < 1.0f)) {
      const uint32_t km = order_key(M);
      kappa = kappa > km ? kappa : km;
      use_m = false;
    }
    // Logits below tau are unlisted: the kept set must lie above it.
    if (covered && kappa < tau && !(use_m && mass_of(key_float(tau - 1u), M, inv_tf) < min_p))
      covered = false;
    if (covered) {
      T bm = neg_inf<T>();
      int32_t bi = kNoIndex;
      for (int q = tid; q < nu; q += kFThreads) {
        const float y = sh.cval[q];
        if (order_key(y) < kappa || (use_m && !(mass_of(y, M, inv_tf) >= min_p))) continue;
        const int32_t i = sh.cidx[q];
        T s;
        if constexpr (!FP64) {
          const Words w = noise_words(a.key, (uint32_t)(i >> 2), rid);
          const uint32_t r = i & 3;
          const uint32_t word = r == 0 ? w.w0 : (r == 1 ? w.w1 : (r == 2 ? w.w2 : w.w3));
          s = T(y * (float)inv_t) + T(gumbel_f32(word));
        } else {
          const Words w = noise_words(a.key, (uint32_t)(i >> 1), rid);
          s = (i & 1) ? T(y) * inv_t + T(gumbel_f64(w.w2, w.w3)) : T(y) * inv_t + T(gumbel_f64(w.w0, w.w1));
        }
        if (beats(s, i, bm, bi)) {
          bm = s;
          bi = i;
        }
      }
      wave_then_block_best(bm, bi, sh.wbest);
      out = bm == neg_inf<T>() ? (int64_t)-1 : (int64_t)bi;
    } else {
      out = filter_row_single<FP64, kSplitCap>(a, b, sh);
    }
    if (tid == 0) {
      a.out[b] = out;
      clear_counter(a.counters + b);
    }
  }
}

}  // namespace

namespace {

__global__ __launch_bounds__(kFThreads) void logits_filter_store_kernel(FilterArgs a) {
  __shared__ FilterShared<float, kCap> sh;
  (void)filter_row_single<false, kCap, true>(a, (int64_t)blockIdx.x, sh);
}

}  // namespace

hipError_t launch_filter_logits(const FilterArgs& a, hipStream_t stream) {
  const int nthr = a.B > kRowsNarrow ? kRowThreadsWide : kFThreads;
  launch(logits_filter_store_kernel, dim3((unsigned)a.B), dim3(nthr), 0, stream, a);
  return hipGetLastError();
}

int filtered_split_chunks(int64_t B, int64_t V) {
  const int64_t G = (V + kChunk - 1) / kChunk;
  return (B <= kSplitTwoLaunchMaxRows && G >= 2 && G <= kSplitMaxChunks) ? (int)G : 0;
}

size_t filtered_split_words(int64_t B, int64_t V) {
  const int G = filtered_split_chunks(B, V);
  return G ? (size_t)B * G * (kHdrWords + kListCap) : 0;
}

template <int MODE>
static void launch_split(const FilterArgs& a, bool fp64, dim3 grid, hipStream_t stream) {
  if (fp64)
    launch((logits_filtered_split_kernel<true, MODE>), grid, dim3(kFThreads), 0, stream, a);
  else
    launch((logits_filtered_split_kernel<false, MODE>), grid, dim3(kFThreads), 0, stream, a);
}

hipError_t launch_logits_filtered(const FilterArgs& a, bool fp64, hipStream_t stream) {
  const int G = a.split && !a.row_flags ? filtered_split_chunks(a.B, a.V) : 0;
  if (G) {
    const dim3 chunks((unsigned)G, (unsigned)a.B), rows(1u, (unsigned)a.B);
    if (a.B <= kSplitMaxRows) {
      launch_split<kSplitOne>(a, fp64, chunks, stream);
    } else {
      launch_split<kSplitChunks>(a, fp64, chunks, stream);
      launch_split<kSplitMerge>(a, fp64, rows, stream);
    }
    return hipGetLastError();
  }
  const dim3 grid((unsigned)a.B);
  const dim3 block(a.B > kRowsNarrow ? kRowThreadsWide : kFThreads);
  if (fp64)
    launch(logits_filtered_kernel<true>, grid, block, 0, stream, a);
  else
    launch(logits_filtered_kernel<false>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace fs
