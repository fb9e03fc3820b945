// fs_verify.hip -- speculative-decoding verification over materialised float32
// target and draft logits, for gfx950.
//
// The spec-decode-ops card describes `verify` as the canonical rejection
// sampler of speculative decoding (Leviathan et al. 2023; Chen et al. 2023):
// draft token x_i is accepted with probability min(1, p_t(x_i) / p_d(x_i)),
// the first rejection is replaced by a draw from max(p_t - p_d, 0)
// renormalised, and a fully accepted row appends a bonus draw from the
// target's last position.  Its usage example fixes the shapes: target logits
// [B, K+1, V], draft logits [B, K, V], draft tokens [B, K].
//
// Two launches:
//  * verify_stats_kernel: one pass over all 2K + 1 rows of every sequence.
//    Each workgroup reduces one chunk of one row: the K target and K draft
//    rows of positions < K to (max, normaliser, first argmax) partials of
//    their temperature softmax; the target's row K to the bonus draw's
//    (score, index) candidate, with the standalone sampler's arithmetic and
//    noise at position offset + K.
//  * verify_draw_kernel: every workgroup of a sequence merges the partials and
//    takes the K acceptance decisions (a few scalar loads and float64
//    arithmetic); the first rejection L fixes the rest.  Fully accepted rows
//    merge the bonus candidates, greedy rows emit the target argmax, and only
//    rows with a sampled rejection stream their two position-L rows once more
//    for the residual draw: Gumbel-max over log max(p_t - p_d, 0) with the
//    noise of position offset + L.  The last workgroup of a row merges the
//    chunks (finish_last); a residual that is all zero (p_t equal to p_d) is
//    replaced by the plain target draw with the same noise, which that
//    workgroup then makes alone.
//
// The acceptance uniform of position i is the 52-bit midpoint value of words
// 0 and 1 of Philox counter (2^32 - 1, row id, offset + i): vocabulary words
// never use that counter value, so the decisions are independent of every
// noise value.
#include <type_traits>

#include "fs_launch.hpp"

namespace fs {
namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 4;  // float4 loads in flight per thread and row
constexpr float kLog2e = 0x1.715476p+0f;
constexpr uint32_t kAcceptCounter = 0xFFFFFFFFu;

__device__ __forceinline__ bool valid_logit(float y) { return !(y != y) && y != -__builtin_inff(); }

// exp((a - m) / t) as exp2((a - m) * c), c = log2(e) / t, for a <= m, with the
// limits the softmax takes: 1 when a == m (also both +inf), 0 when a is -inf
// or m is +inf and a is not.
__device__ __forceinline__ float rel_mass(float a, float m, float c) {
  if (a == m) return 1.0f;
  if (a == -__builtin_inff() || m == __builtin_inff()) return 0.0f;
  return __builtin_amdgcn_exp2f((a - m) * c);
}

// exp2 scale of a row's masses: log2(e) / t (floored at 1e-30 so that t = +inf
// gives masses of 1 rather than NaN at -inf logits; greedy rows use no masses).
__device__ __forceinline__ float mass_scale(float t, bool greedy) {
  return greedy ? kLog2e : __builtin_fmaxf(kLog2e / t, 1e-30f);
}

// (max, normaliser, first argmax) of the valid logits a thread has met.
struct Stat {
  float m;
  float z;
  int32_t idx;
};

// Merge of two partials: larger max wins, equal maxima keep the smaller index.
__device__ __forceinline__ Stat stat_merge(float am, float az, int32_t ai, float bm, float bz,
                                           int32_t bi, float c) {
  const bool a_first = am > bm || (am == bm && ai < bi);
  const float m = a_first ? am : bm;
  float z = az * rel_mass(am, m, c) + bz * rel_mass(bm, m, c);
  if (m == -__builtin_inff()) z = 0.0f;
  return Stat{m, z, a_first ? ai : bi};
}

// Softmax partial of one chunk of one row, as stored between the launches.
struct RowStat {
  float m;
  int32_t idx;
  double z;
};

// (score, index) of the standalone sampler for 4 logits at i0 (i0 % 4 == 0):
// y * (1/t) + g with the noise of counter word i0 / 4 (float32 noise) or
// i0 / 2 and i0 / 2 + 1 (float64 noise); greedy rows score y itself.
template <typename T>
__device__ __forceinline__ void sample4(const NoiseKey& key, bool greedy, T inv_t, uint32_t rid,
                                        int64_t i0, int64_t hi, const float* y, T& bm,
                                        int32_t& bi) {
  T s[4];
  if (greedy) {
#pragma unroll
    for (int j = 0; j < 4; ++j) s[j] = T(y[j]);
  } else if (sizeof(T) == 4) {
    const Words w = noise_words(key, (uint32_t)(i0 >> 2), rid);
    s[0] = T(y[0] * (float)inv_t) + T(gumbel_f32(w.w0));
    s[1] = T(y[1] * (float)inv_t) + T(gumbel_f32(w.w1));
    s[2] = T(y[2] * (float)inv_t) + T(gumbel_f32(w.w2));
    s[3] = T(y[3] * (float)inv_t) + T(gumbel_f32(w.w3));
  } else {
    const Words w0 = noise_words(key, (uint32_t)(i0 >> 1), rid);
    const Words w1 = noise_words(key, (uint32_t)(i0 >> 1) + 1u, rid);
    s[0] = T(y[0]) * inv_t + T(gumbel_f64(w0.w0, w0.w1));
    s[1] = T(y[1]) * inv_t + T(gumbel_f64(w0.w2, w0.w3));
    s[2] = T(y[2]) * inv_t + T(gumbel_f64(w1.w0, w1.w1));
    s[3] = T(y[3]) * inv_t + T(gumbel_f64(w1.w2, w1.w3));
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (i0 + j < hi && s[j] > bm) {
      bm = s[j];
      bi = (int32_t)(i0 + j);
    }
  }
}

// Four logits of a row at i0; past `hi` (or the row end) they read as -inf.
__device__ __forceinline__ void load4(const float* x, int64_t i0, int64_t hi, bool vec4, float* y) {
  if (vec4 && i0 + 3 < hi) {
    const float4 v = *reinterpret_cast<const float4*>(x + i0);
    y[0] = v.x;
    y[1] = v.y;
    y[2] = v.z;
    y[3] = v.w;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = (i0 + j < hi) ? x[i0 + j] : -__builtin_inff();
  }
}

__device__ __forceinline__ uint32_t row_id_of(const VerifyArgs& a, int64_t b) {
  return a.row_ids ? a.row_ids[b] : (uint32_t)b;
}

template <typename T>
__device__ __forceinline__ T block_inv_t(float t) {
  return !(t > 0.0f) ? T(1) : T(1) / T(t);
}

// Launch 1.  Workgroup (q, c): chunk c of logical row q = b (2K + 1) + s, where
// s < K is target row s, K <= s < 2K draft row s - K and s = 2K target row K.
template <bool FP64>
__global__ __launch_bounds__(kThreads) void verify_stats_kernel(VerifyArgs a) {
  typedef typename std::conditional<FP64, double, float>::type T;
  const int64_t K = a.K, V = a.V;
  const int64_t q = (int64_t)blockIdx.x / a.nC;
  const int c = (int)((int64_t)blockIdx.x - q * a.nC);
  const int64_t b = q / (2 * K + 1);
  const int64_t s = q - b * (2 * K + 1);
  const float t = a.temp[b];
  const bool greedy = !(t > 0.0f);
  const float* x = s < K ? a.target + (b * (K + 1) + s) * V
                         : (s < 2 * K ? a.draft + (b * K + (s - K)) * V : a.target + (b * (K + 1) + K) * V);
  const int64_t lo = (int64_t)c * a.chunk;
  const int64_t hi = lo + a.chunk < V ? lo + a.chunk : V;
  constexpr int64_t kStride = 4 * kThreads;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool vec4 = a.vec4 != 0;

  if (s == 2 * K) {
    // The bonus draw's candidate: the standalone sampler at offset + K.
    const T inv_t = block_inv_t<T>(t);
    const NoiseKey key = make_key(a.seed, a.offset + (uint64_t)K);
    const uint32_t rid = row_id_of(a, b);
    T bm = neg_inf<T>();
    int32_t bi = kNoIndex;
    for (int64_t i0 = lo + 4 * (int64_t)threadIdx.x; i0 < hi; i0 += kStride * kInFlight) {
      float y[kInFlight][4];
#pragma unroll
      for (int u = 0; u < kInFlight; ++u) load4(x, i0 + kStride * u, hi, vec4, y[u]);
#pragma unroll
      for (int u = 0; u < kInFlight; ++u)
        if (i0 + kStride * u < hi) sample4<T>(key, greedy, inv_t, rid, i0 + kStride * u, hi, y[u], bm, bi);
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
      reinterpret_cast<Cand<T>*>(a.bonus)[b * a.nC + c] = best;
    }
    return;
  }

  // Softmax partial of a target or draft row of position < K.  Per step of
  // 4 kInFlight logits: their maximum first (NaN read as -inf), the running
  // normaliser rescaled only when it grows, then one exp2 per logit.
  const float cexp = mass_scale(t, greedy);
  constexpr float kInf = __builtin_inff();
  Stat st{-kInf, 0.0f, kNoIndex};
  for (int64_t i0 = lo + 4 * (int64_t)threadIdx.x; i0 < hi; i0 += kStride * kInFlight) {
    float y[kInFlight][4];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) load4(x, i0 + kStride * u, hi, vec4, y[u]);
    float mx = -kInf;
#pragma unroll
    for (int u = 0; u < kInFlight; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        y[u][j] = __builtin_fmaxf(y[u][j], -kInf);  // NaN -> -inf
        mx = __builtin_fmaxf(mx, y[u][j]);
      }
    if (mx > st.m) {
      int32_t id = kNoIndex;  // the first index attaining mx
#pragma unroll
      for (int u = kInFlight - 1; u >= 0; --u)
#pragma unroll
        for (int j = 3; j >= 0; --j)
          if (y[u][j] == mx) id = (int32_t)(i0 + kStride * u + j);
      st.z *= rel_mass(st.m, mx, cexp);
      st.m = mx;
      st.idx = id;
    }
    if (st.m == kInf) {  // +inf maximum: the mass is shared among the +inf logits
#pragma unroll
      for (int u = 0; u < kInFlight; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) st.z += y[u][j] == kInf ? 1.0f : 0.0f;
    } else if (st.m != -kInf) {
      const float m = st.m;
#pragma unroll
      for (int u = 0; u < kInFlight; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) st.z += __builtin_amdgcn_exp2f((y[u][j] - m) * cexp);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float om = __shfl_xor(st.m, o), oz = __shfl_xor(st.z, o);
    const int32_t oi = __shfl_xor(st.idx, o);
    st = stat_merge(st.m, st.z, st.idx, om, oz, oi, cexp);
  }
  __shared__ Stat wst[kThreads / 64];
  if (lane == 0) wst[wave] = st;
  __syncthreads();
  if (threadIdx.x == 0) {
    Stat r = wst[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) r = stat_merge(r.m, r.z, r.idx, wst[w].m, wst[w].z, wst[w].idx, cexp);
    reinterpret_cast<RowStat*>(a.stats)[(b * 2 * K + s) * a.nC + c] = RowStat{r.m, r.idx, (double)r.z};
  }
}

// Probability of token x under a row's merged softmax (float64): greedy rows
// are one-hot on the first argmax; a +inf maximum shares the mass among the
// +inf logits; no valid logit gives 0.
__device__ __forceinline__ double prob_of(float y, int64_t x, bool greedy, double t, float m,
                                          int32_t am, double z) {
  if (!valid_logit(y)) return 0.0;
  if (greedy) return x == (int64_t)am ? 1.0 : 0.0;
  if (m == __builtin_inff()) return y == __builtin_inff() ? 1.0 / z : 0.0;
  return exp(((double)y - (double)m) / t) / z;
}

// Launch 2.  Workgroup (b, c).
template <bool FP64>
__global__ __launch_bounds__(kThreads) void verify_draw_kernel(VerifyArgs a) {
  typedef typename std::conditional<FP64, double, float>::type T;
  const int64_t K = a.K, V = a.V;
  const int64_t b = (int64_t)blockIdx.x / a.nC2;
  const int c = (int)((int64_t)blockIdx.x - b * a.nC2);
  const float t = a.temp[b];
  const bool greedy = !(t > 0.0f);
  const uint32_t rid = row_id_of(a, b);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float cexp = mass_scale(t, greedy);

  // The draft tokens and their two logits (wave 0, lane i: position i), issued
  // before the partials are merged so that the two wait together.
  int64_t xtok = -1;
  float ytx = -__builtin_inff(), ydx = -__builtin_inff();
  if (wave == 0 && lane < K) {
    xtok = a.tokens[b * K + lane];
    if (xtok >= 0 && xtok < V) {
      ytx = a.target[(b * (K + 1) + lane) * V + xtok];
      ydx = a.draft[(b * K + lane) * V + xtok];
    }
  }

  // Merged softmax of the 2K rows (wave w merges rows w, w + 4, ...): one
  // online pass over the chunk partials, then the lanes' merge.
  __shared__ float s_m[2 * kVerifyMaxK];
  __shared__ int32_t s_am[2 * kVerifyMaxK];
  __shared__ double s_z[2 * kVerifyMaxK];
  __shared__ int s_len;
  for (int64_t r = wave; r < 2 * K; r += kThreads / 64) {
    const RowStat* p = reinterpret_cast<const RowStat*>(a.stats) + (b * 2 * K + r) * a.nC;
    float m = -__builtin_inff();
    int32_t idx = kNoIndex;
    double z = 0.0;
    for (int cc = lane; cc < a.nC; cc += 64) {
      const RowStat e = p[cc];
      const bool first = e.m > m || (e.m == m && e.idx < idx);
      const float nm = first ? e.m : m;
      z = z * (double)rel_mass(m, nm, cexp) + e.z * (double)rel_mass(e.m, nm, cexp);
      if (nm == -__builtin_inff()) z = 0.0;
      m = nm;
      idx = first ? e.idx : idx;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float om = __shfl_xor(m, o);
      const int32_t oi = __shfl_xor(idx, o);
      const double oz = __shfl_xor(z, o);
      const bool first = om > m || (om == m && oi < idx);
      const float nm = first ? om : m;
      z = z * (double)rel_mass(m, nm, cexp) + oz * (double)rel_mass(om, nm, cexp);
      if (nm == -__builtin_inff()) z = 0.0;
      m = nm;
      idx = first ? oi : idx;
    }
    if (lane == 0) {
      s_m[r] = m;
      s_am[r] = idx;
      s_z[r] = z;
    }
  }
  __syncthreads();

  // The K acceptance decisions (wave 0, lane i takes position i).
  if (wave == 0) {
    bool acc = true;
    if (lane < K) {
      double pt = 0.0, pq = 0.0;
      if (xtok >= 0 && xtok < V) {
        pt = prob_of(ytx, xtok, greedy, (double)t, s_m[lane], s_am[lane], s_z[lane]);
        pq = prob_of(ydx, xtok, greedy, (double)t, s_m[K + lane], s_am[K + lane], s_z[K + lane]);
      }
      const NoiseKey key = make_key(a.seed, a.offset + (uint64_t)lane);
      const Words w = noise_words(key, kAcceptCounter, rid);
      const uint64_t k52 = ((((uint64_t)w.w0) << 32) | (uint64_t)w.w1) >> 12;
      const double u = (double)(2ull * k52 + 1ull) * 0x1p-53;
      acc = u * pq < pt;
    }
    const uint64_t rejected = __ballot(!acc);
    if (lane == 0) s_len = rejected ? (int)__builtin_ctzll(rejected) : (int)K;
  }
  __syncthreads();
  const int L = s_len;

  if (L == K || greedy) {
    // Bonus draw (merge of launch 1's candidates) or a greedy row's target
    // argmax at the rejected position: one workgroup writes the row.
    if (c != 0) return;
    if (wave == 0) {
      int64_t tok_L;
      if (L == K) {
        tok_L = row_winner(reinterpret_cast<const Cand<T>*>(a.bonus) + b * a.nC, a.nC, lane);
      } else {
        tok_L = s_am[L] == kNoIndex ? (int64_t)-1 : (int64_t)s_am[L];
      }
      for (int64_t j = lane; j <= K; j += 64)
        a.out[b * (K + 1) + j] = j < L ? a.tokens[b * K + j] : (j == L ? tok_L : (int64_t)-1);
      if (lane == 0) a.accept_len[b] = L;
    }
    return;
  }

  // Residual draw at position L: scores log(max(p_t - p_d, 0)) + g.
  const float* xt = a.target + (b * (K + 1) + L) * V;
  const float* xd = a.draft + (b * K + L) * V;
  const float mt = s_m[L], md = s_m[K + L];
  const float izt = s_z[L] > 0.0 ? (float)(1.0 / s_z[L]) : 0.0f;
  const float izd = s_z[K + L] > 0.0 ? (float)(1.0 / s_z[K + L]) : 0.0f;
  const T inv_t = block_inv_t<T>(t);
  const NoiseKey key = make_key(a.seed, a.offset + (uint64_t)L);
  const int64_t lo = (int64_t)c * a.chunk2;
  const int64_t hi = lo + a.chunk2 < V ? lo + a.chunk2 : V;
  constexpr int64_t kStride = 4 * kThreads;
  const bool vec4 = a.vec4 != 0;
  T rm = neg_inf<T>();
  int32_t ri = kNoIndex;
  for (int64_t i0 = lo + 4 * (int64_t)threadIdx.x; i0 < hi; i0 += kStride * kInFlight) {
    float yt[kInFlight][4], yd[kInFlight][4];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      load4(xt, i0 + kStride * u, hi, vec4, yt[u]);
      load4(xd, i0 + kStride * u, hi, vec4, yd[u]);
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int64_t j0 = i0 + kStride * u;
      if (j0 >= hi) continue;
      T g[4];
      if (sizeof(T) == 4) {
        const Words w = noise_words(key, (uint32_t)(j0 >> 2), rid);
        g[0] = T(gumbel_f32(w.w0));
        g[1] = T(gumbel_f32(w.w1));
        g[2] = T(gumbel_f32(w.w2));
        g[3] = T(gumbel_f32(w.w3));
      } else {
        const Words w0 = noise_words(key, (uint32_t)(j0 >> 1), rid);
        const Words w1 = noise_words(key, (uint32_t)(j0 >> 1) + 1u, rid);
        g[0] = T(gumbel_f64(w0.w0, w0.w1));
        g[1] = T(gumbel_f64(w0.w2, w0.w3));
        g[2] = T(gumbel_f64(w1.w0, w1.w1));
        g[3] = T(gumbel_f64(w1.w2, w1.w3));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pt = valid_logit(yt[u][j]) ? rel_mass(yt[u][j], mt, cexp) * izt : 0.0f;
        const float pd = valid_logit(yd[u][j]) ? rel_mass(yd[u][j], md, cexp) * izd : 0.0f;
        const float r = pt - pd;
        const T sr = r > 0.0f ? T(kLn2f * __builtin_amdgcn_logf(r)) + g[j] : neg_inf<T>();
        if (j0 + j < hi && sr > rm) {
          rm = sr;
          ri = (int32_t)(j0 + j);
        }
      }
    }
  }
  wave_argmax_xor(rm, ri, 0);
  __shared__ Cand<T> wres[kThreads / 64];
  __shared__ int64_t s_tok;
  if (lane == 0) wres[wave] = Cand<T>{rm, ri};
  __syncthreads();
  Cand<T>* cres = reinterpret_cast<Cand<T>*>(a.resid) + b * a.nC2;
  if (threadIdx.x == 0) {
    Cand<T> br = wres[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w)
      if (beats(wres[w].m, wres[w].idx, br.m, br.idx)) br = wres[w];
    store_cand(cres + c, br);
    wait_stores_complete();
  }
  if (!finish_last(a.counters + b, (uint32_t)a.nC2)) return;
  // row_winner gives -1 when the best residual score is -inf (all zero)
  if (wave == 0) {
    const int64_t w = row_winner(cres, a.nC2, lane);
    if (lane == 0) s_tok = w;
  }
  __syncthreads();
  int64_t tok_L = s_tok;
  if (tok_L < 0) {
    // A residual that is all zero (p_t equals p_d): the draw from p_t itself,
    // the standalone sampler's on target row L at offset + L, by this
    // workgroup alone (a rare case).
    T bm = neg_inf<T>();
    int32_t bi = kNoIndex;
    for (int64_t i0 = 4 * (int64_t)threadIdx.x; i0 < V; i0 += kStride) {
      float y[4];
      load4(xt, i0, V, vec4, y);
      sample4<T>(key, false, inv_t, rid, i0, V, y, bm, bi);
    }
    wave_argmax_xor(bm, bi, 0);
    if (lane == 0) wres[wave] = Cand<T>{bm, bi};
    __syncthreads();
    Cand<T> best = wres[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w)
      if (beats(wres[w].m, wres[w].idx, best.m, best.idx)) best = wres[w];
    tok_L = best.m == neg_inf<T>() ? (int64_t)-1 : (int64_t)best.idx;
  }
  if (wave == 0) {
    for (int64_t j = lane; j <= K; j += 64)
      a.out[b * (K + 1) + j] = j < L ? a.tokens[b * K + j] : (j == L ? tok_L : (int64_t)-1);
    if (lane == 0) a.accept_len[b] = L;
  }
  if (threadIdx.x == 0) clear_counter(a.counters + b);
}

int chunk_for(int64_t rows, int64_t V) {
  constexpr int64_t kTargetWorkgroups = 2048;  // 8 per CU
  int64_t chunk = kVerifyChunk;
  while (chunk < kVerifyChunkMax && rows * ((V + 2 * chunk - 1) / (2 * chunk)) >= kTargetWorkgroups)
    chunk *= 2;
  return (int)chunk;
}

}  // namespace

size_t verify_stat_bytes() { return sizeof(RowStat); }

void verify_chunks(int64_t B, int64_t K, int64_t V, int* chunk, int* nC, int* chunk2, int* nC2) {
  *chunk = chunk_for(B * (2 * K + 1), V);
  *nC = (int)((V + *chunk - 1) / *chunk);
  *chunk2 = chunk_for(B, 2 * V);
  *nC2 = (int)((V + *chunk2 - 1) / *chunk2);
}

hipError_t launch_verify(const VerifyArgs& a, bool fp64, hipStream_t stream) {
  const dim3 g1((unsigned)(a.B * (2 * a.K + 1) * a.nC)), g2((unsigned)(a.B * a.nC2));
  if (fp64) {
    launch(verify_stats_kernel<true>, g1, dim3(kThreads), 0, stream, a);
    launch(verify_draw_kernel<true>, g2, dim3(kThreads), 0, stream, a);
  } else {
    launch(verify_stats_kernel<false>, g1, dim3(kThreads), 0, stream, a);
    launch(verify_draw_kernel<false>, g2, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace fs
