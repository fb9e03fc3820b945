// fs_device.hpp -- device building blocks shared by the gfx950 kernels:
// counter-based Philox noise, uniform -> exponential -> Gumbel transforms, and
// the (score, index) order that every argmax and reduction uses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fs {

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11, section 4).  Each round
// takes the full 64-bit products of counter words 0 and 2 with the two round
// multipliers; their high halves are xored with words 1 and 3 and the key, the
// low halves pass through.  The key advances by the two Weyl increments between
// rounds.  The key and the offset words are wave-uniform, so the compiler keeps
// the key schedule (and the first round's word-2 product) in scalar registers.
// ---------------------------------------------------------------------------
struct Words {
  uint32_t w0, w1, w2, w3;
};

__device__ __forceinline__ Words philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    // one v_mad_u64_u32 per product gives both halves
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
  }
  return Words{c0, c1, c2, c3};
}

// Noise key of one sampling call: seed -> key, offset -> counter words 2..3.
struct NoiseKey {
  uint32_t k0, k1, off_lo, off_hi;
};

__host__ __device__ inline NoiseKey make_key(uint64_t seed, uint64_t offset) {
  return NoiseKey{(uint32_t)seed, (uint32_t)(seed >> 32), (uint32_t)offset,
                  (uint32_t)(offset >> 32)};
}

// Words of counter (j, row id) -- the row id is the logical id, not the batch
// position, so a row's noise is the same wherever it sits in the batch.
__device__ __forceinline__ Words noise_words(const NoiseKey& k, uint32_t j, uint32_t rid) {
  return philox4x32_10(j, rid, k.off_lo, k.off_hi, k.k0, k.k1);
}

// ---------------------------------------------------------------------------
// Uniform -> exponential -> Gumbel.  u lies on a midpoint grid: (k + 1/2) / 2^23
// from the top 23 bits of one word (float32 noise) or (k + 1/2) / 2^52 from the
// top 52 bits of two words (float64 noise).  E = -log u is standard
// exponential, g = -log E standard Gumbel.
//
// E must keep its relative accuracy where it is tiny (u near 1: the deep tail,
// where g is large).  There E = -log u = 2 atanh(x) with x = (1 - u) / (1 + u);
// 1 - u is exact on both grids, and the odd series 2x (1 + x^2/3 + x^4/5 + ...)
// is summed to its last significant term, the first omitted term below the
// precision's rounding unit: in float32 for u >= 3/4 (x <= 1/7, 5 terms), in
// float64 for u >= 1/2 (x <= 1/3, 16 terms).  Below those points log2 u is
// at least 0.41 in magnitude and the hardware log2 (v_log_f32) times ln 2 is
// accurate to a few float32 ulps.  g = -ln 2 * log2(E) by the hardware log2:
// an absolute error of ~1e-7 in g.
//
// Float64 noise keeps the 52-bit grid exactly and E's float64 relative accuracy
// on u >= 1/2, which is what carries the tail from ~20 to ~40 nats; E for
// u < 1/2 (E in [ln 2, 36.7]) and g are taken to float32 accuracy, and the
// score is then formed and compared in float64.  Both transforms are checked
// against float64 references over the whole float32 grid and on samples of the
// float64 grid.
// ---------------------------------------------------------------------------
constexpr float kLn2f = 0x1.62e43p-1f;

__device__ __forceinline__ float exp1_f32(uint32_t w) {
  const uint32_t k = w >> 9;
  const float u = (float)(2u * k + 1u) * 0x1p-24f;
  const float x = (1.0f - u) * __builtin_amdgcn_rcpf(1.0f + u);
  const float z = x * x;
  float p = 1.0f / 9.0f;
  p = __builtin_fmaf(p, z, 1.0f / 7.0f);
  p = __builtin_fmaf(p, z, 1.0f / 5.0f);
  p = __builtin_fmaf(p, z, 1.0f / 3.0f);
  p = __builtin_fmaf(p, z, 1.0f);
  const float e_tail = 2.0f * x * p;
  const float e_body = -kLn2f * __builtin_amdgcn_logf(u);
  return u >= 0.75f ? e_tail : e_body;
}

__device__ __forceinline__ float gumbel_f32(uint32_t w) {
  return -kLn2f * __builtin_amdgcn_logf(exp1_f32(w));
}

__device__ __forceinline__ double exp1_f64(uint32_t hi, uint32_t lo) {
  const uint64_t k = ((((uint64_t)hi) << 32) | (uint64_t)lo) >> 12;
  const double u = (double)(2ull * k + 1ull) * 0x1p-53;
  if (u >= 0.5) {
    const double x = (1.0 - u) / (1.0 + u);
    const double z = x * x;
    double p = 1.0 / 31.0;
#pragma unroll
    for (int n = 14; n >= 0; --n) p = __builtin_fma(p, z, 1.0 / (2 * n + 1));
    return 2.0 * x * p;
  }
  return (double)(-kLn2f * __builtin_amdgcn_logf((float)u));
}

__device__ __forceinline__ double gumbel_f64(uint32_t hi, uint32_t lo) {
  return (double)(-kLn2f * __builtin_amdgcn_logf((float)exp1_f64(hi, lo)));
}

// ---------------------------------------------------------------------------
// Candidate order: a larger score wins, equal scores go to the smaller index.
// This is a total order on (score, index) for non-NaN scores, so any reduction
// tree (lanes, waves, tiles) returns the result of the serial scan.  NaN never
// wins.  The empty candidate is (-inf, INT32_MAX); a -inf winner is reported as
// "no token" (-1).
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ bool beats(T s, int32_t i, T bs, int32_t bi) {
  return s > bs || (s == bs && i < bi);
}
// The same order with bitwise operators: no branches where it runs in a
// chain (cross-lane reductions, place selection).
template <typename T>
__device__ __forceinline__ bool beats_nb(T s, int32_t i, T bs, int32_t bi) {
  return (s > bs) | ((s == bs) & (i < bi));
}

template <typename T>
struct Cand {
  T m;
  int32_t idx;
};

template <typename T>
__device__ __forceinline__ T neg_inf();
template <>
__device__ __forceinline__ float neg_inf<float>() {
  return -__builtin_inff();
}
template <>
__device__ __forceinline__ double neg_inf<double>() {
  return -__builtin_inf();
}

constexpr int32_t kNoIndex = 0x7fffffff;

// A 32-bit lane exchange by DPP (no LDS): quad_perm [1,0,3,2] and [2,3,0,1]
// swap the lanes of xor 1 and xor 2; row_half_mirror pairs lane j with 7 - j
// of each 8 and row_mirror lane j with 15 - j of each 16.
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kCtrl, 0xf, 0xf, false);
}
template <int kCtrl>
__device__ __forceinline__ float dpp_val(float v) {
  return __uint_as_float(dpp_u32<kCtrl>(__float_as_uint(v)));
}
template <int kCtrl>
__device__ __forceinline__ double dpp_val(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint64_t r = (uint64_t)dpp_u32<kCtrl>((uint32_t)u) | ((uint64_t)dpp_u32<kCtrl>((uint32_t)(u >> 32)) << 32);
  return __longlong_as_double((long long)r);
}
__device__ __forceinline__ float lane_val(float v, int l) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), l));
}
__device__ __forceinline__ double lane_val(double v, int l) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint64_t r = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l) |
                     ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l) << 32);
  return __longlong_as_double((long long)r);
}

// Reduce (m, i) over the lanes of one wave64 that share `mask_bits` low lane
// bits: xor-shuffles over the remaining bits from `lo_bit` to bit 5.  For the
// whole wave (lo_bit = 0, every lane active) the best of each 16 lanes is
// formed by DPP exchanges (each step pairs groups that already agree, so any
// pairing gives the same best) and the four rows meet through readlane: no
// LDS round trips.  The best under the total order is unique, so both ways
// give the same result.
template <typename T>
__device__ __forceinline__ void wave_argmax_xor(T& m, int32_t& i, int lo_bit) {
  if (lo_bit == 0) {
    auto step = [&](T om, int32_t oi) {
      const bool take = beats_nb(om, oi, m, i);
      m = take ? om : m;
      i = take ? oi : i;
    };
    step(dpp_val<0xb1>(m), (int32_t)dpp_u32<0xb1>((uint32_t)i));
    step(dpp_val<0x4e>(m), (int32_t)dpp_u32<0x4e>((uint32_t)i));
    step(dpp_val<0x141>(m), (int32_t)dpp_u32<0x141>((uint32_t)i));
    step(dpp_val<0x140>(m), (int32_t)dpp_u32<0x140>((uint32_t)i));
    T bm = lane_val(m, 0);
    int32_t bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
      const T om = lane_val(m, 16 * r);
      const int32_t oi = __builtin_amdgcn_readlane(i, 16 * r);
      const bool take = beats_nb(om, oi, bm, bi);
      bm = take ? om : bm;
      bi = take ? oi : bi;
    }
    m = bm;
    i = bi;
    return;
  }
  for (int b = lo_bit; b < 6; ++b) {
    const T om = __shfl_xor(m, 1 << b, 64);
    const int32_t oi = __shfl_xor(i, 1 << b, 64);
    const bool take = beats_nb(om, oi, m, i);
    m = take ? om : m;
    i = take ? oi : i;
  }
}

// Reduce (m, i) over each aligned group of kWidth consecutive lanes (8, 16 or
// 32; a group's lanes are all active or all inactive): DPP exchanges within 16
// lanes, one xor-shuffle between the halves of 32.  Every lane of a group ends
// with the group's best (unique under the total order, so the pairing does not
// matter).
template <int kWidth, typename T>
__device__ __forceinline__ void group_argmax(T& m, int32_t& i) {
  static_assert(kWidth == 8 || kWidth == 16 || kWidth == 32, "groups of 8, 16 or 32 lanes");
  auto step = [&](T om, int32_t oi) {
    const bool take = beats_nb(om, oi, m, i);
    m = take ? om : m;
    i = take ? oi : i;
  };
  step(dpp_val<0xb1>(m), (int32_t)dpp_u32<0xb1>((uint32_t)i));
  step(dpp_val<0x4e>(m), (int32_t)dpp_u32<0x4e>((uint32_t)i));
  step(dpp_val<0x141>(m), (int32_t)dpp_u32<0x141>((uint32_t)i));
  if constexpr (kWidth >= 16) step(dpp_val<0x140>(m), (int32_t)dpp_u32<0x140>((uint32_t)i));
  if constexpr (kWidth == 32) step(__shfl_xor(m, 16, 64), __shfl_xor(i, 16, 64));
}

// ---------------------------------------------------------------------------
// Stage 2 inside the sampling kernel [FlashSampling, "algorithm details",
// Stage 2].  The workgroups of one group (a batch tile of the fused kernel, a
// row of the standalone sampler) each publish their candidates and count
// themselves done on the group's counter; the workgroup that counts last
// reduces the group's candidates to out_idx and clears the counter for the
// next call.  No workgroup ever waits for another, so a group cannot stall.
//
// Publishing needs no L2 write-back (an agent-scope release fence writes back
// the whole L2 of the XCD, which serialises at hundreds of nanoseconds per
// workgroup): candidates are written and read with agent-scope relaxed
// atomics, which gfx950 performs at the device coherence point (stores
// written through, loads not served from a possibly stale L1 or L2), and each
// writer waits for its stores to complete before its workgroup counts itself
// done.  A count therefore implies that the counted workgroup's candidates
// are readable by the workgroup that counts last, whatever XCD it runs on.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void cand_store_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t cand_load_u64(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Candidate (m, idx) as one (float) or two (double) 64-bit words, in the
// struct's own byte layout.
__device__ __forceinline__ void store_cand(Cand<float>* p, const Cand<float>& c) {
  cand_store_u64(reinterpret_cast<uint64_t*>(p),
                 (uint64_t)__float_as_uint(c.m) | ((uint64_t)(uint32_t)c.idx << 32));
}
__device__ __forceinline__ void store_cand(Cand<double>* p, const Cand<double>& c) {
  uint64_t* q = reinterpret_cast<uint64_t*>(p);
  cand_store_u64(q, (uint64_t)__double_as_longlong(c.m));
  cand_store_u64(q + 1, (uint64_t)(uint32_t)c.idx);
}
__device__ __forceinline__ Cand<float> load_cand(const Cand<float>* p) {
  const uint64_t v = cand_load_u64(reinterpret_cast<const uint64_t*>(p));
  return Cand<float>{__uint_as_float((uint32_t)v), (int32_t)(uint32_t)(v >> 32)};
}
__device__ __forceinline__ Cand<double> load_cand(const Cand<double>* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  const uint64_t m = cand_load_u64(q);
  const uint64_t i = cand_load_u64(q + 1);
  return Cand<double>{__longlong_as_double((long long)m), (int32_t)(uint32_t)i};
}

// Wait until this thread's stores have completed (vmcnt(0); the other
// counters of the gfx9 s_waitcnt encoding at their maximum, i.e. not waited).
__device__ __forceinline__ void wait_stores_complete() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// True, in every thread, for the workgroup that completes its group of
// `group_size` workgroups on `counter`.  Writer threads call store_cand and
// wait_stores_complete before this.  The workgroup that counts last takes an
// agent-scope acquire fence before it reads the group's candidates: on the
// reading side that is what the memory model asks for, and it costs one cache
// invalidation per group, not per workgroup.  The writing side keeps the
// hardware guarantee stated above (write-through atomic stores, completed
// before the count) instead of a release, whose L2 write-back every workgroup
// would pay.
__device__ __forceinline__ bool finish_last(uint32_t* counter, uint32_t group_size) {
  __shared__ uint32_t last;
  __syncthreads();  // every writer's stores have completed
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   group_size - 1u
               ? 1u
               : 0u;
  __syncthreads();
  if (last == 0u) return false;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return true;
}

// Leave a group's counter at zero for the next call (one thread, after the
// group's Stage 2).
__device__ __forceinline__ void clear_counter(uint32_t* counter) {
  __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The winner of one row's nT candidates, reduced by one wave (lane-strided
// scan, then xor-shuffles; the order is total, so this is the serial scan's
// result): its index, or -1 if the best score is -inf (no finite score).
template <typename T>
__device__ __forceinline__ int64_t row_winner(const Cand<T>* c, int nT, int lane) {
  T bm = neg_inf<T>();
  int32_t bi = kNoIndex;
  for (int t = lane; t < nT; t += 64) {
    const Cand<T> o = load_cand(c + t);
    if (beats(o.m, o.idx, bm, bi)) {
      bm = o.m;
      bi = o.idx;
    }
  }
  wave_argmax_xor(bm, bi, 0);
  return bm == neg_inf<T>() ? (int64_t)-1 : (int64_t)bi;
}

// ---------------------------------------------------------------------------
// Gumbel-top-k [FlashSampling, "limitations" and future work: the k largest
// perturbed scores are k draws without replacement].  Places are ordered by
// larger score, then smaller index; NaN and -inf never take a place.
// ---------------------------------------------------------------------------
constexpr int kTopKMax = 8;  // places kept per (row, tile)

// x comes strictly after w in place order (bitwise operators, as beats_nb).
template <typename T>
__device__ __forceinline__ bool after(T m, int32_t i, T wm, int32_t wi) {
  return (m < wm) | ((m == wm) & (i > wi));
}


// Insert (s, i) into a lane's sorted list (m, id) of K places.  Scores reach
// a lane in increasing index order, so an equal score goes below the places
// already held (strict compares); NaN never enters.
template <typename T, int K>
__device__ __forceinline__ void topk_insert(T (&m)[K], int32_t (&id)[K], T s, int32_t i) {
#pragma unroll
  for (int j = K - 1; j > 0; --j) {
    const bool up = s > m[j - 1];  // s goes above place j - 1: place j takes it
    const bool here = s > m[j];
    m[j] = up ? m[j - 1] : (here ? s : m[j]);
    id[j] = up ? id[j - 1] : (here ? i : id[j]);
  }
  const bool top = s > m[0];
  m[0] = top ? s : m[0];
  id[0] = top ? i : id[0];
}

// The top kTopKMax of two lists of kTopKMax places, each sorted best first
// and holding distinct candidates: a bitonic merge.  The best of a[j] and
// b[K-1-j] for every j is a bitonic sequence holding the top K of both lists;
// three half-cleaner stages sort it best first.  Compares use the place
// order (larger score, then smaller index), so the result is the unique
// sorted top K; (-inf, kNoIndex) fillers stay at the end.
template <typename T>
__device__ __forceinline__ void merge_top(T (&am)[kTopKMax], int32_t (&ai)[kTopKMax],
                                          const T (&bm)[kTopKMax], const int32_t (&bi)[kTopKMax]) {
  static_assert(kTopKMax == 8, "three half-cleaner stages");
#pragma unroll
  for (int j = 0; j < kTopKMax; ++j) {
    const T om = bm[kTopKMax - 1 - j];
    const int32_t oi = bi[kTopKMax - 1 - j];
    const bool take = beats_nb(om, oi, am[j], ai[j]);
    am[j] = take ? om : am[j];
    ai[j] = take ? oi : ai[j];
  }
#pragma unroll
  for (int d = kTopKMax / 2; d >= 1; d >>= 1)
#pragma unroll
    for (int j = 0; j < kTopKMax; ++j)
      if ((j & d) == 0) {
        const bool sw = beats_nb(am[j + d], ai[j + d], am[j], ai[j]);
        const T tm = am[j];
        const int32_t ti = ai[j];
        am[j] = sw ? am[j + d] : am[j];
        ai[j] = sw ? ai[j + d] : ai[j];
        am[j + d] = sw ? tm : am[j + d];
        ai[j + d] = sw ? ti : ai[j + d];
      }
}

// The next place after (pm, pi) among a wave's candidates: every lane offers
// its best candidate that comes after the previous place (first: any), and
// the lanes that differ only in bits lo_bit..5 of the lane id pick the best
// offer (lo_bit = 0: the whole wave).  Returns it in each of those lanes
// ((-inf, kNoIndex) when none is left).
template <typename T, int N>
__device__ __forceinline__ Cand<T> next_place(const Cand<T> (&c)[N], bool first, T pm, int32_t pi,
                                              int lo_bit = 0) {
  T bm = neg_inf<T>();
  int32_t bi = kNoIndex;
#pragma unroll
  for (int q = 0; q < N; ++q) {
    const bool take = (first | after(c[q].m, c[q].idx, pm, pi)) & beats_nb(c[q].m, c[q].idx, bm, bi);
    bm = take ? c[q].m : bm;
    bi = take ? c[q].idx : bi;
  }
  wave_argmax_xor(bm, bi, lo_bit);
  return Cand<T>{bm, bi};
}

}  // namespace fs
