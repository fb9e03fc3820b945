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
    const uint32_t lo0 = 0xD2511F53u * c0;
    const uint32_t hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0;
    const uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
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
// Uniform -> Gumbel.  u lies on a midpoint grid, (k + 1/2) / 2^23 from the top 23
// bits of one word (float32 noise) or (k + 1/2) / 2^52 from the top 52 bits of
// two words (float64 noise); every grid point and u - 1 are exact in the working
// precision, so E = -log u is taken as -log1p(u - 1), which keeps E's relative
// accuracy where u is close to 1 (E tiny, g large: the deep tail).  g = -log E.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float gumbel_f32(uint32_t w) {
  const uint32_t k = w >> 9;
  const float u = (float)(2u * k + 1u) * 0x1p-24f;
  const float E = -log1pf(u - 1.0f);
  return -logf(E);
}

__device__ __forceinline__ double gumbel_f64(uint32_t hi, uint32_t lo) {
  const uint64_t k = ((((uint64_t)hi) << 32) | (uint64_t)lo) >> 12;
  const double u = (double)(2ull * k + 1ull) * 0x1p-53;
  const double E = -log1p(u - 1.0);
  return -log(E);
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

// Reduce (m, i) over the lanes of one wave64 that share `mask_bits` low lane
// bits: xor-shuffles over the remaining bits from `lo_bit` to bit 5.
template <typename T>
__device__ __forceinline__ void wave_argmax_xor(T& m, int32_t& i, int lo_bit) {
  for (int b = lo_bit; b < 6; ++b) {
    const T om = __shfl_xor(m, 1 << b, 64);
    const int32_t oi = __shfl_xor(i, 1 << b, 64);
    if (beats(om, oi, m, i)) {
      m = om;
      i = oi;
    }
  }
}

}  // namespace fs
