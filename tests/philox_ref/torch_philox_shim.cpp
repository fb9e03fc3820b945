// Known-answer source for the oracle's Philox4x32-10: PyTorch's header-only
// engine (ATen/core/PhiloxRNGEngine.h), compiled on the host.  The engine's
// counter words 0-1 hold its "offset", words 2-3 its "subsequence", and its
// key is the 64-bit seed, so any (counter, key) can be reached.  Test-only.
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdint>

extern "C" void torch_philox_block(const uint32_t ctr[4], uint32_t k0, uint32_t k1,
                                   uint32_t out[4]) {
  const uint64_t seed = (uint64_t)k0 | ((uint64_t)k1 << 32);
  const uint64_t offset = (uint64_t)ctr[0] | ((uint64_t)ctr[1] << 32);
  const uint64_t subsequence = (uint64_t)ctr[2] | ((uint64_t)ctr[3] << 32);
  at::philox_engine eng(seed, subsequence, offset);
  for (int i = 0; i < 4; ++i) out[i] = eng();
}
