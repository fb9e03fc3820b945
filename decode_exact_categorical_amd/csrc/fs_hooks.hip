// fs_hooks.hip -- test hooks: the Philox words and the noise transforms the
// samplers use, computed by the same device code (fs_device.hpp).
#include "fs_launch.hpp"

namespace fs {
namespace {

__global__ __launch_bounds__(256) void philox_words_kernel(NoiseKey key, const uint32_t* row_ids,
                                                           int64_t B, int64_t n_ctr, uint32_t* out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= B * n_ctr) return;
  const int64_t b = t / n_ctr;
  const uint32_t j = (uint32_t)(t - b * n_ctr);
  const uint32_t rid = row_ids ? row_ids[b] : (uint32_t)b;
  const Words w = noise_words(key, j, rid);
  uint4 v;
  v.x = w.w0; v.y = w.w1; v.z = w.w2; v.w = w.w3;
  reinterpret_cast<uint4*>(out)[t] = v;
}

__global__ __launch_bounds__(256) void noise_kernel(const uint32_t* words, int64_t n, bool fp64,
                                                    double* E, double* g) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  if (fp64) {
    E[t] = exp1_f64(words[2 * t], words[2 * t + 1]);
    g[t] = gumbel_f64(words[2 * t], words[2 * t + 1]);
  } else {
    E[t] = (double)exp1_f32(words[t]);
    g[t] = (double)gumbel_f32(words[t]);
  }
}

}  // namespace

hipError_t launch_noise(const uint32_t* words, int64_t n, bool fp64, double* E, double* g,
                        hipStream_t stream) {
  const dim3 grid((unsigned)((n + 255) / 256));
  hipLaunchKernelGGL(noise_kernel, grid, dim3(256), 0, stream, words, n, fp64, E, g);
  return hipGetLastError();
}

hipError_t launch_philox_words(NoiseKey key, const uint32_t* row_ids, int64_t B, int64_t n_ctr,
                               uint32_t* out, hipStream_t stream) {
  const int64_t n = B * n_ctr;
  const dim3 grid((unsigned)((n + 255) / 256));
  hipLaunchKernelGGL(philox_words_kernel, grid, dim3(256), 0, stream, key, row_ids, B, n_ctr, out);
  return hipGetLastError();
}

}  // namespace fs
