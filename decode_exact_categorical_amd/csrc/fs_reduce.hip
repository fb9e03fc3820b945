// fs_reduce.hip -- Stage 2 of both samplers, and the Philox and noise test hooks.
//
// Stage 2 follows the FlashSampling page ("algorithm details", Stage 2): for each
// row, the tile whose candidate score is largest gives the sampled index.  One
// wave per row scans the row's candidates (lane-strided, in the candidate
// order of fs_device.hpp) and xor-shuffles the lane results; the order is total,
// so the winner is the serial scan's.  A winner of -inf means the row had no
// finite score and is reported as -1.
#include "fs_launch.hpp"

namespace fs {
namespace {

constexpr int kRowsPerBlock = 4;

template <typename T>
__global__ __launch_bounds__(64 * kRowsPerBlock) void stage2_kernel(const Cand<T>* cand, int64_t B,
                                                                     int nT, int64_t* out) {
  const int lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (b >= B) return;
  const Cand<T>* c = cand + b * nT;
  T bm = neg_inf<T>();
  int32_t bi = kNoIndex;
  for (int t = lane; t < nT; t += 64) {
    const Cand<T> o = c[t];
    if (beats(o.m, o.idx, bm, bi)) {
      bm = o.m;
      bi = o.idx;
    }
  }
  wave_argmax_xor(bm, bi, 0);
  if (lane == 0) out[b] = (bm == neg_inf<T>()) ? (int64_t)-1 : (int64_t)bi;
}

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

hipError_t launch_stage2(const void* cand, int64_t B, int nT, bool fp64, int64_t* out,
                         hipStream_t stream) {
  const dim3 grid((unsigned)((B + kRowsPerBlock - 1) / kRowsPerBlock));
  if (fp64)
    hipLaunchKernelGGL(stage2_kernel<double>, grid, dim3(64 * kRowsPerBlock), 0, stream,
                       reinterpret_cast<const Cand<double>*>(cand), B, nT, out);
  else
    hipLaunchKernelGGL(stage2_kernel<float>, grid, dim3(64 * kRowsPerBlock), 0, stream,
                       reinterpret_cast<const Cand<float>*>(cand), B, nT, out);
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
