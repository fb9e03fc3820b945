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

// A plain streaming read: one workgroup per CU takes a contiguous slice of
// the buffer and each thread keeps eight 16-byte loads in flight per step,
// with the slice's lines read in order.  What one launch achieves is the
// practical read rate an HBM-bound kernel can aim for.  (Of the shapes tried
// on MI355X over 1.245 GB, this was the fastest: 201 us, 6.19 TB/s; two
// workgroups a CU with four loads in flight 206 us, grid-stride reads 218-252.)
constexpr int kStreamThreads = 512;
constexpr int kStreamUnroll = 8;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const uint4* p, int64_t n16,
                                                                    uint64_t* out) {
  const int64_t nwg = gridDim.x;
  const int64_t lo = n16 * (int64_t)blockIdx.x / nwg;
  const int64_t hi = n16 * ((int64_t)blockIdx.x + 1) / nwg;
  uint4 acc = make_uint4(0u, 0u, 0u, 0u);
  const int64_t step = (int64_t)kStreamThreads * kStreamUnroll;
  int64_t i = lo + threadIdx.x;
  for (; i + (kStreamUnroll - 1) * kStreamThreads < hi; i += step) {
    uint4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = p[i + u * kStreamThreads];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      acc.x ^= v[u].x;
      acc.y ^= v[u].y;
      acc.z ^= v[u].z;
      acc.w ^= v[u].w;
    }
  }
  for (; i < hi; i += kStreamThreads) {
    const uint4 v = p[i];
    acc.x ^= v.x;
    acc.y ^= v.y;
    acc.z ^= v.z;
    acc.w ^= v.w;
  }
  // One atomic per workgroup: device-scope atomics on one address are
  // serialised where the memory is, so one per wave (2048 over the chip) would
  // add a tail of tens of microseconds.
  __shared__ uint64_t part[kStreamThreads / 64];
  uint64_t x = ((uint64_t)(acc.x ^ acc.z) << 32) | (uint64_t)(acc.y ^ acc.w);
  for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x / 64] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    x = 0;
#pragma unroll
    for (int w = 0; w < kStreamThreads / 64; ++w) x ^= part[w];
    if (x != 0) atomicXor((unsigned long long*)out, (unsigned long long)x);
  }
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, int cus, uint64_t* out,
                              hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  int64_t wgs = (int64_t)cus;
  if (wgs > n16) wgs = n16;
  launch(stream_read_kernel, dim3((unsigned)wgs), dim3(kStreamThreads), 0, stream,
                     static_cast<const uint4*>(buf), n16, out);
  return hipGetLastError();
}

hipError_t launch_noise(const uint32_t* words, int64_t n, bool fp64, double* E, double* g,
                        hipStream_t stream) {
  const dim3 grid((unsigned)((n + 255) / 256));
  launch(noise_kernel, grid, dim3(256), 0, stream, words, n, fp64, E, g);
  return hipGetLastError();
}

hipError_t launch_philox_words(NoiseKey key, const uint32_t* row_ids, int64_t B, int64_t n_ctr,
                               uint32_t* out, hipStream_t stream) {
  const int64_t n = B * n_ctr;
  const dim3 grid((unsigned)((n + 255) / 256));
  launch(philox_words_kernel, grid, dim3(256), 0, stream, key, row_ids, B, n_ctr, out);
  return hipGetLastError();
}

}  // namespace fs
