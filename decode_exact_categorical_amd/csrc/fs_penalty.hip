// fs_penalty.hip -- the repetition penalty of the spec-decode-ops card's sample
// pipeline (applied before the temperature), over materialised float32 logits,
// for gfx950.
//
// Every token that occurs among a row's previous tokens has its logit y
// replaced by y * penalty when y < 0 and by y / penalty otherwise (the
// transformers processor's rule; a token that occurs several times is
// penalised once).  Workgroup (c, b) takes chunk c of row b: the chunk goes to
// LDS, the penalised values overwrite their places there (each computed from
// the original logit in HBM, so duplicates write the same value), and the
// chunk goes out.  Every read of the input precedes every write of the
// output within the workgroup, and workgroups own disjoint chunks, so the
// output may be the input itself.
#include "fs_launch.hpp"

namespace fs {
namespace {

constexpr int kPThreads = 256;

__global__ __launch_bounds__(kPThreads) void repetition_penalty_kernel(PenaltyArgs a) {
  __shared__ float buf[kPenaltyChunk];
  const int64_t b = blockIdx.y;
  const int64_t V = a.V;
  const int64_t lo = (int64_t)blockIdx.x * kPenaltyChunk;
  const int n = (int)(V - lo < kPenaltyChunk ? V - lo : kPenaltyChunk);
  const float* x = a.X + b * V + lo;
  float* y = a.Y + b * V + lo;
  const int tid = threadIdx.x;
  if (a.vec4) {  // V % 4 == 0, rows 16-byte aligned: n % 4 == 0
    for (int q = 4 * tid; q < n; q += 4 * kPThreads)
      *reinterpret_cast<float4*>(buf + q) = *reinterpret_cast<const float4*>(x + q);
  } else {
    for (int q = tid; q < n; q += kPThreads) buf[q] = x[q];
  }
  const float p = a.penalty[b];
  __syncthreads();
  if (p > 0.0f) {  // NaN and non-positive penalties leave the row as it is
    const int64_t* prev = a.prev + b * a.L;
    for (int64_t j = tid; j < a.L; j += kPThreads) {
      const int64_t t = prev[j] - lo;
      if (t >= 0 && t < n) {
        const float v = x[t];
        buf[t] = v < 0.0f ? v * p : v / p;
      }
    }
  }
  __syncthreads();
  if (a.vec4) {
    for (int q = 4 * tid; q < n; q += 4 * kPThreads)
      *reinterpret_cast<float4*>(y + q) = *reinterpret_cast<const float4*>(buf + q);
  } else {
    for (int q = tid; q < n; q += kPThreads) y[q] = buf[q];
  }
}

}  // namespace

hipError_t launch_repetition_penalty(const PenaltyArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.V + kPenaltyChunk - 1) / kPenaltyChunk), (unsigned)a.B);
  launch(repetition_penalty_kernel, grid, dim3(kPThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fs
