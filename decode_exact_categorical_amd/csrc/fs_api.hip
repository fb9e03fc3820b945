// fs_api.hip -- the C ABI of libfsample.so (declared and documented in
// include/fsample.h): argument checks on the host, workspace sizing, and the
// sampling launches (Stage 1 with Stage 2 in its last workgroups) on the
// caller's stream.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "fs_launch.hpp"
#include "fsample.h"

namespace fs {
LaunchTiming& launch_timing() {
  static thread_local LaunchTiming t;
  return t;
}
}  // namespace fs

namespace {

thread_local char g_last_error[512] = "";

fs_status fail(fs_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

fs_status hip_fail(hipError_t e, const char* what) {
  return fail(FS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxV = (int64_t)1 << 31;  // indices are int32 inside the kernels
constexpr int kMaxDevices = 64;
constexpr int kAssumedCUs = 256;  // MI355X; sizes the workspace without a device query
constexpr size_t kAlign = 256;
constexpr int64_t kMaxFusedB = (int64_t)1 << 22;  // 65536 batch tiles of 64 along grid y

// ---- kernel timing (fs_profile_begin / fs_profile_end) ----
struct Profiler {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;  // 2 events per timed call
  size_t used = 0;               // calls recorded since begin
  static constexpr size_t kMaxCalls = 4096;
};
Profiler g_prof;

// Events (before, after the sampling kernel) for one call, or null if not timing.
hipEvent_t* prof_slot() {
  std::lock_guard<std::mutex> lock(g_prof.mu);
  if (!g_prof.on || g_prof.used >= Profiler::kMaxCalls) return nullptr;
  const size_t need = 2 * (g_prof.used + 1);
  while (g_prof.pool.size() < need) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g_prof.pool.push_back(e);
  }
  hipEvent_t* slot = &g_prof.pool[2 * g_prof.used];
  ++g_prof.used;
  return slot;
}

// A timed call: the call's events go to its launches through launch_timing()
// (fs_launch.hpp).  If the call launched nothing, the events are recorded on
// the stream at the end, so that every timed call has both.
struct ProfScope {
  hipEvent_t* ev;
  hipStream_t st;
  explicit ProfScope(hipStream_t stream) : ev(prof_slot()), st(stream) {
    if (ev) fs::launch_timing() = fs::LaunchTiming{ev[0], ev[1]};
  }
  ~ProfScope() {
    if (!ev) return;
    if (fs::launch_timing().start != nullptr) {
      (void)hipEventRecord(ev[0], st);
      (void)hipEventRecord(ev[1], st);
    }
    fs::launch_timing() = fs::LaunchTiming{};
  }
};

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t cand_bytes(uint32_t flags) { return (flags & FS_FP64_NOISE) ? 16 : 8; }

int logits_tiles(int64_t V) { return (int)((V + fs::kLogitsChunk - 1) / fs::kLogitsChunk); }

// Compute units of the current device, cached per device (first call queries).
fs_status device_cus(int* cus) {
  static int cached[kMaxDevices] = {0};
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(FS_ERR_UNSUPPORTED, "device ordinal %d", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    if (n > kAssumedCUs) n = kAssumedCUs;  // workspace is sized for this many
    cached[dev] = n > 0 ? n : 1;
  }
  *cus = cached[dev];
  return FS_OK;
}

fs_status check_sizes(int64_t B, int64_t V) {
  if (B < 0) return fail(FS_ERR_INVALID_ARG, "B = %lld is negative", (long long)B);
  if (V < 1 || V >= kMaxV) return fail(FS_ERR_INVALID_ARG, "V = %lld outside [1, 2^31)", (long long)V);
  if (B > ((int64_t)1 << 31) / 1) return fail(FS_ERR_INVALID_ARG, "B = %lld too large", (long long)B);
  return FS_OK;
}

size_t align_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

// Workspace layout: a fixed region of kCounterWords completion counters at the
// start (one per batch tile of the fused kernel, one per row of a standalone
// launch), then the [B, tiles] candidates (tiles = the larger tile count of the
// two samplers, at the most CUs the library uses).  Every entry point (the
// fused and standalone samplers, Gumbel-top-k, the filtered sampler's split
// rows, verification) keeps its counters in that region and its other data
// after it, so no call's data overlaps another's counters: the counters stay
// zero between calls whatever entry points and shapes share the workspace.
constexpr int64_t kCounterWords = 65536;
constexpr int64_t kVerifyMaxB = kCounterWords;  // one counter per sequence
constexpr size_t kCounterBytes = (size_t)kCounterWords * sizeof(uint32_t);

size_t cand_region_bytes(int64_t B, int64_t V, uint32_t flags) {
  int64_t tiles = fs::fused_num_tiles(V, kAssumedCUs);
  const int64_t lt = logits_tiles(V);
  if (lt > tiles) tiles = lt;
  return align_up((size_t)B * (size_t)tiles * cand_bytes(flags));
}

uint32_t* counters_of(void* ws) { return static_cast<uint32_t*>(ws); }
void* candidates_of(void* ws) { return static_cast<char*>(ws) + kCounterBytes; }

fs_status check_workspace(void* ws, size_t have, int64_t B, int64_t V, uint32_t flags,
                          bool topk = false) {
  const size_t need = topk ? fs_workspace_bytes_topk(B, V, flags) : fs_workspace_bytes(B, V, flags);
  if (ws == nullptr || have < need)
    return fail(FS_ERR_WORKSPACE, "workspace %p of %zu bytes, need %zu", ws, have, need);
  if (((uintptr_t)ws & 15u) != 0) return fail(FS_ERR_WORKSPACE, "workspace not 16-byte aligned");
  return FS_OK;
}

// Weight formats of the fused calls.
enum WFormat { kFmtBf16 = 0, kFmtFp8 = 1, kFmtMxfp4 = 2 };

// Bytes of one W row.
int64_t row_bytes(int64_t D, int fmt) { return fmt == kFmtBf16 ? 2 * D : (fmt == kFmtFp8 ? D : D / 2); }

// Size and pointer checks shared by the weight formats: bf16 (W), FP8 (W8 +
// float32 row scales) and MXFP4 (W4 + E8M0 block scales).  D % 16 == 0 (FP8)
// and D % 256 == 0 (MXFP4) keep every row's 16-byte lane loads inside the row
// and aligned, and MXFP4's 8-byte scale words (a 256-k chunk's 8 blocks)
// aligned and inside the row.
fs_status check_fused(const fs_bf16* H, const void* W, int fmt, const void* scale, int64_t B,
                      int64_t D, int64_t V) {
  fs_status s = check_sizes(B, V);
  if (s != FS_OK) return s;
  if (B > kMaxFusedB) return fail(FS_ERR_UNSUPPORTED, "B = %lld > 2^22", (long long)B);
  if (D < 1) return fail(FS_ERR_INVALID_ARG, "D = %lld must be positive", (long long)D);
  const int dmul = fmt == kFmtBf16 ? 8 : (fmt == kFmtFp8 ? 16 : 256);
  if (D % dmul != 0)
    return fail(FS_ERR_UNSUPPORTED, "D = %lld is not a multiple of %d", (long long)D, dmul);
  if (D > ((int64_t)1 << 24)) return fail(FS_ERR_UNSUPPORTED, "D = %lld too large", (long long)D);
  if (B > 0 && (H == nullptr || W == nullptr)) return fail(FS_ERR_INVALID_ARG, "H or W is null");
  if (B > 0 && fmt != kFmtBf16 && scale == nullptr)
    return fail(FS_ERR_INVALID_ARG, "weight scales are null");
  if (B > 0 && (!aligned16(H) || !aligned16(W)))
    return fail(FS_ERR_UNSUPPORTED, "H and W must be 16-byte aligned");
  if (B > 0 && fmt == kFmtMxfp4 && ((uintptr_t)scale & 7u) != 0)
    return fail(FS_ERR_UNSUPPORTED, "MXFP4 scales must be 8-byte aligned");
  return FS_OK;
}

// The kernel addresses one wave's W rows through 32-bit offsets.
fs_status check_span(int64_t V, int64_t D, int nT, int fmt) {
  if (fs::fused_wave_span_bytes(V, row_bytes(D, fmt), nT, 1) >= ((int64_t)1 << 31))
    return fail(FS_ERR_UNSUPPORTED, "V * D too large (V = %lld, D = %lld)", (long long)V,
                (long long)D);
  return FS_OK;
}

void set_weights(fs::FusedArgs& a, const void* W, int fmt, const void* scale) {
  a.W = fmt == kFmtBf16 ? static_cast<const uint16_t*>(W) : nullptr;
  a.W8 = fmt == kFmtFp8 ? static_cast<const uint8_t*>(W) : nullptr;
  a.w_scale = fmt == kFmtFp8 ? static_cast<const float*>(scale) : nullptr;
  a.W4 = fmt == kFmtMxfp4 ? static_cast<const uint8_t*>(W) : nullptr;
  a.w4_scale = fmt == kFmtMxfp4 ? static_cast<const uint8_t*>(scale) : nullptr;
}

fs_status launch_sampling(const fs_bf16* H, const void* W, int fmt, const void* scale, int64_t B,
                          int64_t D, int64_t V, const float* temp, const float* bias,
                          uint64_t seed, uint64_t offset, int64_t* out_idx,
                          const uint32_t* row_ids, uint32_t flags, void* cand,
                          uint32_t* counters, int nT, fs_stream_t stream, int k);

// k = 0: one draw per row; 1 <= k <= kTopKMax: Gumbel-top-k (bf16 weights).
fs_status sample_fused(const fs_bf16* H, const void* W, int fmt, const void* scale, int64_t B,
                       int64_t D, int64_t V, const float* temp, const float* bias, uint64_t seed,
                       uint64_t offset, int64_t* out_idx, const uint32_t* row_ids, uint32_t flags,
                       void* workspace, size_t workspace_bytes, fs_stream_t stream, int k = 0) {
  fs_status s = check_fused(H, W, fmt, scale, B, D, V);
  if (s != FS_OK) return s;
  if (flags & ~FS_FP64_NOISE) return fail(FS_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if (k < 0 || k > fs::kTopKMax)
    return fail(FS_ERR_INVALID_ARG, "k = %d outside [1, %d]", k, fs::kTopKMax);
  // Gumbel-top-k tiles hold 16 or 32 rows, one completion counter each.
  if (k > 0 && B > 16 * kCounterWords)
    return fail(FS_ERR_UNSUPPORTED, "B = %lld > 2^20 for Gumbel-top-k", (long long)B);
  if (B == 0) return FS_OK;
  if (temp == nullptr || out_idx == nullptr) return fail(FS_ERR_INVALID_ARG, "temp or out_idx is null");
  s = check_workspace(workspace, workspace_bytes, B, V, flags, k > 0);
  if (s != FS_OK) return s;

  int cus = 0;
  s = device_cus(&cus);
  if (s != FS_OK) return s;
  // (Gumbel-top-k runs the narrow kernel at every batch size)
  const int nT = k > 0 ? fs::fused_num_tiles(V, cus, B <= 64 ? row_bytes(D, fmt) : 0)
                       : fs::fused_call_tiles(B, D, V, fmt == kFmtBf16, cus, row_bytes(D, fmt));
  s = check_span(V, D, nT, fmt);
  if (s != FS_OK) return s;
  return launch_sampling(H, W, fmt, scale, B, D, V, temp, bias, seed, offset, out_idx, row_ids,
                         flags, candidates_of(workspace), counters_of(workspace), nT, stream, k);
}

// The launch of a fused sampling call whose arguments have been checked: the
// per-tile candidates go to `cand`, the batch tiles' completion counters
// (zero on entry, left zero) are `counters`.
fs_status launch_sampling(const fs_bf16* H, const void* W, int fmt, const void* scale, int64_t B,
                          int64_t D, int64_t V, const float* temp, const float* bias,
                          uint64_t seed, uint64_t offset, int64_t* out_idx,
                          const uint32_t* row_ids, uint32_t flags, void* cand,
                          uint32_t* counters, int nT, fs_stream_t stream, int k) {
  const bool fp64 = (flags & FS_FP64_NOISE) != 0;
  fs::FusedArgs a;
  memset(&a, 0, sizeof a);
  a.H = H;
  set_weights(a, W, fmt, scale);
  a.B = B;
  a.D = D;
  a.V = V;
  a.temp = temp;
  a.bias = bias;
  a.row_ids = row_ids;
  a.key = fs::make_key(seed, offset);
  a.cand = cand;
  a.nT = nT;
  a.counters = counters;  // ceil(B / 16) words at most
  a.out = out_idx;
  a.Y = nullptr;
  a.bias_vec4 = bias != nullptr && aligned16(bias) && (V % 4 == 0);
  a.k = k;
  const int epi = k > 0 ? (fp64 ? fs::kEpiTopK64 : fs::kEpiTopK32)
                        : (fp64 ? fs::kEpiSample64 : fs::kEpiSample32);
  hipStream_t st = (hipStream_t)stream;
  ProfScope prof(st);
  hipError_t e = fs::launch_fused_stage1(a, epi, st);
  if (e != hipSuccess) return hip_fail(e, "fused sampling launch");
  return FS_OK;
}

fs_status debug_logits(const fs_bf16* H, const void* W, int fmt, const void* scale, int64_t B,
                       int64_t D, int64_t V, float* Y, fs_stream_t stream) {
  fs_status s = check_fused(H, W, fmt, scale, B, D, V);
  if (s != FS_OK) return s;
  if (B == 0) return FS_OK;
  if (Y == nullptr) return fail(FS_ERR_INVALID_ARG, "Y is null");
  int cus = 0;
  s = device_cus(&cus);
  if (s != FS_OK) return s;
  // (128-column tiles stream W in passes of 32 rows, which 256 tiles divide evenly)
  const int nT = fs::fused_call_tiles(B, D, V, fmt == kFmtBf16, cus, row_bytes(D, fmt));
  s = check_span(V, D, nT, fmt);
  if (s != FS_OK) return s;
  fs::FusedArgs a;
  memset(&a, 0, sizeof a);
  a.H = H;
  set_weights(a, W, fmt, scale);
  a.B = B;
  a.D = D;
  a.V = V;
  a.nT = nT;
  a.Y = Y;
  hipError_t e = fs::launch_fused_stage1(a, fs::kEpiStore, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fused logits launch");
  return FS_OK;
}

// ---- the entry point that allocates nothing (fs_sample_fused_noalloc) ----
// Its scratch memory is this file-scope device array: a counter region, then
// the per-tile candidates of at most kNoAllocMaxB rows (16-byte candidates,
// kMaxFusedTiles tiles).  Each GPU holds its own copy for the life of the
// process; host code reaches it only through the address hipGetSymbolAddress
// returns for the current device (the array's name on the host is not a
// device address).
constexpr int64_t kNoAllocMaxB = 1024;
constexpr size_t kNoAllocCounterBytes = 4096;  // ceil(B / 16) <= 64 counters
constexpr size_t kNoAllocCandBytes = (size_t)kNoAllocMaxB * fs::kMaxFusedTiles * 16;
constexpr size_t kNoAllocBytes = kNoAllocCounterBytes + kNoAllocCandBytes;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

__global__ void clear_words_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The current device's scratch address, looked up (and its counter region
// cleared, by a kernel on `stream`) on the first call on that device.
fs_status noalloc_scratch(hipStream_t stream, unsigned char** out) {
  static unsigned char* ptrs[kMaxDevices] = {nullptr};
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(FS_ERR_UNSUPPORTED, "device ordinal %d", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(FS_ERR_HIP, "hipGetSymbolAddress(scratch) returned null");
    const int64_t words = (int64_t)(kNoAllocCounterBytes / sizeof(uint32_t));
    fs::launch(clear_words_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0,
                       stream, static_cast<uint32_t*>(p), words);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "scratch clear launch");
    ptrs[dev] = static_cast<unsigned char*>(p);
  }
  *out = ptrs[dev];
  return FS_OK;
}

}  // namespace

extern "C" {

fs_status fs_sample_fused_noalloc(const fs_bf16* H, const fs_bf16* W, int64_t B, int64_t D,
                                  int64_t V, const float* temp, const float* bias, uint64_t seed,
                                  uint64_t offset, int64_t* out_idx, const uint32_t* row_ids,
                                  uint32_t flags, fs_stream_t stream) {
  g_last_error[0] = 0;
  fs_status s = check_fused(H, W, kFmtBf16, nullptr, B, D, V);
  if (s != FS_OK) return s;
  if (flags & ~FS_FP64_NOISE) return fail(FS_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if (B > kNoAllocMaxB)
    return fail(FS_ERR_UNSUPPORTED, "B = %lld exceeds the %lld rows of the built-in scratch",
                (long long)B, (long long)kNoAllocMaxB);
  if (B == 0) return FS_OK;
  if (temp == nullptr || out_idx == nullptr) return fail(FS_ERR_INVALID_ARG, "temp or out_idx is null");
  int cus = 0;
  s = device_cus(&cus);
  if (s != FS_OK) return s;
  const int nT = fs::fused_call_tiles(B, D, V, true, cus, row_bytes(D, kFmtBf16));
  s = check_span(V, D, nT, kFmtBf16);
  if (s != FS_OK) return s;
  if ((size_t)B * (size_t)nT * cand_bytes(flags) > kNoAllocCandBytes)
    return fail(FS_ERR_UNSUPPORTED, "B * tiles exceeds the built-in scratch");
  unsigned char* p = nullptr;
  s = noalloc_scratch((hipStream_t)stream, &p);
  if (s != FS_OK) return s;
  return launch_sampling(H, W, kFmtBf16, nullptr, B, D, V, temp, bias, seed, offset, out_idx,
                         row_ids, flags, p + kNoAllocCounterBytes, reinterpret_cast<uint32_t*>(p),
                         nT, stream, 0);
}

size_t fs_workspace_bytes(int64_t B, int64_t V, uint32_t flags) {
  if (B < 0 || V < 1 || V >= kMaxV) return 0;
  return kCounterBytes + cand_region_bytes(B, V, flags);
}

size_t fs_workspace_bytes_topk(int64_t B, int64_t V, uint32_t flags) {
  if (B < 0 || V < 1 || V >= kMaxV) return 0;
  return kCounterBytes + cand_region_bytes(B, V, flags) * fs::kTopKMax;
}

const char* fs_status_string(fs_status status) {
  switch (status) {
    case FS_OK: return "FS_OK";
    case FS_ERR_INVALID_ARG: return "FS_ERR_INVALID_ARG: invalid argument";
    case FS_ERR_UNSUPPORTED: return "FS_ERR_UNSUPPORTED: unsupported size or alignment";
    case FS_ERR_WORKSPACE: return "FS_ERR_WORKSPACE: workspace missing or too small";
    case FS_ERR_HIP: return "FS_ERR_HIP: HIP runtime error";
  }
  return "unknown fs_status";
}

const char* fs_last_error(void) { return g_last_error; }

fs_status fs_sample_fused(const fs_bf16* H, const fs_bf16* W, int64_t B, int64_t D, int64_t V,
                          const float* temp, const float* bias, uint64_t seed, uint64_t offset,
                          int64_t* out_idx, const uint32_t* row_ids, uint32_t flags,
                          void* workspace, size_t workspace_bytes, fs_stream_t stream) {
  g_last_error[0] = 0;
  return sample_fused(H, W, kFmtBf16, nullptr, B, D, V, temp, bias, seed, offset, out_idx, row_ids,
                      flags, workspace, workspace_bytes, stream);
}

fs_status fs_sample_fused_topk(const fs_bf16* H, const fs_bf16* W, int64_t B, int64_t D,
                               int64_t V, const float* temp, const float* bias, uint64_t seed,
                               uint64_t offset, int k, int64_t* out_idx, const uint32_t* row_ids,
                               uint32_t flags, void* workspace, size_t workspace_bytes,
                               fs_stream_t stream) {
  g_last_error[0] = 0;
  if (k < 1) return fail(FS_ERR_INVALID_ARG, "k = %d outside [1, %d]", k, fs::kTopKMax);
  return sample_fused(H, W, kFmtBf16, nullptr, B, D, V, temp, bias, seed, offset, out_idx, row_ids,
                      flags, workspace, workspace_bytes, stream, k);
}

fs_status fs_sample_fused_mxfp4(const fs_bf16* H, const uint8_t* W4, const uint8_t* w4_scale,
                                int64_t B, int64_t D, int64_t V, const float* temp,
                                const float* bias, uint64_t seed, uint64_t offset,
                                int64_t* out_idx, const uint32_t* row_ids, uint32_t flags,
                                void* workspace, size_t workspace_bytes, fs_stream_t stream) {
  g_last_error[0] = 0;
  return sample_fused(H, W4, kFmtMxfp4, w4_scale, B, D, V, temp, bias, seed, offset, out_idx,
                      row_ids, flags, workspace, workspace_bytes, stream);
}

fs_status fs_sample_fused_w8(const fs_bf16* H, const uint8_t* W8, const float* w_scale, int64_t B,
                             int64_t D, int64_t V, const float* temp, const float* bias,
                             uint64_t seed, uint64_t offset, int64_t* out_idx,
                             const uint32_t* row_ids, uint32_t flags, void* workspace,
                             size_t workspace_bytes, fs_stream_t stream) {
  g_last_error[0] = 0;
  return sample_fused(H, W8, kFmtFp8, w_scale, B, D, V, temp, bias, seed, offset, out_idx, row_ids,
                      flags, workspace, workspace_bytes, stream);
}

fs_status fs_sample_logits(const float* logits, int64_t B, int64_t V, const float* temp,
                           uint64_t seed, uint64_t offset, int fp64_noise, int64_t* out_idx,
                           const uint32_t* row_ids, void* workspace, size_t workspace_bytes,
                           fs_stream_t stream) {
  g_last_error[0] = 0;
  fs_status s = check_sizes(B, V);
  if (s != FS_OK) return s;
  if (B == 0) return FS_OK;
  if (logits == nullptr || temp == nullptr || out_idx == nullptr)
    return fail(FS_ERR_INVALID_ARG, "logits, temp or out_idx is null");
  if (((uintptr_t)logits & 3u) != 0) return fail(FS_ERR_UNSUPPORTED, "logits not 4-byte aligned");
  const int nT = logits_tiles(V);
  if ((int64_t)B * nT >= ((int64_t)1 << 31))
    return fail(FS_ERR_INVALID_ARG, "B * ceil(V / %d) exceeds 2^31", fs::kLogitsChunk);
  const uint32_t flags = fp64_noise ? FS_FP64_NOISE : 0u;
  s = check_workspace(workspace, workspace_bytes, B, V, flags);
  if (s != FS_OK) return s;

  // One launch per run of at most kCounterWords rows (one counter per row);
  // the launches follow each other on the stream and reuse the workspace.
  hipStream_t st = (hipStream_t)stream;
  ProfScope prof(st);
  for (int64_t b0 = 0; b0 < B; b0 += kCounterWords) {
    const int64_t nb = B - b0 < kCounterWords ? B - b0 : kCounterWords;
    fs::LogitsArgs a;
    a.X = logits + b0 * V;
    a.B = nb;
    a.V = V;
    a.temp = temp + b0;
    a.row_ids = row_ids ? row_ids + b0 : nullptr;
    a.rid_base = (uint32_t)b0;
    a.key = fs::make_key(seed, offset);
    a.cand = candidates_of(workspace);
    a.chunk = fs::logits_sample_chunk(nb, V);
    a.nT = (int)((V + a.chunk - 1) / a.chunk);  // <= nT at the smallest chunk
    a.counters = counters_of(workspace);
    a.out = out_idx + b0;
    a.vec4 = aligned16(logits) && (V % 4 == 0);
    a.k = 1;
    hipError_t e = fs::launch_logits_stage1(a, fp64_noise != 0, st);
    if (e != hipSuccess) return hip_fail(e, "logits sampling launch");
  }
  return FS_OK;
}

// Workspace of the fused filtered sampler: the counter region (its word 0
// counts the rows flagged for the fallback, words 1 .. B are the rows' flags;
// like every counter they are zero between calls), the per-(row, tile)
// records, then the fallback logits [B, V] (written only for flagged rows).
constexpr int64_t kFusedFilteredMaxB = kCounterWords - 1;
struct FusedFilteredLayout {
  size_t records, logits, total;
};
FusedFilteredLayout fused_filtered_layout(int64_t B, int64_t V) {
  FusedFilteredLayout L;
  L.records = kCounterBytes;
  L.logits = L.records + align_up((size_t)B * fs::kMaxFusedTiles * fs::kFiltRecBytes);
  L.total = L.logits + align_up((size_t)B * (size_t)V * sizeof(float));
  return L;
}

size_t fs_workspace_bytes_fused_filtered(int64_t B, int64_t V) {
  if (B < 0 || B > kFusedFilteredMaxB || V < 1 || V >= kMaxV) return 0;
  return fused_filtered_layout(B, V).total;
}

fs_status fs_sample_fused_filtered(const fs_bf16* H, const fs_bf16* W, int64_t B, int64_t D,
                                   int64_t V, const float* temp, const int32_t* top_k,
                                   const float* top_p, const float* min_p, uint64_t seed,
                                   uint64_t offset, int64_t* out_idx, const uint32_t* row_ids,
                                   uint32_t flags, void* workspace, size_t workspace_bytes,
                                   fs_stream_t stream) {
  g_last_error[0] = 0;
  fs_status s = check_fused(H, W, kFmtBf16, nullptr, B, D, V);
  if (s != FS_OK) return s;
  if (flags & ~FS_FP64_NOISE) return fail(FS_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if (B > kFusedFilteredMaxB)
    return fail(FS_ERR_UNSUPPORTED, "B = %lld > %lld", (long long)B, (long long)kFusedFilteredMaxB);
  if (B == 0) return FS_OK;
  if (temp == nullptr || out_idx == nullptr) return fail(FS_ERR_INVALID_ARG, "temp or out_idx is null");
  const FusedFilteredLayout L = fused_filtered_layout(B, V);
  if (workspace == nullptr || workspace_bytes < L.total)
    return fail(FS_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, L.total);
  if (((uintptr_t)workspace & (kAlign - 1)) != 0)
    return fail(FS_ERR_WORKSPACE, "workspace not %zu-byte aligned", (size_t)kAlign);
  int cus = 0;
  s = device_cus(&cus);
  if (s != FS_OK) return s;
  const int nT = fs::fused_num_tiles(V, cus, row_bytes(D, kFmtBf16));
  s = check_span(V, D, nT, kFmtBf16);
  if (s != FS_OK) return s;
  const bool fp64 = (flags & FS_FP64_NOISE) != 0;
  char* ws = static_cast<char*>(workspace);
  fs::FusedArgs a;
  memset(&a, 0, sizeof a);
  a.H = H;
  a.W = W;
  a.B = B;
  a.D = D;
  a.V = V;
  a.temp = temp;
  a.row_ids = row_ids;
  a.key = fs::make_key(seed, offset);
  a.cand = ws + L.records;
  a.nT = nT;
  a.counters = counters_of(workspace);
  a.out = out_idx;
  a.top_k = top_k;
  a.top_p = top_p;
  a.min_p = min_p;
  a.flag_count = counters_of(workspace);
  a.row_flags = counters_of(workspace) + 1;
  fs::FilterArgs fa;
  memset(&fa, 0, sizeof fa);
  fa.X = reinterpret_cast<const float*>(ws + L.logits);
  fa.B = B;
  fa.V = V;
  fa.temp = temp;
  fa.row_ids = row_ids;
  fa.top_k = top_k;
  fa.top_p = top_p;
  fa.min_p = min_p;
  fa.key = a.key;
  fa.out = out_idx;
  fa.vec4 = (V % 4 == 0);
  fa.row_flags = a.row_flags;
  fa.flag_count = a.flag_count;
  hipStream_t st = (hipStream_t)stream;
  ProfScope prof(st);
  hipError_t e = fs::launch_fused_filtered(a, fp64, fa, st);
  if (e != hipSuccess) return hip_fail(e, "fused filtered sampling launch");
  return FS_OK;
}

size_t fs_workspace_bytes_filtered(int64_t B, int64_t V) {
  if (B < 0 || V < 1 || V >= kMaxV) return 0;
  const size_t words = fs::filtered_split_words(B, V);
  if (words == 0) return 0;
  return kCounterBytes + words * sizeof(uint64_t);
}

fs_status fs_sample_logits_filtered(const float* logits, int64_t B, int64_t V, const float* temp,
                                    const int32_t* top_k, const float* top_p, const float* min_p,
                                    uint64_t seed, uint64_t offset, int fp64_noise,
                                    int64_t* out_idx, const uint32_t* row_ids, void* workspace,
                                    size_t workspace_bytes, fs_stream_t stream) {
  g_last_error[0] = 0;
  fs_status s = check_sizes(B, V);
  if (s != FS_OK) return s;
  if (B == 0) return FS_OK;
  if (logits == nullptr || temp == nullptr || out_idx == nullptr)
    return fail(FS_ERR_INVALID_ARG, "logits, temp or out_idx is null");
  if (((uintptr_t)logits & 3u) != 0) return fail(FS_ERR_UNSUPPORTED, "logits not 4-byte aligned");
  if (B >= ((int64_t)1 << 31)) return fail(FS_ERR_INVALID_ARG, "B = %lld exceeds 2^31 - 1", (long long)B);
  const size_t need = fs_workspace_bytes_filtered(B, V);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need)
      return fail(FS_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    if (((uintptr_t)workspace & (kAlign - 1)) != 0)
      return fail(FS_ERR_WORKSPACE, "workspace not %zu-byte aligned", (size_t)kAlign);
  }

  hipStream_t st = (hipStream_t)stream;
  ProfScope prof(st);
  fs::FilterArgs a;
  a.X = logits;
  a.B = B;
  a.V = V;
  a.temp = temp;
  a.row_ids = row_ids;
  a.top_k = top_k;
  a.top_p = top_p;
  a.min_p = min_p;
  a.key = fs::make_key(seed, offset);
  a.out = out_idx;
  a.vec4 = aligned16(logits) && (V % 4 == 0);
  a.counters = need > 0 ? static_cast<uint32_t*>(workspace) : nullptr;
  a.split = need > 0 ? reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + kCounterBytes)
                     : nullptr;
  a.Y = nullptr;
  a.row_flags = nullptr;
  a.flag_count = nullptr;
  hipError_t e = fs::launch_logits_filtered(a, fp64_noise != 0, st);
  if (e != hipSuccess) return hip_fail(e, "filtered sampling launch");
  return FS_OK;
}

fs_status fs_repetition_penalty(const float* logits, int64_t B, int64_t V,
                                const int64_t* prev_tokens, int64_t L, const float* penalty,
                                float* out_logits, fs_stream_t stream) {
  g_last_error[0] = 0;
  fs_status s = check_sizes(B, V);
  if (s != FS_OK) return s;
  if (B > 65535) return fail(FS_ERR_INVALID_ARG, "B = %lld exceeds 65535", (long long)B);
  if (L < 0) return fail(FS_ERR_INVALID_ARG, "L = %lld is negative", (long long)L);
  if (B == 0) return FS_OK;
  if (logits == nullptr || penalty == nullptr || out_logits == nullptr ||
      (L > 0 && prev_tokens == nullptr))
    return fail(FS_ERR_INVALID_ARG, "logits, prev_tokens, penalty or out_logits is null");
  if (((uintptr_t)logits & 3u) != 0 || ((uintptr_t)out_logits & 3u) != 0)
    return fail(FS_ERR_UNSUPPORTED, "logits or out_logits not 4-byte aligned");
  fs::PenaltyArgs a;
  a.X = logits;
  a.Y = out_logits;
  a.B = B;
  a.V = V;
  a.prev = prev_tokens;
  a.L = L;
  a.penalty = penalty;
  a.vec4 = aligned16(logits) && aligned16(out_logits) && (V % 4 == 0);
  hipStream_t st = (hipStream_t)stream;
  ProfScope prof(st);
  hipError_t e = fs::launch_repetition_penalty(a, st);
  if (e != hipSuccess) return hip_fail(e, "repetition penalty launch");
  return FS_OK;
}

fs_status fs_filter_logits(const float* logits, int64_t B, int64_t V, const float* temp,
                           const int32_t* top_k, const float* top_p, const float* min_p,
                           float* out_logits, fs_stream_t stream) {
  g_last_error[0] = 0;
  fs_status s = check_sizes(B, V);
  if (s != FS_OK) return s;
  if (B >= ((int64_t)1 << 31)) return fail(FS_ERR_INVALID_ARG, "B = %lld exceeds 2^31 - 1", (long long)B);
  if (B == 0) return FS_OK;
  if (logits == nullptr || temp == nullptr || out_logits == nullptr)
    return fail(FS_ERR_INVALID_ARG, "logits, temp or out_logits is null");
  if (((uintptr_t)logits & 3u) != 0 || ((uintptr_t)out_logits & 3u) != 0)
    return fail(FS_ERR_UNSUPPORTED, "logits or out_logits not 4-byte aligned");
  fs::FilterArgs a;
  a.X = logits;
  a.B = B;
  a.V = V;
  a.temp = temp;
  a.row_ids = nullptr;
  a.top_k = top_k;
  a.top_p = top_p;
  a.min_p = min_p;
  a.key = fs::make_key(0, 0);
  a.out = nullptr;
  a.vec4 = aligned16(logits) && aligned16(out_logits) && (V % 4 == 0);
  a.counters = nullptr;
  a.split = nullptr;
  a.Y = out_logits;
  a.row_flags = nullptr;
  a.flag_count = nullptr;
  hipStream_t st = (hipStream_t)stream;
  ProfScope prof(st);
  hipError_t e = fs::launch_filter_logits(a, st);
  if (e != hipSuccess) return hip_fail(e, "filter_logits launch");
  return FS_OK;
}

size_t fs_workspace_bytes_verify(int64_t B, int64_t K, int64_t V) {
  if (B < 0 || B > kVerifyMaxB || K < 0 || K > FS_VERIFY_MAX_K || V < 1 || V >= kMaxV) return 0;
  const int64_t nC = (V + fs::kVerifyChunk - 1) / fs::kVerifyChunk;  // most chunks of a row
  return kCounterBytes + align_up((size_t)B * 2 * K * nC * fs::verify_stat_bytes()) +
         align_up((size_t)B * nC * 16) + align_up((size_t)B * nC * 16);
}

fs_status fs_verify(const float* target, const float* draft, const int64_t* tokens, int64_t B,
                    int64_t K, int64_t V, const float* temp, uint64_t seed, uint64_t offset,
                    int fp64_noise, int64_t* accept_len, int64_t* out, const uint32_t* row_ids,
                    void* workspace, size_t workspace_bytes, fs_stream_t stream) {
  g_last_error[0] = 0;
  fs_status s = check_sizes(B, V);
  if (s != FS_OK) return s;
  if (B > kVerifyMaxB) return fail(FS_ERR_INVALID_ARG, "B = %lld exceeds %lld", (long long)B, (long long)kVerifyMaxB);
  if (K < 0 || K > FS_VERIFY_MAX_K)
    return fail(FS_ERR_INVALID_ARG, "K = %lld outside [0, %d]", (long long)K, FS_VERIFY_MAX_K);
  if (B == 0) return FS_OK;
  if (target == nullptr || temp == nullptr || accept_len == nullptr || out == nullptr ||
      (K > 0 && (draft == nullptr || tokens == nullptr)))
    return fail(FS_ERR_INVALID_ARG, "target, draft, tokens, temp, accept_len or out is null");
  if (((uintptr_t)target & 3u) != 0 || ((uintptr_t)draft & 3u) != 0)
    return fail(FS_ERR_UNSUPPORTED, "target or draft not 4-byte aligned");
  const size_t need = fs_workspace_bytes_verify(B, K, V);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(FS_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  if (((uintptr_t)workspace & (kAlign - 1)) != 0)
    return fail(FS_ERR_WORKSPACE, "workspace not %zu-byte aligned", (size_t)kAlign);

  fs::VerifyArgs a;
  a.target = target;
  a.draft = draft;
  a.tokens = tokens;
  a.B = B;
  a.K = K;
  a.V = V;
  a.temp = temp;
  a.row_ids = row_ids;
  a.seed = seed;
  a.offset = offset;
  fs::verify_chunks(B, K, V, &a.chunk, &a.nC, &a.chunk2, &a.nC2);
  if (B * (2 * K + 1) * a.nC >= ((int64_t)1 << 31) || B * a.nC2 >= ((int64_t)1 << 31))
    return fail(FS_ERR_INVALID_ARG, "B, K, V give more than 2^31 workgroups");
  char* w = static_cast<char*>(workspace);
  const int64_t nCmax = (V + fs::kVerifyChunk - 1) / fs::kVerifyChunk;
  a.counters = counters_of(workspace);
  w += kCounterBytes;
  a.stats = w;
  w += align_up((size_t)B * 2 * K * nCmax * fs::verify_stat_bytes());
  a.bonus = w;
  w += align_up((size_t)B * nCmax * 16);
  a.resid = w;
  a.accept_len = accept_len;
  a.out = out;
  a.vec4 = aligned16(target) && (K == 0 || aligned16(draft)) && (V % 4 == 0);

  hipStream_t st = (hipStream_t)stream;
  ProfScope prof(st);
  hipError_t e = fs::launch_verify(a, fp64_noise != 0, st);
  if (e != hipSuccess) return hip_fail(e, "verify launch");
  return FS_OK;
}

fs_status fs_sample_logits_topk(const float* logits, int64_t B, int64_t V, const float* temp,
                                uint64_t seed, uint64_t offset, int fp64_noise, int k,
                                int64_t* out_idx, const uint32_t* row_ids, void* workspace,
                                size_t workspace_bytes, fs_stream_t stream) {
  g_last_error[0] = 0;
  fs_status s = check_sizes(B, V);
  if (s != FS_OK) return s;
  if (k < 1 || k > fs::kTopKMax)
    return fail(FS_ERR_INVALID_ARG, "k = %d outside [1, %d]", k, fs::kTopKMax);
  if (B == 0) return FS_OK;
  if (logits == nullptr || temp == nullptr || out_idx == nullptr)
    return fail(FS_ERR_INVALID_ARG, "logits, temp or out_idx is null");
  if (((uintptr_t)logits & 3u) != 0) return fail(FS_ERR_UNSUPPORTED, "logits not 4-byte aligned");
  const int nT = logits_tiles(V);
  if ((int64_t)B * nT * fs::kTopKMax >= ((int64_t)1 << 31))
    return fail(FS_ERR_INVALID_ARG, "B * ceil(V / %d) * %d exceeds 2^31", fs::kLogitsChunk,
                fs::kTopKMax);
  const uint32_t flags = fp64_noise ? FS_FP64_NOISE : 0u;
  s = check_workspace(workspace, workspace_bytes, B, V, flags, true);
  if (s != FS_OK) return s;

  hipStream_t st = (hipStream_t)stream;
  ProfScope prof(st);
  for (int64_t b0 = 0; b0 < B; b0 += kCounterWords) {
    const int64_t nb = B - b0 < kCounterWords ? B - b0 : kCounterWords;
    fs::LogitsArgs a;
    a.X = logits + b0 * V;
    a.B = nb;
    a.V = V;
    a.temp = temp + b0;
    a.row_ids = row_ids ? row_ids + b0 : nullptr;
    a.rid_base = (uint32_t)b0;
    a.key = fs::make_key(seed, offset);
    a.cand = candidates_of(workspace);
    a.chunk = fs::logits_chunk(nb, V);
    a.nT = (int)((V + a.chunk - 1) / a.chunk);
    a.counters = counters_of(workspace);
    a.out = out_idx + b0 * k;
    a.vec4 = aligned16(logits) && (V % 4 == 0);
    a.k = k;
    hipError_t e = fs::launch_logits_topk(a, fp64_noise != 0, st);
    if (e != hipSuccess) return hip_fail(e, "logits top-k launch");
  }
  return FS_OK;
}

fs_status fs_profile_begin(void) {
  g_last_error[0] = 0;
  std::lock_guard<std::mutex> lock(g_prof.mu);
  g_prof.on = true;
  g_prof.used = 0;
  return FS_OK;
}

fs_status fs_profile_end_detail(double* kernel_ms, int64_t* calls, float* launch_ms,
                                float* start_to_start_ms, int64_t cap) {
  g_last_error[0] = 0;
  std::lock_guard<std::mutex> lock(g_prof.mu);
  double total = 0.0;
  fs_status status = FS_OK;
  for (size_t c = 0; c < g_prof.used; ++c) {
    hipEvent_t* ev = &g_prof.pool[2 * c];
    float ms = 0.f, gap = 0.f;
    hipError_t e = hipEventSynchronize(ev[1]);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev[0], ev[1]);
    if (e == hipSuccess && start_to_start_ms && (int64_t)c + 1 < cap && c + 1 < g_prof.used) {
      e = hipEventSynchronize(ev[3]);
      if (e == hipSuccess) e = hipEventElapsedTime(&gap, ev[0], ev[2]);
    }
    if (e != hipSuccess) {
      status = hip_fail(e, "profile events");
      break;
    }
    total += ms;
    if (launch_ms && (int64_t)c < cap) launch_ms[c] = ms;
    if (start_to_start_ms && (int64_t)c + 1 < cap && c + 1 < g_prof.used) start_to_start_ms[c] = gap;
  }
  if (kernel_ms) *kernel_ms = total;
  if (calls) *calls = (int64_t)g_prof.used;
  g_prof.on = false;
  g_prof.used = 0;
  return status;
}

fs_status fs_profile_end(double* kernel_ms, int64_t* calls) {
  return fs_profile_end_detail(kernel_ms, calls, nullptr, nullptr, 0);
}

int fs_fused_tiles(int64_t B, int64_t D, int64_t V, int weight_format) {
  g_last_error[0] = 0;
  if (B < 0 || D < 1 || V < 1 || V >= kMaxV || weight_format < 0 || weight_format > 2) {
    fail(FS_ERR_INVALID_ARG, "fs_fused_tiles: invalid sizes or weight format");
    return -1;
  }
  int cus = 0;
  if (device_cus(&cus) != FS_OK) return -1;
  return fs::fused_call_tiles(B, D, V, weight_format == kFmtBf16, cus, row_bytes(D, weight_format));
}

fs_status fs_debug_stream_read(const void* buf, size_t bytes, uint64_t* out, fs_stream_t stream) {
  g_last_error[0] = 0;
  if (out == nullptr || (bytes > 0 && buf == nullptr))
    return fail(FS_ERR_INVALID_ARG, "buf or out is null");
  if (!aligned16(buf) || (bytes & 15u) != 0)
    return fail(FS_ERR_UNSUPPORTED, "buf must be 16-byte aligned and a multiple of 16 bytes");
  int cus = 0;
  fs_status s = device_cus(&cus);
  if (s != FS_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  ProfScope prof(st);
  hipError_t e = fs::launch_stream_read(buf, bytes, cus, out, st);
  if (e != hipSuccess) return hip_fail(e, "stream read launch");
  return FS_OK;
}

fs_status fs_debug_philox_words(uint64_t seed, uint64_t offset, const uint32_t* row_ids,
                                int64_t B, int64_t n_ctr, uint32_t* out, fs_stream_t stream) {
  g_last_error[0] = 0;
  if (B < 0 || n_ctr < 0) return fail(FS_ERR_INVALID_ARG, "negative size");
  if (B == 0 || n_ctr == 0) return FS_OK;
  if (B > (((int64_t)1 << 31) - 1) / n_ctr) return fail(FS_ERR_INVALID_ARG, "B * n_ctr >= 2^31");
  if (out == nullptr) return fail(FS_ERR_INVALID_ARG, "out is null");
  if (!aligned16(out)) return fail(FS_ERR_UNSUPPORTED, "out not 16-byte aligned");
  hipError_t e = fs::launch_philox_words(fs::make_key(seed, offset), row_ids, B, n_ctr, out,
                                         (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "philox words launch");
  return FS_OK;
}

fs_status fs_debug_noise(const uint32_t* words, int64_t n, int fp64, double* E, double* g,
                         fs_stream_t stream) {
  g_last_error[0] = 0;
  if (n < 0 || n >= ((int64_t)1 << 31)) return fail(FS_ERR_INVALID_ARG, "n = %lld", (long long)n);
  if (n == 0) return FS_OK;
  if (words == nullptr || E == nullptr || g == nullptr)
    return fail(FS_ERR_INVALID_ARG, "words, E or g is null");
  hipError_t e = fs::launch_noise(words, n, fp64 != 0, E, g, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "noise launch");
  return FS_OK;
}

fs_status fs_debug_logits(const fs_bf16* H, const fs_bf16* W, int64_t B, int64_t D, int64_t V,
                          float* Y, fs_stream_t stream) {
  g_last_error[0] = 0;
  return debug_logits(H, W, kFmtBf16, nullptr, B, D, V, Y, stream);
}

fs_status fs_debug_logits_w8(const fs_bf16* H, const uint8_t* W8, const float* w_scale, int64_t B,
                             int64_t D, int64_t V, float* Y, fs_stream_t stream) {
  g_last_error[0] = 0;
  return debug_logits(H, W8, kFmtFp8, w_scale, B, D, V, Y, stream);
}

fs_status fs_debug_logits_mxfp4(const fs_bf16* H, const uint8_t* W4, const uint8_t* w4_scale,
                                int64_t B, int64_t D, int64_t V, float* Y, fs_stream_t stream) {
  g_last_error[0] = 0;
  return debug_logits(H, W4, kFmtMxfp4, w4_scale, B, D, V, Y, stream);
}

}  // extern "C"
