// noalloc.hip -- patch_gemm_noalloc: the hybrid GEMM with its scratch in a
// file-scope device array, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).
//
// The only scratch the GEMM path uses is the prefill kernel's K split: the
// fp32 partial sums of the K ranges ([splits][M][N] floats), written in full
// by the GEMM kernel and read by the ordered reduction that follows it on
// the same stream.  Nothing in it has to start at zero, so no call clears
// it.  Every call on a device shares that device's array: calls that
// overlap on one device (concurrent streams, threads) race.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <mutex>

#include "patch.h"

namespace patch {
// sets the text patch_last_error() returns on this thread (patch_api.cpp)
patch_status set_last_error(patch_status s, const char* msg);
}  // namespace patch

namespace {

constexpr uint64_t kScratchBytes = uint64_t(64) << 20;  // 64 MiB a device

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// The array's device address, per device.  In host code `scratch` names a
// host-side stand-in, not device memory: only this address may be passed to
// kernels.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

// the scratch address on the current device, looked up once per device
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

thread_local char g_msg[256];

}  // namespace

extern "C" {

uint64_t patch_noalloc_scratch_bytes(void) { return kScratchBytes; }

patch_status patch_gemm_noalloc(const patch_packed_desc* desc, const void* packed_dev, const void* X_dev, int64_t M,
                                void* Y_dev, patch_dtype y_dtype, void* stream) {
  if (!desc) return patch_gemm(desc, packed_dev, X_dev, M, Y_dev, y_dtype, nullptr, 0, stream);
  // the scratch this shape's launch wants (0: no K split); host arithmetic
  const uint64_t want = patch_gemm_workspace_bytes(desc, M);
  if (want > kScratchBytes) {
    std::snprintf(g_msg, sizeof g_msg,
                  "patch_gemm_noalloc: M=%lld N=%u K=%u wants %llu bytes of scratch, the library holds %llu",
                  (long long)M, desc->N, desc->K, (unsigned long long)want, (unsigned long long)kScratchBytes);
    return patch::set_last_error(PATCH_ERR_BUFFER_TOO_SMALL, g_msg);
  }
  void* ws = nullptr;
  if (want > 0) {
    hipError_t e = scratch_ptr(&ws);
    if (e != hipSuccess) {
      std::snprintf(g_msg, sizeof g_msg, "patch_gemm_noalloc: scratch address: %s", hipGetErrorString(e));
      return patch::set_last_error(PATCH_ERR_HIP, g_msg);
    }
  }
  return patch_gemm(desc, packed_dev, X_dev, M, Y_dev, y_dtype, ws, want, stream);
}

}  // extern "C"
