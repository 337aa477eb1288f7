// fa_bwd_noalloc: the backward of fa_bwd with its workspace in a file-scope device array instead
// of caller memory, for callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).  It enqueues exactly the kernels fa_bwd
// enqueues; only the workspace's address differs.
//
// The array is one per GPU the library runs on (the code object's device globals), held until
// the process ends.  Its address is taken once per device with hipGetSymbolAddress while that
// device is current; host code never uses the array's name as a device address.
#include "../../include/fa.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

namespace {

static_assert(FA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size is a multiple of the alignment");
__device__ __align__(256) char scratch[FA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_init;

// The device address of `scratch` on `dev`, resolved on the first call for that device with the
// device made current (and the caller's current device restored); nullptr on failure.
void* scratch_on(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_init);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (p != nullptr) return p;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* addr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
  if (cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess || addr == nullptr) return nullptr;
  g_scratch[dev].store(addr, std::memory_order_release);
  return addr;
}

}  // namespace

extern "C" int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t Hq,
                              int64_t Hkv, int64_t N, int64_t D, float softmax_scale, int causal, int dtype,
                              void* stream) {
  const size_t need = fa_bwd_workspace_size(B, Hq, Hkv, N, D);
  if (need == 0) {  // invalid shape: fa_bwd reports which check failed, before anything is enqueued
    return fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, nullptr, 0, B, Hq, Hkv, N, D, softmax_scale, causal, dtype,
                  stream);
  }
  if (need > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  int dev = -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((s == nullptr ? hipGetDevice(&dev) : hipStreamGetDevice(s, &dev)) != hipSuccess) return FA_ERR_HIP;
  void* const ws = scratch_on(dev);
  if (ws == nullptr) return FA_ERR_HIP;
  return fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, (size_t)FA_NOALLOC_SCRATCH_BYTES, B, Hq, Hkv, N, D,
                softmax_scale, causal, dtype, stream);
}
