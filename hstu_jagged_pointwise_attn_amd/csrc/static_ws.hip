// hstu_attn_fwd_static: the forward of the attention core with its scratch
// (schedule header, per-sequence descriptors, query-tile offsets and tile
// records) in a static device array instead of a caller workspace, for
// callers that cannot allocate device memory. It runs the same scheduler,
// attention and norm kernels as hstu_attn_fwd.
//
// The array is file-scope device memory: every GPU the library runs on holds
// its own copy, at its own address, until the process ends. In host code the
// array's name is only a host-side stand-in, so its device address is taken
// once per device with hipGetSymbolAddress (with that device current) and
// only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/hstu.h"
#include "hstu_internal.h"

namespace {

constexpr size_t kStaticScratchBytes = size_t(4) << 20;  // 4 MiB per device
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

struct DeviceScratch {
  std::once_flag once;
  hipError_t err = hipSuccess;
  void *ptr = nullptr;
};
DeviceScratch g_scratch[kMaxDevices];

}  // namespace

extern "C" size_t hstu_static_scratch_bytes(void) { return kStaticScratchBytes; }

extern "C" hstu_status_t hstu_attn_fwd_static(const hstu_problem_t *p, const void *Q, const void *K, const void *V,
                                              const void *U, void *Y, void *O, float *mean, float *rstd,
                                              void *stream) {
  if (!p) return hstu::set_last_error(HSTU_ERR_INVALID_ARG, "problem is NULL");
  size_t need = 0;
  hstu_status_t s = hstu_workspace_size(p, HSTU_OP_FWD, 0, 0, 0, &need);
  if (s) return s;
  if (need > kStaticScratchBytes) {
    char msg[160];
    snprintf(msg, sizeof msg, "problem needs %zu bytes of scratch; the static scratch holds %zu (B = %d, T = %lld)",
             need, kStaticScratchBytes, p->B, (long long)p->total_tokens);
    return hstu::set_last_error(HSTU_ERR_WORKSPACE, msg);
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hstu::set_last_error(HSTU_ERR_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return hstu::set_last_error(HSTU_ERR_UNSUPPORTED, "device index out of range");
  DeviceScratch &ds = g_scratch[dev];
  std::call_once(ds.once, [&] { ds.err = hipGetSymbolAddress(&ds.ptr, HIP_SYMBOL(scratch)); });
  if (ds.err != hipSuccess || !ds.ptr) {
    char msg[160];
    snprintf(msg, sizeof msg, "hipGetSymbolAddress of the static scratch on device %d: %s", dev,
             hipGetErrorString(ds.err));
    return hstu::set_last_error(HSTU_ERR_HIP, msg);
  }
  return hstu_attn_fwd(p, Q, K, V, U, Y, O, mean, rstd, ds.ptr, kStaticScratchBytes, stream);
}
