// Library-held device scratch for paged_attn_decode_noalloc: the split-K
// partial results of paged_attn_decode live in this file-scope array instead
// of a caller-allocated workspace, for callers that cannot allocate device
// memory (code under graph capture, tight serving loops).  Every GPU the
// library runs on holds one copy of the array, at its own address, until the
// process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address comes from hipGetSymbolAddress, looked up once per device
// with that device current and kept here; only that address is ever passed
// to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/attn.h"

namespace attn {

// Largest scratch a call may use (ATTN_DECODE_SCRATCH_BYTES, 40 MiB): the
// partials of 2,048 persistent waves for up to 16 query heads per KV head at
// head_dim 128 (32.5 MiB), plus the per-(sequence, KV head) records.
constexpr size_t kScratchBytes = ATTN_DECODE_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

size_t scratch_capacity() { return kScratchBytes; }

// Device address of `scratch` on `device`, looked up on first use (with that
// device made current for the lookup) and cached.  Returns the HIP status.
hipError_t scratch_address(int device, void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  *out = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[device] == nullptr) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != device) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    addr[device] = ptr;
  }
  *out = addr[device];
  return hipSuccess;
}

}  // namespace attn
