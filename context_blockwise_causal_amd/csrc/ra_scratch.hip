// The static scratch of ra_chunk_bwd_ds_noalloc and the lookup of its device address.  The array
// and the hipGetSymbolAddress call that resolves it live in this one source file; the kernels
// that use the memory (kern_bwd.hip) take the resolved address as an argument, like the caller's
// scratch of ra_chunk_bwd_ds.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ra_internal.h"

namespace ra {

// Scratch of ra_chunk_bwd_ds_noalloc (the stored dS of one call): one copy per GPU, held until the
// process ends.  Host code never uses this name as an address: noalloc_scratch_address returns
// the device address of each GPU's copy.
static __device__ __align__(256) unsigned char scratch[RA_NOALLOC_SCRATCH_BYTES];

int noalloc_scratch_address(int device, void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    void* p = nullptr;  // the calling thread has `device` current
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    addr[device] = p;
  }
  *out = addr[device];
  return 0;
}

}  // namespace ra
