// Scratch memory for the paged decode entry point that allocates nothing
// (attn_decode_paged_noalloc): the split partials of the decode live in a
// file-scope device array instead of a caller-provided workspace.
//
// Each GPU the library runs on holds its own copy of the array for the rest of
// the process.  In host code `scratch` names a host-side stand-in, not a
// device address, so the array's device address is looked up once per
// device (with that device current) and only that address is ever handed to
// kernels.  The decode kernels need no part of the array cleared: every
// partial result is written before it is read, and the counts are written by
// the workgroup that owns them, so stale contents of an earlier call do no
// harm.  Calls that overlap on one GPU share the array and race.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "kernels.h"

namespace attn {
namespace {

static __device__ __align__(256) unsigned char scratch[kDecodeNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

hipError_t decode_noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = (g_err[dev] == hipSuccess) ? p : nullptr;
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  *ptr = g_ptr[dev];
  return *ptr ? hipSuccess : hipErrorInvalidSymbol;
}

}  // namespace attn
