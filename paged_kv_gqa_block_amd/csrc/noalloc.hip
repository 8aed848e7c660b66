// The device array behind pkv_attend_noalloc (noalloc_api.cpp): the partial
// states of the allocation-free decode step live here instead of in caller
// buffers.
//
// `scratch` is a file-scope device variable: every GPU the library runs on
// holds its own copy (PKV_NOALLOC_SCRATCH_BYTES) until the process ends.
// Host code never passes the variable's name to a kernel -- on the host that
// name is only a stand-in -- but the device address that hipGetSymbolAddress
// returns for it, looked up once per device (with that device current) and
// kept in g_scratch.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pkv_internal.h"
#include "selfplan_args.h"

namespace pkv {
namespace {

static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

pkv_status noalloc_scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return PKV_ERANGE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PKV_EHIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return PKV_OK;
}

}  // namespace pkv
