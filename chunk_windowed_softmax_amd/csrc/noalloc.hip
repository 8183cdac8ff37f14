// Static device workspace of wa_forward_noalloc: one file-scope device array per GPU,
// reached from host code only through the address hipGetSymbolAddress returns for the
// current device (the array's name in host code is a host-side stand-in, not a device
// address).
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace wa {
namespace {

// The workspace: plan tables (work items, launch order, queue counters), the global leg's
// partial results and, for fp32 inputs, their bf16 staging copies.  Every GPU that runs
// the library holds its own copy until the process ends.
__device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_workspace(int device, void** ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[device]) {
    // once per device, with that device current (the caller's current device)
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[device] = p;
  }
  *ptr = g_ptr[device];
  return hipSuccess;
}

}  // namespace wa
