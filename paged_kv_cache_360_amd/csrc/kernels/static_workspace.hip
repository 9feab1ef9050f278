// A library-owned decode workspace in device memory that no call allocates:
// a file-scope device array of fixed size.  Each GPU the library runs on holds
// its own copy until the process ends.
//
// In host code the array's name is only a host-side stand-in; its device
// address differs per device and is taken once per device, with that device
// current, by hipGetSymbolAddress.  Every use from host code (kernel
// arguments) goes through that address.

#include <hip/hip_runtime.h>

#include <cstddef>
#include <mutex>

#include "../../../include/pagedkv.h"
#include "../pkv_internal.hpp"

namespace pkv {

namespace {

constexpr size_t kStaticWorkspaceBytes = PKV_STATIC_WORKSPACE_BYTES;

static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

size_t static_workspace_capacity() { return kStaticWorkspaceBytes; }

int static_workspace(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return e != hipSuccess ? (int)e : (int)hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  *out = g_addr[dev];
  return 0;
}

}  // namespace pkv
