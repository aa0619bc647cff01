// A fixed device workspace for tkv_attend_decode_noalloc: the plan and the
// split-K partial records of a decode call, in a file-scope device array, so
// that the call itself allocates no device memory.
//
// Each GPU the library runs on holds its own copy of the array, from the first
// cache created on it until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol):
// the device address is looked up once per device with hipGetSymbolAddress,
// with that device current, and only that address is used.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace tkv {

static __device__ __align__(256) char scratch[kStaticWorkspaceBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

int static_workspace_init(int device) {
  if (device < 0 || device >= kMaxDevices) return -1;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_ptr[device]) return 0;
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) return -1;
  if (prev != device && hipSetDevice(device) != hipSuccess) return -1;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (prev != device) (void)hipSetDevice(prev);
  if (e != hipSuccess || p == nullptr) return -1;
  g_ptr[device] = p;
  return 0;
}

void* static_workspace(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  return g_ptr[device];
}

}  // namespace tkv
