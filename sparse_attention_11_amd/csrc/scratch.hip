// scratch.hip -- the library's static device scratch buffer, for the entry
// point that allocates nothing (dsa_sparse_attn_decode_noalloc).
//
// The buffer is a file-scope __device__ array: every GPU the library runs on
// holds its own copy from module load until the process ends. In host code
// the array's name is only a host-side stand-in, never a device address, so
// host code obtains each device's address once, with that device current,
// through hipGetSymbolAddress, and uses that address everywhere (kernel
// arguments, copies). All calls on one GPU share its copy.
#include <mutex>

#include "kernels.h"

namespace dsa {
namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace dsa
