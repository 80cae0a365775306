// Library-owned device scratch for gca_retrieve_noalloc: the per-slice partial
// top-k keys of a sliced retrieval live in a file-scope device array instead of
// a caller workspace, so that call allocates nothing.
//
// Host code never passes `scratch` itself to a kernel: on the host that name
// is only a stand-in for the symbol.  Its device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and kept; every GPU
// holds its own copy of the array at its own address, for the life of the
// process.

#include <mutex>

#include "gca_launch.h"

namespace gca {

static __device__ __align__(256) uint64_t scratch[kScratchBytes / sizeof(uint64_t)];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

}  // namespace

hipError_t scratch_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace gca
