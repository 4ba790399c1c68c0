// Static device scratch for pka_run_noalloc: the split-KV partial states
// (fp32 partial O rows, then their lse) of a run live in this file-scope
// array instead of the plan's float workspace, so that a caller that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc) needs no float workspace for its runs.
//
// Every GPU holds its own copy of the array, at its own address, from the
// moment the library's code object is loaded on it until the process ends.
// Host code never uses the array's name as an address: the device address
// is looked up once per device with hipGetSymbolAddress, with that device
// current, and kept.  All runs on one GPU share the array, and it keeps the
// last run's contents; nothing in it must start at zero (every partial row
// is written by its unit before the merge reads it), but runs that overlap on
// one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace pka {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // the current device's copy
    if (e != hipSuccess) return e;
    g_addr[dev] = p;
  }
  *out = g_addr[dev];
  return hipSuccess;
}

}  // namespace pka
