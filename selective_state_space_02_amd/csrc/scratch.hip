// scratch.hip -- device scratch of the allocation-free entry point (ssm_scan_fwd_noalloc).
//
// The scan's scratch (the fp32 B/C tiles, the time-segment aggregates) lives in one
// statically sized device array per GPU instead of a caller workspace or a stream-ordered
// allocation, for callers that cannot allocate.  Its device address is looked up once per
// device (with that device current) and kept; host code never passes the array's own name
// to a kernel, since on the host that name is only a stand-in for the symbol.
//
// Nothing in the scratch has to start at zero: every kernel that reads a scratch region
// reads only what an earlier kernel of the same call wrote there.  All calls on one GPU
// share its array, so calls that overlap in time on one GPU (two streams, two threads)
// race on it.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "scan_plan.h"

namespace ssm {
namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;   // 32 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

size_t scratch_capacity() { return kScratchBytes; }

int scratch_address(void** out, char* msg, size_t msg_len) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    std::snprintf(msg, msg_len, "hipGetDevice: %s", hipGetErrorString(e));
    return SSM_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    std::snprintf(msg, msg_len, "device %d beyond the %d devices the static scratch table covers", dev, kMaxDevices);
    return SSM_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      std::snprintf(msg, msg_len, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      return SSM_ERR_HIP;
    }
    g_addr[dev] = p;
  }
  *out = g_addr[dev];
  return SSM_OK;
}

}  // namespace ssm
