// Allocation-free forward (cgtp_conv_forward_static): the channelwise forward of cgtp_conv_forward
// with its per-chunk G rows in a file-scope device array instead of a caller workspace, for callers
// that cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).
//
// `scratch` is a static device array of kStaticScratchBytes; every GPU the library runs on holds
// its own copy until the process ends.  In host code its name is only a host-side stand-in, so the
// device address of each GPU's copy is looked up once per device (hipGetSymbolAddress with that
// device current) and kept; kernels receive that address, never the name.  Calls on one GPU share
// its copy: calls that overlap in time on one GPU (two streams) race on it.  The forward writes
// every row it later reads (the prep kernel fills a chunk's rows before the contraction reads them),
// so nothing in the array needs clearing between calls.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <string>

#include "cgtp.h"
#include "errors.hpp"
#include "forward.hpp"

namespace {

constexpr size_t kStaticScratchBytes = CGTP_STATIC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;  // device ordinal -> address of that device's `scratch`

// Address of the current device's copy of `scratch`, looked up on the first call per device.
cgtp_status_t device_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return cgtp::set_error(CGTP_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *out = it->second;
    return CGTP_OK;
  }
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || ptr == nullptr)
    return cgtp::set_error(CGTP_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
  g_scratch_ptr[dev] = ptr;
  *out = ptr;
  return CGTP_OK;
}

}  // namespace

extern "C" {

cgtp_status_t cgtp_conv_forward_static(cgtp_plan_t plan, cgtp_graph_t g, cgtp_schedule_t schedule, const void* x,
                                       const void* pos, const void* shift, const void* phi, const void* A, void* out,
                                       void* stream) {
  if (!plan || !g) return cgtp::set_error(CGTP_ERR_INVALID_ARG, "null plan or graph");
  void* ptr = nullptr;
  cgtp_status_t st = device_scratch(&ptr);
  if (st != CGTP_OK) return st;
  return cgtp::forward_in_scratch(plan, g, schedule, x, pos, shift, phi, A, out, ptr, kStaticScratchBytes, stream);
}

}  // extern "C"
