// Allocation-free variant of the backward: the workspace is a fixed
// file-scope device array instead of a caller buffer, for callers that
// cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// Each GPU the library runs on holds its own copy of `scratch` (from the
// code object's load on that device until the process ends).  Host code
// never passes the array's name to a kernel or a copy: the name is a
// host-side stand-in.  The device address comes from hipGetSymbolAddress,
// taken once per device with that device current, and kept per device.
#include <mutex>

#include "../../include/sparse_attn.h"

#include <hip/hip_runtime.h>

namespace sa {
sa_status_t bwd_entry(const sa_desc_t* desc, const sa_bwd_args_t* a, void* workspace, size_t workspace_bytes,
                      void* stream, void* ev_main_start, void* ev_main_stop, int allow_side);
}

namespace {

constexpr size_t kScratchBytes = size_t(128) << 20;   // 128 MiB per GPU
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices];   // device address of `scratch` on each device (null: not looked up yet)

// The device `stream` runs on (the current device for the null stream).
hipError_t stream_device(hipStream_t stream, int* dev) {
  if (!stream) return hipGetDevice(dev);
  hipDevice_t d;
  const hipError_t e = hipStreamGetDevice(stream, &d);
  if (e == hipSuccess) *dev = (int)d;
  return e;
}

// Address of this device's `scratch`, looked up on the first call on the
// device with that device current (the caller's current device restored).
sa_status_t scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return SA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return SA_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return SA_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return SA_ERR_HIP;
    if (e != hipSuccess || !p) return SA_ERR_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return SA_OK;
}

}  // namespace

extern "C" {

sa_status_t sparse_attn_bwd_noalloc(const sa_desc_t* desc, const sa_bwd_args_t* args, void* stream) {
  size_t need = 0;
  sa_status_t st = sparse_attn_bwd_workspace_size(desc, &need);
  if (st != SA_OK) return st;
  if (need > kScratchBytes) return SA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int dev = -1;
  if (stream_device(s, &dev) != hipSuccess) return SA_ERR_HIP;
  void* ws = nullptr;
  st = scratch_address(dev, &ws);
  if (st != SA_OK) return st;
  // the same launch sequence as sparse_attn_bwd, every launch on the
  // caller's stream (no library-owned stream), on the fixed workspace; it
  // clears whatever must start at zero itself (it never relies on the
  // contents a previous call left)
  return sa::bwd_entry(desc, args, ws, kScratchBytes, stream, nullptr, nullptr, 0);
}

}  // extern "C"
