// moe_decode_stack_static: moe_decode_stack on a workspace that lives in the
// library itself, for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The workspace is the file-scope device array `scratch` (kScratchBytes, one
// copy per GPU, held until the process ends). Host code never passes the
// array's name to a kernel: in host code that name is a host-side stand-in,
// not a device address. Instead, on the first call on each device (with that
// device current) hipGetSymbolAddress gives the array's address on that
// device, which is kept per device and passed on as the workspace pointer.
// Nothing here allocates: no hipMalloc / hipFree and no allocating library
// routine. What a call needs zeroed (the exchange words and status word of
// the streaming stack kernel) is cleared by the launches themselves.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace moe {
namespace {

constexpr size_t kScratchBytes = size_t(4) << 20;  // 4 MiB
constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device id (nullptr: not looked up yet)

}  // namespace
}  // namespace moe

static __device__ __align__(256) uint8_t scratch[moe::kScratchBytes];

namespace moe {
namespace {

// Address of this device's copy of `scratch` (looked up once per device).
int32_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return set_error(MOE_ERR_UNSUPPORTED, "device %d beyond the scratch table", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(MOE_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int32_t moe_decode_stack_static(const moe_shape_t* shape, const void* const* layers_host, int32_t n_layers,
                                           int32_t T, const uint16_t* h_in_dev, uint16_t* h_out_dev, int32_t* ids_dev,
                                           float* w_dev, uint16_t* h_trace_dev, moe_stream_t stream) {
  clear_error();
  int32_t rc = check_shape(shape);
  if (rc) return rc;
  if (T < 1 || T > kMaxT) return set_error(MOE_ERR_INVALID_ARG, "T %d not in [1, %d]", T, kMaxT);
  const int64_t need = ws_map(*shape, T).total;
  if (need > (int64_t)kScratchBytes)
    return set_error(MOE_ERR_WORKSPACE, "this shape at T = %d needs %lld bytes of workspace; the static scratch holds %zu",
                     T, (long long)need, kScratchBytes);
  void* ws = nullptr;
  if ((rc = scratch_ptr(&ws))) return rc;
  return decode_stack_ws(shape, layers_host, n_layers, T, h_in_dev, h_out_dev, ids_dev, w_dev, h_trace_dev, ws,
                         kScratchBytes, stream);
}
