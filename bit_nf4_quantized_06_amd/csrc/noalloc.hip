// qlora_linear_fwd_noalloc: the forward of the linear layer for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  It takes the workspace from a
// fixed device array of this library instead of a caller buffer; the caller
// still passes inputs and outputs, and nothing here allocates or frees.
//
// The array, `scratch`, is a file-scope __device__ object: every GPU the
// library runs on holds its own copy (kScratchBytes) until the process ends.
// Host code never uses its name as an address (on the host that name is only
// a stand-in); the device address comes from hipGetSymbolAddress, resolved
// once per device with that device current, and is kept per device.  All
// calls on one GPU share that GPU's array and it keeps the last call's
// contents: the forward's kernels fully overwrite the parts they read (split
// partials, the rounded U; the GEMM's arrival counters are zeroed by the
// launch before it), so nothing needs clearing, but calls that overlap on
// one GPU (two streams at once) race on it.  When the fused GEMM's K-split
// partials would not fit, the forward runs the plain tile schedule (same
// results up to the float32 summation order of those tiles).  The weight is
// always decoded inside the GEMM here: its 16-bit copy (2 bytes a weight)
// would not fit the array for any but small weights.
#include <hip/hip_runtime.h>

#include <mutex>

#include "abi_internal.h"
#include "qlora_nf4.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;   // 32 MiB per device
constexpr int kMaxDevices = 64;

__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device (guarded)

// The device address of this device's scratch array (resolved on first use).
qlora_status scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    qlora::set_last_hip_error((int)e);
    return QLORA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return QLORA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      qlora::set_last_hip_error((int)e);
      return QLORA_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return QLORA_OK;
}

}  // namespace

extern "C" {

size_t qlora_linear_fwd_noalloc_max_scratch(void) { return kScratchBytes; }

qlora_status qlora_linear_fwd_noalloc(const qlora_nf4_weight* w, const uint16_t* X, int64_t T,
                                      const uint16_t* A, const uint16_t* B, int32_t r,
                                      float alpha, uint16_t* Y, uint16_t* U_save, void* stream) {
  using namespace qlora;
  // the sizes first: a call whose workspace would not fit is rejected before
  // any device work
  WeightDims d;
  qlora_status s = check_linear_args(w, T, r, alpha, &d);
  if (s != QLORA_OK) return s;
  if (T == 0)   // an empty batch needs no workspace
    return qlora_linear_fwd(w, X, T, A, B, r, alpha, Y, U_save, nullptr, 0, stream);
  // the fused GEMM's K-split of its last tiles when its partials fit, else
  // the plain tile schedule
  const bool split = linear_ws_layout(T, d, r, false, false, true, false).total <= kScratchBytes;
  if (!split && linear_ws_layout(T, d, r, false, false, false, false).total > kScratchBytes)
    return QLORA_ERR_SCRATCH;
  s = check_device();
  if (s != QLORA_OK) return s;
  void* ws = nullptr;
  s = scratch_for_current_device(&ws);
  if (s != QLORA_OK) return s;
  return linear_fwd_impl(w, X, T, A, B, r, alpha, Y, U_save, ws, kScratchBytes, stream, split,
                         false);
}

}  // extern "C"
