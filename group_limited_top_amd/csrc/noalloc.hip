// noalloc.hip -- moe_layer_forward_noalloc: the layer forward with its
// workspace in a static per-device buffer, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).
//
// The buffer is a file-scope __device__ array: every GPU the library runs on
// holds its own copy at its own address until the process ends.  In host code
// the array's name is only a stand-in for the symbol, so its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address is ever passed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe.h"

#include "layer_check.h"

namespace {

__device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_err[kMaxDevices];

// Device address of the current device's copy of `scratch`, looked up on the
// first call on that device and kept for the process's lifetime.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = p;
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  if (!g_scratch[dev]) return hipErrorInvalidSymbol;
  *out = g_scratch[dev];
  return hipSuccess;
}

// The status word (the first 256 bytes of a workspace) accumulates flags and
// must start at zero: cleared by a kernel, not a memset, so that a captured
// graph holds no memset node.
__global__ void k_clear_status(uint32_t* status) { status[threadIdx.x] = 0u; }

}  // namespace

extern "C" int moe_layer_forward_noalloc(const moe_desc_t* desc, const void* x,
                                         const moe_weights_t* weights, void* y,
                                         int32_t* topk_idx_out, float* topk_w_out,
                                         float* logits_out, int32_t* counts_out,
                                         int64_t* tracking, hipStream_t stream) {
  // checks that need no device: the desc, its flags and its scratch size
  int rc = moe::validate_desc(desc);
  if (rc) return rc;
  if (desc->flags & MOE_F_CHECK_FINITE) return MOE_ERR_UNSUPPORTED;  // no readable status word
  if (moe_workspace_size(desc) > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  if (desc->T == 0) return MOE_OK;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return MOE_ERR_HIP;
  // every other check of the workspace entry point, before anything is enqueued
  rc = moe::layer_forward_check(desc, x, weights, y, topk_idx_out, topk_w_out, logits_out,
                                counts_out, tracking, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  if (rc) return rc;
  hipLaunchKernelGGL(k_clear_status, dim3(1), dim3(64), 0, stream, static_cast<uint32_t*>(ws));
  if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  return moe_layer_forward(desc, x, weights, y, topk_idx_out, topk_w_out, logits_out, counts_out,
                           tracking, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}
