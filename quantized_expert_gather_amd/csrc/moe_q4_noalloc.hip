// Allocation-free variant of moe_swiglu_q4_forward, for callers that cannot
// allocate device memory (work recorded under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  The workspace is a file-scope
// device array of this library instead of a caller buffer.
//
// Each GPU the library runs on holds its own copy of `scratch` from the
// library's load until the process ends.  Host code never passes the array's
// name to a kernel or a copy (on the host it is a stand-in symbol, not a
// device address): the first call on a device looks its device address up
// with hipGetSymbolAddress, with that device current, and every call uses that
// address as the workspace pointer of the ordinary entry point.
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>

#include "moe_q4.h"

namespace {

__device__ __align__(256) unsigned char scratch[MOE_Q4_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device (null until looked up)

// Device address of the current device's copy of `scratch`.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_Q4_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_Q4_ERR_LAUNCH;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_Q4_OK;
}

}  // namespace

extern "C" int moe_swiglu_q4_forward_noalloc(const void* x, const int32_t* topk_ids, const float* topk_weights,
                                             const uint32_t* wg, const void* sg, const void* bg, const uint32_t* wu,
                                             const void* su, const void* bu, const uint32_t* wd, const void* sd,
                                             const void* bd, int L, int k, int E, int H, int I, int group_size,
                                             int bits, void* out, int out_dtype, hipStream_t stream) {
  // argument errors first, exactly as the ordinary entry point reports them
  // (it returns before any use of the workspace for every one of them)
  const int path = moe_swiglu_q4_select_path(L, k, E, H, I);
  if (path < 0) return -path;
  if (path == MOE_Q4_PATH_NONE || group_size != 64 || bits != 4)
    return moe_swiglu_q4_forward(x, topk_ids, topk_weights, wg, sg, bg, wu, su, bu, wd, sd, bd, L, k, E, H, I,
                                 group_size, bits, out, out_dtype, nullptr, 0, stream);
  if (moe_swiglu_q4_workspace_bytes(L, k, E, H, I) > (size_t)MOE_Q4_NOALLOC_SCRATCH_BYTES)
    return MOE_Q4_ERR_SCRATCH;
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st) return st;
  // the workspace regions need no initialisation: every call writes what it
  // later reads (the status word included)
  return moe_swiglu_q4_forward(x, topk_ids, topk_weights, wg, sg, bg, wu, su, bu, wd, sd, bd, L, k, E, H, I,
                               group_size, bits, out, out_dtype, ws, (size_t)MOE_Q4_NOALLOC_SCRATCH_BYTES, stream);
}
