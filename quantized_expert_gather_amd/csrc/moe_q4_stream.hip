// Streaming-read reference of the measurement: reads a device buffer once
// with 16-byte nontemporal loads and nothing else, the analogue of the plain
// sum() over a large array that the mlx issue "gather_qmm at M=1 streams
// 4-bit expert weights at ~half the bandwidth of M=4" (section "Numbers")
// quotes beside its layer timings.  The layer kernels' byte rates are read
// against this kernel's rate on the same chip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_q4.h"

namespace {

typedef int v4i_t __attribute__((ext_vector_type(4)));

// Grid-stride loop, one 16-byte load per lane in flight per iteration; the
// XOR of everything read goes to one word per block so the loads stay.
__global__ __launch_bounds__(1024) void k_stream_read(const v4i_t* __restrict__ p, size_t n16,
                                                      const unsigned char* __restrict__ tail, size_t ntail,
                                                      uint32_t* __restrict__ sink) {
  const size_t st = (size_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += st) {
    const v4i_t v = __builtin_nontemporal_load(p + i);
    acc ^= (uint32_t)(v.x ^ v.y ^ v.z ^ v.w);
  }
  if (blockIdx.x == 0 && threadIdx.x < ntail) acc ^= tail[threadIdx.x];
  // wave XOR, then one word per block
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  __shared__ uint32_t wv[16];
  if ((threadIdx.x & 63) == 0) wv[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) r ^= wv[w];
    sink[blockIdx.x] = r;
  }
}

}  // namespace

extern "C" int moe_q4_stream_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words,
                                  hipStream_t stream) {
  if (!buf || !sink) return MOE_Q4_ERR_NULL;
  if (((uintptr_t)buf & 15) || ((uintptr_t)sink & 3)) return MOE_Q4_ERR_ALIGN;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
    return MOE_Q4_ERR_LAUNCH;
  const size_t grid = (size_t)2 * ncu;  // two 1024-thread blocks per CU
  if (sink_words < grid) return MOE_Q4_ERR_WORKSPACE;
  if (bytes == 0) return MOE_Q4_OK;
  const size_t n16 = bytes / 16;
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)grid), dim3(1024), 0, stream,
                     static_cast<const v4i_t*>(buf), n16, static_cast<const unsigned char*>(buf) + n16 * 16,
                     bytes - n16 * 16, sink);
  return hipGetLastError() == hipSuccess ? MOE_Q4_OK : MOE_Q4_ERR_LAUNCH;
}
