// Streaming-read reference for the decode roofline.
//
// Decode attention reads every context byte of K and V once, so its ceiling
// is what HBM delivers to a plain read stream.  This kernel reads a buffer
// once with the same 16-byte non-temporal loads the decode kernels use and
// no other work, so the rate it reaches on a large buffer is the ceiling the
// decode kernels are measured against, beside the nominal 8 TB/s.  It folds
// every 32-bit word into one XOR per workgroup so that the result can be
// checked (and the loads cannot be dropped).
#include <cstdint>

#include "pkv_internal.h"
#include <hip/hip_runtime.h>

namespace pkv {
namespace {

typedef unsigned int u32x4v_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fold(const u32x4v_t v) { return (v.x ^ v.y) ^ (v.z ^ v.w); }

// Grid-stride over n16 16-byte pieces, four loads in flight per thread and
// iteration; out[blockIdx.x] = XOR of every word the workgroup read.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4v_t* __restrict__ src,
                                                          size_t n16, uint32_t* __restrict__ out) {
  const size_t stride = size_t(gridDim.x) * 256;
  size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4v_t a = __builtin_nontemporal_load(src + i);
    const u32x4v_t b = __builtin_nontemporal_load(src + i + stride);
    const u32x4v_t c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4v_t d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= (fold(a) ^ fold(b)) ^ (fold(c) ^ fold(d));
  }
  for (; i < n16; i += stride) acc ^= fold(__builtin_nontemporal_load(src + i));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o);
  __shared__ uint32_t s_acc[4];
  if ((threadIdx.x & 63) == 0) s_acc[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = (s_acc[0] ^ s_acc[1]) ^ (s_acc[2] ^ s_acc[3]);
}

}  // namespace
}  // namespace pkv

using pkv::fail;

extern "C" pkv_status pkv_stream_read(const void* src, size_t bytes, uint32_t* out,
                                      int32_t workgroups, void* stream) {
  if (!src || !out)
    return fail(PKV_ERR_INVALID_ARG, "stream_read: NULL pointer argument");
  if ((reinterpret_cast<uintptr_t>(src) & 15u) || bytes % 16 != 0)
    return fail(PKV_ERR_INVALID_ARG,
                "stream_read: source must be 16-byte aligned and bytes (%zu) a multiple of 16",
                bytes);
  if (workgroups < 1 || workgroups > (1 << 20))
    return fail(PKV_ERR_INVALID_ARG, "stream_read: workgroups=%d outside [1, 2^20]", workgroups);
  hipLaunchKernelGGL(pkv::stream_read_kernel, dim3(workgroups), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const pkv::u32x4v_t*>(src),
                     bytes / 16, out);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(PKV_ERR_HIP, "stream_read: launch failed: %s", hipGetErrorString(e));
  return pkv::ok();
}
