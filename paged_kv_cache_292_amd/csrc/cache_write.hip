// Cache writes for gfx950: new tokens' K/V rows through a slot mapping, and
// whole-block copies.
//
// A sequence's cache grows one token at a time; each new token's rows go to
// the slot the allocator gave its position ("vLLM in Production …", section
// "PagedAttention — Virtual Memory for the KV Cache").  With the cache laid
// out [num_blocks][block_size][num_kv_heads][head_dim], slot s = block *
// block_size + row starts at element s * num_kv_heads * head_dim, so a token
// is one contiguous copy of num_kv_heads * head_dim elements per cache.
// Block copies give a sequence its own copy of a block that others still
// share ("What Is vLLM …", section "How does PagedAttention work?"), and swap
// copies move whole blocks between the device cache and a pinned host pool
// when sequences are preempted (same page, "What is continuous batching in
// vLLM?", step 2).
#include <algorithm>
#include <cstdint>

#include "pkv_internal.h"
#include <hip/hip_runtime.h>

namespace pkv {
namespace {

// One workgroup per token; 16-byte vectors, K and V interleaved over threads.
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, const int64_t* __restrict__ slots, int64_t key_stride_vec,
    int64_t value_stride_vec, int row_vec, int64_t num_slots) {
  const int i = blockIdx.x;
  const int64_t slot = slots[i];
  if (slot < 0 || slot >= num_slots) return;
  const uint4* ks = key + i * key_stride_vec;
  const uint4* vs = value + i * value_stride_vec;
  uint4* kd = k_cache + slot * row_vec;
  uint4* vd = v_cache + slot * row_vec;
  for (int j = threadIdx.x; j < 2 * row_vec; j += blockDim.x) {
    if (j < row_vec)
      kd[j] = ks[j];
    else
      vd[j - row_vec] = vs[j - row_vec];
  }
}

// One workgroup per (pair, cache); copies a whole block.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* __restrict__ k_cache,
                                                          uint4* __restrict__ v_cache,
                                                          const int64_t* __restrict__ pairs,
                                                          int64_t block_vec, int32_t num_blocks) {
  const int64_t src = pairs[2 * blockIdx.x];
  const int64_t dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  uint4* c = blockIdx.y == 0 ? k_cache : v_cache;
  const uint4* s = c + src * block_vec;
  uint4* d = c + dst * block_vec;
  for (int64_t j = threadIdx.x; j < block_vec; j += blockDim.x) d[j] = s[j];
}

// Copy of mapped pinned host memory into device memory by the GPU itself.
__global__ __launch_bounds__(256) void upload_kernel(const uint4* __restrict__ src,
                                                     uint4* __restrict__ dst, int64_t n_vec) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n_vec;
       i += int64_t(gridDim.x) * 256)
    dst[i] = src[i];
}

// Swap copy between the device cache and a pinned host pool (mapped into the
// device's address space): one workgroup per (pair, cache, slice of up to
// kSwapSlice 16-byte vectors of the block).  Each thread issues all of its
// loads before its stores, so a workgroup keeps 16 KB in flight over the
// host link.
constexpr int kSwapSlice = 1024;
__global__ __launch_bounds__(256) void swap_blocks_kernel(
    const uint4* __restrict__ k_src, const uint4* __restrict__ v_src, uint4* __restrict__ k_dst,
    uint4* __restrict__ v_dst, const int64_t* __restrict__ pairs, int64_t block_vec,
    int32_t src_blocks, int32_t dst_blocks) {
  const int64_t s = pairs[2 * int64_t(blockIdx.x)];
  const int64_t d = pairs[2 * int64_t(blockIdx.x) + 1];
  if (s < 0 || s >= src_blocks || d < 0 || d >= dst_blocks) return;
  const uint4* src = (blockIdx.y == 0 ? k_src : v_src) + s * block_vec;
  uint4* dst = (blockIdx.y == 0 ? k_dst : v_dst) + d * block_vec;
  const int64_t lo = int64_t(blockIdx.z) * kSwapSlice;
  const int64_t hi = std::min<int64_t>(lo + kSwapSlice, block_vec);
  constexpr int kPer = kSwapSlice / 256;
  uint4 r[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int64_t i = lo + threadIdx.x + k * 256;
    if (i < hi) r[k] = src[i];
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int64_t i = lo + threadIdx.x + k * 256;
    if (i < hi) dst[i] = r[k];
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

// Device address of pinned, mapped host memory; nullptr (and no sticky
// runtime error left behind) if the pointer is not such memory.
void* mapped_host(void* host) {
  void* dev = nullptr;
  const hipError_t e = hipHostGetDevicePointer(&dev, host, 0);
  if (e != hipSuccess || !dev) {
    (void)hipGetLastError();
    return nullptr;
  }
  return dev;
}

}  // namespace pkv

using pkv::fail;

extern "C" pkv_status pkv_kv_reshape_and_cache(const void* key, const void* value,
                                               void* k_cache, void* v_cache,
                                               const int64_t* slot_mapping, int32_t num_tokens,
                                               int32_t num_kv_heads, int32_t head_dim,
                                               int32_t block_size, int32_t num_blocks,
                                               int64_t key_token_stride,
                                               int64_t value_token_stride, pkv_dtype dtype,
                                               void* stream) {
  if (dtype != PKV_F32 && dtype != PKV_BF16)
    return fail(PKV_ERR_INVALID_ARG, "kv_reshape_and_cache: unknown dtype %d", int(dtype));
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "kv_reshape_and_cache: head_dim=%d (64 or 128)", head_dim);
  if (num_tokens < 0 || num_kv_heads <= 0 || block_size <= 0 || num_blocks < 0)
    return fail(PKV_ERR_INVALID_ARG,
                "kv_reshape_and_cache: num_tokens=%d num_kv_heads=%d block_size=%d "
                "num_blocks=%d", num_tokens, num_kv_heads, block_size, num_blocks);
  const int64_t esize = dtype == PKV_F32 ? 4 : 2;
  const int64_t row = int64_t(num_kv_heads) * head_dim;
  if (key_token_stride < row || value_token_stride < row ||
      (key_token_stride * esize) % 16 || (value_token_stride * esize) % 16)
    return fail(PKV_ERR_INVALID_ARG,
                "kv_reshape_and_cache: token strides (%lld, %lld) must be >= %lld elements "
                "and multiples of 16 bytes", (long long)key_token_stride,
                (long long)value_token_stride, (long long)row);
  if (num_tokens == 0) return pkv::ok();
  if (!key || !value || !k_cache || !v_cache || !slot_mapping)
    return fail(PKV_ERR_INVALID_ARG, "kv_reshape_and_cache: NULL pointer argument");
  if (!pkv::aligned16(key) || !pkv::aligned16(value) || !pkv::aligned16(k_cache) ||
      !pkv::aligned16(v_cache))
    return fail(PKV_ERR_INVALID_ARG, "kv_reshape_and_cache: tensors must be 16-byte aligned");
  const int row_vec = int(row * esize / 16);
  hipLaunchKernelGGL(pkv::reshape_and_cache_kernel, dim3(num_tokens), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(key),
                     static_cast<const uint4*>(value), static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), slot_mapping, key_token_stride * esize / 16,
                     value_token_stride * esize / 16, row_vec,
                     int64_t(num_blocks) * block_size);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(PKV_ERR_HIP, "kv_reshape_and_cache: launch failed: %s", hipGetErrorString(e));
  return pkv::ok();
}

extern "C" pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs,
                                      int32_t num_pairs, int32_t num_blocks, int32_t block_size,
                                      int32_t num_kv_heads, int32_t head_dim, pkv_dtype dtype,
                                      void* stream) {
  if (dtype != PKV_F32 && dtype != PKV_BF16)
    return fail(PKV_ERR_INVALID_ARG, "copy_blocks: unknown dtype %d", int(dtype));
  if (num_pairs < 0 || num_pairs > 0x7FFFFFFF || num_blocks < 0 || block_size <= 0 ||
      num_kv_heads <= 0 || head_dim <= 0)
    return fail(PKV_ERR_INVALID_ARG, "copy_blocks: bad sizes");
  const int64_t esize = dtype == PKV_F32 ? 4 : 2;
  const int64_t block_bytes = int64_t(block_size) * num_kv_heads * head_dim * esize;
  if (block_bytes % 16)
    return fail(PKV_ERR_UNSUPPORTED, "copy_blocks: block of %lld bytes is not a multiple of 16",
                (long long)block_bytes);
  if (num_pairs == 0) return pkv::ok();
  if (!k_cache || !v_cache || !pairs)
    return fail(PKV_ERR_INVALID_ARG, "copy_blocks: NULL pointer argument");
  if (!pkv::aligned16(k_cache) || !pkv::aligned16(v_cache))
    return fail(PKV_ERR_INVALID_ARG, "copy_blocks: caches must be 16-byte aligned");
  hipLaunchKernelGGL(pkv::copy_blocks_kernel, dim3(num_pairs, 2), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), pairs, block_bytes / 16, num_blocks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(PKV_ERR_HIP, "copy_blocks: launch failed: %s", hipGetErrorString(e));
  return pkv::ok();
}

extern "C" pkv_status pkv_swap_blocks(void* k_cache, void* v_cache, void* k_host, void* v_host,
                                      const int64_t* pairs, int32_t num_pairs,
                                      int32_t num_blocks, int32_t num_host_blocks,
                                      int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                                      pkv_dtype dtype, int32_t direction, void* stream) {
  if (dtype != PKV_F32 && dtype != PKV_BF16)
    return fail(PKV_ERR_INVALID_ARG, "swap_blocks: unknown dtype %d", int(dtype));
  if (direction != PKV_SWAP_OUT && direction != PKV_SWAP_IN)
    return fail(PKV_ERR_INVALID_ARG, "swap_blocks: unknown direction %d", direction);
  if (num_pairs < 0 || num_blocks < 0 || num_host_blocks < 0 || block_size <= 0 ||
      num_kv_heads <= 0 || head_dim <= 0)
    return fail(PKV_ERR_INVALID_ARG, "swap_blocks: bad sizes");
  const int64_t esize = dtype == PKV_F32 ? 4 : 2;
  const int64_t block_bytes = int64_t(block_size) * num_kv_heads * head_dim * esize;
  if (block_bytes % 16)
    return fail(PKV_ERR_UNSUPPORTED, "swap_blocks: block of %lld bytes is not a multiple of 16",
                (long long)block_bytes);
  const int64_t slices = (block_bytes / 16 + pkv::kSwapSlice - 1) / pkv::kSwapSlice;
  if (slices > 65535)
    return fail(PKV_ERR_UNSUPPORTED, "swap_blocks: block of %lld bytes is too large",
                (long long)block_bytes);
  if (num_pairs == 0) return pkv::ok();
  if (!k_cache || !v_cache || !k_host || !v_host || !pairs)
    return fail(PKV_ERR_INVALID_ARG, "swap_blocks: NULL pointer argument");
  if (!pkv::aligned16(k_cache) || !pkv::aligned16(v_cache) || !pkv::aligned16(k_host) ||
      !pkv::aligned16(v_host))
    return fail(PKV_ERR_INVALID_ARG, "swap_blocks: caches and pools must be 16-byte aligned");
  void* kh = pkv::mapped_host(k_host);
  void* vh = pkv::mapped_host(v_host);
  if (!kh || !vh)
    return fail(PKV_ERR_INVALID_ARG,
                "swap_blocks: the host pools must be pinned, device-mapped host memory");
  const bool out = direction == PKV_SWAP_OUT;
  hipLaunchKernelGGL(pkv::swap_blocks_kernel, dim3(num_pairs, 2, unsigned(slices)), dim3(256), 0,
                     static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(out ? k_cache : kh),
                     static_cast<const uint4*>(out ? v_cache : vh),
                     static_cast<uint4*>(out ? kh : k_cache), static_cast<uint4*>(out ? vh : v_cache),
                     pairs, block_bytes / 16, out ? num_blocks : num_host_blocks,
                     out ? num_host_blocks : num_blocks);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(PKV_ERR_HIP, "swap_blocks: launch failed: %s", hipGetErrorString(e));
  return pkv::ok();
}

extern "C" pkv_status pkv_upload_pinned(void* dst, const void* src_host, size_t bytes,
                                        void* stream) {
  if (bytes == 0) return pkv::ok();
  if (!dst || !src_host)
    return fail(PKV_ERR_INVALID_ARG, "upload_pinned: NULL pointer argument");
  if (bytes % 16 || !pkv::aligned16(dst) || !pkv::aligned16(src_host))
    return fail(PKV_ERR_INVALID_ARG,
                "upload_pinned: size (%zu) and both addresses must be multiples of 16 bytes", bytes);
  void* src_dev = pkv::mapped_host(const_cast<void*>(src_host));
  if (!src_dev)
    return fail(PKV_ERR_INVALID_ARG,
                "upload_pinned: source is not pinned, device-mapped host memory");
  const int64_t n_vec = int64_t(bytes / 16);
  const int64_t blocks = std::min<int64_t>((n_vec + 255) / 256, 1024);
  hipLaunchKernelGGL(pkv::upload_kernel, dim3(unsigned(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src_dev),
                     static_cast<uint4*>(dst), n_vec);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(PKV_ERR_HIP, "upload_pinned: launch failed: %s", hipGetErrorString(e));
  return pkv::ok();
}
