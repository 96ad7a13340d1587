// Device-side helpers for the gfx950 kernels: wave64 lane arithmetic, DPP row
// reductions, bf16 <-> f32 conversion and 16-byte loads.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pkv {
namespace dev {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

// DPP move within 16-lane rows; CTRL is the dpp_ctrl encoding.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
// Steps: swap neighbours, swap pairs, mirror within 8, mirror within 16.
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bfloat16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Read of a wave-uniform address through the scalar data cache.  The pointer
// goes to the constant address space, which only takes scalar loads when the
// address is uniform; the data must not change while the kernel runs.
template <typename T>
__device__ __forceinline__ T scalar_read(const T* p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) T*>(
      reinterpret_cast<uintptr_t>(p));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Dot product of two packed bf16 pairs, accumulated in f32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

#ifndef PKV_NT_LOADS
#define PKV_NT_LOADS 1
#endif

// Streaming 16- and 8-byte loads of K/V: each byte is read once, so the loads
// carry the non-temporal hint (on MI355X this raises a pure read stream from
// about 6.3 to about 7.1 TB/s).
__device__ __forceinline__ uint4 load16_stream(const void* p) {
#if PKV_NT_LOADS
  const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
#else
  return *reinterpret_cast<const uint4*>(p);
#endif
}
// The same load, non-temporal or not by a compile-time choice.
template <bool NT>
__device__ __forceinline__ uint4 load16(const void* p) {
  if constexpr (NT) {
    const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}
template <bool NT>
__device__ __forceinline__ uint2 load8(const void* p) {
  if constexpr (NT) {
    const u32x2_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    return make_uint2(t.x, t.y);
  } else {
    return *reinterpret_cast<const uint2*>(p);
  }
}
__device__ __forceinline__ uint2 load8_stream(const void* p) {
#if PKV_NT_LOADS
  const u32x2_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(t.x, t.y);
#else
  return *reinterpret_cast<const uint2*>(p);
#endif
}

// WORDS 32-bit words per lane, loaded with 16-byte (or 8-byte) vector loads.
template <int WORDS>
struct Frag {
  uint32_t w[WORDS];
};

template <int WORDS>
__device__ __forceinline__ void load_frag(Frag<WORDS>& f, const void* p) {
  if constexpr (WORDS % 4 == 0) {
    const uint4* v = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < WORDS / 4; ++i) {
      uint4 x = v[i];
      f.w[4 * i + 0] = x.x;
      f.w[4 * i + 1] = x.y;
      f.w[4 * i + 2] = x.z;
      f.w[4 * i + 3] = x.w;
    }
  } else {
    static_assert(WORDS == 2, "8- or 16-byte multiples only");
    uint2 x = *reinterpret_cast<const uint2*>(p);
    f.w[0] = x.x;
    f.w[1] = x.y;
  }
}

template <int WORDS>
__device__ __forceinline__ void load_frag_stream(Frag<WORDS>& f, const void* p) {
  if constexpr (WORDS % 4 == 0) {
#pragma unroll
    for (int i = 0; i < WORDS / 4; ++i) {
      const uint4 x = load16_stream(static_cast<const char*>(p) + 16 * i);
      f.w[4 * i + 0] = x.x;
      f.w[4 * i + 1] = x.y;
      f.w[4 * i + 2] = x.z;
      f.w[4 * i + 3] = x.w;
    }
  } else {
    static_assert(WORDS == 2, "8- or 16-byte multiples only");
    const uint2 x = load8_stream(p);
    f.w[0] = x.x;
    f.w[1] = x.y;
  }
}

template <int WORDS>
__device__ __forceinline__ void zero_frag(Frag<WORDS>& f) {
#pragma unroll
  for (int i = 0; i < WORDS; ++i) f.w[i] = 0u;
}

// Element e of a fragment as float.
template <typename T, int WORDS>
__device__ __forceinline__ float elem(const Frag<WORDS>& f, int e) {
  if constexpr (sizeof(T) == 4) {
    return __uint_as_float(f.w[e]);
  } else {
    return (e & 1) ? bf16_hi(f.w[e >> 1]) : bf16_lo(f.w[e >> 1]);
  }
}

// Store one element from a float.
template <typename T>
__device__ __forceinline__ void store_elem(void* base, size_t idx, float v) {
  if constexpr (sizeof(T) == 4) {
    reinterpret_cast<float*>(base)[idx] = v;
  } else {
    reinterpret_cast<uint16_t*>(base)[idx] = f32_to_bf16(v);
  }
}

}  // namespace dev
}  // namespace pkv
