// Device-side helpers shared by the gfx950 kernels of libpkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));   // one 16-byte chunk in 4 VGPRs

__device__ __forceinline__ u32x4_t load16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// Reinterpret a 32-bit word as two packed bf16.  Done through memcpy on a
// value: clang's __builtin_bit_cast applied to an element of a vector held by
// reference was seen to read element 0 for every element.
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) {
  bf16x2_t r;
  __builtin_memcpy(&r, &w, sizeof(r));
  return r;
}
__device__ __forceinline__ void store16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Storage element types: float, or bf16 kept as its 16-bit pattern.
struct Bf16 {};

template <typename ET> struct Storage;
template <> struct Storage<float> { using T = float; static constexpr int bytes = 4; };
template <> struct Storage<Bf16> { using T = uint16_t; static constexpr int bytes = 2; };

// bf16 <-> f32.  Widening is exact (the bf16 bits are the high half of the f32).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even f32 -> bf16 bits; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename ET> __device__ __forceinline__ void store_out(typename Storage<ET>::T* p, float v);
template <> __device__ __forceinline__ void store_out<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_out<Bf16>(uint16_t* p, float v) { *p = f32_to_bf16_rne(v); }

// ---------------------------------------------------------------------------
// DPP reductions over one row of 16 lanes (every lane of the row gets the
// result).  Pairs, then quads, then half-row mirror, then row mirror.
// ---------------------------------------------------------------------------
template <int CTRL> __device__ __forceinline__ float dpp_f(float x) {
  return __builtin_amdgcn_update_dpp(0.0f, x, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp_f<0x140>(x));  // row_mirror
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x141>(x);
  x += dpp_f<0x140>(x);
  return x;
}

// Full-wave (64 lanes) reductions; lanes 16/32 apart are reached with ds_swizzle-free
// cross-row shuffles.
__device__ __forceinline__ float wave_max(float x) {
  x = row16_max(x);
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  x = row16_sum(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Workgroup ids are handed to the 8 XCDs of the chip round-robin.  This maps
// the hardware id to a logical id so that runs of `chunk` consecutive logical
// ids execute on one XCD (sharing its L2).  Bijective when the grid is a
// multiple of 8*chunk.
__device__ __forceinline__ uint32_t xcd_logical_id(uint32_t w, uint32_t chunk) {
  const uint32_t xcd = w & 7u, slot = w >> 3;
  return ((slot / chunk) * 8u + xcd) * chunk + (slot % chunk);
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

}  // namespace pkv
