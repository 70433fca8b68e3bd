// KV append with rotary position embedding fused in (gfx950).
//
// The Llama-style decoder rotates every key (and query) by its position
// before attention ("LLM Inference from Scratch", Architecture overview: a
// Llama-style transformer with RoPE; "warpllama", Milestones: fused RoPE
// kernel).  Fusing the rotation into the append writes each new key into its
// cache slot already rotated, in one pass over k_new.  Pairing is Llama's:
// dimension i < D/2 with i + D/2, angle p * theta^(-2i/D) at position
// p = lens_pre[b] + t.
//
// One workgroup per (sequence, new token): the D/2 angles are computed once
// in float64 (the angle p * w_i reaches 1e5 radians at long contexts, where
// float32 would lose the phase) and kept in LDS; each thread rotates pairs of
// key (and optionally query) elements in float64 and rounds once to the
// storage type: float32 round to nearest even, or bf16 through a
// round-to-odd float32, which equals rounding the float64 value directly.
// The value row is copied with 16-byte moves.
#include <cmath>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

// float64 -> bf16, round to nearest even (via round-to-odd float32).
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  const float f = (float)x;
  uint32_t u = __float_as_uint(f);
  if ((double)f != x && isfinite(f)) {
    if (fabs((double)f) > fabs(x)) u -= 1;   // the truncated float32
    u |= 1;                                   // sticky: odd marks "inexact"
  }
  return f32_to_bf16_rne(__uint_as_float(u));
}

template <typename ET> struct RopeIO;
template <> struct RopeIO<float> {
  using T = float;
  __device__ static double get(const T* p) { return (double)*p; }
  __device__ static void put(T* p, double v) { *p = (float)v; }
};
template <> struct RopeIO<Bf16> {
  using T = uint16_t;
  __device__ static double get(const T* p) { return (double)__uint_as_float((uint32_t)*p << 16); }
  __device__ static void put(T* p, double v) { *p = f64_to_bf16_rne(v); }
};

constexpr int kMaxHalf = 64;   // D/2 for D <= 128

template <typename ET>
__global__ __launch_bounds__(256) void append_rope_kernel(typename RopeIO<ET>::T* q, int Hq,
                                                          const typename RopeIO<ET>::T* __restrict__ k_new,
                                                          const uint4* __restrict__ v_new,
                                                          typename RopeIO<ET>::T* __restrict__ k_pool,
                                                          uint4* __restrict__ v_pool, const int32_t* __restrict__ tables,
                                                          const int32_t* __restrict__ lens_pre, int T, int Hkv, int D,
                                                          int block_size, int max_blocks, int N_blocks, double theta) {
  using IO = RopeIO<ET>;
  __shared__ double s_cos[kMaxHalf], s_sin[kMaxHalf];
  const int bt = blockIdx.x;   // (b, t)
  const int b = bt / T, t = bt - (bt / T) * T;
  const int pos = lens_pre[b] + t;
  const int half = D / 2;
  if (pos < 0) return;   // no position: nothing to rotate or write
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const double ang = (double)pos * pow(theta, -2.0 * i / D);
    double sn, cs;
    sincos(ang, &sn, &cs);
    s_cos[i] = cs;
    s_sin[i] = sn;
  }
  __syncthreads();

  auto rotate = [&](const typename IO::T* src, typename IO::T* dst, int e) {
    const int h = e / half, i = e - (e / half) * half;
    const double x0 = IO::get(src + (size_t)h * D + i), x1 = IO::get(src + (size_t)h * D + i + half);
    const double c = s_cos[i], sn = s_sin[i];
    IO::put(dst + (size_t)h * D + i, x0 * c - x1 * sn);
    IO::put(dst + (size_t)h * D + i + half, x1 * c + x0 * sn);
  };

  if (q) {   // queries of this token, rotated in place
    typename IO::T* qrow = q + (size_t)bt * Hq * D;
    for (int e = threadIdx.x; e < Hq * half; e += blockDim.x) rotate(qrow, qrow, e);
  }
  const int lb = pos / block_size;
  if (lb >= max_blocks) return;                       // outside the table: nothing to write
  const int phys = tables[(size_t)b * max_blocks + lb];
  if (phys < 0 || phys >= N_blocks) return;           // bad table entry: never write outside the pool
  const size_t slot = (size_t)phys * block_size + pos % block_size;
  const typename IO::T* krow = k_new + (size_t)bt * Hkv * D;
  typename IO::T* kdst = k_pool + slot * Hkv * D;
  for (int e = threadIdx.x; e < Hkv * half; e += blockDim.x) rotate(krow, kdst, e);
  const int row_chunks = Hkv * D * (int)sizeof(typename IO::T) / 16;
  for (int c = threadIdx.x; c < row_chunks; c += blockDim.x) v_pool[slot * row_chunks + c] = v_new[(size_t)bt * row_chunks + c];
}

}  // namespace

hipError_t launch_append_rope(void* q, int Hq, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                              const int32_t* block_tables, const int32_t* lens_pre, int B, int T, int Hkv, int D,
                              int block_size, int max_blocks, int N_blocks, double theta, bool bf16,
                              hipStream_t stream) {
  if (D / 2 > kMaxHalf) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL(append_rope_kernel<Bf16>, dim3(B * T), dim3(256), 0, stream, static_cast<uint16_t*>(q), Hq,
                       static_cast<const uint16_t*>(k_new), static_cast<const uint4*>(v_new),
                       static_cast<uint16_t*>(k_pool), static_cast<uint4*>(v_pool), block_tables, lens_pre, T, Hkv, D,
                       block_size, max_blocks, N_blocks, theta);
  else
    hipLaunchKernelGGL(append_rope_kernel<float>, dim3(B * T), dim3(256), 0, stream, static_cast<float*>(q), Hq,
                       static_cast<const float*>(k_new), static_cast<const uint4*>(v_new),
                       static_cast<float*>(k_pool), static_cast<uint4*>(v_pool), block_tables, lens_pre, T, Hkv, D,
                       block_size, max_blocks, N_blocks, theta);
  return hipGetLastError();
}

}  // namespace pkv
