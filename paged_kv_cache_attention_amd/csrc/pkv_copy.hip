// KV append, diagnostic gather and the device-side contract check (gfx950).
//
// Append writes this step's new key/value rows at positions
// lens_pre[b] .. lens_pre[b]+T-1 of each sequence, through the block table
// ("LLM Inference from Scratch", M1: the cache keeps past keys/values and a
// decode step adds the new token's rows).  Gather copies each sequence's
// cached rows out into a contiguous buffer ("The Project", M10: paged_gather).
// Both move bytes in 16-byte chunks; a (token, all KV heads) row is
// Hkv*D*elem_bytes contiguous bytes in both the pool and the dense arrays.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

__global__ __launch_bounds__(256) void append_kernel(const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
                                                     uint4* __restrict__ k_pool, uint4* __restrict__ v_pool,
                                                     const int32_t* __restrict__ tables,
                                                     const int32_t* __restrict__ lens_pre, int T, int row_chunks,
                                                     int block_size, int max_blocks, int N_blocks) {
  const int bt = blockIdx.x;              // (b, t)
  const int b = bt / T, t = bt % T;
  const int pos = lens_pre[b] + t;
  const int lb = pos / block_size;
  if (pos < 0 || lb >= max_blocks) return;          // outside the table: nothing to write
  const int phys = tables[(size_t)b * max_blocks + lb];
  if (phys < 0 || phys >= N_blocks) return;          // bad table entry: never write outside the pool
  const size_t dst = ((size_t)phys * block_size + pos % block_size) * row_chunks;
  const size_t src = (size_t)bt * row_chunks;
  for (int c = threadIdx.x; c < row_chunks; c += blockDim.x) {
    k_pool[dst + c] = k_new[src + c];
    v_pool[dst + c] = v_new[src + c];
  }
}

__global__ __launch_bounds__(256) void gather_kernel(const uint4* __restrict__ k_pool, const uint4* __restrict__ v_pool,
                                                     const int32_t* __restrict__ tables, const int32_t* __restrict__ lens,
                                                     uint4* __restrict__ k_out, uint4* __restrict__ v_out, int max_len,
                                                     int row_chunks, int block_size, int max_blocks, int N_blocks,
                                                     size_t total) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % row_chunks);
    const size_t tok = i / row_chunks;               // b * max_len + j
    const int j = (int)(tok % max_len);
    const int b = (int)(tok / max_len);
    uint4 kv = make_uint4(0u, 0u, 0u, 0u), vv = kv;
    if (j < lens[b]) {
      const int lb = j / block_size;
      const int phys = lb < max_blocks ? tables[(size_t)b * max_blocks + lb] : -1;
      if (phys >= 0 && phys < N_blocks) {
        const size_t s = ((size_t)phys * block_size + j % block_size) * row_chunks + c;
        kv = k_pool[s];
        vv = v_pool[s];
      }
    }
    k_out[i] = kv;
    v_out[i] = vv;
  }
}

__global__ __launch_bounds__(256) void validate_kernel(const int32_t* __restrict__ tables, const int32_t* __restrict__ lens,
                                                       int B, int T, int len_add, int block_size, int max_blocks,
                                                       int N_blocks, int* bad) {
  const int b = blockIdx.x;
  const int L = lens[b] + len_add;
  if (L < T || L > max_blocks * block_size) {
    if (threadIdx.x == 0) *bad = 1;
    return;
  }
  const int nb = (L + block_size - 1) / block_size;
  for (int i = threadIdx.x; i < nb; i += blockDim.x) {
    const int ph = tables[(size_t)b * max_blocks + i];
    if (ph < 0 || ph >= N_blocks) *bad = 1;
  }
}

}  // namespace

hipError_t launch_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool, const int32_t* block_tables,
                         const int32_t* lens_pre, int B, int T, int Hkv, int D, int block_size, int max_blocks,
                         int N_blocks, int elem_bytes, hipStream_t stream) {
  const int row_chunks = Hkv * D * elem_bytes / 16;
  const int threads = row_chunks >= 256 ? 256 : (row_chunks + 63) / 64 * 64;
  hipLaunchKernelGGL(append_kernel, dim3(B * T), dim3(threads), 0, stream, static_cast<const uint4*>(k_new),
                     static_cast<const uint4*>(v_new), static_cast<uint4*>(k_pool), static_cast<uint4*>(v_pool),
                     block_tables, lens_pre, T, row_chunks, block_size, max_blocks, N_blocks);
  return hipGetLastError();
}

// Copy-on-write support: block dst[i] of both pools becomes a copy of block
// src[i]; pairs with an id outside [0, N_blocks) are skipped.  One workgroup
// per pair and 16-byte moves.  Sources must not be destinations of the same
// call (the engine never plans that).
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* __restrict__ k_pool, uint4* __restrict__ v_pool,
                                                          const int32_t* __restrict__ src,
                                                          const int32_t* __restrict__ dst, int block_chunks,
                                                          int N_blocks) {
  const int s = src[blockIdx.x], d = dst[blockIdx.x];
  if (s < 0 || s >= N_blocks || d < 0 || d >= N_blocks) return;
  const size_t so = (size_t)s * block_chunks, dof = (size_t)d * block_chunks;
  for (int c = threadIdx.x; c < block_chunks; c += blockDim.x) {
    k_pool[dof + c] = k_pool[so + c];
    v_pool[dof + c] = v_pool[so + c];
  }
}

hipError_t launch_copy_blocks(void* k_pool, void* v_pool, const int32_t* src, const int32_t* dst, int n, int Hkv,
                              int D, int block_size, int N_blocks, int elem_bytes, hipStream_t stream) {
  const int block_chunks = block_size * Hkv * D * elem_bytes / 16;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n), dim3(256), 0, stream, static_cast<uint4*>(k_pool),
                     static_cast<uint4*>(v_pool), src, dst, block_chunks, N_blocks);
  return hipGetLastError();
}

hipError_t launch_gather(const void* k_pool, const void* v_pool, const int32_t* block_tables, const int32_t* lens,
                         void* k_out, void* v_out, int B, int max_len, int Hkv, int D, int block_size, int max_blocks,
                         int N_blocks, int elem_bytes, hipStream_t stream) {
  const int row_chunks = Hkv * D * elem_bytes / 16;
  const size_t total = (size_t)B * max_len * row_chunks;
  const size_t want = (total + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(gather_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const uint4*>(k_pool),
                     static_cast<const uint4*>(v_pool), block_tables, lens, static_cast<uint4*>(k_out),
                     static_cast<uint4*>(v_out), max_len, row_chunks, block_size, max_blocks, N_blocks, total);
  return hipGetLastError();
}

hipError_t launch_validate(const int32_t* block_tables, const int32_t* lens, int B, int T, int len_add, int block_size,
                           int max_blocks, int N_blocks, int* bad, hipStream_t stream) {
  hipLaunchKernelGGL(validate_kernel, dim3(B), dim3(256), 0, stream, block_tables, lens, B, T, len_add, block_size,
                     max_blocks, N_blocks, bad);
  return hipGetLastError();
}

}  // namespace pkv
