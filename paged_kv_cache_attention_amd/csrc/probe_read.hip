// Diagnostic read-bandwidth probe (libpkv_probe.so, not part of the pkv ABI).
//
// Reads every byte of a pool of 32 KB blocks in a caller-given random block
// order, the way paged attention reads a KV pool: each wave takes one 4 KB
// slice (16 rows of 256 B, 2 KB apart) of one block with 16-byte loads, and 8
// consecutive waves cover the 8 slices of a block.  No arithmetic beyond an
// XOR into a per-thread sink, so the time is the memory system's.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace {

constexpr int kBlockBytes = 32768;

__global__ __launch_bounds__(256) void slice_read_kernel(const unsigned char* __restrict__ pool,
                                                         const int32_t* __restrict__ order, int nblocks,
                                                         uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int wave = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  const int nwaves = (int)((gridDim.x * blockDim.x) >> 6);
  const int h = wave & 7, c = lane & 15, tg = lane >> 4;
  uint32_t acc = 0;
  for (int k = wave >> 3; k < nblocks; k += nwaves >> 3) {
    const unsigned char* base = pool + (size_t)order[k] * kBlockBytes + (size_t)(tg * 8 + h) * 256 + c * 16;
    u32x4_t v[4];
#pragma unroll
    for (int l = 0; l < 4; ++l) v[l] = *reinterpret_cast<const u32x4_t*>(base + (size_t)l * 8192);
#pragma unroll
    for (int l = 0; l < 4; ++l) acc ^= v[l].x ^ v[l].w;
  }
  sink[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

// pool: nblocks * 32 KB; order: nblocks entries, a permutation of [0, nblocks);
// sink: grid*256 uint32.  grid must be a multiple of 2 (8 waves per block).
extern "C" int pkv_probe_slice_read(const void* pool, const int32_t* order, int nblocks, int grid, uint32_t* sink,
                                    void* stream) {
  if (!pool || !order || !sink || nblocks <= 0 || grid <= 0 || grid % 2) return 1;
  hipLaunchKernelGGL(slice_read_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const unsigned char*>(pool), order, nblocks, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
