// Log-sum-exp merge of split-KV partials (gfx950).
//
// Partials over disjoint key ranges, each normalised within its range and
// carrying lse_p = log sum exp(scores), merge exactly:
//   M = max_p lse_p,  w_p = exp(lse_p - M),
//   out = sum_p w_p o_p / sum_p w_p,  lse = M + log sum_p w_p
// ("Inference From Scratch", ch. 8: softmax over pieces combined through the
// running max and sum).  Partitions with lse = -inf are empty and skipped by
// selection, so their o_p is never read.  One wave per output row, the sum
// over p runs in a fixed order: results are deterministic.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kRowsPerGroup = 4;

template <typename ET, int D>
__global__ __launch_bounds__(64 * kRowsPerGroup) void lse_reduce_kernel(
    const float* __restrict__ po, const float* __restrict__ pl, typename Storage<ET>::T* __restrict__ out,
    float* __restrict__ lse_out, int rows, int THq, int P_max, const int32_t* __restrict__ lens, int part_tokens) {
  constexpr int DPL = D / 64;  // output elements per lane
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerGroup + (threadIdx.x >> 6);
  if (row >= rows) return;
  int P = P_max;
  if (lens) {
    const int L = lens[row / THq];
    const int Pb = L > part_tokens ? (L + part_tokens - 1) / part_tokens : 1;
    if (Pb <= 1) return;   // written directly by the decode kernel
    P = min(Pb, P_max);
  }
  const float* lrow = pl + (size_t)row * P_max;
  const float* orow = po + (size_t)row * P_max * D;

  float M = kNegInf;
  for (int p = lane; p < P; p += 64) M = fmaxf(M, lrow[p]);
  M = wave_max(M);

  float acc[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
  float wsum = 0.f;
  if (M != kNegInf) {
    for (int p0 = 0; p0 < P; p0 += 64) {
      const int pp = p0 + lane;
      const float lv = pp < P ? lrow[pp] : kNegInf;
      const float wl = lv == kNegInf ? 0.f : __builtin_amdgcn_exp2f((lv - M) * kLog2e);
      const int n = min(64, P - p0);
      for (int k2 = 0; k2 < n; ++k2) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), k2));
        if (w == 0.f) continue;  // empty partition: its o_p is not read
        wsum += w;
        const float* op = orow + (size_t)(p0 + k2) * D + lane * DPL;
#pragma unroll
        for (int k = 0; k < DPL; ++k) acc[k] = fmaf(w, op[k], acc[k]);
      }
    }
  }
  const float inv = wsum != 0.f ? 1.f / wsum : 0.f;   // NaN inputs stay NaN
#pragma unroll
  for (int k = 0; k < DPL; ++k) store_out<ET>(out + (size_t)row * D + lane * DPL + k, acc[k] * inv);
  if (lse_out && lane == 0) lse_out[row] = wsum != 0.f ? M + logf(wsum) : kNegInf;
}

template <typename ET>
hipError_t launch_r(const float* po, const float* pl, void* out, float* lse_out, int rows, int THq, int D,
                    int P_max, const int32_t* lens, int part_tokens, hipStream_t stream) {
  using OT = typename Storage<ET>::T;
  const dim3 grid((rows + kRowsPerGroup - 1) / kRowsPerGroup), block(64 * kRowsPerGroup);
  if (D == 64)
    hipLaunchKernelGGL((lse_reduce_kernel<ET, 64>), grid, block, 0, stream, po, pl, static_cast<OT*>(out), lse_out,
                       rows, THq, P_max, lens, part_tokens);
  else
    hipLaunchKernelGGL((lse_reduce_kernel<ET, 128>), grid, block, 0, stream, po, pl, static_cast<OT*>(out), lse_out,
                       rows, THq, P_max, lens, part_tokens);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_reduce(const float* part_out, const float* part_lse, void* out, float* lse_out, int B, int T,
                             int Hq, int D, int P_max, bool bf16, const int32_t* lens, int part_tokens,
                             hipStream_t stream) {
  const int rows = B * T * Hq;
  if (bf16) return launch_r<Bf16>(part_out, part_lse, out, lse_out, rows, T * Hq, D, P_max, lens, part_tokens, stream);
  return launch_r<float>(part_out, part_lse, out, lse_out, rows, T * Hq, D, P_max, lens, part_tokens, stream);
}

}  // namespace pkv
