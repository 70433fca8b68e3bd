// Chunked-prefill attention over the paged cache on MFMA (gfx950).
//
// A prefill chunk appends T new tokens of a sequence to the cache and lets
// each of them attend causally to everything before it: query t sits at
// position L - T + t and sees keys 0 .. L - T + t.  Attending a prompt chunk
// by chunk this way equals attending the whole prefix at once ("Efficient LLM
// Inference", KV Caching: Verify Reuse, Positions and Windows; "LLM Inference
// from Scratch", Architecture overview, M1: prefill/decode equivalence).
// Unlike single-token decode this is a real GEMM pair per KV head:
// T * Hq/Hkv query rows against the same keys.
//
// Work item = (row group of kRows query rows, sequence, KV head); rows are
// r = t * G + g (G = Hq/Hkv).  A workgroup of kWaves waves owns one item; wave
// w holds rows 32w .. 32w+31 as two 16-row MFMA tiles.  Keys advance kStep
// (32) at a time, staged once per workgroup through LDS (double-buffered: the
// next step's global loads are in flight while the tiles work on the current
// one):
//   K[token][d]  row-major, padded rows        -> A operand of S^T = K Q^T
//   V^T[d][token] transposed when staged        -> B operand of O += P V
// Per wave and step, for each row tile:
//   S^T[token][row] = K . Q^T   v_mfma_f32_16x16x32_bf16, two 16-token halves
//   online softmax per row (base 2, running max raised lazily)
//   O[row][d] += P . V          v_mfma_f32_16x16x32_bf16, k = the step's 32
//     keys; P split into bf16 hi + lo so the product keeps about 16 bits of P
// Keys at or past the group's last visible position are never used: their V
// columns are zeroed when staged and their scores masked.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kBS = 16;
constexpr int kWaves = 4;
constexpr int kTilesPerWave = 2;
constexpr int kRows = 16 * kTilesPerWave * kWaves;   // query rows per item
constexpr int kStep = 32;                            // keys per step
constexpr int kThreads = 64 * kWaves;
constexpr float kSlack = 8.f;

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8_v as_bf16x8(u32x4_t v) {
  bf16x8_v r;
  __builtin_memcpy(&r, &v, sizeof(r));
  return r;
}

template <int D>
struct PLds {
  static constexpr int KROW = 2 * D + 16;            // K row bytes (conflict-free 16-byte reads)
  static constexpr int VROW = 2 * kStep + 8;         // V^T row bytes: one d, 32 keys
  static constexpr int KBYTES = kStep * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int BYTES = 2 * (KBYTES + VBYTES);
};

struct PrefillArgs {
  DecodeArgs a;
  int groups;   // row groups per (sequence, KV head)
};

// Two waves per SIMD: two workgroups per CU (registers of both tiles, 256 per lane).
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_kernel(PrefillArgs pa, float scale_log2e) {
  constexpr int KS = D / 32;                          // k-steps of QK^T
  constexpr int DT = D / 16;                          // output column tiles
  constexpr int RC = D * 2 / 16;                      // 16-byte chunks per token row
  constexpr int PER_T = kStep * RC / kThreads;        // staged chunks per thread (K, and again V)
  static_assert(PER_T * kThreads == kStep * RC, "even staging split");
  using LD = PLds<D>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[LD::BYTES];
  auto kst = [&](int buf) { return lds + buf * LD::KBYTES; };
  auto vst = [&](int buf) { return lds + 2 * LD::KBYTES + buf * LD::VBYTES; };

  const DecodeArgs& a = pa.a;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.Hq / a.Hkv;
  const int R = a.T * G;
  // row groups with the most keys first: the last group of every (b, kv)
  const int per_g = a.B * a.Hkv;
  const int rg = pa.groups - 1 - (int)blockIdx.x / per_g;
  const int rem = (int)blockIdx.x % per_g;
  const int b = rem / a.Hkv, kv = rem - (rem / a.Hkv) * a.Hkv;
  const int max_tokens = a.max_blocks * kBS;
  const int L = clampi(a.context_lens[b], 0, max_tokens);
  const int r0 = rg * kRows;
  const int t_last = (min(R, r0 + kRows) - 1) / G;
  const int kv_len = clampi(L - a.T + t_last + 1, 0, L);   // keys any row of the group sees
  const int nsteps = (kv_len + kStep - 1) / kStep;
  const int nblk = (kv_len + kBS - 1) / kBS;

  // ---- this wave's rows: tile j holds rows r0 + 32 wave + 16 j + (lane % 16) ----
  const int row = lane & 15, quad = lane >> 4;
  const uint16_t* qbase = static_cast<const uint16_t*>(a.q);
  u32x4_t qreg[kTilesPerWave][KS];
  int hi_row[kTilesPerWave];
#pragma unroll
  for (int j = 0; j < kTilesPerWave; ++j) {
    const int r = r0 + 32 * wave + 16 * j + row;
    const bool ok = r < R;
    const int rq = ok ? r : r0;
    const int t = rq / G, g = rq - (rq / G) * G;
    hi_row[j] = ok ? clampi(L - a.T + t + 1, 0, L) : 0;
    const unsigned char* qp = reinterpret_cast<const unsigned char*>(
                                  qbase + ((size_t)(b * a.T + t) * a.Hq + kv * G + g) * D) + quad * 16;
#pragma unroll
    for (int c = 0; c < KS; ++c) {
      const u32x4_t v = load16(qp + c * 64);
      qreg[j][c] = ok ? v : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  const bool wave_active = r0 + 32 * wave < R;

  floatx4_t acc[kTilesPerWave][DT];
  float m_row[kTilesPerWave], l_part[kTilesPerWave];
#pragma unroll
  for (int j = 0; j < kTilesPerWave; ++j) {
#pragma unroll
    for (int d = 0; d < DT; ++d) acc[j][d] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    m_row[j] = kNegInf;
    l_part[j] = 0.f;
  }

  // ---- staging: chunk i = tid + k * kThreads -> key i / RC of the step, columns 8 (i % RC) .. +7 ----
  const size_t kv_row_bytes = (size_t)a.Hkv * D * 2;
  const size_t block_bytes = (size_t)kBS * kv_row_bytes;
  const int nmax = a.N_blocks - 1;
  const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks;
  const unsigned char* kpool = static_cast<const unsigned char*>(a.k_pool) + (size_t)kv * D * 2;
  const unsigned char* vpool = static_cast<const unsigned char*>(a.v_pool) + (size_t)kv * D * 2;
  u32x4_t kreg[PER_T], vreg[PER_T];
  auto issue = [&](int s) {
#pragma unroll
    for (int k = 0; k < PER_T; ++k) {
      const int i = tid + k * kThreads;
      const int pos = s * kStep + i / RC;
      const int ph = clampi(trow[min(pos / kBS, nblk - 1)], 0, nmax);
      const size_t off = (size_t)ph * block_bytes + (size_t)(pos % kBS) * kv_row_bytes + (i % RC) * 16;
      kreg[k] = load16(kpool + off);
      vreg[k] = load16(vpool + off);
    }
  };
  auto commit = [&](int s, int buf) {
#pragma unroll
    for (int k = 0; k < PER_T; ++k) {
      const int i = tid + k * kThreads;
      const int key = i / RC, c = i % RC;
      store16(kst(buf) + key * LD::KROW + c * 16, kreg[k]);
      // keys past the group's last visible one may hold anything: zero their V
      const u32x4_t v = s * kStep + key < kv_len ? vreg[k] : u32x4_t{0u, 0u, 0u, 0u};
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
      uint16_t* vt = reinterpret_cast<uint16_t*>(vst(buf) + (8 * c) * LD::VROW) + key;
#pragma unroll
      for (int e = 0; e < 8; ++e) vt[e * (LD::VROW / 2)] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
    }
  };

  auto compute = [&](int s, int buf) {
    const unsigned char* ks = kst(buf);
    const unsigned char* vs = vst(buf);
    // S^T for both 16-key halves of the step and both row tiles
    floatx4_t sacc[kTilesPerWave][2];
#pragma unroll
    for (int j = 0; j < kTilesPerWave; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) sacc[j][h] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const unsigned char* kr = ks + (16 * h + row) * LD::KROW + quad * 16;
#pragma unroll
      for (int c = 0; c < KS; ++c) {
        const bf16x8_v kv8 = as_bf16x8(*reinterpret_cast<const u32x4_t*>(kr + c * 64));
#pragma unroll
        for (int j = 0; j < kTilesPerWave; ++j)
          sacc[j][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv8, as_bf16x8(qreg[j][c]), sacc[j][h], 0, 0, 0);
      }
    }
    // softmax; k-slot 8*quad + i of P holds key 4*quad + i (i < 4) or 16 + 4*quad + i - 4
    bf16x8_v phi[kTilesPerWave], plo[kTilesPerWave];
#pragma unroll
    for (int j = 0; j < kTilesPerWave; ++j) {
      float sv[8];
      bool need = false;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int key = s * kStep + 16 * (i >> 2) + 4 * quad + (i & 3);
        sv[i] = key < hi_row[j] ? sacc[j][i >> 2][i & 3] * scale_log2e : kNegInf;
        need |= sv[i] > m_row[j] + kSlack;
      }
      if (__builtin_amdgcn_ballot_w64(need)) {
        float mx = sv[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_row[j], mx);
        // 1 while a row is still empty (both -inf), 0 on its first key
        const float alpha = m_row[j] == m_new ? 1.f : __builtin_amdgcn_exp2f(m_row[j] - m_new);
        l_part[j] *= alpha;
        m_row[j] = m_new;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float ak = __shfl(alpha, 4 * quad + k);
#pragma unroll
          for (int d = 0; d < DT; ++d) acc[j][d][k] *= ak;
        }
      }
      uint16_t hb[8], lb[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = sv[i] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(sv[i] - m_row[j]);
        l_part[j] += p;
        hb[i] = f32_to_bf16_rne(p);
        lb[i] = f32_to_bf16_rne(p - __uint_as_float((uint32_t)hb[i] << 16));
      }
      __builtin_memcpy(&phi[j], hb, 16);
      __builtin_memcpy(&plo[j], lb, 16);
    }
    // O += P V: B operand = V^T[d][keys 4*quad .. +3 and 16 + 4*quad .. +3]
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      const unsigned char* vr = vs + (16 * d + row) * LD::VROW + quad * 8;
      const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vr);
      const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vr + 32);
      const u32x4_t w = {lo.x, lo.y, hi.x, hi.y};
      const bf16x8_v bv = as_bf16x8(w);
#pragma unroll
      for (int j = 0; j < kTilesPerWave; ++j) {
        acc[j][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi[j], bv, acc[j][d], 0, 0, 0);
        acc[j][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo[j], bv, acc[j][d], 0, 0, 0);
      }
    }
  };

  if (nsteps > 0) {
    issue(0);
    commit(0, 0);
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
      const int buf = s & 1;
      if (s + 1 < nsteps) issue(s + 1);
      if (wave_active) compute(s, buf);
      if (s + 1 < nsteps) commit(s + 1, buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: O / l in bf16, lse in natural log ----
  if (!wave_active) return;
  uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int j = 0; j < kTilesPerWave; ++j) {
    float l = l_part[j] + __shfl_xor(l_part[j], 16);
    l += __shfl_xor(l, 32);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int rr = r0 + 32 * wave + 16 * j + 4 * quad + k;   // O row held in acc[j][*][k]
      const float lr = __shfl(l, 4 * quad + k);
      const float mr = __shfl(m_row[j], 4 * quad + k);
      if (rr < R) {
        const int t = rr / G, h = kv * G + (rr - (rr / G) * G);
        const size_t orow = ((size_t)b * a.T + t) * a.Hq + h;
        const float inv = lr != 0.f ? 1.f / lr : 0.f;
#pragma unroll
        for (int d = 0; d < DT; ++d) out[orow * D + 16 * d + row] = f32_to_bf16_rne(acc[j][d][k] * inv);
        if (row == 0 && a.lse_out) a.lse_out[orow] = lr != 0.f ? (mr + log2f(lr)) * kLn2 : kNegInf;
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill(const DecodeArgs& a, hipStream_t stream) {
  PrefillArgs pa{};
  pa.a = a;
  const int G = a.Hq / a.Hkv;
  pa.groups = (a.T * G + kRows - 1) / kRows;
  const long long items = (long long)pa.groups * a.B * a.Hkv;
  if (items <= 0) return hipSuccess;
  if (items > 0x7fffffff) return hipErrorInvalidValue;
  const float sl2 = a.scale * kLog2e;
  if (a.D == 64)
    hipLaunchKernelGGL(prefill_kernel<64>, dim3((unsigned)items), dim3(kThreads), 0, stream, pa, sl2);
  else
    hipLaunchKernelGGL(prefill_kernel<128>, dim3((unsigned)items), dim3(kThreads), 0, stream, pa, sl2);
  return hipGetLastError();
}

}  // namespace pkv
