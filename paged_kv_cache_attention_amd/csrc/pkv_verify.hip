// Multi-query (speculative verify) paged attention on MFMA (gfx950).
//
// The verify step of speculative decoding scores T drafted tokens of a
// sequence in one pass ("LLM Inference from Scratch", Architecture overview,
// M7: small draft + big target verify).  With GQA, the T*G query rows that
// share one KV head form a real small GEMM against the cached keys, so here a
// wave owns one KV head of one sequence and its rows r = t*G + g (r < 16):
//
//   S^T[token][row] = K[token][:] . Q[row][:]      v_mfma_f32_16x16x32_bf16
//   (A = K straight from the 16-byte global loads, B = Q^T from registers;
//    the result layout puts one row and 4 consecutive tokens in each lane)
//   online softmax per row, causal limit L - T + t per row
//   O[row][d] += P[row][token] . V[token][d]       v_mfma_f32_16x16x16_bf16
//   (A = P: exactly the S^T result layout; P is split into bf16 hi + lo so the
//    product keeps about 16 bits of P; B = V transposed through LDS)
//
// Work distribution is the balanced one of the VALU path: a fixed grid of
// persistent workgroups, one wave per KV head, splits the block list of all
// sequences into equal ranges; sequences cut by range boundaries leave
// normalised partials merged by log-sum-exp weights.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kBS = 16;
constexpr int kMaxWpg = 8;
constexpr float kSlack = 8.f;
constexpr int kVRow = 272;   // LDS row stride of the V tile (bytes): 256 + 16 keeps reads and writes conflict-free

typedef __bf16 bf16x4_v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));

struct VerifyArgs {
  DecodeArgs a;
  const int* hdr;     // [total, per, tbtot]
  const int* prefix;  // [B + 1] blocks per sequence, prefix sums
  const int* first;   // [ranges]
  float* part;        // [(ranges + B)][T][Hq][D + 1]
  int ranges;
};

__device__ __forceinline__ bf16x8_v as_bf16x8(u32x4_t v) {
  bf16x8_v r;
  __builtin_memcpy(&r, &v, sizeof(r));
  return r;
}

__device__ __forceinline__ uint32_t pack_bf16(uint16_t lo, uint16_t hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

template <int D, int PD>
__global__ __launch_bounds__(64 * kMaxWpg) void verify_mfma_kernel(VerifyArgs va, float scale_log2e) {
  constexpr int KSTEPS = D / 32;   // 16x16x32 steps over the head dimension
  constexpr int DT = D / 16;       // 16-wide output column tiles
  const DecodeArgs& a = va.a;
  const int lane = threadIdx.x & 63;
  const int wpg = blockDim.x >> 6;
  const int rng = blockIdx.x / (a.Hkv / wpg);
  const int kv = (blockIdx.x % (a.Hkv / wpg)) * wpg + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int total = va.hdr[0], per = va.hdr[1];
  const int F0 = rng * per;
  if (F0 >= total) return;
  const int F1 = min(total, F0 + per);
  int b = va.first[rng];

  __shared__ __attribute__((aligned(16))) unsigned char vtile_all[kMaxWpg][kBS * kVRow];
  unsigned char* vtile = vtile_all[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)];

  const int G = a.Hq / a.Hkv;
  const int R = a.T * G;                 // query rows of this KV head (<= 16)
  const int row = lane & 15;             // this lane's row in S^T / P
  const int quad = lane >> 4;            // token quad (4 tokens) in S^T / P, row quad in O
  const bool row_ok = row < R;
  const int t_row = row / G;
  const size_t kv_row_bytes = (size_t)a.Hkv * D * 2;          // one token, all KV heads
  const size_t block_bytes = (size_t)kBS * kv_row_bytes;
  // byte offset of this lane's 16-byte chunk for MFMA step c: token = lane%16, d = 32c + 8*quad
  const uint32_t lane_off = (uint32_t)((size_t)row * kv_row_bytes + (size_t)kv * D * 2 + quad * 16);
  const unsigned char* kpool = static_cast<const unsigned char*>(a.k_pool) + lane_off;
  const unsigned char* vpool = static_cast<const unsigned char*>(a.v_pool) + lane_off;
  const int nmax = a.N_blocks - 1;
  const int max_tokens = a.max_blocks * kBS;

  while (true) {
    const int pstart = va.prefix[b], plen = va.prefix[b + 1] - pstart;
    const int js = max(F0, pstart) - pstart;
    const int je = min(F1, pstart + plen) - pstart;
    const bool direct = pstart >= F0 && pstart + plen <= F1;
    if (je > js) {
      const int L = clampi(a.context_lens[b], 0, max_tokens);
      // keys visible to this lane's row, cut at the end of the piece
      const int hi_row = row_ok ? min(L - a.T + t_row + 1, je * kBS) : 0;

      // Q^T as the B operand: lane (row, quad) holds Q[row][32c + 8*quad .. +8]
      u32x4_t qreg[KSTEPS];
      {
        const int rq = row_ok ? row : 0;   // padding rows read row 0 and are zeroed
        const int tq = rq / G, g = rq - tq * G;
        const unsigned char* qp = reinterpret_cast<const unsigned char*>(static_cast<const uint16_t*>(a.q)) +
                                  (((size_t)(b * a.T + tq) * a.Hq + kv * G + g) * D + quad * 8) * 2;
#pragma unroll
        for (int c = 0; c < KSTEPS; ++c) {
          const u32x4_t v = load16(qp + c * 64);
          qreg[c] = row_ok ? v : u32x4_t{0u, 0u, 0u, 0u};
        }
      }

      float m_row = kNegInf, l_part = 0.f;
      floatx4_t acc[DT];
#pragma unroll
      for (int d = 0; d < DT; ++d) acc[d] = floatx4_t{0.f, 0.f, 0.f, 0.f};

      const int nb = je - js;
      const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks + js;
      u32x4_t kbuf[PD][KSTEPS], vbuf[PD][KSTEPS];
      int tbl = 0, cn = 0;
      auto load_block = [&](u32x4_t (&dst)[KSTEPS], const unsigned char* pool, int ph) {
        const unsigned char* base = pool + (size_t)ph * block_bytes;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < KSTEPS; ++c) dst[c] = load16(base + c * 64);
        __builtin_amdgcn_sched_barrier(0);
      };
      auto phys = [&](int i) { return __builtin_amdgcn_readlane(tbl, i < cn ? i : cn - 1); };

      auto body = [&](u32x4_t (&kcur)[KSTEPS], u32x4_t (&vcur)[KSTEPS], int kb, int i) {
        const int ph_ahead = phys(i + PD);
        // V tile -> LDS rows (token-major, padded), to be read back transposed.  Rows
        // past the sequence end are zeroed: p = 0 there, and 0 * poison is NaN.
        const bool vok = kb * kBS + row < L;
#pragma unroll
        for (int c = 0; c < KSTEPS; ++c)
          store16(vtile + row * kVRow + (32 * c + 8 * quad) * 2, vok ? vcur[c] : u32x4_t{0u, 0u, 0u, 0u});
        // S^T = K Q^T
        floatx4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KSTEPS; ++c)
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kcur[c]), as_bf16x8(qreg[c]), s, 0, 0, 0);
        load_block(kcur, kpool, ph_ahead);
        load_block(vcur, vpool, ph_ahead);
        // online softmax: lane holds row `row`, tokens 4*quad .. 4*quad+3 of the block
        const int tok0 = kb * kBS + 4 * quad;
        float sv[4];
        bool need = false;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          sv[k] = tok0 + k < hi_row ? s[k] * scale_log2e : kNegInf;
          need |= sv[k] > m_row + kSlack;
        }
        if (__builtin_amdgcn_ballot_w64(need)) {
          float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
          mx = fmaxf(mx, __shfl_xor(mx, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          const float m_new = fmaxf(m_row, mx);
          // 1 for rows that are still empty (both -inf), 0 on a row's first key
          const float alpha = m_row == m_new ? 1.f : __builtin_amdgcn_exp2f(m_row - m_new);
          l_part *= alpha;
          m_row = m_new;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float ak = __shfl(alpha, 4 * quad + k);   // O rows 4*quad + k
#pragma unroll
            for (int d = 0; d < DT; ++d) acc[d][k] *= ak;
          }
        }
        float p[4];
        uint16_t ph[4], pl[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          p[k] = sv[k] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(sv[k] - m_row);
          l_part += p[k];
          ph[k] = f32_to_bf16_rne(p[k]);
          pl[k] = f32_to_bf16_rne(p[k] - __uint_as_float((uint32_t)ph[k] << 16));
        }
        bf16x4_v phi, plo;
        {
          const uint32_t h2[2] = {pack_bf16(ph[0], ph[1]), pack_bf16(ph[2], ph[3])};
          const uint32_t l2[2] = {pack_bf16(pl[0], pl[1]), pack_bf16(pl[2], pl[3])};
          __builtin_memcpy(&phi, h2, 8);
          __builtin_memcpy(&plo, l2, 8);
        }
        __asm__ volatile("" ::: "memory");
        // O += P V, one 16-column tile at a time; V^T read from LDS as B[token][d]
        const uint16_t* vt16 = reinterpret_cast<const uint16_t*>(vtile);
#pragma unroll
        for (int d = 0; d < DT; ++d) {
          const int col = 16 * d + row;
          uint16_t vv[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) vv[k] = vt16[((4 * quad + k) * kVRow) / 2 + col];
          bf16x4_v bv;
          const uint32_t v2[2] = {pack_bf16(vv[0], vv[1]), pack_bf16(vv[2], vv[3])};
          __builtin_memcpy(&bv, v2, 8);
          acc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, bv, acc[d], 0, 0, 0);
          acc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, bv, acc[d], 0, 0, 0);
        }
        __asm__ volatile("" ::: "memory");
      };

      for (int c0 = 0; c0 < nb; c0 += 64) {
        cn = min(64, nb - c0);
        tbl = lane < cn ? clampi(trow[c0 + lane], 0, nmax) : 0;
#pragma unroll
        for (int s = 0; s < PD; ++s) {
          load_block(kbuf[s], kpool, phys(s));
          load_block(vbuf[s], vpool, phys(s));
        }
        for (int i = 0; i < cn; i += PD) {
#pragma unroll
          for (int s = 0; s < PD; ++s) body(kbuf[s], vbuf[s], js + c0 + i + s, i + s);
        }
      }

      // ---- finish the piece ----
      float l_row = l_part + __shfl_xor(l_part, 16);
      l_row += __shfl_xor(l_row, 32);
      const size_t out_row0 = (size_t)b * a.T * a.Hq;   // + t * Hq + h
      float* slot = va.part + (size_t)(rng + b) * a.T * a.Hq * (D + 1);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = 4 * quad + k;                // O row held in acc[*][k]
        const float lr = __shfl(l_row, r);
        const float mr = __shfl(m_row, r);
        if (r < R) {
          const int t = r / G, h = kv * G + (r - t * G);
          const float inv = lr != 0.f ? 1.f / lr : 0.f;
          const float lse = lr != 0.f ? (mr + log2f(lr)) * kLn2 : kNegInf;
          if (direct) {
            uint16_t* o = static_cast<uint16_t*>(a.out) + (out_row0 + (size_t)t * a.Hq + h) * D;
#pragma unroll
            for (int d = 0; d < DT; ++d) o[16 * d + row] = f32_to_bf16_rne(acc[d][k] * inv);
            if (row == 0 && a.lse_out) a.lse_out[out_row0 + (size_t)t * a.Hq + h] = lse;
          } else {
            float* od = slot + ((size_t)t * a.Hq + h) * (D + 1);
#pragma unroll
            for (int d = 0; d < DT; ++d) od[16 * d + row] = acc[d][k] * inv;
            if (row == 0) od[D] = lse;
          }
        }
      }
    }
    if (pstart + plen >= F1) break;
    ++b;
  }
}

// Merge of the pieces of sequences cut by range boundaries: one wave per
// (sequence, query token, 4 heads); 16 lanes per head.
template <int D>
__global__ __launch_bounds__(256) void verify_merge_kernel(VerifyArgs va) {
  constexpr int EPL = D / 16;
  constexpr int BATCH = 8;
  const DecodeArgs& a = va.a;
  const int lane = threadIdx.x & 63;
  const int gidx = blockIdx.x * 4 + (threadIdx.x >> 6);     // ((b * T + t) * Hq/4 + hq)
  const int HG = a.Hq / 4;
  if (gidx >= a.B * a.T * HG) return;
  const int per = va.hdr[1];
  const int hq = gidx % HG, bt = gidx / HG;
  const int b = bt / a.T, t = bt - b * a.T;
  const int pstart = va.prefix[b], plen = va.prefix[b + 1] - pstart;
  const int h = hq * 4 + (lane >> 4), d0 = (lane & 15) * EPL;
  uint16_t* out = static_cast<uint16_t*>(a.out) + (((size_t)b * a.T + t) * a.Hq + h) * D + d0;
  float* lse_out = a.lse_out ? a.lse_out + ((size_t)b * a.T + t) * a.Hq + h : nullptr;
  if (plen == 0) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) out[e] = 0;
    if (lse_out && (lane & 15) == 0) *lse_out = kNegInf;
    return;
  }
  const int w0 = pstart / per, w1 = (pstart + plen - 1) / per;
  if (w0 == w1) return;
  float m = kNegInf, ssum = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int w = w0; w <= w1; w += BATCH) {
    float lv[BATCH], ov[BATCH][EPL];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      lv[k] = kNegInf;
      if (w + k <= w1) {
        const float* slot = va.part + (((size_t)(w + k + b) * a.T + t) * a.Hq + h) * (D + 1);
        lv[k] = slot[D];
#pragma unroll
        for (int e = 0; e < EPL; ++e) ov[k][e] = slot[d0 + e];
      }
    }
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      if (lv[k] == kNegInf) continue;
      const float nm = fmaxf(m, lv[k]);
      const float sa = __builtin_amdgcn_exp2f((m - nm) * kLog2e);
      const float sb = __builtin_amdgcn_exp2f((lv[k] - nm) * kLog2e);
      ssum = ssum * sa + sb;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = acc[e] * sa + sb * ov[k][e];
      m = nm;
    }
  }
  const float inv = ssum != 0.f ? 1.f / ssum : 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) out[e] = f32_to_bf16_rne(acc[e] * inv);
  if (lse_out && (lane & 15) == 0) *lse_out = ssum != 0.f ? m + logf(ssum) : kNegInf;
}

int verify_ranges(int Hkv) { return kStreamWaves / Hkv; }   // one wave per KV head and range

}  // namespace

bool verify_mfma_supported(const DecodeArgs& a) {
  const int G = a.Hq / a.Hkv;
  return a.bf16 && (a.D == 64 || a.D == 128) && a.T >= 2 && a.T * G <= 16 && a.B <= kStreamMaxTB &&
         (a.Hkv <= kMaxWpg || a.Hkv % kMaxWpg == 0) && (long long)a.B * a.max_blocks < (1ll << 30);
}

size_t verify_workspace_bytes(int B, int T, int Hq, int D) {
  const size_t R = kStreamWaves;   // upper bound on ranges (Hkv = 1)
  size_t off = 256;
  off += (((size_t)B + 1) * 4 + 255) / 256 * 256;
  off += (R * 4 + 255) / 256 * 256;
  off += (R + (size_t)B) * T * Hq * (D + 1) * 4;
  return off;
}

hipError_t launch_verify_mfma(const DecodeArgs& a, void* workspace, hipStream_t stream) {
  VerifyArgs va{};
  va.a = a;
  va.ranges = verify_ranges(a.Hkv);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  int* hdr = reinterpret_cast<int*>(ws);
  int* prefix = reinterpret_cast<int*>(ws + 256);
  int* first = reinterpret_cast<int*>(ws + 256 + (((size_t)a.B + 1) * 4 + 255) / 256 * 256);
  float* part = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(first) +
                                         ((size_t)kStreamWaves * 4 + 255) / 256 * 256);
  va.hdr = hdr; va.prefix = prefix; va.first = first; va.part = part;
  // one unit per sequence: blocks = ceil(L / 16)
  hipError_t e = launch_plan(a.context_lens, a.B, 1, va.ranges, a.max_blocks * kBS, hdr, prefix, first, stream);
  if (e != hipSuccess) return e;
  const int wpg = a.Hkv < kMaxWpg ? a.Hkv : kMaxWpg;
  const float sl2 = a.scale * kLog2e;
  if (a.D == 64)
    hipLaunchKernelGGL((verify_mfma_kernel<64, 2>), dim3(va.ranges * (a.Hkv / wpg)), dim3(64 * wpg), 0, stream, va, sl2);
  else
    hipLaunchKernelGGL((verify_mfma_kernel<128, 2>), dim3(va.ranges * (a.Hkv / wpg)), dim3(64 * wpg), 0, stream, va, sl2);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int waves = a.B * a.T * (a.Hq / 4);
  if (a.D == 64)
    hipLaunchKernelGGL((verify_merge_kernel<64>), dim3((waves + 3) / 4), dim3(256), 0, stream, va);
  else
    hipLaunchKernelGGL((verify_merge_kernel<128>), dim3((waves + 3) / 4), dim3(256), 0, stream, va);
  return hipGetLastError();
}

}  // namespace pkv
