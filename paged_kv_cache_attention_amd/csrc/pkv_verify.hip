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
// normalised partials merged by log-sum-exp weights.  While B + 1 fits the
// workgroup's LDS list (kInlinePerWave entries per wave) every workgroup scans
// the lengths itself and keeps the per-sequence block prefix sums in LDS;
// otherwise the planning kernel writes them to the workspace first.
#include "pkv_device.h"
#include "pkv_internal.h"
#include "pkv_tile.h"

namespace pkv {
namespace {

constexpr int kBS = 16;
constexpr int kMaxWpg = 8;
// Blocks whose K and V are in flight while a wave works on one.  One measured
// faster than two and three on the 8B shared-prefix decode batch (216.1,
// 218.2, 222.3 us), the 1B batch (53.8, 54.8, 57.3 us) and the long-context
// verify batch (432.6, 436.6, 439.8 us).
constexpr int kTilePD = 1;

constexpr int kInlinePerWave = 512;            // LDS prefix entries per wave
constexpr int kInlinePT = kInlinePerWave / 64;  // sequences per thread
constexpr int kMinBlocksPerRange = 16;

struct VerifyArgs {
  DecodeArgs a;
  int* hdr;           // [total, per, tbtot]
  int* prefix;        // [B + 1] blocks per sequence, prefix sums
  const int* first;   // [ranges] first non-empty sequence of each range (index into udesc)
  const int4* udesc;  // [B + 1] non-empty sequences, x = sequence
  float* part;        // [(ranges + B)][T][Hq][D + 1]
  int ranges;
};

// Block prefix sums of the sequences (blocks = ceil(L / 16)) into sp[0..B],
// by the whole workgroup; returns the total.  Workgroup g publishes entries
// g*threads + tid (+ multiples of all threads) and workgroup 0 the header, for
// the merge kernel.
__device__ __forceinline__ int verify_inline_prefix(const VerifyArgs& va, int* sp, int* wsc) {
  const DecodeArgs& a = va.a;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), nw = blockDim.x >> 6;
  const int max_tokens = a.max_blocks * kBS;
  int nb[kInlinePT];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < kInlinePT; ++j) {
    const int i = tid * kInlinePT + j;
    nb[j] = i < a.B ? (clampi(a.context_lens[i], 0, max_tokens) + kBS - 1) / kBS : 0;
    sum += nb[j];
  }
  int is = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(is, off);
    if (lane >= off) is += y;
  }
  if (lane == 63) wsc[wave] = is;
  __syncthreads();
  int run = is - sum, total = 0;
  for (int w = 0; w < nw; ++w) {
    const int v = wsc[w];
    if (w < wave) run += v;
    total += v;
  }
#pragma unroll
  for (int j = 0; j < kInlinePT; ++j) {
    const int i = tid * kInlinePT + j;
    if (i <= a.B) sp[i] = run;   // i = B: the total
    run += nb[j];
  }
  __syncthreads();
  {   // the merge kernel reads prefix and per
    for (int k = blockIdx.x * blockDim.x + tid; k <= a.B; k += gridDim.x * blockDim.x) va.prefix[k] = sp[k];
    if (blockIdx.x == 0 && tid == 0) {
      va.hdr[0] = total;
      va.hdr[1] = max(kMinBlocksPerRange, (total + va.ranges - 1) / va.ranges);
      va.hdr[2] = total;
    }
  }
  return total;
}

// INL: prefix sums computed in the kernel (LDS); otherwise read from the
// workspace written by the planning kernel.  LDS (dynamic): one V tile per
// wave, then with INL the prefix list.
template <int D, int PD, bool INL>
__global__ __launch_bounds__(64 * kMaxWpg) void verify_mfma_kernel(VerifyArgs va, float scale_log2e) {
  constexpr int DT = D / 16;
  const DecodeArgs& a = va.a;
  const int lane = threadIdx.x & 63;
  const int wpg = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  extern __shared__ __attribute__((aligned(16))) unsigned char vlds[];
  constexpr int kTileBytes = tile::run_tile_bytes<D, PD>();
  unsigned char* vtiles = vlds + wave * kTileBytes;
  int* sprefix = reinterpret_cast<int*>(vlds + wpg * kTileBytes);
  __shared__ int wsc[16];
  int total, per;
  if constexpr (INL) {
    total = __builtin_amdgcn_readfirstlane(verify_inline_prefix(va, sprefix, wsc));
    per = max(kMinBlocksPerRange, (total + va.ranges - 1) / va.ranges);
  } else {
    total = va.hdr[0];
    per = va.hdr[1];
  }
  auto prefix_of = [&](int i) -> int {
    if constexpr (INL) return sprefix[i];
    else return va.prefix[i];
  };
  // Workgroup -> range: as in the decode stream, each XCD takes a
  // contiguous run of ranges when they are longer than the minimum, so that
  // neighbouring sequences sharing prefix blocks re-read them through one L2.
  const bool contiguous = INL && gridDim.x % 8 == 0 && per > kMinBlocksPerRange;
  const int wid = __builtin_amdgcn_readfirstlane(contiguous ? (int)xcd_logical_id(blockIdx.x, gridDim.x / 8)
                                                            : (int)blockIdx.x);
  const int rng = wid / (a.Hkv / wpg);
  const int kv = (wid % (a.Hkv / wpg)) * wpg + wave;
  const int F0 = rng * per;
  if (F0 >= total) return;
  const int F1 = min(total, F0 + per);
  int b;
  if constexpr (INL) {
    // the sequence holding block F0: largest b < B with prefix[b] <= F0
    int lo = 0, hi = a.B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (sprefix[mid] <= F0) lo = mid; else hi = mid;
    }
    b = __builtin_amdgcn_readfirstlane(lo);
  } else {
    b = va.udesc[va.first[rng]].x;
  }

  const int G = a.Hq / a.Hkv;
  const int R = a.T * G;                 // query rows of this KV head (<= 16)
  const int row = lane & 15;             // this lane's row in S^T / P
  const int quad = lane >> 4;            // row quad in O
  const bool row_ok = row < R;
  const int rq = row_ok ? row : 0;
  const int t_row = rq / G;
  const size_t kv_row_bytes = (size_t)a.Hkv * D * 2;
  const size_t block_bytes = (size_t)kBS * kv_row_bytes;
  const uint32_t lane_off = (uint32_t)((size_t)row * kv_row_bytes + (size_t)kv * D * 2 + quad * 16);
  const unsigned char* kpool = static_cast<const unsigned char*>(a.k_pool) + lane_off;
  const unsigned char* vhead = static_cast<const unsigned char*>(a.v_pool) + (size_t)kv * D * 2;
  const int nmax = a.N_blocks - 1;
  const int max_tokens = a.max_blocks * kBS;

  while (true) {
    const int pstart = prefix_of(b), plen = prefix_of(b + 1) - pstart;
    const int js = max(F0, pstart) - pstart;
    const int je = min(F1, pstart + plen) - pstart;
    const bool direct = pstart >= F0 && pstart + plen <= F1;
    if (je > js) {
      const int L = clampi(a.context_lens[b], 0, max_tokens);
      const int hi_row = row_ok ? L - a.T + t_row + 1 : 0;   // causal limit of this row's query token
      u32x4_t qreg[D / 32];
      tile::load_q<D>(qreg, static_cast<const uint16_t*>(a.q) +
                                ((size_t)(b * a.T + t_row) * a.Hq + kv * G + (rq - t_row * G)) * D,
                      row_ok, lane);
      tile::State<D> st;
      tile::init(st);
      tile::run<D, PD>(st, qreg, hi_row, L, a.block_tables + (size_t)b * a.max_blocks + js, js, je - js, nmax, kpool,
                       vhead, kv_row_bytes, block_bytes, vtiles, scale_log2e, lane);

      // ---- finish the piece ----
      const float l_row = tile::row_sum(st);
      const size_t out_row0 = (size_t)b * a.T * a.Hq;   // + t * Hq + h
      float* slot = va.part + (size_t)(rng + b) * a.T * a.Hq * (D + 1);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = 4 * quad + k;                // O row held in acc[*][k]
        const float lr = __shfl(l_row, r);
        const float mr = __shfl(st.m_row, r);
        if (r < R) {
          const int t = r / G, h = kv * G + (r - t * G);
          const float inv = lr != 0.f ? 1.f / lr : 0.f;
          const float lse = lr != 0.f ? (mr + log2f(lr)) * kLn2 : kNegInf;
          if (direct) {
            uint16_t* o = static_cast<uint16_t*>(a.out) + (out_row0 + (size_t)t * a.Hq + h) * D;
#pragma unroll
            for (int d = 0; d < DT; ++d) o[16 * d + row] = f32_to_bf16_rne(st.acc[d][k] * inv);
            if (row == 0 && a.lse_out) a.lse_out[out_row0 + (size_t)t * a.Hq + h] = lse;
          } else {
            float* od = slot + ((size_t)t * a.Hq + h) * (D + 1);
#pragma unroll
            for (int d = 0; d < DT; ++d) od[16 * d + row] = st.acc[d][k] * inv;
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
  constexpr int BATCH = 16;   // pieces whose loads are issued together
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
  return a.bf16 && (a.D == 64 || a.D == 128) && a.T >= 1 && a.T * G <= 16 && a.B <= kStreamMaxTB &&
         (a.Hkv <= kMaxWpg || a.Hkv % kMaxWpg == 0) && (long long)a.B * a.max_blocks < (1ll << 30);
}

// Every shape the tile supports takes it, single-token decode included (its
// T = 1 rows are the G query heads of a KV head, 1 to 8 of the 16 tile rows).
// Measured against the VALU stream kernel at T = 1: faster for every head
// group size at D = 64 (Llama-3.2-1B shape 57.0 -> 55.1 us; 64 query heads
// over 8 KV heads 97.0 -> 66.5 us) and for the 8B shared-prefix batch
// (222.7 -> 217.9 us); about 3 % slower on a 64-sequence D = 128, G = 4
// batch without shared blocks, and 1.2 us slower on an 8-sequence batch of
// 1,681 tokens.  The stream kernel serves fp32 and the shapes with more than
// 16 query rows per KV head.
bool verify_tile_for(const DecodeArgs& a) { return verify_mfma_supported(a); }

size_t verify_workspace_bytes(int B, int T, int Hq, int D) {
  const size_t R = kStreamWaves;   // upper bound on ranges (Hkv = 1)
  size_t off = 256;
  off += (((size_t)B + 1) * 4 + 255) / 256 * 256;
  off += (R * 4 + 255) / 256 * 256;
  off += (((size_t)B + 1) * 16 + 255) / 256 * 256;
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
  int4* udesc = reinterpret_cast<int4*>(reinterpret_cast<unsigned char*>(first) +
                                        ((size_t)kStreamWaves * 4 + 255) / 256 * 256);
  float* part = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(udesc) +
                                         (((size_t)a.B + 1) * 16 + 255) / 256 * 256);
  va.hdr = hdr; va.prefix = prefix; va.first = first; va.udesc = udesc; va.part = part;
  // the V tiles of every wave of a workgroup share its LDS: fewer waves per
  // workgroup where they would not fit (the grid then has more workgroups)
  const size_t tile_bytes = a.D == 64 ? tile::run_tile_bytes<64, kTilePD>() : tile::run_tile_bytes<128, kTilePD>();
  int wpg = a.Hkv < kMaxWpg ? a.Hkv : kMaxWpg;
  // At D = 64, workgroups of at most 4 waves (twice as many per CU, the same
  // waves per SIMD) measured faster: 1B decode batch 51.4 against 53.0 us.
  // At D = 128 they were not (8B batch 216.5 against 215.7, long-context
  // verify 433.3 against 429.5).  Halving keeps Hkv a multiple of wpg.
  if (a.D == 64)
    while (wpg > 4 && wpg % 2 == 0) wpg /= 2;
  while (wpg % 2 == 0 && (size_t)wpg * tile_bytes + 64 > (size_t)device_lds_per_block()) wpg /= 2;
  const size_t tiles = (size_t)wpg * tile_bytes;
  const size_t lds_inl = tiles + (size_t)kInlinePerWave * wpg * 4;
  const bool inl = a.B + 1 <= kInlinePerWave * wpg && lds_inl + 64 <= (size_t)device_lds_per_block();
  hipError_t e = hipSuccess;
  // one unit per sequence: blocks = ceil(L / 16)
  if (!inl) e = launch_plan(a.context_lens, a.B, 1, va.ranges, a.max_blocks, hdr, prefix, first, udesc, stream);
  if (e != hipSuccess) return e;
  const float sl2 = a.scale * kLog2e;
  const dim3 grid(va.ranges * (a.Hkv / wpg)), block(64 * wpg);
  if (a.D == 64) {
    if (inl) hipLaunchKernelGGL((verify_mfma_kernel<64, kTilePD, true>), grid, block, lds_inl, stream, va, sl2);
    else hipLaunchKernelGGL((verify_mfma_kernel<64, kTilePD, false>), grid, block, tiles, stream, va, sl2);
  } else {
    if (inl) hipLaunchKernelGGL((verify_mfma_kernel<128, kTilePD, true>), grid, block, lds_inl, stream, va, sl2);
    else hipLaunchKernelGGL((verify_mfma_kernel<128, kTilePD, false>), grid, block, tiles, stream, va, sl2);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int waves = a.B * a.T * (a.Hq / 4);
  if (a.D == 64)
    hipLaunchKernelGGL((verify_merge_kernel<64>), dim3((waves + 3) / 4), dim3(256), 0, stream, va);
  else
    hipLaunchKernelGGL((verify_merge_kernel<128>), dim3((waves + 3) / 4), dim3(256), 0, stream, va);
  return hipGetLastError();
}

}  // namespace pkv
