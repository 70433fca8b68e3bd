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
//
// Split-KV partitions (partition_size > 0): the same balanced ranges, and a
// wave cuts its piece of a sequence at the partition boundaries (every PB
// blocks from position 0).  A partition inside one range leaves its
// normalised partial and log-sum-exp in the documented [B, T, Hq, P_max]
// layout (or goes straight to `out` when the sequence has one partition).  A
// partition cut by range boundaries leaves a piece per range in per-range
// slots: a range holds at most two such pieces, the one its start cuts and
// the one its end cuts.  The partition merge kernel combines those pieces into
// the partition's partial (written back to the documented layout), then
// merges every sequence's partitions by log-sum-exp.
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
// Partition staging area per wave: 16 rows of D + 4 floats.
template <int D>
constexpr int kStageFloats = 16 * (D + 4);

struct VerifyArgs {
  DecodeArgs a;       // with partitions: a.part_out [B, T, Hq, P_max, D], a.part_lse [B, T, Hq, P_max]
  int* hdr;           // [total, per, tbtot]
  int* prefix;        // [B + 1] blocks per sequence, prefix sums
  const int* first;   // [ranges] first non-empty sequence of each range (index into udesc)
  const int4* udesc;  // [B + 1] non-empty sequences, x = sequence
  float* part;        // single pass: [(ranges + B)][T][Hq][D + 1]; partitions: [2 * ranges][T][Hq][D + 1]
  int ranges;
  int PB;             // blocks per partition (partitions only)
};

// Prefix sums over n counts (count(i) for i < n) into sp[0..n] by the whole
// workgroup, kInlinePT consecutive entries per thread; returns the total.
template <typename CountFn>
__device__ __forceinline__ int inline_scan(int n, CountFn count, int* sp, int* wsc) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), nw = blockDim.x >> 6;
  int nb[kInlinePT];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < kInlinePT; ++j) {
    const int i = tid * kInlinePT + j;
    nb[j] = i < n ? count(i) : 0;
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
    if (i <= n) sp[i] = run;   // i = n: the total
    run += nb[j];
  }
  __syncthreads();
  return total;
}

// The plan inside the kernel, by the whole workgroup: each sequence's block
// count (ceil(L / 16)) and their prefix sums into sp[0 .. B] (LDS).
// Workgroup g publishes entries g * threads + tid (+ multiples of all
// threads) and workgroup 0 the header, for the merge kernel.  Returns the
// total.
__device__ __forceinline__ int verify_inline_plan(const VerifyArgs& va, int* sp, int* wsc) {
  const DecodeArgs& a = va.a;
  const int tid = threadIdx.x;
  const int max_tokens = a.max_blocks * kBS;
  const int total = inline_scan(a.B, [&](int b) { return (clampi(a.context_lens[b], 0, max_tokens) + kBS - 1) / kBS; },
                                sp, wsc);
  for (int k = blockIdx.x * blockDim.x + tid; k <= a.B; k += gridDim.x * blockDim.x) va.prefix[k] = sp[k];
  if (blockIdx.x == 0 && tid == 0) {
    va.hdr[0] = total;
    va.hdr[1] = max(kMinBlocksPerRange, (total + va.ranges - 1) / va.ranges);
    va.hdr[2] = total;
  }
  return total;
}

// Normalise the tile's rows and store them: bf16 rows of `out` (and lse_out)
// when `to_out`, else fp32 rows `o_at(t, h)` of D values with their natural-log
// lse at `lse_at(t, h)`.  Rows with no visible key get o = 0, lse = -inf.
template <int D, typename OAt, typename LAt>
__device__ __forceinline__ void emit_rows(const tile::State<D>& st, const DecodeArgs& a, int b, int kv, int G, int R,
                                          bool to_out, OAt o_at, LAt lse_at, int lane) {
  constexpr int DT = D / 16;
  const int row = lane & 15, quad = lane >> 4;
  const float l_row = tile::row_sum(st);
  const size_t out_row0 = (size_t)b * a.T * a.Hq;   // + t * Hq + h
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = 4 * quad + k;                // O row held in acc[*][k]
    const float lr = __shfl(l_row, r);
    const float mr = __shfl(st.m_row, r);
    if (r < R) {
      const int t = r / G, h = kv * G + (r - t * G);
      const float inv = lr != 0.f ? 1.f / lr : 0.f;
      const float lse = lr != 0.f ? (mr + log2f(lr)) * kLn2 : kNegInf;
      if (to_out) {
        uint16_t* o = static_cast<uint16_t*>(a.out) + (out_row0 + (size_t)t * a.Hq + h) * D;
#pragma unroll
        for (int d = 0; d < DT; ++d) o[16 * d + row] = f32_to_bf16_rne(st.acc[d][k] * inv);
        if (row == 0 && a.lse_out) a.lse_out[out_row0 + (size_t)t * a.Hq + h] = lse;
      } else {
        float* od = o_at(t, h);
#pragma unroll
        for (int d = 0; d < DT; ++d) od[16 * d + row] = st.acc[d][k] * inv;
        if (row == 0) *lse_at(t, h) = lse;
      }
    }
  }
}

// A partition's normalised rows, staged through the wave's LDS area so that
// they leave as whole rows of 16-byte stores (each row D contiguous floats
// of part_out) instead of 4-byte stores scattered over the rows: rows r < R
// of the tile, row r being query token t = r / G, head kv G + r % G; lse to
// part_lse.  The area holds 16 rows of D + 4 floats (the padding puts the 4
// rows a store instruction writes on distinct banks).
template <int D>
__device__ __forceinline__ void emit_partition_staged(const tile::State<D>& st, const DecodeArgs& a, size_t prow,
                                                      int p, int kv, int G, int R, float* stage, int lane) {
  constexpr int DT = D / 16, STR = D + 4, C4 = D / 4;   // 16-byte chunks per row
  const int row = lane & 15, quad = lane >> 4;
  const float l_row = tile::row_sum(st);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = 4 * quad + k;
    const float lr = __shfl(l_row, r);
    const float inv = lr != 0.f ? 1.f / lr : 0.f;
#pragma unroll
    for (int d = 0; d < DT; ++d) stage[r * STR + 16 * d + row] = st.acc[d][k] * inv;
  }
  if (quad == 0 && row < R) {   // row lane r holds its own max and sum
    const float lr = l_row;
    const int t = row / G, h = kv * G + (row - t * G);
    a.part_lse[(prow + (size_t)t * a.Hq + h) * a.P_max + p] = lr != 0.f ? (st.m_row + log2f(lr)) * kLn2 : kNegInf;
  }
  // (LDS operations of one wave complete in order: the reads see the writes)
  for (int c = lane; c < R * C4; c += 64) {
    const int r = c / C4, c4 = c - r * C4;
    const int t = r / G, h = kv * G + (r - t * G);
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + r * STR + 4 * c4);
    store16(a.part_out + ((prow + (size_t)t * a.Hq + h) * a.P_max + p) * D + 4 * c4, v);
  }
}

// INL: the plan is computed in the kernel (LDS); otherwise read from the
// workspace written by the planning kernel.  LDS (dynamic): one V tile per
// wave, then with INL the prefix list; with PART a staging area of 16 rows
// per wave.  PART: split-KV partitions of va.PB blocks.
template <int D, int PD, bool INL, bool PART>
__global__ __launch_bounds__(64 * kMaxWpg) void verify_mfma_kernel(VerifyArgs va, float scale_log2e) {
  const DecodeArgs& a = va.a;
  const int lane = threadIdx.x & 63;
  const int wpg = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  extern __shared__ __attribute__((aligned(16))) unsigned char vlds[];
  constexpr int kTileBytes = tile::run_tile_bytes<D, PD>();
  unsigned char* vtiles = vlds + wave * kTileBytes;
  int* sprefix = reinterpret_cast<int*>(vlds + wpg * kTileBytes);
  float* stage = reinterpret_cast<float*>(vlds + wpg * kTileBytes + (INL ? kInlinePerWave * wpg * 4 : 0)) +
                 wave * kStageFloats<D>;
  __shared__ int wsc[16];
  int total, per;
  if constexpr (INL) {
    total = __builtin_amdgcn_readfirstlane(verify_inline_plan(va, sprefix, wsc));
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

  const size_t slot_floats = (size_t)a.T * a.Hq * (D + 1);
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
      const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks;
      if constexpr (PART) {
        // the partitions this range holds of sequence b, one at a time
        const int PB = va.PB;
        const int Pb = (plen + PB - 1) / PB;
        for (int p0 = js; p0 < je;) {
          const int p = p0 / PB;
          const int pe = min(je, (p + 1) * PB);
          tile::State<D> st;
          tile::init(st);
          tile::run<D, PD>(st, qreg, hi_row, L, trow + p0, p0, pe - p0, nmax, kpool, vhead, kv_row_bytes,
                           block_bytes, vtiles, scale_log2e, lane);
          const bool whole = p0 == p * PB && pe == min(plen, (p + 1) * PB);
          if (whole && Pb > 1) {
            emit_partition_staged<D>(st, a, (size_t)b * a.T * a.Hq, p, kv, G, R, stage, lane);
          } else if (whole) {
            emit_rows<D>(st, a, b, kv, G, R, true, [&](int, int) { return (float*)nullptr; },
                         [&](int, int) { return (float*)nullptr; }, lane);
          } else {
            // a piece of a partition cut by this range's start (slot 0) or,
            // starting inside the range, by its end (slot 1)
            float* slot = va.part + (size_t)(2 * rng + (p0 == p * PB ? 1 : 0)) * slot_floats;
            emit_rows<D>(st, a, b, kv, G, R, false,
                         [&](int t, int h) { return slot + ((size_t)t * a.Hq + h) * (D + 1); },
                         [&](int t, int h) { return slot + ((size_t)t * a.Hq + h) * (D + 1) + D; }, lane);
          }
          p0 = pe;
        }
      } else {
        tile::State<D> st;
        tile::init(st);
        tile::run<D, PD>(st, qreg, hi_row, L, trow + js, js, je - js, nmax, kpool, vhead, kv_row_bytes, block_bytes,
                         vtiles, scale_log2e, lane);
        float* slot = va.part + (size_t)(rng + b) * slot_floats;
        emit_rows<D>(st, a, b, kv, G, R, direct,
                     [&](int t, int h) { return slot + ((size_t)t * a.Hq + h) * (D + 1); },
                     [&](int t, int h) { return slot + ((size_t)t * a.Hq + h) * (D + 1) + D; }, lane);
      }
    }
    if (pstart + plen >= F1) break;
    ++b;
  }
}

// Merge of the pieces of sequences cut by range boundaries: one wave per
// (sequence, query token, 4 heads); 16 lanes per head.  A sequence inside one
// range was written directly.
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

// Log-sum-exp of two normalised partials (o, lse) into the first; an empty
// one (lse = -inf) is never read.
template <int N>
__device__ __forceinline__ void lse_pair(float& l, float (&o)[N], float l2, const float (&o2)[N]) {
  if (l2 == kNegInf) return;
  if (l == kNegInf) {
    l = l2;
#pragma unroll
    for (int e = 0; e < N; ++e) o[e] = o2[e];
    return;
  }
  const float m = fmaxf(l, l2);
  const float w1 = __builtin_amdgcn_exp2f((l - m) * kLog2e), w2 = __builtin_amdgcn_exp2f((l2 - m) * kLog2e);
  const float inv = 1.f / (w1 + w2);
#pragma unroll
  for (int e = 0; e < N; ++e) o[e] = (w1 * o[e] + w2 * o2[e]) * inv;
  l = m + logf(w1 + w2);
}

// Merge of the split-KV partitions, one wave per output row (b, t, h): lane
// group g (16 lanes, D/16 elements each) takes partitions g, g + 4, ... in
// batches whose loads are issued together, and the four groups' running
// states are combined at the end.  A partition cut by range boundaries is
// first rebuilt from its pieces (the range holding its first block wrote slot
// 1, every later range slot 0) and, when the sequence has several
// partitions, written back to the documented partial layout.  Sequences with
// one partition inside one range were written directly and are skipped.
template <int D>
__global__ __launch_bounds__(256) void partition_merge_kernel(VerifyArgs va) {
  constexpr int EPL = D / 16;
  constexpr int NB = 4;   // partitions per group whose loads are issued together
  const DecodeArgs& a = va.a;
  const int lane = threadIdx.x & 63, grp = lane >> 4, d0 = (lane & 15) * EPL;
  const int rowi = blockIdx.x * 4 + (threadIdx.x >> 6);   // (b * T + t) * Hq + h
  if (rowi >= a.B * a.T * a.Hq) return;
  const int h = rowi % a.Hq, bt = rowi / a.Hq;
  const int b = bt / a.T, t = bt - b * a.T;
  const int per = va.hdr[1], PB = va.PB;
  const int pstart = va.prefix[b], plen = va.prefix[b + 1] - pstart;
  const int Pb = (plen + PB - 1) / PB;
  uint16_t* out = static_cast<uint16_t*>(a.out) + (size_t)rowi * D + d0;
  float* lse_out = a.lse_out ? a.lse_out + rowi : nullptr;
  if (plen > 0 && Pb == 1 && pstart / per == (pstart + plen - 1) / per) return;   // written by the tile
  const size_t slot_floats = (size_t)a.T * a.Hq * (D + 1);
  const size_t srow = ((size_t)t * a.Hq + h) * (D + 1);
  float* po = a.part_out + (size_t)rowi * a.P_max * D + d0;
  float* pl = a.part_lse + (size_t)rowi * a.P_max;

  float m = kNegInf, ssum = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int p0 = grp; p0 < Pb; p0 += 4 * NB) {
    float lv[NB], ov[NB][EPL];
    int cut_lo[NB], cut_hi[NB];   // ranges of a cut partition (cut_lo < cut_hi), else equal
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int p = p0 + 4 * k;
      lv[k] = kNegInf;
      cut_lo[k] = cut_hi[k] = 0;
      if (p < Pb) {
        const int s0 = pstart + p * PB, e0 = pstart + min(plen, (p + 1) * PB);
        const int r0 = s0 / per, r1 = (e0 - 1) / per;
        const float* src = r0 == r1 ? nullptr : va.part + (size_t)(2 * r0 + 1) * slot_floats + srow;
        lv[k] = src ? src[D] : pl[p];
#pragma unroll
        for (int e = 0; e < EPL; ++e) ov[k][e] = src ? src[d0 + e] : po[(size_t)p * D + e];
        cut_lo[k] = r0;
        cut_hi[k] = r1;
      }
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (cut_lo[k] == cut_hi[k]) continue;
      for (int r = cut_lo[k] + 1; r <= cut_hi[k]; ++r) {   // the later pieces (slot 0 of each later range)
        const float* src = va.part + (size_t)(2 * r) * slot_floats + srow;
        float o2[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) o2[e] = src[d0 + e];
        lse_pair<EPL>(lv[k], ov[k], src[D], o2);
      }
      if (Pb > 1) {   // the partition's partial, in the documented layout
        const int p = p0 + 4 * k;
#pragma unroll
        for (int e = 0; e < EPL; ++e) po[(size_t)p * D + e] = lv[k] == kNegInf ? 0.f : ov[k][e];
        if ((lane & 15) == 0) pl[p] = lv[k];
      }
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (lv[k] == kNegInf) continue;   // absent or empty partition: its o is not read
      const float nm = fmaxf(m, lv[k]);
      const float sa = __builtin_amdgcn_exp2f((m - nm) * kLog2e);
      const float sb = __builtin_amdgcn_exp2f((lv[k] - nm) * kLog2e);
      ssum = ssum * sa + sb;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = acc[e] * sa + sb * ov[k][e];
      m = nm;
    }
  }
  // combine the four groups (partners 16 and 32 lanes away)
#pragma unroll
  for (int off = 16; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(ssum, off);
    const float nm = fmaxf(m, m2);
    const float sa = m == kNegInf ? 0.f : __builtin_amdgcn_exp2f((m - nm) * kLog2e);
    const float sb = m2 == kNegInf ? 0.f : __builtin_amdgcn_exp2f((m2 - nm) * kLog2e);
    ssum = ssum * sa + s2 * sb;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = acc[e] * sa + __shfl_xor(acc[e], off) * sb;
    m = nm;
  }
  if (grp == 0) {
    const float inv = ssum != 0.f ? 1.f / ssum : 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) out[e] = f32_to_bf16_rne(acc[e] * inv);
    if (lse_out && lane == 0) *lse_out = ssum != 0.f ? m + logf(ssum) : kNegInf;
  }
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

namespace {
// The tile's plan area: header, per-sequence block prefix sums, each range's
// first sequence and the sequence descriptors (the last two written only by
// the planning kernel).
struct PlanLayout {
  size_t prefix, first, udesc, end;
};
size_t align256(size_t n) { return (n + 255) / 256 * 256; }
PlanLayout plan_layout(int B) {
  PlanLayout l{};
  l.prefix = 256;
  l.first = l.prefix + align256(((size_t)B + 1) * 4);
  l.udesc = l.first + align256((size_t)kStreamWaves * 4);
  l.end = l.udesc + align256(((size_t)B + 1) * 16);
  return l;
}
}  // namespace

// Single pass.  Piece slots: (ranges + B) slots of T * Hq rows, where
// ranges * T * Hq = kStreamWaves * T * G <= kStreamWaves * min(16, T * Hq)
// for every shape the tile takes.
size_t verify_workspace_bytes(int B, int T, int Hq, int D) {
  const size_t rows = (size_t)kStreamWaves * (T * Hq < 16 ? T * Hq : 16) + (size_t)B * T * Hq;
  return plan_layout(B).end + rows * (D + 1) * 4;
}

// Beyond the documented partials: the plan and two piece slots per range.
size_t verify_partition_extra_bytes(int B, int T, int Hq, int D) {
  const size_t rows = (size_t)kStreamWaves * (T * Hq < 16 ? T * Hq : 16);
  return plan_layout(B).end + 2 * rows * (D + 1) * 4;
}

hipError_t launch_verify_mfma(const DecodeArgs& a, void* workspace, hipStream_t stream) {
  VerifyArgs va{};
  va.a = a;
  va.ranges = verify_ranges(a.Hkv);
  const bool part = a.part_tokens > 0;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  if (part) {   // the documented partials first, then the plan and the piece slots
    va.a.part_out = reinterpret_cast<float*>(ws);
    va.a.part_lse = va.a.part_out + (size_t)a.B * a.T * a.Hq * a.P_max * a.D;
    ws += align256((size_t)a.B * a.T * a.Hq * a.P_max * (a.D + 1) * 4);
    va.PB = a.part_tokens / kBS;
  }
  const PlanLayout pl = plan_layout(a.B);
  int* hdr = reinterpret_cast<int*>(ws);
  int* prefix = reinterpret_cast<int*>(ws + pl.prefix);
  int* first = reinterpret_cast<int*>(ws + pl.first);
  int4* udesc = reinterpret_cast<int4*>(ws + pl.udesc);
  va.hdr = hdr; va.prefix = prefix; va.first = first; va.udesc = udesc;
  va.part = reinterpret_cast<float*>(ws + pl.end);
  // the V tiles of every wave of a workgroup share its LDS: fewer waves per
  // workgroup where they would not fit (the grid then has more workgroups)
  const size_t tile_bytes = a.D == 64 ? tile::run_tile_bytes<64, kTilePD>() : tile::run_tile_bytes<128, kTilePD>();
  const size_t stage_bytes = part ? (a.D == 64 ? kStageFloats<64> : kStageFloats<128>) * 4 : 0;
  int wpg = a.Hkv < kMaxWpg ? a.Hkv : kMaxWpg;
  // At D = 64, workgroups of at most 4 waves (twice as many per CU, the same
  // waves per SIMD) measured faster: 1B decode batch 51.4 against 53.0 us.
  // At D = 128 they were not (8B batch 216.5 against 215.7, long-context
  // verify 433.3 against 429.5).  Halving keeps Hkv a multiple of wpg.
  if (a.D == 64)
    while (wpg > 4 && wpg % 2 == 0) wpg /= 2;
  const size_t lds_cap = (size_t)device_lds_per_block() - 64;
  while (wpg % 2 == 0 && (size_t)wpg * (tile_bytes + stage_bytes) > lds_cap) wpg /= 2;
  const size_t tiles = (size_t)wpg * tile_bytes;
  const size_t lds_inl = tiles + (size_t)kInlinePerWave * wpg * 4 + (size_t)wpg * stage_bytes;
  const bool inl = a.B + 1 <= kInlinePerWave * wpg && lds_inl <= lds_cap;
  hipError_t e = hipSuccess;
  // one unit per sequence: blocks = ceil(L / 16)
  if (!inl) e = launch_plan(a.context_lens, a.B, 1, va.ranges, a.max_blocks, hdr, prefix, first, udesc, stream);
  if (e != hipSuccess) return e;
  const float sl2 = a.scale * kLog2e;
  const dim3 grid(va.ranges * (a.Hkv / wpg)), block(64 * wpg);
  const size_t lds = inl ? lds_inl : tiles + (size_t)wpg * stage_bytes;
#define PKV_VERIFY_LAUNCH(DD, INLV, PARTV) \
  hipLaunchKernelGGL((verify_mfma_kernel<DD, kTilePD, INLV, PARTV>), grid, block, lds, stream, va, sl2)
  if (a.D == 64) {
    if (part) { if (inl) PKV_VERIFY_LAUNCH(64, true, true); else PKV_VERIFY_LAUNCH(64, false, true); }
    else { if (inl) PKV_VERIFY_LAUNCH(64, true, false); else PKV_VERIFY_LAUNCH(64, false, false); }
  } else {
    if (part) { if (inl) PKV_VERIFY_LAUNCH(128, true, true); else PKV_VERIFY_LAUNCH(128, false, true); }
    else { if (inl) PKV_VERIFY_LAUNCH(128, true, false); else PKV_VERIFY_LAUNCH(128, false, false); }
  }
#undef PKV_VERIFY_LAUNCH
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (part) {
    const int rows = a.B * a.T * a.Hq;
    if (a.D == 64)
      hipLaunchKernelGGL((partition_merge_kernel<64>), dim3((rows + 3) / 4), dim3(256), 0, stream, va);
    else
      hipLaunchKernelGGL((partition_merge_kernel<128>), dim3((rows + 3) / 4), dim3(256), 0, stream, va);
    return hipGetLastError();
  }
  const int waves = a.B * a.T * (a.Hq / 4);
  if (a.D == 64)
    hipLaunchKernelGGL((verify_merge_kernel<64>), dim3((waves + 3) / 4), dim3(256), 0, stream, va);
  else
    hipLaunchKernelGGL((verify_merge_kernel<128>), dim3((waves + 3) / 4), dim3(256), 0, stream, va);
  return hipGetLastError();
}

}  // namespace pkv
