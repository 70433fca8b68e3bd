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
// Split-KV partitions (partition_size > 0): the same balanced ranges, walked
// the same way, and the walk cuts at the partition boundaries (every PB
// blocks from position 0) without stopping its loads.  A partition inside one
// range leaves its normalised partial and log-sum-exp in the documented
// [B, T, Hq, P_max] layout; each partition is also folded by log-sum-exp into
// a running state of the wave (LDS), which becomes the range's piece of the
// sequence, exactly as in the single pass.  A partition cut by range
// boundaries leaves a piece per range in per-range slots: a range holds at
// most two such pieces, the one its start cuts and the one its end cuts.  The
// finishing kernel merges each sequence's range pieces into `out` and
// rebuilds every cut partition's partial from its pieces.
#include "pkv_device.h"
#include "pkv_internal.h"
#include "pkv_tile.h"

namespace pkv {
namespace {

constexpr int kBS = 16;
constexpr int kMaxWpg = 8;
// Blocks whose K and V are in flight while a wave works on one.
constexpr int kTilePD = 1;
// Running partition state of a wave: 16 rows of D + 4 floats (the padding
// puts the 4 rows one LDS instruction touches on distinct banks).
template <int D>
constexpr int kRunFloats = 16 * (D + 4);

// LDS bytes per wave: the V tile; with partitions as many bytes again (the
// two together stage a partition's 16 x D float partial, while the V tile is
// idle) and the running state.
template <int D, bool PART>
constexpr int verify_wave_lds() {
  return tile::run_tile_bytes<D>() * (PART ? 2 : 1) + (PART ? kRunFloats<D> * 4 : 0);
}
static_assert(2 * tile::run_tile_bytes<64>() == 16 * 64 * 4 && 2 * tile::run_tile_bytes<128>() == 16 * 128 * 4,
              "the partition stage is the V tile and as many bytes after it");

constexpr int kInlinePerWave = 512;            // LDS prefix entries per wave
constexpr int kInlinePT = kInlinePerWave / 64;  // sequences per thread
constexpr int kMinBlocksPerRange = 16;
// V is streamed (non-temporal loads, tile::run) when the call's K and V
// exceed twice the device's 256 MB last-level cache; a batch that fits keeps
// its rows cached from one decode step to the next (Llama-3.2-1B batch, 257
// MB: 53.0 us per call with the default policy, 54.0 streamed).
constexpr long long kStreamVBytes = 512ll << 20;

struct VerifyArgs {
  DecodeArgs a;       // with partitions: a.part_out [B, T, Hq, P_max, D], a.part_lse [B, T, Hq, P_max]
  int* hdr;           // [total, per, tbtot]
  int* prefix;        // [B + 1] blocks per sequence, prefix sums
  const int* first;   // [ranges] first non-empty sequence of each range (index into udesc)
  const int4* udesc;  // [B + 1] non-empty sequences, x = sequence
  float* part;        // range pieces: [(ranges + B)][T][Hq][D + 1], piece of sequence b in range r at r + b
  float* cut;         // partitions: pieces of cut partitions, [2 * ranges][T][Hq][D + 1]
  int ranges;
  int PB;             // blocks per partition (partitions only)
};

// Prefix sums over n counts (count(i) for i < n) into sp[0..n] by the whole
// workgroup, kInlinePT consecutive entries per thread; returns the total.
// count(i, raw) turns raw = load(min(i, n - 1)) into the count of entry i;
// every thread loads its kInlinePT raw values first, unconditionally (n >= 1),
// so that the loads are in flight together rather than one at a time.
template <typename LoadFn, typename CountFn>
__device__ __forceinline__ int inline_scan(int n, LoadFn load, CountFn count, int* sp, int* wsc) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), nw = blockDim.x >> 6;
  int nb[kInlinePT];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < kInlinePT; ++j) nb[j] = load(min(tid * kInlinePT + j, n - 1));
#pragma unroll
  for (int j = 0; j < kInlinePT; ++j) {
    const int i = tid * kInlinePT + j;
    nb[j] = i < n ? count(i, nb[j]) : 0;
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
  const int total = inline_scan(a.B, [&](int b) { return a.context_lens[b]; },
                                [&](int, int L) { return (clampi(L, 0, max_tokens) + kBS - 1) / kBS; }, sp, wsc);
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

// A whole partition's normalised rows r < R (query token t = r / G, head
// kv G + r % G) to the documented partials, through the wave's LDS stage so
// that they leave as whole rows of 16-byte stores (row D contiguous floats)
// rather than 64-byte pieces of 16 rows far apart (measured about twice as
// costly); lse from the row lanes.  Stage row r: D floats, 16-byte chunk c
// at chunk c ^ 4 ((r / 4) % 4), which puts the 4 rows one write instruction
// touches on distinct banks.
template <int D>
__device__ __forceinline__ void emit_partition_staged(const tile::State<D>& st, const DecodeArgs& a, size_t prow,
                                                      int p, int kv, int G, int R, float* stage, int lane) {
  constexpr int DT = D / 16, C4 = D / 4;
  const int row = lane & 15, quad = lane >> 4;
  const float l_row = tile::row_sum(st);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = 4 * quad + k;
    const float lr = __shfl(l_row, r);
    const float inv = lr != 0.f ? 1.f / lr : 0.f;
#pragma unroll
    for (int d = 0; d < DT; ++d)
      stage[r * D + 4 * ((4 * d + (row >> 2)) ^ (4 * quad)) + (row & 3)] = st.acc[d][k] * inv;
  }
  if (quad == 0 && row < R) {   // the row lanes hold their row's max and sum
    const int t = row / G, h = kv * G + (row - t * G);
    a.part_lse[(prow + (size_t)t * a.Hq + h) * a.P_max + p] = l_row != 0.f ? (st.m_row + log2f(l_row)) * kLn2
                                                                           : kNegInf;
  }
  // (one wave's LDS operations complete in order: the reads see the writes)
  for (int c = lane; c < R * C4; c += 64) {
    const int r = c / C4, c4 = c - r * C4;
    const int t = r / G, h = kv * G + (r - t * G);
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + r * D + 4 * (c4 ^ (4 * ((r >> 2) & 3))));
    store16(a.part_out + ((prow + (size_t)t * a.Hq + h) * a.P_max + p) * D + 4 * c4, v);
  }
}

// Fold a partition's tile state into the wave's running state: O rows in
// LDS (row r at run + r * (D + 4), unnormalised, scaled to the running max;
// each lane keeps to the elements its accumulators hold), the running max
// (base 2) and denominator of row lane % 16 in registers.  `first`: the
// running state is empty.
template <int D>
__device__ __forceinline__ void fold_partition(const tile::State<D>& st, float* run, float& mrun, float& lrun,
                                               bool first, int lane) {
  constexpr int DT = D / 16, STR = D + 4;
  const int row = lane & 15, quad = lane >> 4;
  const float l_p = tile::row_sum(st);
  const float m_new = fmaxf(mrun, st.m_row);
  // 1 for a side that holds the new max (two empty sides included)
  const float sa = mrun == m_new ? 1.f : __builtin_amdgcn_exp2f(mrun - m_new);
  const float sb = st.m_row == m_new ? 1.f : __builtin_amdgcn_exp2f(st.m_row - m_new);
  lrun = first ? l_p : lrun * sa + l_p * sb;
  mrun = first ? st.m_row : m_new;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = 4 * quad + k;
    const float ak = __shfl(sa, r), bk = __shfl(sb, r);
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      float* x = run + r * STR + 16 * d + row;
      *x = first ? st.acc[d][k] : *x * ak + st.acc[d][k] * bk;
    }
  }
}

// The running state as a tile state (for emit_rows): row sums whole in the
// quad-0 lanes.
template <int D>
__device__ __forceinline__ void load_running(tile::State<D>& st, const float* run, float mrun, float lrun, int lane) {
  constexpr int DT = D / 16, STR = D + 4;
  const int row = lane & 15, quad = lane >> 4;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int d = 0; d < DT; ++d) st.acc[d][k] = run[(4 * quad + k) * STR + 16 * d + row];
  st.m_row = mrun;
  st.l_part = quad == 0 ? lrun : 0.f;
}

// INL: the plan is computed in the kernel (LDS); otherwise read from the
// workspace written by the planning kernel.  LDS (dynamic): per wave its V
// tile and with PART its running state, then with INL the prefix list.
// PART: split-KV partitions of va.PB blocks.
template <int D, bool INL, bool PART>
__global__ __launch_bounds__(64 * kMaxWpg) void verify_mfma_kernel(VerifyArgs va, float scale_log2e) {
  const DecodeArgs& a = va.a;
  const int lane = threadIdx.x & 63;
  const int wpg = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  extern __shared__ __attribute__((aligned(16))) unsigned char vlds[];
  constexpr int kWaveLds = verify_wave_lds<D, PART>();
  unsigned char* vtile = vlds + wave * kWaveLds;
  float* stage = reinterpret_cast<float*>(vtile);                                      // PART only
  float* run = reinterpret_cast<float*>(vtile + 2 * tile::run_tile_bytes<D>());   // PART only
  int* sprefix = reinterpret_cast<int*>(vlds + wpg * kWaveLds);
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
  const bool stream_v = (long long)total * kBS * a.Hkv * D * 4 > kStreamVBytes;
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
      // the neighbours' table entries at the same logical blocks (within
      // their rows: js .. je - 1 < max_blocks); equal ids mark shared blocks
      const int32_t* tprev = b > 0 ? trow - a.max_blocks + js : nullptr;
      const int32_t* tnext = b + 1 < a.B ? trow + a.max_blocks + js : nullptr;
      float* piece = va.part + (size_t)(rng + b) * slot_floats;
      tile::State<D> st;
      tile::init(st);
      if constexpr (PART) {
        const int PB = va.PB;
        const int Pb = (plen + PB - 1) / PB;
        const size_t prow = (size_t)b * a.T * a.Hq;   // + t * Hq + h: the row's partials
        float mrun = kNegInf, lrun = 0.f;
        bool first = true;
        // partition p ends before block kb_end: its partial (whole in this
        // range) or its piece (cut by a range boundary) when the sequence has
        // several partitions, and its fold into the running state
        auto flush = [&](tile::State<D>& s, int kb_end) {
          // the lane index through an empty asm: what the flush derives from
          // it (LDS and global addresses) is then computed here, not hoisted
          // out of the walk's loop, where those registers would crowd the
          // P.V step (its eight V reads, otherwise issued together, went one
          // at a time at 247 VGPRs)
          int ln = lane;
          __asm__ volatile("" : "+v"(ln));
          const int p = (kb_end - 1) / PB;
          const bool starts = js <= p * PB;
          const bool ends = kb_end == min(plen, (p + 1) * PB);
          if (Pb > 1) {
            if (starts && ends) {
              emit_partition_staged<D>(s, a, prow, p, kv, G, R, stage, ln);
            } else {
              // cut by this range's start (slot 0) or, starting in it, by its end (slot 1)
              float* slot = va.cut + (size_t)(2 * rng + (starts ? 1 : 0)) * slot_floats;
              emit_rows<D>(s, a, b, kv, G, R, false,
                           [&](int t, int h) { return slot + ((size_t)t * a.Hq + h) * (D + 1); },
                           [&](int t, int h) { return slot + ((size_t)t * a.Hq + h) * (D + 1) + D; }, ln);
            }
          }
          fold_partition<D>(s, run, mrun, lrun, first, ln);
          first = false;
          tile::init(s);
        };
        tile::run<D, kTilePD>(st, qreg, hi_row, L, trow + js, js, je - js, nmax, kpool, vhead, kv_row_bytes,
                                   block_bytes, vtile, scale_log2e, lane, PB, flush, stream_v, tprev, tnext);
        flush(st, je);
        load_running<D>(st, run, mrun, lrun, lane);
      } else {
        tile::run<D, kTilePD>(st, qreg, hi_row, L, trow + js, js, je - js, nmax, kpool, vhead, kv_row_bytes,
                                   block_bytes, vtile, scale_log2e, lane, 0, tile::NoFlush(), stream_v, tprev, tnext);
      }
      emit_rows<D>(st, a, b, kv, G, R, direct,
                   [&](int t, int h) { return piece + ((size_t)t * a.Hq + h) * (D + 1); },
                   [&](int t, int h) { return piece + ((size_t)t * a.Hq + h) * (D + 1) + D; }, lane);
    }
    if (pstart + plen >= F1) break;
    ++b;
  }
}

// Merge of the pieces of sequences cut by range boundaries: one wave per
// (sequence, query token, 4 heads); 16 lanes per head.  A sequence inside one
// range was written directly.
template <int D>
__device__ __forceinline__ void merge_pieces(const VerifyArgs& va, int gidx, int lane) {
  constexpr int EPL = D / 16;
  constexpr int BATCH = 16;   // pieces whose loads are issued together
  const DecodeArgs& a = va.a;
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

// The partial of a partition cut by range boundaries, rebuilt from its pieces
// and written to the documented layout: one wave per (range boundary r >= 1,
// query token, 4 heads).  The partition cut by boundary r, if any, is handled
// at the first boundary that cuts it; the range holding its first block wrote
// the piece to slot 1, every later range to slot 0.  Sequences with a single
// partition have no partials.
template <int D>
__device__ __forceinline__ void rebuild_cut_partition(const VerifyArgs& va, int gidx, int lane) {
  constexpr int EPL = D / 16;
  const DecodeArgs& a = va.a;
  const int HG = a.Hq / 4;
  if (gidx >= (va.ranges - 1) * a.T * HG) return;
  const int hq = gidx % HG, rt = gidx / HG;
  const int t = rt % a.T, r = rt / a.T + 1;
  const int total = va.hdr[0], per = va.hdr[1], PB = va.PB;
  const int F = r * per;
  if (F >= total) return;
  int lo = 0, hi = a.B;   // the sequence holding block F: prefix[lo] <= F < prefix[lo + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (va.prefix[mid] <= F) lo = mid; else hi = mid;
  }
  const int b = lo;
  const int pstart = va.prefix[b], plen = va.prefix[b + 1] - pstart;
  const int off = F - pstart;
  if (off % PB == 0 || plen <= PB) return;   // no partition cut here, or a single partition
  const int p = off / PB;
  const int r0 = (pstart + p * PB) / per;
  if (r != r0 + 1) return;
  const int r1 = (pstart + min(plen, (p + 1) * PB) - 1) / per;
  const int h = hq * 4 + (lane >> 4), d0 = (lane & 15) * EPL;
  const size_t slot_floats = (size_t)a.T * a.Hq * (D + 1);
  const size_t srow = ((size_t)t * a.Hq + h) * (D + 1);
  const float* src = va.cut + (size_t)(2 * r0 + 1) * slot_floats + srow;
  float l = src[D], o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = src[d0 + e];
  for (int rr = r0 + 1; rr <= r1; ++rr) {
    const float* s2 = va.cut + (size_t)(2 * rr) * slot_floats + srow;
    float o2[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o2[e] = s2[d0 + e];
    lse_pair<EPL>(l, o, s2[D], o2);
  }
  const size_t prow = ((size_t)b * a.T + t) * a.Hq + h;
  float* po = a.part_out + (prow * a.P_max + p) * D + d0;
#pragma unroll
  for (int e = 0; e < EPL; ++e) po[e] = l == kNegInf ? 0.f : o[e];
  if ((lane & 15) == 0) a.part_lse[prow * a.P_max + p] = l;
}

// After the tile: workgroups [0, merge_blocks) merge range pieces into `out`,
// the rest (partitions only) rebuild cut partitions.  Four waves per workgroup.
template <int D>
__global__ __launch_bounds__(256) void verify_finish_kernel(VerifyArgs va, int merge_blocks) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if ((int)blockIdx.x < merge_blocks)
    merge_pieces<D>(va, blockIdx.x * 4 + wave, lane);
  else
    rebuild_cut_partition<D>(va, (blockIdx.x - merge_blocks) * 4 + wave, lane);
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

// Beyond the documented partials: the plan, the range-piece slots of the
// single pass, then two slots per range for pieces of cut partitions.
size_t verify_partition_extra_bytes(int B, int T, int Hq, int D) {
  return verify_workspace_bytes(B, T, Hq, D) + 2 * (size_t)kStreamWaves * (T * Hq < 16 ? T * Hq : 16) * (D + 1) * 4;
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
  va.cut = va.part + ((size_t)va.ranges + a.B) * a.T * a.Hq * (a.D + 1);
  // the per-wave LDS of a workgroup: fewer waves per workgroup where it
  // would not fit (the grid then has more workgroups)
  const size_t wave_lds = a.D == 64 ? (part ? verify_wave_lds<64, true>() : verify_wave_lds<64, false>())
                                    : (part ? verify_wave_lds<128, true>() : verify_wave_lds<128, false>());
  int wpg = a.Hkv < kMaxWpg ? a.Hkv : kMaxWpg;
  // At D = 64, workgroups of at most 4 waves (twice as many per CU, the same
  // waves per SIMD) measured faster: 1B decode batch 51.4 against 53.0 us.
  // At D = 128 they were not (8B batch 216.5 against 215.7, long-context
  // verify 433.3 against 429.5).  Halving keeps Hkv a multiple of wpg.
  if (a.D == 64)
    while (wpg > 4 && wpg % 2 == 0) wpg /= 2;
  const size_t lds_cap = (size_t)device_lds_per_block() - 64;
  while (wpg % 2 == 0 && (size_t)wpg * wave_lds > lds_cap) wpg /= 2;
  const size_t lds_waves = (size_t)wpg * wave_lds;
  const size_t lds_inl = lds_waves + (size_t)kInlinePerWave * wpg * 4;
  const bool inl = a.B + 1 <= kInlinePerWave * wpg && lds_inl <= lds_cap;
  hipError_t e = hipSuccess;
  // one unit per sequence: blocks = ceil(L / 16)
  if (!inl) e = launch_plan(a.context_lens, a.B, 1, va.ranges, a.max_blocks, hdr, prefix, first, udesc, stream);
  if (e != hipSuccess) return e;
  const float sl2 = a.scale * kLog2e;
  const dim3 grid(va.ranges * (a.Hkv / wpg)), block(64 * wpg);
  const size_t lds = inl ? lds_inl : lds_waves;
#define PKV_VERIFY_LAUNCH(DD, INLV, PARTV) \
  hipLaunchKernelGGL((verify_mfma_kernel<DD, INLV, PARTV>), grid, block, lds, stream, va, sl2)
  if (a.D == 64) {
    if (part) { if (inl) PKV_VERIFY_LAUNCH(64, true, true); else PKV_VERIFY_LAUNCH(64, false, true); }
    else { if (inl) PKV_VERIFY_LAUNCH(64, true, false); else PKV_VERIFY_LAUNCH(64, false, false); }
  } else {
    if (part) { if (inl) PKV_VERIFY_LAUNCH(128, true, true); else PKV_VERIFY_LAUNCH(128, false, true); }
    else { if (inl) PKV_VERIFY_LAUNCH(128, true, false); else PKV_VERIFY_LAUNCH(128, false, false); }
  }
#undef PKV_VERIFY_LAUNCH
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int merge_blocks = (a.B * a.T * (a.Hq / 4) + 3) / 4;
  const int fix_blocks = part ? ((va.ranges - 1) * a.T * (a.Hq / 4) + 3) / 4 : 0;
  if (merge_blocks + fix_blocks == 0) return hipSuccess;
  const dim3 fgrid(merge_blocks + fix_blocks);
  if (a.D == 64)
    hipLaunchKernelGGL((verify_finish_kernel<64>), fgrid, dim3(256), 0, stream, va, merge_blocks);
  else
    hipLaunchKernelGGL((verify_finish_kernel<128>), fgrid, dim3(256), 0, stream, va, merge_blocks);
  return hipGetLastError();
}

}  // namespace pkv
