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

// Shared prefixes (single pass, in-kernel plan): the sequences are taken in
// windows of M = 16 / (T G) adjacent ones (M >= 2), as many as one tile has
// rows for.  The leading blocks a window's sequences have in common (the same
// physical ids as its longest member, up to kShareMaxBlocks) form the window's
// prefix unit, attended once for all of them with every member's query rows in
// the one tile; each sequence's own unit is the rest of its blocks.  The flat
// block list is then, window by window: the prefix unit, then each member's
// own unit, so unit u = w (M + 1) + k is window w's prefix unit for k = 0 and
// the own unit of sequence w M + k - 1 otherwise.  Without sharing (M = 1
// here) unit u is sequence u.
constexpr int kShareMaxBlocks = 64;   // prefix blocks a window may share (1024 tokens)
constexpr int kShareSeg = 16;         // table entries one thread compares

struct VerifyArgs {
  DecodeArgs a;       // with partitions: a.part_out [B, T, Hq, P_max, D], a.part_lse [B, T, Hq, P_max]
  int* hdr;           // [total, per, tbtot]
  int* prefix;        // [units + 1] blocks per unit, prefix sums
  int* wshare;        // [windows] prefix blocks of each window (shared prefixes only)
  const int* first;   // [ranges] first non-empty sequence of each range (index into udesc)
  const int4* udesc;  // [B + 1] non-empty sequences, x = sequence
  float* part;        // single pass: [(ranges + B)][T][Hq][D + 1]; partitions: [2 * ranges][T][Hq][D + 1]
  float* gpart;       // shared prefixes: [(ranges + windows)][M * T][Hq][D + 1]
  int ranges;
  int PB;             // blocks per partition (partitions only)
  int M;              // sequences per window (1: no sharing)
};

__host__ __device__ inline int units_of(int B, int M) { return M > 1 ? (B + M - 1) / M * (M + 1) : B; }

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

// Shared prefix blocks of every window into sS[w] (M >= 2).  snb[b] holds
// each sequence's block count and sfirst[b] its first physical block.  A
// window's lead is its longest member (the first of equals); member m agrees
// with it up to d_m, the first block i < nb_m whose id differs (nb_m if none).
// The window shares S = min(nb_lead, kShareMaxBlocks, min over members with
// d_m < nb_m of d_m) blocks: every member that has block i < S holds the
// lead's block there.  Windows whose members do not all start with the lead's
// first block share nothing and load no table entries.  Threads take
// (sequence, 16-entry segment) pairs and issue all their loads at once.
__device__ __forceinline__ void detect_shared_prefixes(const DecodeArgs& a, int M, const int* snb, const int* sfirst,
                                                       int* sd, int* sS) {
  const int nwin = (a.B + M - 1) / M;
  constexpr int NSEG = kShareMaxBlocks / kShareSeg;
  const int pairs = a.B * NSEG;
  auto lead_of = [&](int w) {
    const int m0 = w * M, m1 = min(a.B, m0 + M);
    int ld = m0;
    for (int m = m0 + 1; m < m1; ++m)
      if (snb[m] > snb[ld]) ld = m;
    return ld;
  };
  for (int pr = threadIdx.x; pr < pairs; pr += blockDim.x) {
    const int m = pr / NSEG, sg = pr - m * NSEG;
    const int ld = lead_of(m / M);
    const int lim = min(min(snb[m], snb[ld]), kShareMaxBlocks);
    const int i0 = sg * kShareSeg;
    int d = kShareSeg;   // first differing entry of this segment, kShareSeg if none
    if (m != ld && sfirst[m] == sfirst[ld] && i0 < lim) {
      const int32_t* tm = a.block_tables + (size_t)m * a.max_blocks + i0;
      const int32_t* tl = a.block_tables + (size_t)ld * a.max_blocks + i0;
      int xm[kShareSeg], xl[kShareSeg];
#pragma unroll
      for (int k = 0; k < kShareSeg; ++k) {
        const bool ok = i0 + k < lim;
        xm[k] = ok ? tm[k] : 0;
        xl[k] = ok ? tl[k] : 0;
      }
#pragma unroll
      for (int k = kShareSeg - 1; k >= 0; --k)
        if (i0 + k < lim && xm[k] != xl[k]) d = k;
    }
    // a segment at or past lim holds no comparison; the lead agrees with itself
    sd[pr] = (m == ld || i0 >= lim) ? kShareSeg : (sfirst[m] == sfirst[ld] ? d : 0);
  }
  __syncthreads();
  for (int w = threadIdx.x; w < nwin; w += blockDim.x) {
    const int m0 = w * M, m1 = min(a.B, m0 + M);
    const int ld = lead_of(w);
    int S = min(snb[ld], kShareMaxBlocks);
    int members = 0;
    for (int m = m0; m < m1; ++m) {
      if (snb[m] == 0) continue;
      ++members;
      if (m == ld) continue;
      int dm = min(snb[m], kShareMaxBlocks);   // agreement over every block of m compared
      for (int sg = 0; sg < NSEG; ++sg) {
        const int v = sd[m * NSEG + sg];
        if (v < kShareSeg) {
          dm = min(dm, sg * kShareSeg + v);
          break;
        }
      }
      if (dm < min(snb[m], kShareMaxBlocks)) S = min(S, dm);   // m diverges inside its own blocks
    }
    sS[w] = members >= 2 ? S : 0;
  }
  __syncthreads();
}

// The plan inside the kernel, by the whole workgroup: unit block counts and
// their prefix sums into sp[0 .. units] (LDS), and with shared prefixes
// (va.M >= 2) each window's prefix blocks into sS (LDS; snb, sfirst and sd are
// LDS scratch of B, B and 4 B entries).  Workgroup g publishes entries
// g * threads + tid (+ multiples of all threads) of the prefix sums and the
// windows' prefix blocks, and workgroup 0 the header, for the merge kernel.
// Returns the total.
__device__ __forceinline__ int verify_inline_plan(const VerifyArgs& va, int* sp, int* wsc, int* snb, int* sfirst,
                                                  int* sd, int* sS) {
  const DecodeArgs& a = va.a;
  const int tid = threadIdx.x;
  const int max_tokens = a.max_blocks * kBS;
  const int M = va.M;
  auto nb_of = [&](int b) { return (clampi(a.context_lens[b], 0, max_tokens) + kBS - 1) / kBS; };
  int total;
  if (M > 1) {
    for (int b = tid; b < a.B; b += blockDim.x) {
      // both loads issued together (entry 0 of a row exists whatever the length)
      const int L = a.context_lens[b];
      const int f = a.block_tables[(size_t)b * a.max_blocks];
      const int n = (clampi(L, 0, max_tokens) + kBS - 1) / kBS;
      snb[b] = n;
      sfirst[b] = n > 0 ? f : -1 - b;
    }
    __syncthreads();
    detect_shared_prefixes(a, M, snb, sfirst, sd, sS);
    const int US = M + 1;
    total = inline_scan(units_of(a.B, M), [&](int u) {
      const int w = u / US, k = u - w * US;
      if (k == 0) return sS[w];
      const int b = w * M + k - 1;
      return b < a.B ? snb[b] - min(sS[w], snb[b]) : 0;
    }, sp, wsc);
    const int nwin = (a.B + M - 1) / M;
    for (int w = blockIdx.x * blockDim.x + tid; w < nwin; w += gridDim.x * blockDim.x) va.wshare[w] = sS[w];
  } else {
    total = inline_scan(a.B, nb_of, sp, wsc);
  }
  const int nu = units_of(a.B, M);
  for (int k = blockIdx.x * blockDim.x + tid; k <= nu; k += gridDim.x * blockDim.x) va.prefix[k] = sp[k];
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

// INL: the plan is computed in the kernel (LDS); otherwise read from the
// workspace written by the planning kernel.  LDS (dynamic): one V tile per
// wave, then with INL the unit prefix list (kInlinePerWave entries per wave)
// and, with shared prefixes, the detection scratch.  PART: split-KV partitions
// of va.PB blocks (no shared prefixes).
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
  int* snb = sprefix + kInlinePerWave * wpg;   // shared prefixes: [B] blocks per sequence
  int* sfirst = snb + a.B;                      // [B] first physical block
  int* sd = sfirst + a.B;                       // [B * 4] detection scratch
  int* sS = sd + a.B * (kShareMaxBlocks / kShareSeg);   // [windows] prefix blocks per window
  __shared__ int wsc[16];
  const int M = PART ? 1 : va.M;
  const int US = M > 1 ? M + 1 : 1;
  const int NU = units_of(a.B, M);
  int total, per;
  if constexpr (INL) {
    total = __builtin_amdgcn_readfirstlane(verify_inline_plan(va, sprefix, wsc, snb, sfirst, sd, sS));
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
  int u;   // the unit holding block F0
  if constexpr (INL) {
    // largest u < NU with prefix[u] <= F0 (a non-empty unit: F0 < total)
    int lo = 0, hi = NU;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (sprefix[mid] <= F0) lo = mid; else hi = mid;
    }
    u = __builtin_amdgcn_readfirstlane(lo);
  } else {
    u = va.udesc[va.first[rng]].x;
  }

  const int G = a.Hq / a.Hkv;
  const int R = a.T * G;                 // query rows of one sequence for this KV head (<= 16)
  const int row = lane & 15;             // this lane's row in S^T / P
  const int quad = lane >> 4;            // row quad in O
  const size_t kv_row_bytes = (size_t)a.Hkv * D * 2;
  const size_t block_bytes = (size_t)kBS * kv_row_bytes;
  const uint32_t lane_off = (uint32_t)((size_t)row * kv_row_bytes + (size_t)kv * D * 2 + quad * 16);
  const unsigned char* kpool = static_cast<const unsigned char*>(a.k_pool) + lane_off;
  const unsigned char* vhead = static_cast<const unsigned char*>(a.v_pool) + (size_t)kv * D * 2;
  const int nmax = a.N_blocks - 1;
  const int max_tokens = a.max_blocks * kBS;
  const uint16_t* qbase = static_cast<const uint16_t*>(a.q);

  const size_t slot_floats = (size_t)a.T * a.Hq * (D + 1);
  while (true) {
    const int ustart = prefix_of(u), ulen = prefix_of(u + 1) - ustart;
    const int js = max(F0, ustart) - ustart;
    const int je = min(F1, ustart + ulen) - ustart;
    const int w = u / US, k = u - w * US;
    if (je > js && M > 1 && k == 0) {
      // ---- prefix unit of window w: its blocks [0, S) for every member ----
      const int m0 = w * M, mc = min(M, a.B - m0);
      const int S = sS[w];
      int ld = m0;   // the longest member: the window's blocks are its table entries
      for (int m = m0 + 1; m < m0 + mc; ++m)
        if (snb[m] > snb[ld]) ld = m;
      ld = __builtin_amdgcn_readfirstlane(ld);
      // row r of the tile: member r / R, its query token and head
      const int jm = row / R;
      const bool rok = jm < mc;
      const int rr = rok ? row - jm * R : 0;
      const int tm = rr / G;
      const int bm = m0 + (rok ? jm : 0);
      const int Lm = clampi(a.context_lens[bm], 0, max_tokens);
      const int sm = min(S, (Lm + kBS - 1) / kBS);   // blocks of the prefix this member has
      const int hi = rok ? min(Lm - a.T + tm + 1, sm * kBS) : 0;
      // V rows at or past every member's shared length are zeroed
      int vl = rok ? min(Lm, sm * kBS) : 0;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) vl = max(vl, __shfl_xor(vl, off));
      u32x4_t qreg[D / 32];
      tile::load_q<D>(qreg, qbase + ((size_t)(bm * a.T + tm) * a.Hq + kv * G + (rr - tm * G)) * D, rok, lane);
      tile::State<D> st;
      tile::init(st);
      tile::run<D, PD>(st, qreg, hi, vl, a.block_tables + (size_t)ld * a.max_blocks + js, js, je - js, nmax, kpool,
                       vhead, kv_row_bytes, block_bytes, vtiles, scale_log2e, lane);
      // rows (member j, token t) as (j T + t) of the window's slot
      float* slot = va.gpart + (size_t)(rng + w) * M * slot_floats;
      emit_rows<D>(st, a, m0, kv, G, mc * R, false,
                   [&](int t, int h) { return slot + ((size_t)t * a.Hq + h) * (D + 1); },
                   [&](int t, int h) { return slot + ((size_t)t * a.Hq + h) * (D + 1) + D; }, lane);
    } else if (je > js) {
      // ---- own unit of sequence b: its blocks [sb, nb) ----
      const int b = M > 1 ? w * M + k - 1 : u;
      const int L = clampi(a.context_lens[b], 0, max_tokens);
      const int sb = M > 1 ? min(sS[w], (L + kBS - 1) / kBS) : 0;   // blocks its window's prefix unit took
      const bool row_ok = row < R;
      const int rq = row_ok ? row : 0;
      const int t_row = rq / G;
      const int hi_row = row_ok ? L - a.T + t_row + 1 : 0;   // causal limit of this row's query token
      u32x4_t qreg[D / 32];
      tile::load_q<D>(qreg, qbase + ((size_t)(b * a.T + t_row) * a.Hq + kv * G + (rq - t_row * G)) * D, row_ok,
                      lane);
      const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks;
      if constexpr (PART) {
        // the partitions this range holds of sequence b, one at a time
        const int PB = va.PB;
        const int Pb = (ulen + PB - 1) / PB;
        for (int p0 = js; p0 < je;) {
          const int p = p0 / PB;
          const int pe = min(je, (p + 1) * PB);
          tile::State<D> st;
          tile::init(st);
          tile::run<D, PD>(st, qreg, hi_row, L, trow + p0, p0, pe - p0, nmax, kpool, vhead, kv_row_bytes,
                           block_bytes, vtiles, scale_log2e, lane);
          const bool whole = p0 == p * PB && pe == min(ulen, (p + 1) * PB);
          if (whole) {
            const size_t prow = (size_t)b * a.T * a.Hq;   // (+ t * Hq + h) * P_max + p
            emit_rows<D>(st, a, b, kv, G, R, Pb == 1,
                         [&](int t, int h) { return a.part_out + ((prow + t * a.Hq + h) * a.P_max + p) * D; },
                         [&](int t, int h) { return a.part_lse + (prow + t * a.Hq + h) * a.P_max + p; }, lane);
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
        tile::run<D, PD>(st, qreg, hi_row, L, trow + sb + js, sb + js, je - js, nmax, kpool, vhead, kv_row_bytes,
                         block_bytes, vtiles, scale_log2e, lane);
        // straight to out when the sequence shares nothing and this range holds all of it
        const bool direct = sb == 0 && ustart >= F0 && ustart + ulen <= F1;
        float* slot = va.part + (size_t)(rng + b) * slot_floats;
        emit_rows<D>(st, a, b, kv, G, R, direct,
                     [&](int t, int h) { return slot + ((size_t)t * a.Hq + h) * (D + 1); },
                     [&](int t, int h) { return slot + ((size_t)t * a.Hq + h) * (D + 1) + D; }, lane);
      }
    }
    if (ustart + ulen >= F1 || u + 1 >= NU) break;
    ++u;
  }
}

// Merge of the pieces of each sequence: one wave per (sequence, query token,
// 4 heads); 16 lanes per head.  A sequence's pieces are those of its own unit
// (one per range it spans) and, with a shared prefix, those of its window's
// prefix unit.  A sequence that shares nothing and lies inside one range was
// written directly.
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
  const int M = va.M, US = M > 1 ? M + 1 : 1;
  const int w = M > 1 ? b / M : 0, j = M > 1 ? b - w * M : 0;
  const int uo = M > 1 ? w * US + 1 + j : b;
  const int ostart = va.prefix[uo], olen = va.prefix[uo + 1] - ostart;
  const int L = clampi(a.context_lens[b], 0, a.max_blocks * kBS);
  const int sb = M > 1 ? min(va.wshare[w], (L + kBS - 1) / kBS) : 0;
  const int h = hq * 4 + (lane >> 4), d0 = (lane & 15) * EPL;
  uint16_t* out = static_cast<uint16_t*>(a.out) + (((size_t)b * a.T + t) * a.Hq + h) * D + d0;
  float* lse_out = a.lse_out ? a.lse_out + ((size_t)b * a.T + t) * a.Hq + h : nullptr;
  if (sb == 0) {
    if (olen == 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) out[e] = 0;
      if (lse_out && (lane & 15) == 0) *lse_out = kNegInf;
      return;
    }
    if (ostart / per == (ostart + olen - 1) / per) return;
  }
  float m = kNegInf, ssum = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  // the pieces of one unit over ranges w0 .. w1, slot(r) its piece in range r
  auto absorb_unit = [&](int w0, int w1, auto slot) {
    for (int r = w0; r <= w1; r += BATCH) {
      float lv[BATCH], ov[BATCH][EPL];
#pragma unroll
      for (int k = 0; k < BATCH; ++k) {
        lv[k] = kNegInf;
        if (r + k <= w1) {
          const float* sl = slot(r + k);
          lv[k] = sl[D];
#pragma unroll
          for (int e = 0; e < EPL; ++e) ov[k][e] = sl[d0 + e];
        }
      }
#pragma unroll
      for (int k = 0; k < BATCH; ++k) {
        if (lv[k] == kNegInf) continue;
        const float nm = fmaxf(m, lv[k]);
        const float sa = __builtin_amdgcn_exp2f((m - nm) * kLog2e);
        const float sbw = __builtin_amdgcn_exp2f((lv[k] - nm) * kLog2e);
        ssum = ssum * sa + sbw;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = acc[e] * sa + sbw * ov[k][e];
        m = nm;
      }
    }
  };
  const size_t slot_floats = (size_t)a.T * a.Hq * (D + 1);
  if (sb > 0) {
    const int up = w * US;
    const int pstart = va.prefix[up], plen = va.prefix[up + 1] - pstart;
    const size_t prow = (((size_t)j * a.T + t) * a.Hq + h) * (D + 1);   // member j, token t in the window slot
    absorb_unit(pstart / per, (pstart + plen - 1) / per,
                [&](int r) { return va.gpart + (size_t)(r + w) * M * slot_floats + prow; });
  }
  if (olen > 0) {
    const size_t orow = ((size_t)t * a.Hq + h) * (D + 1);
    absorb_unit(ostart / per, (ostart + olen - 1) / per,
                [&](int r) { return va.part + (size_t)(r + b) * slot_floats + orow; });
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
// The tile's plan area: header, unit block prefix sums (at most 2 B + 17
// entries: with shared prefixes M >= 2 windows of M + 1 units), the windows'
// shared prefix blocks, each range's first sequence and the sequence
// descriptors (the last two written only by the planning kernel).
struct PlanLayout {
  size_t prefix, wshare, first, udesc, end;
};
size_t align256(size_t n) { return (n + 255) / 256 * 256; }
PlanLayout plan_layout(int B) {
  PlanLayout l{};
  l.prefix = 256;
  l.wshare = l.prefix + align256(((size_t)2 * B + 18) * 4);
  l.first = l.wshare + align256(((size_t)B + 1) * 4);
  l.udesc = l.first + align256((size_t)kStreamWaves * 4);
  l.end = l.udesc + align256(((size_t)B + 1) * 16);
  return l;
}

// Members per shared-prefix window for a shape: one tile's rows, 16 / (T G).
int window_members(int T, int G) { return 16 / (T * G); }

// Shared-prefix detection runs inside every workgroup (one pass over the
// windows' table entries): only for batches up to this size.
constexpr int kShareMaxB = 1024;
}  // namespace

// Single pass.  Piece slots of sequences: (ranges + B) slots of T * Hq rows,
// where ranges * T * Hq = kStreamWaves * T * G <= kStreamWaves * min(16,
// T * Hq) for every shape the tile takes.  Piece slots of shared prefixes:
// (ranges + windows) slots of M T Hq rows, with ranges M T Hq = kStreamWaves
// M T G <= kStreamWaves * 16 and windows M T Hq <= (B + M) T Hq <= (B + 16)
// T Hq.
size_t verify_workspace_bytes(int B, int T, int Hq, int D) {
  const size_t own = (size_t)kStreamWaves * (T * Hq < 16 ? T * Hq : 16) + (size_t)B * T * Hq;
  const size_t shared = (size_t)kStreamWaves * 16 + ((size_t)B + 16) * T * Hq;
  return plan_layout(B).end + (own + shared) * (D + 1) * 4;
}

// Beyond the documented partials: the plan and two piece slots per range.
// ranges * T * Hq = kStreamWaves * T * G <= kStreamWaves * 16 for every shape
// the tile takes.
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
  float* slots = reinterpret_cast<float*>(ws + pl.end);
  va.hdr = hdr; va.prefix = prefix; va.wshare = reinterpret_cast<int*>(ws + pl.wshare); va.first = first;
  va.udesc = udesc; va.part = slots;
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
  const size_t lds_list = tiles + (size_t)kInlinePerWave * wpg * 4;
  const size_t lds_cap = (size_t)device_lds_per_block() - 64;
  const bool inl = a.B + 1 <= kInlinePerWave * wpg && lds_list <= lds_cap;
  // shared prefixes: single pass, planned in the kernel, two or more
  // sequences per tile, and room for the units and the detection scratch
  int M = window_members(a.T, a.Hq / a.Hkv);
  const size_t lds_share = lds_list + ((size_t)6 * a.B + a.B / 2 + 8) * 4;
  if (part || !inl || M < 2 || a.B > kShareMaxB || units_of(a.B, M) + 1 > kInlinePerWave * wpg ||
      lds_share > lds_cap)
    M = 1;
  va.M = M;
  va.gpart = slots + ((size_t)va.ranges + a.B) * a.T * a.Hq * (a.D + 1);
  hipError_t e = hipSuccess;
  // one unit per sequence: blocks = ceil(L / 16)
  if (!inl) e = launch_plan(a.context_lens, a.B, 1, va.ranges, a.max_blocks, hdr, prefix, first, udesc, stream);
  if (e != hipSuccess) return e;
  const float sl2 = a.scale * kLog2e;
  const dim3 grid(va.ranges * (a.Hkv / wpg)), block(64 * wpg);
  const size_t lds = !inl ? tiles : M > 1 ? lds_share : lds_list;
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
