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
// Work item = (row group, sequence, KV head); rows are r = t * G + g
// (G = Hq/Hkv).  A workgroup of WAVES waves owns one item; each wave holds
// TPW 16-row MFMA tiles (two in the shipped configuration: 128 rows per item
// with 4 waves, 256 with the 8 waves of a key-piece launch at D = 128).
// Keys are staged in LDS once per workgroup, a stage of 64 keys at D = 128
// (32 at D = 64) per workgroup barrier, computed as 32-key steps
// (global_load_lds_dwordx4, double-buffered: the next stage's loads are in
// flight while the tiles work on the current one), with the item's
// block-table entries cached in LDS 512 at a time:
//   K[token][d]  row-major, chunks XOR-swizzled by row -> A operand of S^T = K Q^T
//   V[token][d]  row-major, chunks XOR-swizzled by row, read back transposed
//                (gfx950 ds_read_b64_tr_b16)          -> B operand of O += P V
// Per wave and step, for each row tile:
//   S^T[token][row] = K . Q^T   v_mfma_f32_16x16x32_bf16, two 16-token halves
//   online softmax per row (base 2, running max raised lazily)
//   O[row][d] += P . V          v_mfma_f32_16x16x32_bf16, k = the step's 32
//     keys; P rounded once to bf16 (the operand), fp32 accumulation.  bf16
//     keeps 8 significant bits: p~ = p (1 + e), |e| <= 2^-8, and with the
//     denominator l summed from the fp32 p an output element is off by at
//     most 2^-8 sum_j p_j |v_j| / l.  A second product with the rounding
//     residual of P (the decode tile's hi + lo split, good to about 2^-16)
//     measured 18 % of this kernel's time on the 8B chunked batch (231
//     against 190 us) and 17 % on one long prompt.
// Keys at or past the group's last visible position are never used: their V
// columns are zeroed when staged and their scores masked.
//
// Items start longest first (piece_of_rank).  With key pieces (piece_tokens
// > 0, for grids too small to fill the device) an item of n steps is cut into
// ceil(n / piece_steps) pieces of near-equal length, one workgroup each; the
// pieces of an item with more than one leave normalised partials and
// log-sum-exps in a workspace, and prefill_merge_kernel combines them.
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kBS = 16;
constexpr int kTblWin = 512;   // block-table entries cached in LDS at a time
constexpr float kSlack = 8.f;
// K/V steps staged in LDS at once: the loads of the next step are in flight
// while the tiles work on this one.  Three stages measured no faster than two
// on the Llama-3-8B-shaped chunked batch and on one long prompt (the staging
// loads cost their issue and LDS writes, not their latency).  The step loop
// runs two steps per iteration, so that each step's stage is a constant and
// its LDS offsets fold into the read instructions.
constexpr int kStages = 2;

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));
typedef short i16x4_v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_v as_bf16x8(u32x4_t v) {
  bf16x8_v r;
  __builtin_memcpy(&r, &v, sizeof(r));
  return r;
}

// 16 bytes from global memory straight to LDS (global_load_lds_dwordx4):
// lane l of the wave writes lds_run + 16 l, lds_run being wave-uniform.
__device__ __forceinline__ void load_lds16(const void* g, unsigned char* lds_run) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_run, 16, 0, 0);
}

// Two floats to packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  const bf16x2_v r = __builtin_convertvector((f32x2_v){a, b}, bf16x2_v);
  uint32_t u;
  __builtin_memcpy(&u, &r, 4);
  return u;
}

// V^T operands of four column tiles: two ds_read_b64_tr_b16 each, at ad[i]
// (keys 4 quad .. +3 of a 32-key chunk) and HI bytes further (16 keys on),
// issued together in one asm block that waits for them (lgkmcnt(0)) before
// it ends.  As builtins, these reads got an s_waitcnt vmcnt(0) from the
// compiler (it cannot tell the staged step from the one being loaded by
// global_load_lds), which waited for the next step's loads, just issued:
// every step then ran with its prefetch drained.
// ad[i] addresses the V staging area's start; OFF (the stage and the
// 32-key half within it, a multiple of 8 KB at D = 128) goes into the
// instructions' offset field, so the addresses stay the same from step to
// step.
typedef uint32_t u32x2_v __attribute__((ext_vector_type(2)));
template <int HI, int OFF>
__device__ __forceinline__ void vt_reads4(u32x2_v (&lo)[4], u32x2_v (&hi)[4], const uint32_t (&ad)[4]) {
  static_assert(HI == 4096, "16 staged rows of 2 D bytes, D = 128");
  static_assert(OFF % 8192 == 0 && OFF + HI < 65536, "offset field");
#define PKV_VT_READS4(OFF0, OFF1)                                                                                 \
  __asm__ volatile(                                                                                               \
      "ds_read_b64_tr_b16 %0, %8 offset:" OFF0 "\n\t"                                                          \
      "ds_read_b64_tr_b16 %4, %8 offset:" OFF1 "\n\t"                                                          \
      "ds_read_b64_tr_b16 %1, %9 offset:" OFF0 "\n\t"                                                          \
      "ds_read_b64_tr_b16 %5, %9 offset:" OFF1 "\n\t"                                                          \
      "ds_read_b64_tr_b16 %2, %10 offset:" OFF0 "\n\t"                                                         \
      "ds_read_b64_tr_b16 %6, %10 offset:" OFF1 "\n\t"                                                         \
      "ds_read_b64_tr_b16 %3, %11 offset:" OFF0 "\n\t"                                                         \
      "ds_read_b64_tr_b16 %7, %11 offset:" OFF1 "\n\t"                                                         \
      "s_waitcnt lgkmcnt(0)"                                                                                      \
      : "=&v"(lo[0]), "=&v"(lo[1]), "=&v"(lo[2]), "=&v"(lo[3]), "=&v"(hi[0]), "=&v"(hi[1]), "=&v"(hi[2]),       \
        "=&v"(hi[3])                                                                                              \
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])                                                            \
      : "memory")
  if constexpr (OFF == 0) PKV_VT_READS4("0", "4096");
  else if constexpr (OFF == 8192) PKV_VT_READS4("8192", "12288");
  else if constexpr (OFF == 16384) PKV_VT_READS4("16384", "20480");
  else PKV_VT_READS4("24576", "28672");
#undef PKV_VT_READS4
  static_assert(OFF <= 24576, "two stages of two halves");
}

// TPW 16-row tiles per wave, STEP keys per staged step, WAVES waves per
// workgroup (one item).
template <int D, int TPW, int STEP, int WAVES = 4>
struct PGeo {
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int ROWS = 16 * TPW * WAVES;      // query rows per item
  static constexpr int NQ = STEP / 16;               // 16-key quarters per step (S^T tiles)
  static constexpr int NK = STEP / 32;               // 32-key MFMA k-chunks per step (P.V)
  static constexpr int ROWB = 2 * D;                 // staged K or V row bytes (unpadded: loads land
                                                     // in LDS as whole 1 KB runs per wave)
  // 32-key steps per staged stage (one barrier and one load wait per
  // stage): two at D = 128 (chunked 8B batch 193.4 -> 183.8 us, one long
  // prompt 107.8 -> 102.8, interleaved A/B, identical bits); one at D = 64,
  // where the staging offsets of a second step spilled at the 128-VGPR
  // budget of four waves per SIMD.
  static constexpr int SUBS = D == 128 ? 2 : 1;
  static constexpr int SKEYS = SUBS * STEP;          // keys per staged stage
  static constexpr int KBYTES = SKEYS * ROWB;
  static constexpr int VBYTES = SKEYS * ROWB;
  static constexpr int OROW = 2 * D + 16;            // epilogue row bytes (the 4 rows a quad writes sit 16
                                                     // banks apart)
  static constexpr int LDS = kStages * (KBYTES + VBYTES) > ROWS * OROW ? kStages * (KBYTES + VBYTES) : ROWS * OROW;
  static constexpr int RC = D * 2 / 16;              // 16-byte chunks per token row
  static constexpr int PER_T = SKEYS * RC / THREADS;  // staged chunks per thread (K, and again V)
  static_assert(PER_T * THREADS == SKEYS * RC, "even staging split");
  // Chunk c of staged row r sits in slot c ^ swz(r) of the row (an XOR
  // swizzle instead of padding).  K: the 16 rows a 16-lane group reads at one
  // chunk fall on 16 distinct 4-bank slots.  V: the 4 rows x 2 chunks of one
  // transposing read of a 16-lane group fall on 8 distinct slots, and at
  // D = 128 (a row is exactly the 64 banks) the neighbouring group, 4 rows
  // further, on the other half of the banks: without that bit the chunked 8B
  // batch counted 9.0 M LDS bank-conflict cycles per call, with it 0.13 M
  // (190.2 -> 181.2 us, interleaved A/B, identical bits).  At D = 64 a row
  // is half the 64 banks, so its parity picks the half.
  static __device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  static __device__ __forceinline__ int swz_v(int r) {
    return D == 128 ? (2 * (r & 3)) | (8 * ((r >> 2) & 1)) : 2 * ((r >> 1) & 1);
  }
};

static_assert(PGeo<64, kPrefillTPW, kPrefillStep>::ROWS == kPrefillRows &&
                  PGeo<128, kPrefillTPW, kPrefillStep>::ROWS == kPrefillRows &&
                  PGeo<128, kPrefillTPW, kPrefillStep, 8>::ROWS == kPrefillRowsWide,
              "work item rows shared with the host-side sizing");

struct PrefillArgs {
  DecodeArgs a;
  int groups;        // row groups per (sequence, KV head)
  int pieces;        // key pieces per item in the grid (1: no split)
  int piece_steps;   // keys per piece / STEP (0: no split)
  float* part;       // split items' partials: [B][groups][Hkv][pieces] slots of ROWS x (D + 1) floats
};

// Start order of the work items.  Without key pieces the workgroup of rank
// p = blockIdx / Hkv takes the item (b, rg) with the p-th largest key count
//   work(b, rg) = L_b - T + min(T, (rg + 1) * tpg)    (tpg = chunk tokens per row group)
// (ties: smaller b first), so the longest items start first and never run
// alone at the end of the grid.  work is strictly increasing in rg, so the
// number of items of sequence b with work >= w has a closed form, and the
// item of rank p follows from a binary search on w: a bijection from ranks to
// items for any lengths.  Wave 0 computes it with the lengths in registers
// (kOrderMaxB sequences at most; larger batches keep the plain order).  Every
// workgroup pays for this search before its first load, so it avoids
// cross-lane shuffles (LDS round trips) and integer division.
constexpr int kOrderMaxB = 512;

// floor(n / d) for 0 <= n < 2^20 and 0 < d, from inv = 1 / d in fp32: the
// product is within 1/8 of n / d, so at most one step of correction either way.
__device__ __forceinline__ int div_floor_small(int n, int d, float inv) {
  int q = (int)((float)n * inv);
  q -= q * d > n ? 1 : 0;
  q += (q + 1) * d <= n ? 1 : 0;
  return q;
}

// Branch-free: the division runs on x clamped to [1, T] (n < 2^14) and its
// result is used only where tpg < x <= T.
__device__ __forceinline__ int count_work_ge(int Lc, int w, int T, int tpg, float inv_tpg, int groups) {
  const int x = w - Lc + T;   // rg counts iff min(T, (rg + 1) tpg) >= x
  const int mid = groups + 1 - div_floor_small(min(max(x, 1), T) + tpg - 1, tpg, inv_tpg);
  return x > T ? 0 : (x <= tpg ? groups : mid);
}

// Sum over the wave of values in [0, 2^bits): one ballot per bit.
__device__ __forceinline__ int wave_sum_bits(int x, int bits) {
  int s = 0;
  for (int k = 0; k < bits; ++k) s += __builtin_popcountll(__builtin_amdgcn_ballot_w64((x >> k) & 1)) << k;
  return s;
}

// Launch order with key pieces.  Workgroups are handed to the XCDs and, in
// each, to its shader engines in turn, and a full engine holds back the
// launch of every later workgroup; so a grid whose pieces alternate between
// heavy and empty would pile the heavy ones onto some engines.  The ranks
// therefore run: piece 0 of every split item (longest first), then piece 1 of
// them, piece 2 of those with three or more, and so on; then the unsplit
// items, longest first; then ranks with no piece.  The split items are the
// top-ranked ones (work > piece_keys), and the items with more than k pieces
// are the top count(work > k * piece_keys) ones, so each rank maps to an item
// rank and a piece with a few counts.
//
// Wave 0 only: for launch rank p, writes item[0] = b (or -1: no piece),
// item[1] = rg, item[2] = L_b clamped to [0, max_tokens], item[3] = piece.
// NK = 64-sequence chunks of the lengths held per lane (straight-line code
// for batches of up to 64 sequences).
template <int NK>
__device__ __forceinline__ void piece_of_rank(const int32_t* lens, int B, int T, int max_tokens, int tpg, int groups,
                                              int piece_keys, int pieces, int p, int lane, int* item) {
  const float inv_tpg = 1.f / (float)tpg;
  const bool one = B == 1;   // every lane then holds sequence 0, and counts need no sum
  int lc[NK];
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const int bb = one ? 0 : lane + 64 * k;
    lc[k] = bb < B ? clampi(lens[bb], 0, max_tokens) : 0;
  }
  // a lane's count is at most NK * groups
  const int bits = 32 - __builtin_clz((unsigned)(NK * groups));
  auto total_ge = [&](int w) {
    int c = 0;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int ck = count_work_ge(lc[k], w, T, tpg, inv_tpg, groups);
      c += one || lane + 64 * k < B ? ck : 0;
    }
    return one ? c : wave_sum_bits(c, bits);
  };
  // item rank r and piece of launch rank p
  int r = p, piece = 0;
  if (piece_keys > 0) {
    const int split = total_ge(piece_keys + 1);   // items of two or more pieces
    if (p >= split) {
      int q = p - split;
      piece = -1;
      for (int k = 1; k < pieces; ++k) {
        const int ck = k == 1 ? split : total_ge(k * piece_keys + 1);   // items of more than k pieces
        if (q < ck) {
          r = q;
          piece = k;
          break;
        }
        q -= ck;
        if (ck == 0) break;
      }
      if (piece < 0) {
        r = split + q;
        piece = 0;
        if (r >= B * groups) {   // past the last piece
          if (lane == 0) item[0] = -1;
          return;
        }
      }
    }
  }
  if (one) {   // work grows with rg
    if (lane == 0) {
      item[0] = 0;
      item[1] = groups - 1 - r;
      item[2] = lc[0];
      item[3] = piece;
    }
    return;
  }
  // the item of rank r: binary search on its work w,
  // total_ge(lo) = B * groups > r >= total_ge(hi) = 0
  int lo = -T, hi = max_tokens + 1;
  while (hi - lo > 1) {
    const int mid = lo + (hi - lo) / 2;
    if (total_ge(mid) > r) lo = mid;
    else hi = mid;
  }
  // the item has work lo; o = its rank among the items of that work, which
  // are one per sequence at most, taken in order of b
  int o = r - total_ge(hi);
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const int bb = lane + 64 * k;
    const int ge = count_work_ge(lc[k], lo, T, tpg, inv_tpg, groups);
    const bool has = bb < B && ge > count_work_ge(lc[k], hi, T, tpg, inv_tpg, groups);
    const uint64_t m = __builtin_amdgcn_ballot_w64(has);
    const int n = __builtin_popcountll(m);
    if (o < n) {
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
      if (has && below == o) {
        item[0] = bb;
        item[1] = groups - ge;
        item[2] = lc[k];
        item[3] = piece;
      }
      break;
    }
    o -= n;
  }
}

// Waves per SIMD the register budget is sized for (that many workgroups per
// CU, 20 KB of LDS each at D = 64, 66 KB at D = 128): four with one tile per wave,
// or two tiles at D = 64; two otherwise.
template <int D, int TPW, int STEP>
constexpr int prefill_waves_per_eu() { return STEP == 32 && (TPW == 1 || D == 64) ? 4 : 2; }

template <int D, int TPW, int STEP, int WAVES>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(prefill_waves_per_eu<D, TPW, STEP>())))
void prefill_kernel(PrefillArgs pa, float scale_log2e) {
  using PG = PGeo<D, TPW, STEP, WAVES>;
  constexpr int kThreads = PG::THREADS;
  constexpr int KS = D / 32;                          // k-steps of QK^T
  constexpr int DT = D / 16;                          // output column tiles
  constexpr int NQ = PG::NQ, NK = PG::NK, RC = PG::RC, PER_T = PG::PER_T;
  __shared__ __attribute__((aligned(16))) unsigned char lds[PG::LDS];
  __shared__ int stbl[kTblWin];   // physical ids of blocks [win0, win0 + kTblWin)
  auto kst = [&](int buf) { return lds + buf * PG::KBYTES; };
  auto vst = [&](int buf) { return lds + kStages * PG::KBYTES + buf * PG::VBYTES; };

  const DecodeArgs& a = pa.a;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.Hq / a.Hkv;
  const int R = a.T * G;
  // the KV heads of one piece of an item are consecutive workgroups; pieces
  // and items in the order of piece_of_rank
  const int max_tokens = a.max_blocks * kBS;
  const int kv = (int)blockIdx.x % a.Hkv;
  int b, rg, L, piece;
  if (a.B > kOrderMaxB) {   // plain order: the last row group of every sequence first, its pieces together
    const int q = (int)blockIdx.x / a.Hkv;
    const int p = q / pa.pieces;
    piece = q % pa.pieces;
    b = p % a.B;
    rg = pa.groups - 1 - p / a.B;
    L = clampi(a.context_lens[b], 0, max_tokens);
  } else {
    __shared__ int sitem[4];
    if (tid < 64) {
      if (a.B <= 64)
        piece_of_rank<1>(a.context_lens, a.B, a.T, max_tokens, PG::ROWS / G, pa.groups, pa.piece_steps * STEP,
                         pa.pieces, (int)blockIdx.x / a.Hkv, tid, sitem);
      else
        piece_of_rank<kOrderMaxB / 64>(a.context_lens, a.B, a.T, max_tokens, PG::ROWS / G, pa.groups,
                                       pa.piece_steps * STEP, pa.pieces, (int)blockIdx.x / a.Hkv, tid, sitem);
    }
    __syncthreads();
    b = sitem[0];
    if (b < 0) return;   // a rank past the last piece: whole workgroup
    rg = sitem[1];
    L = sitem[2];
    piece = sitem[3];
  }
  const int r0 = rg * PG::ROWS;
  const int t_last = (min(R, r0 + PG::ROWS) - 1) / G;
  const int kv_len = clampi(L - a.T + t_last + 1, 0, L);   // keys any row of the group sees
  const int nsteps = (kv_len + STEP - 1) / STEP;
  const int nblk = __builtin_amdgcn_readfirstlane((kv_len + kBS - 1) / kBS);
  // This workgroup's steps [s0, s1): the whole item, or piece `piece` of
  // npc = ceil(nsteps / piece_steps) near-equal pieces.  An item of npc > 1
  // pieces leaves normalised partials.
  int s0 = 0, s1 = nsteps, npc = 1;
  if (pa.piece_steps > 0) {
    npc = max(1, (nsteps + pa.piece_steps - 1) / pa.piece_steps);
    if (piece >= npc) return;   // the item is shorter than this piece: whole workgroup
    s0 = piece * nsteps / npc;
    s1 = (piece + 1) * nsteps / npc;
  }

  // ---- this wave's rows: tile j holds rows rw + 16 j + (lane % 16) ----
  const int row = lane & 15, quad = lane >> 4;
  const int rw = r0 + 16 * TPW * wave;
  const bool wave_active = rw < R;
  // keys below the wave's smallest causal limit need no mask
  const int hi_min = clampi(L - a.T + rw / G + 1, 0, L);
  const uint16_t* qbase = static_cast<const uint16_t*>(a.q);
  u32x4_t qreg[TPW][KS];
  int hi_row[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int r = rw + 16 * j + row;
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

  floatx4_t acc[TPW][DT];
  float m_row[TPW], m_thr[TPW], l_part[TPW];   // m_thr = m_row + kSlack: a larger score rescales
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
#pragma unroll
    for (int d = 0; d < DT; ++d) acc[j][d] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    m_row[j] = kNegInf;
    m_thr[j] = kNegInf;
    l_part[j] = 0.f;
  }

  // ---- staging: straight from global memory into LDS
  // (global_load_lds_dwordx4: lane l of a wave writes bytes 16 l .. 16 l + 15
  // of the instruction's 1 KB run).  Tile position i = tid + k * kThreads is
  // row i / RC, slot i % RC; the lane loads the chunk that belongs there
  // (chunk = slot ^ swizzle(row)): columns 8 chunk .. +7 of that key.  V is
  // read back transposed by the P.V products. ----
  const size_t kv_row_bytes = (size_t)a.Hkv * D * 2;
  const size_t block_bytes = (size_t)kBS * kv_row_bytes;
  const int nmax = a.N_blocks - 1;
  const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks;
  const unsigned char* kpool = static_cast<const unsigned char*>(a.k_pool) + (size_t)kv * D * 2;
  const unsigned char* vpool = static_cast<const unsigned char*>(a.v_pool) + (size_t)kv * D * 2;
  // The block-table window: kTblWin entries from block win0 on, loaded once
  // per kTblWin blocks instead of once per stage, so the K/V loads of a stage
  // depend on no global load of their own.  It slides to a stage's first
  // block when the stage's last one is past it.
  int win0 = 0;
  auto load_window = [&](int first) {
    win0 = first;
    for (int e = tid; e < kTblWin; e += kThreads) {
      const int blk = min(first + e, nblk - 1);
      stbl[e] = clampi(trow[blk], 0, nmax);
    }
  };
  // Per thread and staged chunk k: the block of the stage it reads (relative
  // to the stage's first block) and its byte offset inside a physical block;
  // only the physical id changes from stage to stage.  The 64 lanes of a wave
  // stage 64 / RC consecutive keys of one row-aligned run (4 keys at D = 128,
  // 8 at D = 64), never across a block boundary, so the block is the same
  // for the whole wave: its base address is formed in scalar registers and
  // the lanes add only their 32-bit offset.
  constexpr int NB = STEP / kBS;                      // blocks per step
  static_assert(kBS % (64 / RC) == 0 && (kThreads / RC) % kBS == 0, "a wave's staged keys stay in one block");
  int kblk[PER_T];
  uint32_t koff[PER_T], voff[PER_T];
#pragma unroll
  for (int k = 0; k < PER_T; ++k) {
    const int i = tid + k * kThreads;
    const int key = i / RC, slot = i % RC;
    kblk[k] = __builtin_amdgcn_readfirstlane(key / kBS);
    koff[k] = (uint32_t)((key % kBS) * kv_row_bytes + (slot ^ PG::swz_k(key)) * 16);
    voff[k] = (uint32_t)((key % kBS) * kv_row_bytes + (slot ^ PG::swz_v(key)) * 16);
  }
  auto issue = [&](int s, int buf) {
    const int b0 = s * NB;
#pragma unroll
    for (int k = 0; k < PER_T; ++k) {
      const int te = __builtin_amdgcn_readfirstlane(min(b0 + kblk[k], nblk - 1) - win0);
      const uint32_t ph = (uint32_t)__builtin_amdgcn_readfirstlane(stbl[te]);
      uint64_t kb = (uint64_t)(uintptr_t)kpool + (uint64_t)ph * block_bytes;
      uint64_t vb = (uint64_t)(uintptr_t)vpool + (uint64_t)ph * block_bytes;
      uint32_t ko = koff[k], vo = voff[k];
      // opaque to the optimiser, so that neither the pool base is folded into
      // the lanes' offsets nor the offsets widened out of the loop: the loads
      // then take the scalar-base + 32-bit-offset form
      __asm__ volatile("" : "+s"(kb), "+s"(vb), "+v"(ko), "+v"(vo));
      const int run = (k * kThreads + 64 * wave) * 16;   // this wave's 1 KB run of the tile
      load_lds16(reinterpret_cast<const unsigned char*>(kb) + ko, kst(buf) + run);
      load_lds16(reinterpret_cast<const unsigned char*>(vb) + vo, vst(buf) + run);
    }
  };
  // After this the stage starting at step s has its K and V in LDS as far as
  // this wave's loads go (the barrier that follows covers the other waves).
  auto land = [&](int s, int buf) {
    __builtin_amdgcn_s_waitcnt(0);
    if (s * STEP + PG::SKEYS > kv_len) {   // the stage holds keys past the group's last visible one:
#pragma unroll                            // they may hold anything, so zero their V (each lane its own chunk)
      for (int k = 0; k < PER_T; ++k) {
        const int i = tid + k * kThreads;
        if (s * STEP + i / RC >= kv_len) store16(vst(buf) + i * 16, u32x4_t{0u, 0u, 0u, 0u});
      }
    }
  };

  // One 32-key step for this wave's tiles: half HALF of the stage in buffer
  // BUF.  MASKED: some key of the step is at or past the causal limit of one
  // of the wave's rows.
  auto compute = [&](int s, auto buf_tag, auto half_tag, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr int BUF = decltype(buf_tag)::value, HALF = decltype(half_tag)::value;
    constexpr int R0 = HALF * STEP;   // the step's first row in the stage
    const unsigned char* ks = kst(BUF);
    // at D = 128 the V^T reads address the V area's start and add the stage
    // and half in their offset field
    const unsigned char* vs = D == 128 ? vst(0) : vst(BUF) + R0 * PG::ROWB;
    constexpr int kVtOff = BUF * PG::VBYTES + R0 * PG::ROWB;
    static_assert(D != 128 || PG::VBYTES == 16384, "V stage size in vt_reads4's offsets");
    floatx4_t sacc[TPW][NQ];
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
      for (int h = 0; h < NQ; ++h) sacc[j][h] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    // all of the step's K chunks first, so that the LDS latency is paid once
    // and the NQ * TPW accumulation chains interleave
    u32x4_t kc[NQ][KS];
#pragma unroll
    for (int h = 0; h < NQ; ++h)
#pragma unroll
      for (int c = 0; c < KS; ++c)
        kc[h][c] = *reinterpret_cast<const u32x4_t*>(ks + (R0 + 16 * h + row) * PG::ROWB +
                                                     ((quad + 4 * c) ^ PG::swz_k(R0 + 16 * h + row)) * 16);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < KS; ++c)
#pragma unroll
      for (int h = 0; h < NQ; ++h)
#pragma unroll
        for (int j = 0; j < TPW; ++j)
          sacc[j][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kc[h][c]), as_bf16x8(qreg[j][c]), sacc[j][h],
                                                               0, 0, 0);
    // the step's V^T chunks, read while the QK^T products run: keys
    // 32 kk + 4 quad .. +3, then 16 keys further, for column 16 d + row, two
    // transposing reads each (ds_read_b64_tr_b16: lane i of each 16-lane group
    // receives element i % 4 of the 8-byte chunk that lane 4 k + i / 4 of the
    // group addresses, k = 0..3).  At D = 128 four column tiles go per asm
    // block (vt_reads4); at D = 64 the asm blocks spilled at the 128-VGPR
    // budget of four waves per SIMD, so the reads stay builtins there.
    bf16x8_v vb[NK][DT];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const int vrow = 32 * kk + 4 * quad + (row >> 2);   // row in the step; R0 + vrow in the stage
      auto vaddr = [&](int d) {
        return vs + vrow * PG::ROWB + (((2 * d + ((row & 3) >> 1)) ^ PG::swz_v(R0 + vrow)) * 16) + 8 * (row & 1);
      };
      if constexpr (D == 128) {
#pragma unroll
        for (int d0 = 0; d0 < DT; d0 += 4) {
          uint32_t ad[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            ad[i] = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)(
                const_cast<unsigned char*>(vaddr(d0 + i)));
          u32x2_v lo[4], hi[4];
          vt_reads4<16 * PG::ROWB, kVtOff>(lo, hi, ad);
#pragma unroll
          for (int i = 0; i < 4; ++i) vb[kk][d0 + i] = as_bf16x8(u32x4_t{lo[i].x, lo[i].y, hi[i].x, hi[i].y});
        }
      } else {
#pragma unroll
        for (int d = 0; d < DT; ++d) {
          const unsigned char* vr = vaddr(d);
          const i16x4_v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_v*)(const_cast<unsigned char*>(vr)));
          const i16x4_v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_v*)(const_cast<unsigned char*>(vr + 16 * PG::ROWB)));
          u32x4_t w;
          __builtin_memcpy(&w, &lo, 8);
          __builtin_memcpy(reinterpret_cast<unsigned char*>(&w) + 8, &hi, 8);
          vb[kk][d] = as_bf16x8(w);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // softmax.  Score i of the lane (i = 4 h + k) is key 16 h + 4 quad + k of
    // the step; k-slot 8 quad + e of P chunk kk holds score 8 kk + e.  The
    // running max m is kept in scaled base-2 units; since the scale is
    // positive, max(score) * scale is the max of the scaled scores, and each
    // p is exp2(score * scale - m) with one rounding (an fma).
    u32x4_t pb[TPW][NK];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      float sv[4 * NQ];   // raw scores, masked ones -inf
#pragma unroll
      for (int i = 0; i < 4 * NQ; ++i) {
        if constexpr (MASKED) {
          const int key = s * STEP + 16 * (i >> 2) + 4 * quad + (i & 3);
          sv[i] = key < hi_row[j] ? sacc[j][i >> 2][i & 3] : kNegInf;
        } else {
          sv[i] = sacc[j][i >> 2][i & 3];
        }
      }
      float mx = sv[0];
#pragma unroll
      for (int i = 1; i < 4 * NQ; ++i) mx = fmaxf(mx, sv[i]);
      // rare (the running max rises by more than the slack): marked
      // unlikely, the rescale is laid out after the loop (chunked 8B batch
      // 187.2 -> 181.5 us, interleaved A/B, identical bits)
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(mx * scale_log2e > m_thr[j]) != 0, 0)) {
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_row[j], mx * scale_log2e);
        // 1 while a row is still empty (both -inf), 0 on its first key
        const float alpha = m_row[j] == m_new ? 1.f : __builtin_amdgcn_exp2f(m_row[j] - m_new);
        l_part[j] *= alpha;
        m_row[j] = m_new;
        m_thr[j] = m_new + kSlack;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float ak = __shfl(alpha, 4 * quad + k);
#pragma unroll
          for (int d = 0; d < DT; ++d) acc[j][d][k] *= ak;
        }
      }
      const float neg_m = -m_row[j];
      float pv[4 * NQ];
#pragma unroll
      for (int i = 0; i < 4 * NQ; ++i) {
        // masked keys (and rows that have seen none) give p = 0; in unmasked
        // steps every row has seen a key, so m is finite
        pv[i] = MASKED && sv[i] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i], scale_log2e, neg_m));
        l_part[j] += pv[i];
      }
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        uint32_t h4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h4[e] = cvt_pk_bf16(pv[8 * kk + 2 * e], pv[8 * kk + 2 * e + 1]);
        pb[j][kk] = u32x4_t{h4[0], h4[1], h4[2], h4[3]};
      }
    }
    // O += P V: B operand = V^T[d][keys 32 kk + 4 quad .. +3 and 32 kk + 16 + 4 quad .. +3]
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int d = 0; d < DT; ++d)
#pragma unroll
        for (int j = 0; j < TPW; ++j)
          acc[j][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(pb[j][kk]), vb[kk][d], acc[j][d], 0, 0, 0);
  };

  if (s1 > s0) {
    static_assert(kStages == 2, "two stages");
    constexpr int SUBS = PG::SUBS;
    using Buf0 = std::integral_constant<int, 0>;
    using Buf1 = std::integral_constant<int, 1>;
    using Half0 = std::integral_constant<int, 0>;
    using Half1 = std::integral_constant<int, 1>;
    // Stages of SUBS steps from s0 on, alternating the two buffers.  A
    // stage's loads start one stage before it is computed; if its last block
    // is past the table window, the window slides to its first block first
    // (every load of earlier stages has its address by then).
    auto start = [&](int sa, int buf) {
      if ((sa + SUBS) * NB - 1 >= win0 + kTblWin) {
        __syncthreads();
        load_window(sa * NB);
        __syncthreads();
      }
      issue(sa, buf);
    };
    load_window(s0 * NB);
    __syncthreads();
    start(s0, 0);
    land(s0, 0);
    __syncthreads();
    // One stage: step s and (SUBS = 2, when `two`) step s + 1.
    auto stage = [&](int s, auto buf_tag, auto masked_tag, bool two) {
      constexpr int BUF = decltype(buf_tag)::value;
      if (s + SUBS < s1) start(s + SUBS, 1 - BUF);
      if (wave_active) {
        compute(s, buf_tag, Half0{}, masked_tag);
        if constexpr (SUBS == 2)
          if (two) compute(s + 1, buf_tag, Half1{}, masked_tag);
      }
      if (s + SUBS < s1) land(s + SUBS, 1 - BUF);
      __syncthreads();
    };
    // Steps before s_mask hold only keys every row of the wave sees; the
    // rest are masked.  One loop per kind, so each keeps its registers in
    // place (the barrier count per stage is the same for every wave); each
    // runs two stages per iteration, buffer 0 then buffer 1, and each step
    // variant is written once (so that it is inlined).  Unmasked steps left
    // over from whole iterations run in the masked loop, whose code also
    // serves steps that every row sees.
    const int s_mask = wave_active ? clampi(hi_min / STEP, s0, s1) : s1;
    const int s_whole = s0 + ((s_mask - s0) / (2 * SUBS)) * (2 * SUBS);
    int s = s0;
    for (; s < s_whole; s += 2 * SUBS) {
      stage(s, Buf0{}, std::false_type{}, true);
      stage(s + SUBS, Buf1{}, std::false_type{}, true);
    }
    for (; s < s1; s += 2 * SUBS) {
      stage(s, Buf0{}, std::true_type{}, s + 1 < s1);
      if (s + SUBS < s1) stage(s + SUBS, Buf1{}, std::true_type{}, s + SUBS + 1 < s1);
    }
  }

  // ---- epilogue: O / l in bf16 (or, for a piece of a split item, in fp32
  // to the item's slot), lse in natural log.  bf16 rows are staged in LDS
  // (free after the loop's last barrier) and leave as 16-byte row chunks:
  // the rows of one query token are consecutive heads, so the stores cover
  // contiguous runs of G * D * 2 bytes. ----
  constexpr int OROW = PG::OROW;
  static_assert(PG::ROWS * OROW <= PG::LDS, "output tile fits the staging buffers");
  float* slot = npc > 1 ? pa.part + ((((size_t)b * pa.groups + rg) * a.Hkv + kv) * pa.pieces + piece) *
                                        (size_t)(PG::ROWS * (D + 1))
                        : nullptr;
  if (wave_active) {
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      float l = l_part[j] + __shfl_xor(l_part[j], 16);
      l += __shfl_xor(l, 32);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int rr = rw + 16 * j + 4 * quad + k;   // O row held in acc[j][*][k]
        const float lr = __shfl(l, 4 * quad + k);
        const float mr = __shfl(m_row[j], 4 * quad + k);
        const float inv = lr != 0.f ? 1.f / lr : 0.f;
        const float lse = lr != 0.f ? (mr + log2f(lr)) * kLn2 : kNegInf;
        if (slot) {   // partial of a piece: rows with no visible key here give (0, -inf)
          if (rr < R) {
            float* o = slot + (size_t)(rr - r0) * D;
#pragma unroll
            for (int d = 0; d < DT; ++d) o[16 * d + row] = acc[j][d][k] * inv;
            if (row == 0) slot[PG::ROWS * D + (rr - r0)] = lse;
          }
        } else {   // rows at or past R are staged but never copied out
          uint16_t* o = reinterpret_cast<uint16_t*>(lds + (rr - r0) * OROW);
#pragma unroll
          for (int d = 0; d < DT; ++d) o[16 * d + row] = f32_to_bf16_rne(acc[j][d][k] * inv);
          if (rr < R && row == 0 && a.lse_out) {
            const int t = rr / G;
            a.lse_out[((size_t)b * a.T + t) * a.Hq + kv * G + (rr - t * G)] = lse;
          }
        }
      }
    }
  }
  if (slot) return;
  __syncthreads();
  constexpr int CPR = D / 8;   // 16-byte chunks per row
  unsigned char* out = static_cast<unsigned char*>(a.out);
  const int nrows = min(R, r0 + PG::ROWS) - r0;
  for (int i = tid; i < nrows * CPR; i += kThreads) {
    const int rl = i / CPR, c = i % CPR;
    const int r = r0 + rl, t = r / G;
    const size_t orow = ((size_t)b * a.T + t) * a.Hq + kv * G + (r - t * G);
    store16(out + orow * (D * 2) + c * 16, *reinterpret_cast<const u32x4_t*>(lds + rl * OROW + c * 16));
  }
}

// Merges the pieces of each split item.  Pieces cover disjoint key ranges of
// the same rows and carry normalised partials with their log-sum-exp, so
//   M = max_p lse_p,  w_p = exp(lse_p - M),
//   out = sum_p w_p o_p / sum_p w_p,  lse = M + ln sum_p w_p
// ("Inference From Scratch", ch. 8: softmax over pieces combined through the
// running max and sum).  A piece where a row sees no key has lse = -inf,
// weight 0 and o = 0.  One workgroup per kMergeRows rows of an item, D / 4
// threads per row with 4 columns each; the loads of every piece are
// independent and the sum runs in piece order.
constexpr int kMergeThreads = 256;

template <int D, int ROWS, int STEP>
__global__ __launch_bounds__(kMergeThreads) void prefill_merge_kernel(PrefillArgs pa) {
  constexpr int TPR = D / 4, RPW = kMergeThreads / TPR, CHUNKS = ROWS / RPW;
  static_assert(CHUNKS * RPW == ROWS, "whole chunks of rows");
  const DecodeArgs& a = pa.a;
  const int item = (int)blockIdx.x / CHUNKS, chunk = (int)blockIdx.x % CHUNKS;
  const int kv = item % a.Hkv, rest = item / a.Hkv;
  const int rg = rest % pa.groups, b = rest / pa.groups;
  const int G = a.Hq / a.Hkv, R = a.T * G;
  const int L = clampi(a.context_lens[b], 0, a.max_blocks * kBS);
  const int r0 = rg * ROWS;
  const int t_last = (min(R, r0 + ROWS) - 1) / G;
  const int kv_len = clampi(L - a.T + t_last + 1, 0, L);   // as the tile computes it
  const int npc = max(1, ((kv_len + STEP - 1) / STEP + pa.piece_steps - 1) / pa.piece_steps);
  if (npc <= 1) return;   // written directly by the tile
  const int i = chunk * RPW + (int)threadIdx.x / TPR;   // row within the item
  if (r0 + i >= R) return;
  constexpr size_t SLOT = (size_t)ROWS * (D + 1);
  const float* base = pa.part + (((size_t)b * pa.groups + rg) * a.Hkv + kv) * pa.pieces * SLOT;
  const float* lp = base + (size_t)ROWS * D + i;
  const float* opp = base + (size_t)i * D + ((int)threadIdx.x % TPR) * 4;
  float M = kNegInf;
  for (int q = 0; q < npc; ++q) M = fmaxf(M, lp[q * SLOT]);
  float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f, wsum = 0.f;
  if (M != kNegInf) {
#pragma unroll 4
    for (int q = 0; q < npc; ++q) {
      const float lq = lp[q * SLOT];
      const float4 v = *reinterpret_cast<const float4*>(opp + q * SLOT);
      const float w = lq == kNegInf ? 0.f : __builtin_amdgcn_exp2f((lq - M) * kLog2e);
      wsum += w;
      o0 = fmaf(w, v.x, o0);
      o1 = fmaf(w, v.y, o1);
      o2 = fmaf(w, v.z, o2);
      o3 = fmaf(w, v.w, o3);
    }
  }
  const float inv = wsum != 0.f ? 1.f / wsum : 0.f;
  const int rr = r0 + i, t = rr / G, h = kv * G + (rr - t * G);
  const size_t orow = ((size_t)b * a.T + t) * a.Hq + h;
  const int c = ((int)threadIdx.x % TPR) * 4;
  uint16_t* op = static_cast<uint16_t*>(a.out) + orow * D + c;
  op[0] = f32_to_bf16_rne(o0 * inv);
  op[1] = f32_to_bf16_rne(o1 * inv);
  op[2] = f32_to_bf16_rne(o2 * inv);
  op[3] = f32_to_bf16_rne(o3 * inv);
  if (c == 0 && a.lse_out) a.lse_out[orow] = wsum != 0.f ? M + logf(wsum) : kNegInf;
}

template <int D, int TPW, int STEP, int WAVES>
hipError_t launch_pf(const PrefillArgs& pa0, int piece_tokens, hipStream_t stream) {
  using PG = PGeo<D, TPW, STEP, WAVES>;
  PrefillArgs pa = pa0;
  const int G = pa.a.Hq / pa.a.Hkv;
  pa.groups = (pa.a.T * G + PG::ROWS - 1) / PG::ROWS;
  const long long items = (long long)pa.groups * pa.a.B * pa.a.Hkv;
  if (items <= 0) return hipSuccess;
  pa.pieces = prefill_pieces(pa.a.max_blocks, piece_tokens);
  pa.piece_steps = pa.pieces > 1 ? piece_tokens / STEP : 0;
  if (items * pa.pieces > 0x7fffffff || items * PG::ROWS > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_kernel<D, TPW, STEP, WAVES>), dim3((unsigned)(items * pa.pieces)), dim3(PG::THREADS), 0,
                     stream, pa, pa.a.scale * kLog2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pa.pieces <= 1) return e;
  constexpr int kChunks = PG::ROWS / (kMergeThreads / (D / 4));
  hipLaunchKernelGGL((prefill_merge_kernel<D, PG::ROWS, STEP>), dim3((unsigned)(items * kChunks)),
                     dim3(kMergeThreads), 0, stream, pa);
  return hipGetLastError();
}

// Two 16-row tiles per wave and 32-key steps: measured fastest on the
// chunked-prefill batch of the Llama-3-8B shape.  The tiles share each K and
// V read from LDS, which outweighs the occupancy given up at D = 128 (two
// workgroups per CU instead of four with one tile: 312 against 346 us);
// 64-key steps and 8-wave workgroups of one tile per wave were slower.
// Items of 4 waves (128 rows) normally; with key pieces at D = 128, items of
// 8 waves (256 rows), which stage each key once for twice the rows: one long
// prompt chunk 100.2 -> 95.6 us per call (interleaved A/B), where the pieces
// already give every CU work, while the unsplit 8-sequence chunked batch
// schedules its coarser items worse (187.7 -> 194.5 us).  At D = 64 a
// second step per stage, which 8-wave staging needs, spills.
template <int D>
hipError_t launch_pf_d(const PrefillArgs& pa, int piece_tokens, hipStream_t stream) {
  if constexpr (D == 128)
    if (prefill_pieces(pa.a.max_blocks, piece_tokens) > 1)
      return launch_pf<D, kPrefillTPW, kPrefillStep, 8>(pa, piece_tokens, stream);
  return launch_pf<D, kPrefillTPW, kPrefillStep, 4>(pa, piece_tokens, stream);
}

}  // namespace

int prefill_pieces(int max_blocks, int piece_tokens) {
  if (piece_tokens <= 0) return 1;
  const long long keys = (long long)max_blocks * kBS;
  return (int)max(1LL, (keys + piece_tokens - 1) / piece_tokens);
}

size_t prefill_workspace_bytes(int B, int T, int Hq, int Hkv, int D, int max_blocks, int piece_tokens) {
  const int pieces = prefill_pieces(max_blocks, piece_tokens);
  if (pieces <= 1 || B <= 0 || T <= 0 || Hkv <= 0) return 0;
  const int rows = D == 128 ? kPrefillRowsWide : kPrefillRows;   // items of the split launch (launch_pf_d)
  const long long groups = ((long long)T * (Hq / Hkv) + rows - 1) / rows;
  return (size_t)B * groups * Hkv * pieces * rows * (D + 1) * sizeof(float);
}

int prefill_piece_tokens(int B, int T, int Hq, int Hkv, int D, int max_blocks, int cus) {
  if (B <= 0 || T <= 0 || Hkv <= 0 || Hq % Hkv) return 0;
  const long long groups = ((long long)T * (Hq / Hkv) + kPrefillRows - 1) / kPrefillRows;
  const long long items = (long long)B * groups * Hkv;
  // one workgroup per slot (prefill_waves_per_eu workgroups per CU): fewer
  // items leave CUs idle.  More pieces than that only add partials to write
  // and merge (measured on one sequence with an 8192-token prefix: 4 pieces
  // 170-180 us, 2 about 208, 8 about 225, none 330).
  const long long want = (long long)cus * (D == 64 ? prefill_waves_per_eu<64, kPrefillTPW, kPrefillStep>()
                                                   : prefill_waves_per_eu<128, kPrefillTPW, kPrefillStep>());
  if (items >= want) return 0;
  const long long keys = (long long)max_blocks * kBS;
  const long long pieces = (want + items - 1) / items;
  long long tokens = (keys + pieces - 1) / pieces;
  tokens = (tokens + kPrefillStep - 1) / kPrefillStep * kPrefillStep;
  tokens = max(tokens, (long long)kPrefillMinPiece);
  return tokens >= keys ? 0 : (int)tokens;
}

hipError_t launch_prefill(const DecodeArgs& a, int piece_tokens, float* workspace, hipStream_t stream) {
  PrefillArgs pa{};
  pa.a = a;
  pa.part = workspace;
  return a.D == 64 ? launch_pf_d<64>(pa, piece_tokens, stream) : launch_pf_d<128>(pa, piece_tokens, stream);
}

}  // namespace pkv
