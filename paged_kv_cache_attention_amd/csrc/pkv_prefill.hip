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
// (G = Hq/Hkv).  A workgroup of kWaves waves owns one item; each wave holds
// TPW 16-row MFMA tiles (two in the shipped configuration: 128 rows per item).
// Keys advance STEP (32) at a time, staged once per workgroup through LDS
// (double-buffered: the next step's global loads are in flight while the
// tiles work on the current one), with the item's block-table entries cached
// in LDS 512 at a time:
//   K[token][d]  row-major, padded rows        -> A operand of S^T = K Q^T
//   V^T[d][token] transposed when staged        -> B operand of O += P V
// Per wave and step, for each row tile:
//   S^T[token][row] = K . Q^T   v_mfma_f32_16x16x32_bf16, two 16-token halves
//   online softmax per row (base 2, running max raised lazily)
//   O[row][d] += P . V          v_mfma_f32_16x16x32_bf16, k = the step's 32
//     keys; P split into bf16 hi + lo so the product keeps about 16 bits of P
// Keys at or past the group's last visible position are never used: their V
// columns are zeroed when staged and their scores masked.
//
// Items start longest first (item_of_rank).  With key pieces (piece_tokens
// > 0, for grids too small to fill the device) an item's keys are cut into
// pieces from position 0, one workgroup each; the pieces of an item with more
// than one leave normalised partials and log-sum-exps in a workspace, and
// prefill_merge_kernel combines them.
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kBS = 16;
constexpr int kTblWin = 512;   // block-table entries cached in LDS at a time
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kSlack = 8.f;

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8_v as_bf16x8(u32x4_t v) {
  bf16x8_v r;
  __builtin_memcpy(&r, &v, sizeof(r));
  return r;
}

// Two floats to packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  const bf16x2_v r = __builtin_convertvector((f32x2_v){a, b}, bf16x2_v);
  uint32_t u;
  __builtin_memcpy(&u, &r, 4);
  return u;
}

// TPW 16-row tiles per wave, STEP keys per staged step.
template <int D, int TPW, int STEP>
struct PGeo {
  static constexpr int ROWS = 16 * TPW * kWaves;     // query rows per item
  static constexpr int NQ = STEP / 16;               // 16-key quarters per step (S^T tiles)
  static constexpr int NK = STEP / 32;               // 32-key MFMA k-chunks per step (P.V)
  static constexpr int KROW = 2 * D + 16;            // K row bytes (conflict-free 16-byte reads)
  static constexpr int VROW = 2 * STEP + 8;          // V^T row bytes: one d, STEP keys
  static constexpr int KBYTES = STEP * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int LDS = 2 * (KBYTES + VBYTES);
  static constexpr int RC = D * 2 / 16;              // 16-byte chunks per token row
  static constexpr int PER_T = STEP * RC / kThreads;  // staged chunks per thread (K, and again V)
  static_assert(PER_T * kThreads == STEP * RC, "even staging split");
};

static_assert(PGeo<64, kPrefillTPW, kPrefillStep>::ROWS == kPrefillRows &&
                  PGeo<128, kPrefillTPW, kPrefillStep>::ROWS == kPrefillRows,
              "work item rows shared with the host-side sizing");

struct PrefillArgs {
  DecodeArgs a;
  int groups;        // row groups per (sequence, KV head)
  int pieces;        // key pieces per item in the grid (1: no split)
  int piece_steps;   // keys per piece / STEP (0: no split)
  float* part;       // split items' partials: [B][groups][Hkv][pieces] slots of ROWS x (D + 1) floats
};

// Start order of the work items.  The workgroup of rank p = blockIdx / Hkv
// takes the item (b, rg) with the p-th largest key count
//   work(b, rg) = L_b - T + min(T, (rg + 1) * tpg)    (tpg = chunk tokens per row group)
// (ties: smaller b first), so the longest items start first and never run
// alone at the end of the grid.  work is strictly increasing in rg, so the
// number of items of sequence b with work >= w has a closed form, and the
// item of rank p follows from a binary search on w: a bijection from ranks to
// items for any lengths.  Wave 0 computes it with the lengths in registers
// (kOrderMaxB sequences at most; larger batches keep the plain order).
constexpr int kOrderMaxB = 512;

__device__ __forceinline__ int count_work_ge(int Lc, int w, int T, int tpg, int groups) {
  const int x = w - Lc + T;   // rg counts iff min(T, (rg + 1) tpg) >= x
  if (x > T) return 0;
  if (x <= tpg) return groups;
  return groups + 1 - (x + tpg - 1) / tpg;
}

__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Wave 0 only: the item of rank p, written to item[0] (b) and item[1] (rg).
__device__ void item_of_rank(const int32_t* lens, int B, int T, int max_tokens, int tpg, int groups, int p,
                             int lane, int* item) {
  constexpr int KB = kOrderMaxB / 64;
  const int nk = (B + 63) / 64;
  int lc[KB];
  int lo = max_tokens, hi = 0;
#pragma unroll
  for (int k = 0; k < KB; ++k) {
    lc[k] = 0;
    if (k < nk) {
      const int bb = lane + 64 * k;
      if (bb < B) {
        lc[k] = clampi(lens[bb], 0, max_tokens);
        lo = min(lo, lc[k]);
        hi = max(hi, lc[k]);
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = min(lo, __shfl_xor(lo, o));
    hi = max(hi, __shfl_xor(hi, o));
  }
  auto total_ge = [&](int w) {
    int c = 0;
#pragma unroll
    for (int k = 0; k < KB; ++k)
      if (k < nk && lane + 64 * k < B) c += count_work_ge(lc[k], w, T, tpg, groups);
    return wave_sum_int(c);
  };
  // total_ge(lo) = B * groups > p >= total_ge(hi) = 0
  lo -= T;
  hi += 1;
  while (hi - lo > 1) {
    const int mid = lo + (hi - lo) / 2;
    if (total_ge(mid) > p) lo = mid;
    else hi = mid;
  }
  // the item has work lo; o = its rank among the items of that work, which
  // are one per sequence at most, taken in order of b
  int o = p - total_ge(hi);
#pragma unroll
  for (int k = 0; k < KB; ++k) {
    if (k >= nk) break;
    const int bb = lane + 64 * k;
    const int ge = bb < B ? count_work_ge(lc[k], lo, T, tpg, groups) : 0;
    const bool has = bb < B && ge > count_work_ge(lc[k], hi, T, tpg, groups);
    const uint64_t m = __builtin_amdgcn_ballot_w64(has);
    const int n = __builtin_popcountll(m);
    if (o < n) {
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
      if (has && below == o) {
        item[0] = bb;
        item[1] = groups - ge;
      }
      break;
    }
    o -= n;
  }
}

// Waves per SIMD the register budget is sized for (that many workgroups per
// CU, 20 or 39 KB of LDS each at 32-key steps): four with one tile per wave,
// or two tiles at D = 64; two otherwise.
template <int D, int TPW, int STEP>
constexpr int prefill_waves_per_eu() { return STEP == 32 && (TPW == 1 || D == 64) ? 4 : 2; }

template <int D, int TPW, int STEP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(prefill_waves_per_eu<D, TPW, STEP>())))
void prefill_kernel(PrefillArgs pa, float scale_log2e) {
  using PG = PGeo<D, TPW, STEP>;
  constexpr int KS = D / 32;                          // k-steps of QK^T
  constexpr int DT = D / 16;                          // output column tiles
  constexpr int NQ = PG::NQ, NK = PG::NK, RC = PG::RC, PER_T = PG::PER_T;
  __shared__ __attribute__((aligned(16))) unsigned char lds[PG::LDS];
  __shared__ int stbl[kTblWin];   // physical ids of blocks [win * kTblWin, (win + 1) * kTblWin)
  auto kst = [&](int buf) { return lds + buf * PG::KBYTES; };
  auto vst = [&](int buf) { return lds + 2 * PG::KBYTES + buf * PG::VBYTES; };

  const DecodeArgs& a = pa.a;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.Hq / a.Hkv;
  const int R = a.T * G;
  // items longest first (item_of_rank); the KV heads of one piece of an item
  // are consecutive workgroups, and the pieces of an item follow each other
  const int max_tokens = a.max_blocks * kBS;
  const int kv = (int)blockIdx.x % a.Hkv;
  const int piece = ((int)blockIdx.x / a.Hkv) % pa.pieces;
  const int p = (int)blockIdx.x / a.Hkv / pa.pieces;
  int b, rg;
  if (a.B == 1) {
    b = 0;
    rg = pa.groups - 1 - p;
  } else if (a.B > kOrderMaxB) {   // plain order: the last row group of every sequence first
    b = p % a.B;
    rg = pa.groups - 1 - p / a.B;
  } else {
    __shared__ int sitem[2];
    if (tid < 64)
      item_of_rank(a.context_lens, a.B, a.T, max_tokens, PG::ROWS / G, pa.groups, p, tid, sitem);
    __syncthreads();
    b = sitem[0];
    rg = sitem[1];
  }
  const int L = clampi(a.context_lens[b], 0, max_tokens);
  const int r0 = rg * PG::ROWS;
  const int t_last = (min(R, r0 + PG::ROWS) - 1) / G;
  const int kv_len = clampi(L - a.T + t_last + 1, 0, L);   // keys any row of the group sees
  const int nsteps = (kv_len + STEP - 1) / STEP;
  const int nblk = (kv_len + kBS - 1) / kBS;
  // This workgroup's steps [s0, s1): the whole item, or one piece of
  // piece_steps steps.  An item of npc > 1 pieces leaves normalised partials.
  int s0 = 0, s1 = nsteps, npc = 1;
  if (pa.piece_steps > 0) {
    npc = max(1, (nsteps + pa.piece_steps - 1) / pa.piece_steps);
    if (piece >= npc) return;   // the item is shorter than this piece: whole workgroup
    s0 = piece * pa.piece_steps;
    s1 = min(nsteps, s0 + pa.piece_steps);
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

  // ---- staging: chunk i = tid + k * kThreads.  K: key i / RC, columns
  // 8 (i % RC) .. +7 (a row's chunks on consecutive lanes: coalesced, and the
  // rows land as 16-byte LDS writes).  V: key i % STEP, columns 8 (i / STEP)
  // .. +7 (consecutive lanes on consecutive keys, so each 16-bit write of the
  // transpose covers one contiguous run of V^T: few bank conflicts). ----
  const size_t kv_row_bytes = (size_t)a.Hkv * D * 2;
  const size_t block_bytes = (size_t)kBS * kv_row_bytes;
  const int nmax = a.N_blocks - 1;
  const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks;
  const unsigned char* kpool = static_cast<const unsigned char*>(a.k_pool) + (size_t)kv * D * 2;
  const unsigned char* vpool = static_cast<const unsigned char*>(a.v_pool) + (size_t)kv * D * 2;
  // The table window holding step s: entries are loaded once per kTblWin
  // blocks instead of once per step, so the K/V loads of a step depend on no
  // global load of their own.
  auto load_window = [&](int win) {
    for (int e = tid; e < kTblWin; e += kThreads) {
      const int blk = min(win * kTblWin + e, nblk - 1);
      stbl[e] = clampi(trow[blk], 0, nmax);
    }
  };
  // Per thread and staged chunk k: the block of the step it reads (relative
  // to the step's first block) and its byte offset inside a physical block;
  // only the physical id changes from step to step.
  constexpr int NB = STEP / kBS;                      // blocks per step
  int kblk[PER_T], vblk[PER_T];
  uint32_t koff[PER_T], voff[PER_T];
#pragma unroll
  for (int k = 0; k < PER_T; ++k) {
    const int i = tid + k * kThreads;
    const int key = i / RC, vkey = i % STEP;
    kblk[k] = key / kBS;
    vblk[k] = vkey / kBS;
    koff[k] = (uint32_t)((key % kBS) * kv_row_bytes + (i % RC) * 16);
    voff[k] = (uint32_t)((vkey % kBS) * kv_row_bytes + (i / STEP) * 16);
  }
  u32x4_t kreg[PER_T], vreg[PER_T];
  auto issue = [&](int s) {
    const int b0 = s * NB;
#pragma unroll
    for (int k = 0; k < PER_T; ++k) {
      const uint32_t kph = (uint32_t)stbl[(uint32_t)min(b0 + kblk[k], nblk - 1) % kTblWin];
      const uint32_t vph = (uint32_t)stbl[(uint32_t)min(b0 + vblk[k], nblk - 1) % kTblWin];
      kreg[k] = load16(kpool + (uint64_t)kph * block_bytes + koff[k]);
      vreg[k] = load16(vpool + (uint64_t)vph * block_bytes + voff[k]);
    }
  };
  auto commit = [&](int s, int buf) {
    if ((s + 1) * STEP > kv_len) {   // the step holds keys past the group's last visible one:
#pragma unroll                      // they may hold anything, so zero their V
      for (int k = 0; k < PER_T; ++k)
        if (s * STEP + (tid + k * kThreads) % STEP >= kv_len) vreg[k] = u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < PER_T; ++k) {
      const int i = tid + k * kThreads;
      store16(kst(buf) + (i / RC) * PG::KROW + (i % RC) * 16, kreg[k]);
      const int vkey = i % STEP, vc = i / STEP;
      const u32x4_t v = vreg[k];
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
      uint16_t* vt = reinterpret_cast<uint16_t*>(vst(buf) + (8 * vc) * PG::VROW) + vkey;
#pragma unroll
      for (int e = 0; e < 8; ++e) vt[e * (PG::VROW / 2)] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
    }
  };

  // One step for this wave's tiles.  MASKED: some key of the step is at or
  // past the causal limit of one of the wave's rows.
  auto compute = [&](int s, int buf, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const unsigned char* ks = kst(buf);
    const unsigned char* vs = vst(buf);
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
        kc[h][c] = *reinterpret_cast<const u32x4_t*>(ks + (16 * h + row) * PG::KROW + quad * 16 + c * 64);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < KS; ++c)
#pragma unroll
      for (int h = 0; h < NQ; ++h)
#pragma unroll
        for (int j = 0; j < TPW; ++j)
          sacc[j][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kc[h][c]), as_bf16x8(qreg[j][c]), sacc[j][h],
                                                               0, 0, 0);
    // the step's V^T chunks, in flight during the softmax
    bf16x8_v vb[NK][DT];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int d = 0; d < DT; ++d) {
        const unsigned char* vr = vs + (16 * d + row) * PG::VROW + 64 * kk + quad * 8;
        const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vr);
        const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vr + 32);
        vb[kk][d] = as_bf16x8(u32x4_t{lo.x, lo.y, hi.x, hi.y});
      }
    __builtin_amdgcn_sched_barrier(0);
    // softmax.  Score i of the lane (i = 4 h + k) is key 16 h + 4 quad + k of
    // the step; k-slot 8 quad + e of P chunk kk holds score 8 kk + e.  The
    // running max m is kept in scaled base-2 units; since the scale is
    // positive, max(score) * scale is the max of the scaled scores, and each
    // p is exp2(score * scale - m) with one rounding (an fma).
    u32x4_t phi[TPW][NK], plo[TPW][NK];
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
      if (__builtin_amdgcn_ballot_w64(mx * scale_log2e > m_thr[j])) {
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
        uint32_t h4[4], l4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = pv[8 * kk + 2 * e], p1 = pv[8 * kk + 2 * e + 1];
          const uint32_t h = cvt_pk_bf16(p0, p1);
          h4[e] = h;
          l4[e] = cvt_pk_bf16(p0 - __uint_as_float(h << 16), p1 - __uint_as_float(h & 0xffff0000u));
        }
        phi[j][kk] = u32x4_t{h4[0], h4[1], h4[2], h4[3]};
        plo[j][kk] = u32x4_t{l4[0], l4[1], l4[2], l4[3]};
      }
    }
    // O += P V: B operand = V^T[d][keys 32 kk + 4 quad .. +3 and 32 kk + 16 + 4 quad .. +3]
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
#pragma unroll
      for (int d = 0; d < DT; ++d)
#pragma unroll
        for (int j = 0; j < TPW; ++j)
          acc[j][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(phi[j][kk]), vb[kk][d], acc[j][d], 0, 0, 0);
#pragma unroll
      for (int d = 0; d < DT; ++d)
#pragma unroll
        for (int j = 0; j < TPW; ++j)
          acc[j][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(plo[j][kk]), vb[kk][d], acc[j][d], 0, 0, 0);
    }
  };

  constexpr int kStepsPerWin = kTblWin * kBS / STEP;
  if (s1 > s0) {
    load_window(s0 / kStepsPerWin);
    __syncthreads();
    issue(s0);
    commit(s0, s0 & 1);
    __syncthreads();
    auto step = [&](int s, auto masked_tag) {
      const int buf = s & 1;
      if (s + 1 < s1 && (s + 1) % kStepsPerWin == 0) {   // step s + 1 opens a new table window
        __syncthreads();
        load_window((s + 1) / kStepsPerWin);
        __syncthreads();
      }
      if (s + 1 < s1) issue(s + 1);
      if (wave_active) compute(s, buf, masked_tag);
      if (s + 1 < s1) commit(s + 1, buf ^ 1);
      __syncthreads();
    };
    // Steps before s_mask hold only keys every row of the wave sees; the
    // rest are masked.  Two loops, one per kind, so each keeps its registers
    // in place (the barrier count per step is the same for every wave).
    const int s_mask = wave_active ? clampi(hi_min / STEP, s0, s1) : s1;
    int s = s0;
    for (; s < s_mask; ++s) step(s, std::false_type{});
    for (; s < s1; ++s) step(s, std::true_type{});
  }

  // ---- epilogue: O / l in bf16 (or, for a piece of a split item, in fp32
  // to the item's slot), lse in natural log ----
  if (!wave_active) return;
  uint16_t* out = static_cast<uint16_t*>(a.out);
  float* slot = npc > 1 ? pa.part + ((((size_t)b * pa.groups + rg) * a.Hkv + kv) * pa.pieces + piece) *
                                        (size_t)(PG::ROWS * (D + 1))
                        : nullptr;
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    float l = l_part[j] + __shfl_xor(l_part[j], 16);
    l += __shfl_xor(l, 32);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int rr = rw + 16 * j + 4 * quad + k;   // O row held in acc[j][*][k]
      const float lr = __shfl(l, 4 * quad + k);
      const float mr = __shfl(m_row[j], 4 * quad + k);
      if (rr < R) {
        const float inv = lr != 0.f ? 1.f / lr : 0.f;
        const float lse = lr != 0.f ? (mr + log2f(lr)) * kLn2 : kNegInf;
        if (slot) {   // partial of a piece: rows with no visible key here give (0, -inf)
          float* o = slot + (size_t)(rr - r0) * D;
#pragma unroll
          for (int d = 0; d < DT; ++d) o[16 * d + row] = acc[j][d][k] * inv;
          if (row == 0) slot[PG::ROWS * D + (rr - r0)] = lse;
        } else {
          const int t = rr / G, h = kv * G + (rr - (rr / G) * G);
          const size_t orow = ((size_t)b * a.T + t) * a.Hq + h;
#pragma unroll
          for (int d = 0; d < DT; ++d) out[orow * D + 16 * d + row] = f32_to_bf16_rne(acc[j][d][k] * inv);
          if (row == 0 && a.lse_out) a.lse_out[orow] = lse;
        }
      }
    }
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

template <int D, int TPW, int STEP>
hipError_t launch_pf(const PrefillArgs& pa0, int piece_tokens, hipStream_t stream) {
  using PG = PGeo<D, TPW, STEP>;
  PrefillArgs pa = pa0;
  const int G = pa.a.Hq / pa.a.Hkv;
  pa.groups = (pa.a.T * G + PG::ROWS - 1) / PG::ROWS;
  const long long items = (long long)pa.groups * pa.a.B * pa.a.Hkv;
  if (items <= 0) return hipSuccess;
  pa.pieces = prefill_pieces(pa.a.max_blocks, piece_tokens);
  pa.piece_steps = pa.pieces > 1 ? piece_tokens / STEP : 0;
  if (items * pa.pieces > 0x7fffffff || items * PG::ROWS > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_kernel<D, TPW, STEP>), dim3((unsigned)(items * pa.pieces)), dim3(kThreads), 0, stream,
                     pa, pa.a.scale * kLog2e);
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
template <int D>
hipError_t launch_pf_d(const PrefillArgs& pa, int piece_tokens, hipStream_t stream) {
  return launch_pf<D, kPrefillTPW, kPrefillStep>(pa, piece_tokens, stream);
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
  const long long groups = ((long long)T * (Hq / Hkv) + kPrefillRows - 1) / kPrefillRows;
  return (size_t)B * groups * Hkv * pieces * kPrefillRows * (D + 1) * sizeof(float);
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
