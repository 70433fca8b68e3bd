// Shared-prefix groups for single-token decode: device code (gfx950).
//
// When several sequences of a batch point their block tables at the same
// physical blocks (a common prompt prefix: "vLLM and PagedAttention",
// memory sharing), the per-sequence path reads those blocks once per
// sequence.  Here the shared blocks are attended once per group instead: all
// members' query rows of one KV head (members x G rows, up to 64) run as MFMA
// tiles against the group's blocks, and each member's result over its own
// remaining blocks is merged with the group partials by log-sum-exp weights
// (softmax over a union of key sets combines through the pieces' max and
// sum, "Inference From Scratch", ch. 8).
//
// Detection (one wave per aligned window of kGroupWindow sequences, run by
// the planning kernel):
//   key(b)     = first physical block of b (sequences with no tokens never group)
//   groups     = runs of equal keys inside the window, cut every M_max members
//   canonical  = the member with the most blocks (lowest index on ties)
//   s(b)       = common prefix length of b's and the canonical's tables,
//                limited to both block counts
//   d          = max s(b) over the non-canonical members; the canonical's
//                share is d (its table is the one the group walks)
// A group with fewer than kGroupMinShare common blocks is dissolved.  Member b
// then sees the group's blocks [0, d) up to position min(L_b, 16 s(b)); its
// own path covers blocks [s(b), n_b).  Only adjacent sequences are grouped;
// sharing between sequences far apart in the batch is left to the
// per-sequence path (still correct, only not deduplicated).
//
// Group items (group chunk x KV head) run on extra workgroups of the decode
// launch, beside the decode workgroups on every CU.
#pragma once

#include "pkv_device.h"
#include "pkv_internal.h"
#include "pkv_tile.h"

namespace pkv {
namespace grp {

constexpr int kBS = 16;
constexpr int kTiles = 4;                   // 16-row tiles (waves) per group item: 64 rows
constexpr int kThreads = 64 * kTiles;

// Sub-chunks staged through LDS (double-buffered): 52 KB for D = 128 and
// 36 KB for D = 64.
template <int D> struct Stage {
  static constexpr int SUB = D == 128 ? 3 : 4;   // blocks per sub-chunk
  static constexpr int ROWS = SUB * kBS;
  static constexpr int ROW = 2 * D + 16;          // padded row bytes
  static constexpr int BYTES = 2 * 2 * ROWS * ROW;
};

// Detection of the groups of the window starting at sequence w0 by one wave.
// Writes sfx / nch / cnt for the window's sequences to LDS (indexed by
// sequence) and to the plan, and the descriptor of each group leader.
__device__ __forceinline__ void detect_window(int w0, const int32_t* __restrict__ tables,
                                              const int32_t* __restrict__ lens, int B, int max_blocks, int GM,
                                              const GroupPlan& gp, int* ssfx, int* snch, int* scnt) {
  const int lane = threadIdx.x & 63;
  const int m = lane >> 2, sub = lane & 3;      // 4 lanes per member
  const int j = w0 + m;
  const bool valid = j < B;
  const int max_tokens = max_blocks * kBS;
  const int L = valid ? clampi(lens[j], 0, max_tokens) : 0;
  const int n = (L + kBS - 1) / kBS;
  const int32_t* trow = tables + (size_t)(valid ? j : 0) * max_blocks;
  const int key = n > 0 ? trow[0] : -1 - m;     // members without tokens stay alone
  const int prev = __shfl(key, lane - 4);
  const bool start = m == 0 || key != prev || (m % GM) == 0;
  const unsigned long long smask = __builtin_amdgcn_ballot_w64(start && sub == 0);
  // group of m: [gs, ge) in member units
  const unsigned long long below = smask & ((2ull << (4 * m)) - 1);
  const int gs = (63 - __builtin_clzll(below)) >> 2;
  const unsigned long long above = smask & ~((2ull << (4 * m)) - 1);
  const int ge_raw = above ? (__builtin_ctzll(above) >> 2) : kGroupWindow;
  const int ge = min(ge_raw, B - w0);
  const int M = ge - gs;
  // canonical: most blocks, lowest index on ties
  int cm = gs, cn = -1;
  for (int mm = 0; mm < kGroupWindow; ++mm) {
    const int nn = __shfl(n, 4 * mm);
    if (mm >= gs && mm < ge && nn > cn) { cn = nn; cm = mm; }
  }
  const int32_t* crow = tables + (size_t)(w0 + cm) * max_blocks;
  const int lim = min(n, cn);
  // common prefix with the canonical: 64 entries per member and pass
  int s = lim;
  bool done = !valid || M < 2 || m == cm || lim == 0;
  for (int i0 = 0;; i0 += 64) {
    const bool active = !done && i0 < lim;
    if (!__builtin_amdgcn_ballot_w64(active)) break;
    int fm = 0x7fffffff;
    if (active) {
      int tv[16], cv[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {   // all loads first, then the compare chain
        const int i = min(i0 + sub * 16 + e, lim - 1);
        tv[e] = trow[i];
        cv[e] = crow[i];
      }
#pragma unroll
      for (int e = 15; e >= 0; --e)
        if (i0 + sub * 16 + e < lim && tv[e] != cv[e]) fm = i0 + sub * 16 + e;
    }
    fm = min(fm, __shfl_xor(fm, 1));
    fm = min(fm, __shfl_xor(fm, 2));
    if (active) {
      if (fm != 0x7fffffff) { s = fm; done = true; }
      else if (i0 + 64 >= lim) done = true;
    }
  }
  // shared blocks of the group: max over non-canonical members
  int d = 0;
  for (int mm = 0; mm < kGroupWindow; ++mm) {
    const int sm = __shfl(s, 4 * mm);
    if (mm >= gs && mm < ge && mm != cm) d = max(d, sm);
  }
  const bool grouped = valid && M >= 2 && d >= kGroupMinShare;
  const int sfx = grouped ? (m == cm ? d : s) : 0;
  int vlim = 0;                                 // last V row any member reads
  for (int mm = 0; mm < kGroupWindow; ++mm) {
    const int v = __shfl(min(L, kBS * sfx), 4 * mm);
    if (mm >= gs && mm < ge) vlim = max(vlim, v);
  }
  const int nch = grouped ? (d + group_chunk_blocks(d) - 1) / group_chunk_blocks(d) : 0;
  if (valid && sub == 0) {
    const int c = m == gs ? nch : 0;
    ssfx[j] = sfx;
    snch[j] = nch;
    scnt[j] = c;
    gp.sfx[j] = sfx;
    gp.nch[j] = nch;
    if (m == gs) gp.desc[j] = make_int4(w0 + cm, M, d, vlim);
  }
}

// Group items on one workgroup of kTiles waves: item = (group chunk, KV
// head); wave w owns rows 16w .. 16w+15 of the group's member-major rows
// r = member * G + head.  The chunk's K and V rows of the KV head are staged
// through LDS in sub-chunks (double-buffered: the next sub-chunk's loads are
// in flight while the tiles work on the current one), so each shared block is
// read once per item and reused by every member tile.  lds: Stage<D>::BYTES.
template <int D>
__device__ __forceinline__ void group_items(const DecodeArgs& a, const GroupPlan& gp, int items, int first, int step,
                                            unsigned char* lds, float scale_log2e) {
  constexpr int DT = D / 16;
  constexpr int kSub = Stage<D>::SUB, kSubRows = Stage<D>::ROWS, ROW = Stage<D>::ROW;
  constexpr int RC = D * 2 / 16;                     // 16-byte chunks per token row
  constexpr int PER_T = kSubRows * RC / kThreads;    // chunks per thread and sub-chunk (K, and again V)
  static_assert(PER_T * kThreads == kSubRows * RC, "even staging split");
  unsigned char* kst[2] = {lds, lds + kSubRows * ROW};
  unsigned char* vst[2] = {lds + 2 * kSubRows * ROW, lds + 3 * kSubRows * ROW};
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.Hq / a.Hkv;
  const int row = lane & 15, quad = lane >> 4;
  const size_t kv_row_bytes = (size_t)a.Hkv * D * 2;
  const size_t block_bytes = (size_t)kBS * kv_row_bytes;
  const int nmax = a.N_blocks - 1;
  const int max_tokens = a.max_blocks * kBS;
  const int scol = tid % RC;   // staging: chunk i = tid + k * kThreads -> token row i / RC, column i % RC

  for (int item = first; item < items; item += step) {
    const int jc = item / a.Hkv, kv = item - jc * a.Hkv;
    const int e = gp.clist[jc];
    const int bl = e / kGroupChunks, ch = e - bl * kGroupChunks;
    const int4 desc = gp.desc[bl];
    const int rows = desc.y * G;
    const int gc = group_chunk_blocks(desc.z);
    const int kb0 = ch * gc, nb = min(desc.z, kb0 + gc) - kb0;
    const int32_t* trow = a.block_tables + (size_t)desc.x * a.max_blocks + kb0;
    const unsigned char* kbase = static_cast<const unsigned char*>(a.k_pool) + (size_t)kv * D * 2 + scol * 16;
    const unsigned char* vbase = static_cast<const unsigned char*>(a.v_pool) + (size_t)kv * D * 2 + scol * 16;

    u32x4_t kreg[PER_T], vreg[PER_T];
    auto issue = [&](int sub) {   // loads of sub-chunk `sub` (rows past the chunk repeat its last block)
#pragma unroll
      for (int k = 0; k < PER_T; ++k) {
        const int r = (tid + k * kThreads) / RC;
        const int blk = min(sub * kSub + r / kBS, nb - 1);
        const int ph = clampi(trow[blk], 0, nmax);
        const size_t off = (size_t)ph * block_bytes + (size_t)(r % kBS) * kv_row_bytes;
        kreg[k] = load16(kbase + off);
        vreg[k] = load16(vbase + off);
      }
    };
    auto commit = [&](int sub, int buf) {   // V rows at or past the V limit are zeroed (poison never meets p = 0)
#pragma unroll
      for (int k = 0; k < PER_T; ++k) {
        const int r = (tid + k * kThreads) / RC;
        const int pos = (kb0 + sub * kSub) * kBS + r;
        store16(kst[buf] + r * ROW + scol * 16, kreg[k]);
        store16(vst[buf] + r * ROW + scol * 16, pos < desc.w ? vreg[k] : u32x4_t{0u, 0u, 0u, 0u});
      }
    };

    // this wave's rows
    const bool active = wave * 16 < rows;
    const int r = wave * 16 + row;
    const bool row_ok = r < rows;
    const int rq = row_ok ? r : (active ? wave * 16 : 0);
    const int mq = rq / G, hq = kv * G + (rq - mq * G);
    const int bq = bl + mq;
    const int Lq = clampi(a.context_lens[bq], 0, max_tokens);
    const int hi_row = row_ok ? min(Lq, kBS * gp.sfx[bq]) : 0;
    u32x4_t qreg[D / 32];
    tile::load_q<D>(qreg, static_cast<const uint16_t*>(a.q) + ((size_t)bq * a.Hq + hq) * D, row_ok, lane);
    tile::State<D> st;
    tile::init(st);

    const int nsub = (nb + kSub - 1) / kSub;
    issue(0);
    commit(0, 0);
    __syncthreads();
    for (int sub = 0; sub < nsub; ++sub) {
      const int buf = sub & 1;
      if (sub + 1 < nsub) issue(sub + 1);
      if (active)
        tile::run_lds<D, ROW>(st, qreg, hi_row, kb0 + sub * kSub, min(kSub, nb - sub * kSub), kst[buf], vst[buf],
                              scale_log2e, lane);
      if (sub + 1 < nsub) commit(sub + 1, buf ^ 1);
      __syncthreads();
    }

    if (active) {
      const float l_row = tile::row_sum(st);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int ro = wave * 16 + 4 * quad + k;    // O row held in acc[*][k]
        const float lr = __shfl(l_row, 4 * quad + k);
        const float mr = __shfl(st.m_row, 4 * quad + k);
        if (ro < rows) {
          const int mo = ro / G, ho = kv * G + (ro - mo * G);
          float* od = gp.part + (((size_t)(bl + mo) * kGroupChunks + ch) * a.Hq + ho) * (D + 1);
          const float inv = lr != 0.f ? 1.f / lr : 0.f;
#pragma unroll
          for (int d = 0; d < DT; ++d) od[16 * d + row] = st.acc[d][k] * inv;
          if (row == 0) od[D] = lr != 0.f ? (mr + log2f(lr)) * kLn2 : kNegInf;
        }
      }
    }
  }
}

}  // namespace grp
}  // namespace pkv
