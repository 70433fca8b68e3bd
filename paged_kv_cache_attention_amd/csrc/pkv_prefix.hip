// Shared-prefix groups for single-token decode (gfx950).
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
// Detection (one wave per aligned window of kGroupWindow sequences):
//   key(b)     = first physical block of b (sequences with no tokens never group)
//   groups     = runs of equal keys inside the window, cut every M_max members
//   canonical  = the member with the most blocks (lowest index on ties)
//   s(b)       = common prefix length of b's and the canonical's tables,
//                limited to both block counts
//   d          = max s(b) over the non-canonical members; the canonical's
//                share is d (its tables are the ones the group walks)
// A group with fewer than kGroupMinShare common blocks is dissolved.  Member b
// then sees the group's blocks [0, d) up to position min(L_b, 16 s(b)); its
// own path covers blocks [s(b), n_b).  Only adjacent sequences are grouped;
// sharing between sequences far apart in the batch is left to the
// per-sequence path (still correct, only not deduplicated).
#include "pkv_device.h"
#include "pkv_internal.h"
#include "pkv_tile.h"

namespace pkv {
namespace {

constexpr int kBS = 16;
constexpr int kTiles = 4;            // 16-row tiles per group item (64 rows)
constexpr int kDetectWaves = 4;

__global__ __launch_bounds__(64 * kDetectWaves) void group_detect_kernel(const int32_t* __restrict__ tables,
                                                                      const int32_t* __restrict__ lens, int B,
                                                                      int max_blocks, int GM, GroupPlan gp) {
  const int lane = threadIdx.x & 63;
  const int w0 = (blockIdx.x * kDetectWaves + (threadIdx.x >> 6)) * kGroupWindow;
  if (w0 >= B) return;
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
    gp.sfx[j] = sfx;
    gp.nch[j] = nch;
    gp.cnt[j] = m == gs ? nch : 0;
    if (m == gs) gp.desc[j] = make_int4(w0 + cm, M, d, vlim);
  }
}

// One workgroup of kTiles waves per (group chunk, KV head) item; wave w owns
// rows 16w .. 16w+15 of the group's member-major rows r = member * G + head.
// The chunk's K and V rows of the KV head are staged through LDS in
// sub-chunks of kSub blocks (double-buffered: the next sub-chunk's loads are
// in flight while the tiles work on the current one), so each shared block is
// read from memory once per item and reused by every member tile.
constexpr int kStageThreads = 64 * kTiles;
// sub-chunk blocks: a 52 KB double buffer for D = 128 and 36 KB for D = 64,
// small enough for the kernel to sit beside the decode kernel on every CU
template <int D> struct Stage {
  static constexpr int SUB = D == 128 ? 3 : 4;
  static constexpr int ROWS = SUB * 16;
  static constexpr int ROW = 2 * D + 16;   // padded row bytes
};

template <int D>
__global__ __launch_bounds__(kStageThreads) __attribute__((amdgpu_waves_per_eu(3))) void group_prefix_kernel(DecodeArgs a, GroupPlan gp, const int* hdr,
                                                                   float scale_log2e) {
  constexpr int DT = D / 16;
  constexpr int kSub = Stage<D>::SUB, kSubRows = Stage<D>::ROWS, ROW = Stage<D>::ROW;
  constexpr int RC = D * 2 / 16;                        // 16-byte chunks per token row
  constexpr int PER_T = kSubRows * RC / kStageThreads;  // chunks per thread and sub-chunk (K, and again V)
  static_assert(PER_T * kStageThreads == kSubRows * RC, "even staging split");
  __shared__ __attribute__((aligned(16))) unsigned char kst[2][kSubRows * ROW];
  __shared__ __attribute__((aligned(16))) unsigned char vst[2][kSubRows * ROW];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.Hq / a.Hkv;
  const int row = lane & 15, quad = lane >> 4;
  const size_t kv_row_bytes = (size_t)a.Hkv * D * 2;
  const size_t block_bytes = (size_t)kBS * kv_row_bytes;
  const int nmax = a.N_blocks - 1;
  const int max_tokens = a.max_blocks * kBS;
  const int items = hdr[3] * a.Hkv;
  // staging map: chunk i = tid + k * kStageThreads -> token row i / RC, 16-byte column i % RC
  const int scol = tid % RC;

  for (int item = blockIdx.x; item < items; item += gridDim.x) {
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
        const int r = (tid + k * kStageThreads) / RC;
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
        const int r = (tid + k * kStageThreads) / RC;
        const int pos = (kb0 + sub * kSub) * kBS + r;
        store16(&kst[buf][r * ROW + scol * 16], kreg[k]);
        store16(&vst[buf][r * ROW + scol * 16], pos < desc.w ? vreg[k] : u32x4_t{0u, 0u, 0u, 0u});
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

constexpr int kMaxDevices = 64;
GroupSide g_side[kMaxDevices];
bool g_side_ready[kMaxDevices];

}  // namespace

std::mutex& group_side_mutex() {
  static std::mutex mu;
  return mu;
}

hipError_t group_side(GroupSide* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(group_side_mutex());
  if (!g_side_ready[dev]) {
    GroupSide s{};
    if ((e = hipDeviceGetAttribute(&s.cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if ((e = hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&s.fork, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&s.join, hipEventDisableTiming)) != hipSuccess) return e;
    g_side[dev] = s;
    g_side_ready[dev] = true;
  }
  *out = g_side[dev];
  return hipSuccess;
}

bool groups_supported(const DecodeArgs& a) {
  const int G = a.Hq / a.Hkv;
  return a.bf16 && a.T == 1 && a.B >= 2 && (a.D == 64 || a.D == 128) && G <= 32;
}

size_t group_workspace_bytes(int B, int Hq, int D) {
  const size_t r = 256;
  size_t off = 0;
  off += ((size_t)B * 4 + r - 1) / r * r * 3;                         // sfx, nch, cnt
  off += ((size_t)B * 16 + r - 1) / r * r;                            // desc
  off += ((size_t)B * kGroupChunks / 2 * 4 + r - 1) / r * r;          // clist
  off += (size_t)B * kGroupChunks * Hq * (D + 1) * 4;                 // partials
  return off;
}

GroupPlan group_plan_layout(void* base, int B, int Hq, int D) {
  const size_t r = 256;
  unsigned char* p = static_cast<unsigned char*>(base);
  GroupPlan gp{};
  const size_t vec = ((size_t)B * 4 + r - 1) / r * r;
  gp.sfx = reinterpret_cast<int*>(p); p += vec;
  gp.nch = reinterpret_cast<int*>(p); p += vec;
  gp.cnt = reinterpret_cast<int*>(p); p += vec;
  gp.desc = reinterpret_cast<int4*>(p); p += ((size_t)B * 16 + r - 1) / r * r;
  gp.clist = reinterpret_cast<int*>(p); p += ((size_t)B * kGroupChunks / 2 * 4 + r - 1) / r * r;
  gp.part = reinterpret_cast<float*>(p);
  (void)Hq; (void)D;
  return gp;
}

hipError_t launch_group_detect(const DecodeArgs& a, const GroupPlan& gp, hipStream_t stream) {
  const int windows = (a.B + kGroupWindow - 1) / kGroupWindow;
  const int GM = group_members(a.Hq / a.Hkv);
  hipLaunchKernelGGL(group_detect_kernel, dim3((windows + kDetectWaves - 1) / kDetectWaves), dim3(64 * kDetectWaves), 0,
                     stream, a.block_tables, a.context_lens, a.B, a.max_blocks, GM, gp);
  return hipGetLastError();
}

hipError_t launch_group_prefix(const DecodeArgs& a, const GroupPlan& gp, const int* hdr, int grid, hipStream_t stream) {
  // persistent: at most one workgroup per item (B/2 groups, kGroupChunks
  // chunks each, one item per KV head) and per CU
  const long long items = (long long)(a.B / 2) * kGroupChunks * a.Hkv;
  if (items < grid) grid = (int)items;
  if (grid < 1) grid = 1;
  const float sl2 = a.scale * kLog2e;
  if (a.D == 64)
    hipLaunchKernelGGL((group_prefix_kernel<64>), dim3(grid), dim3(kStageThreads), 0, stream, a, gp, hdr, sl2);
  else
    hipLaunchKernelGGL((group_prefix_kernel<128>), dim3(grid), dim3(kStageThreads), 0, stream, a, gp, hdr, sl2);
  return hipGetLastError();
}

}  // namespace pkv
