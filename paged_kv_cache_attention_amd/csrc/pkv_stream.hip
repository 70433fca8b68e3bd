// Paged decode attention, balanced persistent VALU path (gfx950).
//
// Work is the flattened list of 16-token KV blocks of all (query token t,
// sequence b) pairs:  flat = prefix[t*B + b] + j,  j < ceil(visible(b,t)/16).
// A fixed grid of persistent workgroups splits that list into equal
// contiguous ranges, so every workgroup streams the same number of blocks
// whatever the mix of sequence lengths.  A workgroup has one wave per group of
// 4 query heads (U = Hq/4 waves); its waves walk the same blocks together, so
// each CU reads whole physical blocks (all KV heads, contiguous) at once.
// A (t, b) pair that lies inside one range is finished by its workgroup; a
// pair cut by range boundaries leaves one normalised partial (o, lse) per
// piece and head, merged afterwards by log-sum-exp weights ("Inference From
// Scratch", ch. 8: softmax pieces combine through their max and sum).
//
// Inside a wave everything stays in registers:
//   * lane (c, kl, tg) loads 16-byte chunk c of token rows of KV head kl; a
//     block of K (or V) is LOADS such loads per lane;
//   * each lane dots its K chunk with the matching q chunk of the GW query
//     heads of that KV head (v_dot2 on bf16 pairs), and a DPP reduce-scatter
//     over the NC lanes of a row leaves one complete score per lane;
//   * online softmax per query head with a lazily raised running maximum
//     (exponents stay <= 2^8; a rescale happens only when a score exceeds the
//     maximum by more than 8 in base-2 units, detected with one ballot);
//   * p is broadcast back along the row with DPP and multiplies the lane's
//     own V chunk into fp32 accumulators;
//   * K and V of the next PD blocks are in flight while a block is processed.
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kBS = 16;
constexpr int kHPW = 4;              // query heads per work unit
constexpr int kWaves = kStreamWaves;   // about 8 waves per CU
// Head groups (waves) per decode workgroup: one workgroup per range and CU
// (a second workgroup on a CU measured about 8 % slower than the first).
constexpr int kMaxU = 8;
constexpr int kMinBlocksPerRange = 16;
constexpr float kSlack = 8.f;

struct StreamArgs {
  DecodeArgs a;
  int* hdr;            // [total, per, total, unused, nu]
  int* prefix;         // [TB + 1] (written by the planning kernel only)
  int* first;          // [ranges] first non-empty unit (compact index) of each range, -1 if idle
  int4* mdesc;         // [ranges] merge at boundary r: {unit, first range, last range} or x = -1
  int4* udesc;         // [nu + 1] non-empty units: {tb, flat start, table offset, visible tokens}
  float* part;         // partial slots [(ranges + TB)][Hq][D + 1]
  int stream_wgs;      // decode workgroups
  int TB;
  int ranges;          // workgroups splitting the block list
  bool inl;            // plan computed inside the decode kernel (no planning kernel)
};

template <typename ET, int D, int GW>
struct SGeo {
  static constexpr int EB = Storage<ET>::bytes;
  static constexpr int EC = 16 / EB;
  static constexpr int RB = D * EB;
  static constexpr int NC = RB / 16;              // lanes per token row (8 or 16)
  static constexpr int KW = kHPW / GW;            // KV heads per unit
  static constexpr int LOADS = KW * NC / 4;       // 16-byte loads per lane per block
  static constexpr int RPL = 64 / (NC * KW);      // tokens per load and KV head
  static constexpr int NCOMB = LOADS * GW;        // (load, head) score combos per row group
  static_assert(NCOMB == NC, "one score per lane after the reduce-scatter");
  static_assert(NC == 8 || NC == 16, "rows of 8 or 16 lanes");
};

template <int CTRL> __device__ __forceinline__ float dppf(float x) {
  return __builtin_amdgcn_update_dpp(0.0f, x, CTRL, 0xf, 0xf, false);
}

// One reduce-scatter stage: lanes whose `bit` is clear keep the lower half of
// v[0..2n), the others the upper half, each adding its partner's copy.
template <int CTRL, int N>
__device__ __forceinline__ void rs_stage(float* v, bool upper) {
#pragma unroll
  for (int m = 0; m < N; ++m) {
    const float mine = upper ? v[m + N] : v[m];
    const float theirs = upper ? v[m] : v[m + N];
    v[m] = mine + dppf<CTRL>(theirs);
  }
}

// Reduce-scatter of NC partial sums over a group of NC lanes (a 16-lane row
// or an 8-lane half row): afterwards v[0] of lane c holds the group sum of
// combo c.  Partners: c^8 (row rotate by 8), c^7 (half-row mirror), c^2, c^1.
template <int NC>
__device__ __forceinline__ float reduce_scatter(float* v, int c) {
  if constexpr (NC == 16) rs_stage<0x128, 8>(v, c & 8);   // row_ror:8
  rs_stage<0x141, 4>(v, c & 4);                            // row_half_mirror (c^7): split on bit 2
  rs_stage<0x4E, 2>(v, c & 2);                             // quad_perm [2,3,0,1]
  rs_stage<0xB1, 1>(v, c & 1);                             // quad_perm [1,0,3,2]
  return v[0];
}

// p of combo k from lane k of the lane's own group.
template <int NC>
__device__ __forceinline__ float group_bcast(float p, int k, bool upper_half) {
  if constexpr (NC == 16) {
    switch (k) {
      case 0: return dppf<0x150>(p); case 1: return dppf<0x151>(p); case 2: return dppf<0x152>(p);
      case 3: return dppf<0x153>(p); case 4: return dppf<0x154>(p); case 5: return dppf<0x155>(p);
      case 6: return dppf<0x156>(p); case 7: return dppf<0x157>(p); case 8: return dppf<0x158>(p);
      case 9: return dppf<0x159>(p); case 10: return dppf<0x15A>(p); case 11: return dppf<0x15B>(p);
      case 12: return dppf<0x15C>(p); case 13: return dppf<0x15D>(p); case 14: return dppf<0x15E>(p);
      default: return dppf<0x15F>(p);
    }
  } else {
    float lo, hi;
    switch (k) {
      case 0: lo = dppf<0x150>(p); hi = dppf<0x158>(p); break;
      case 1: lo = dppf<0x151>(p); hi = dppf<0x159>(p); break;
      case 2: lo = dppf<0x152>(p); hi = dppf<0x15A>(p); break;
      case 3: lo = dppf<0x153>(p); hi = dppf<0x15B>(p); break;
      case 4: lo = dppf<0x154>(p); hi = dppf<0x15C>(p); break;
      case 5: lo = dppf<0x155>(p); hi = dppf<0x15D>(p); break;
      case 6: lo = dppf<0x156>(p); hi = dppf<0x15E>(p); break;
      default: lo = dppf<0x157>(p); hi = dppf<0x15F>(p); break;
    }
    return upper_half ? hi : lo;
  }
}

// Reduce over all lanes that hold the same query head: every lane bit except
// the head-selecting ones (the low log2(GW) bits of c and the kl bits).
template <int NC, int GW, int KW, bool MAX>
__device__ __forceinline__ float head_reduce(float x) {
#pragma unroll
  for (int bit = 0; bit < 6; ++bit) {
    const int m = 1 << bit;
    const bool head_bit = (m < GW) || (m >= NC && m < NC * KW);
    if (head_bit) continue;
    const float y = __shfl_xor(x, m);
    x = MAX ? fmaxf(x, y) : x + y;
  }
  return x;
}

template <typename ET> __device__ __forceinline__ float chunk_dot4(u32x4_t k, u32x4_t q, float acc);
template <> __device__ __forceinline__ float chunk_dot4<Bf16>(u32x4_t k, u32x4_t q, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(k.x), as_bf16x2(q.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(k.y), as_bf16x2(q.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(k.z), as_bf16x2(q.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(k.w), as_bf16x2(q.w), acc, false);
  return acc;
}
template <> __device__ __forceinline__ float chunk_dot4<float>(u32x4_t k, u32x4_t q, float acc) {
  acc = fmaf(__uint_as_float(k.x), __uint_as_float(q.x), acc);
  acc = fmaf(__uint_as_float(k.y), __uint_as_float(q.y), acc);
  acc = fmaf(__uint_as_float(k.z), __uint_as_float(q.z), acc);
  acc = fmaf(__uint_as_float(k.w), __uint_as_float(q.w), acc);
  return acc;
}

template <typename ET> __device__ __forceinline__ void widen(u32x4_t v, float* f);
template <> __device__ __forceinline__ void widen<Bf16>(u32x4_t v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}
template <> __device__ __forceinline__ void widen<float>(u32x4_t v, float* f) {
  f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y); f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}

template <typename ET> __device__ __forceinline__ void store_chunk(void* dst, const float* v);
template <> __device__ __forceinline__ void store_chunk<Bf16>(void* dst, const float* v) {
  u32x4_t w;
  w.x = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
  w.y = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
  w.z = (uint32_t)f32_to_bf16_rne(v[4]) | ((uint32_t)f32_to_bf16_rne(v[5]) << 16);
  w.w = (uint32_t)f32_to_bf16_rne(v[6]) | ((uint32_t)f32_to_bf16_rne(v[7]) << 16);
  store16(dst, w);
}
template <> __device__ __forceinline__ void store_chunk<float>(void* dst, const float* v) {
  store16(dst, u32x4_t{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
}

// ---------------------------------------------------------------------------
// Planning: blocks per (t, b) unit, their prefix sums, the compact list of
// non-empty units with everything a wave needs to walk them, and each range's
// first non-empty unit.
// ---------------------------------------------------------------------------
constexpr int kPlanThreads = 1024;

__device__ __forceinline__ int unit_visible(const int32_t* lens, int tb, int B, int T, int max_tokens) {
  const int t = tb / B, b = tb - t * B;
  const int L = clampi(lens[b], 0, max_tokens);
  return max(0, L - T + t + 1);
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ lens, int B, int T,
                                                            int ranges, int max_blocks, int TB, int* __restrict__ hdr,
                                                            int* __restrict__ prefix, int* __restrict__ first,
                                                            int4* __restrict__ udesc, int4* __restrict__ mdesc,
                                                            PlanFinish fin, bool finish) {
  __shared__ int part[kPlanThreads];
  __shared__ int npart[kPlanThreads];
  __shared__ int spref[kStreamMaxTB + 1];   // flat start of each non-empty unit
  __shared__ int sid[kStreamMaxTB];         // its unit index
  const int tid = threadIdx.x;
  const int max_tokens = max_blocks * kBS;
  const int per_t = (TB + kPlanThreads - 1) / kPlanThreads;
  const int s0 = min(TB, tid * per_t), s1 = min(TB, s0 + per_t);
  auto blocks_of = [&](int vis) { return (vis + kBS - 1) / kBS; };
  int sum = 0, ne = 0;
  for (int i = s0; i < s1; ++i) {
    const int nb = blocks_of(unit_visible(lens, i, B, T, max_tokens));
    sum += nb;
    ne += nb > 0;
  }
  part[tid] = sum;
  npart[tid] = ne;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    const int nv = tid >= off ? npart[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    npart[tid] += nv;
    __syncthreads();
  }
  int run = tid ? part[tid - 1] : 0;
  int krun = tid ? npart[tid - 1] : 0;
  for (int i = s0; i < s1; ++i) {
    prefix[i] = run;
    const int vis = unit_visible(lens, i, B, T, max_tokens);
    const int nb = blocks_of(vis);
    if (nb > 0) {
      const int b = i % B;
      // {unit, flat start, table offset of its first block, visible tokens}
      udesc[krun] = make_int4(i, run, b * max_blocks, vis);
      spref[krun] = run;
      sid[krun] = i;
      ++krun;
    }
    run += nb;
  }
  const int tbtot = part[kPlanThreads - 1];
  const int nu = npart[kPlanThreads - 1];
  if (tid == 0) {
    prefix[TB] = tbtot;
    spref[nu] = tbtot;
    udesc[nu] = make_int4(0, tbtot, 0, 0);   // sentinel: start of "unit nu" = end of the list
  }
  __syncthreads();
  const int per = max(kMinBlocksPerRange, (tbtot + ranges - 1) / ranges);
  if (tid == 0) {
    hdr[0] = tbtot;
    hdr[1] = per;
    hdr[2] = tbtot;
    hdr[3] = 0;
    hdr[4] = nu;
  }
  if (finish) {
    // units with nothing visible: out = 0, lse = -inf
    for (int i = s0; i < s1; ++i) {
      const int nb = blocks_of(unit_visible(lens, i, B, T, max_tokens));
      if (nb > 0) continue;
      const int t = i / B, b = i - t * B;
      const size_t row = ((size_t)b * T + t) * fin.Hq;
      for (int e = 0; e < fin.Hq * fin.D; ++e) {
        if (fin.bf16) static_cast<uint16_t*>(fin.out)[row * fin.D + e] = 0;
        else static_cast<float*>(fin.out)[row * fin.D + e] = 0.f;
      }
      if (fin.lse_out)
        for (int h = 0; h < fin.Hq; ++h) fin.lse_out[row + h] = kNegInf;
    }
  }
  for (int w = tid; w < ranges; w += kPlanThreads) {
    const long long F0 = (long long)w * per;
    if (F0 >= tbtot) {
      first[w] = -1;
      if (mdesc) mdesc[w] = make_int4(-1, 0, 0, 0);
      continue;
    }
    const int r = (int)F0;
    int lo = 0, hi = nu;   // spref[lo] <= r < spref[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (spref[mid] <= r) lo = mid; else hi = mid;
    }
    first[w] = lo;
    // the unit cut by boundary w is merged there if boundary w cuts it first
    if (mdesc) {
      const int us = spref[lo], ue = spref[lo + 1];
      mdesc[w] = w > 0 && us < r && us >= r - per ? make_int4(sid[lo], w - 1, (ue - 1) / per, 0) : make_int4(-1, 0, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// The same plan computed inside the decode kernel, when the unit list fits in
// LDS (B*T + 1 <= kInlineUnitsPerWave entries per wave of the workgroup):
// every workgroup derives it from the lengths, so no planning launch precedes
// the decode launch.  Thread i counts the blocks of units 4i .. 4i+3; a wave
// scan plus a pass over the waves' totals gives their flat starts; the
// compact descriptors go to LDS.  Each range publishes the merge descriptor
// of its boundary to the workspace for the merge kernel.
// ---------------------------------------------------------------------------
constexpr int kInlineUnitsPerWave = 256;
constexpr int kInlinePT = kInlineUnitsPerWave / 64;   // units per thread

struct InlinePlan {
  int total, per, nu;
};

__device__ __forceinline__ InlinePlan inline_plan(const StreamArgs& sa, int4* lud, int* wsc) {
  const DecodeArgs& a = sa.a;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), nw = blockDim.x >> 6;
  const int max_tokens = a.max_blocks * kBS;
  int vis[kInlinePT];
  int sum = 0, ne = 0;
#pragma unroll
  for (int j = 0; j < kInlinePT; ++j) {
    const int i = tid * kInlinePT + j;
    vis[j] = i < sa.TB ? unit_visible(a.context_lens, i, a.B, a.T, max_tokens) : 0;
    const int nb = (vis[j] + kBS - 1) / kBS;
    sum += nb;
    ne += nb > 0;
  }
  int is = sum, in = ne;   // inclusive scans over the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int ys = __shfl_up(is, off), yn = __shfl_up(in, off);
    if (lane >= off) {
      is += ys;
      in += yn;
    }
  }
  if (lane == 63) {
    wsc[wave] = is;
    wsc[16 + wave] = in;
  }
  __syncthreads();
  int run = is - sum, krun = in - ne, total = 0, nu = 0;
  for (int w = 0; w < nw; ++w) {
    const int vs = wsc[w], vn = wsc[16 + w];
    if (w < wave) {
      run += vs;
      krun += vn;
    }
    total += vs;
    nu += vn;
  }
#pragma unroll
  for (int j = 0; j < kInlinePT; ++j) {
    const int i = tid * kInlinePT + j;
    const int nb = (vis[j] + kBS - 1) / kBS;
    if (nb > 0) lud[krun++] = make_int4(i, run, (i % a.B) * a.max_blocks, vis[j]);
    run += nb;
  }
  if (tid == 0) lud[nu] = make_int4(0, total, 0, 0);   // sentinel
  __syncthreads();
  const int per = max(kMinBlocksPerRange, (total + sa.ranges - 1) / sa.ranges);
  return InlinePlan{total, per, nu};
}

// Largest k < nu with lud[k].y <= F, by one wave (unit starts strictly
// increase and lud[0].y = 0 <= F): 64-way splits of the candidate interval.
__device__ __forceinline__ int find_unit(const int4* lud, int nu, int F) {
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = nu;   // the answer lies in [lo, hi); lud[lo].y <= F
  while (hi - lo > 64) {
    const int step = (hi - lo + 63) / 64;
    const int k = lo + lane * step;
    const unsigned long long m = __builtin_amdgcn_ballot_w64(k < hi && lud[min(k, hi - 1)].y <= F);
    lo += (63 - __builtin_clzll(m)) * step;
    hi = min(hi, lo + step);
  }
  const int k = lo + lane;
  const unsigned long long m = __builtin_amdgcn_ballot_w64(k < hi && lud[min(k, hi - 1)].y <= F);
  return lo + 63 - __builtin_clzll(m);
}

// ---------------------------------------------------------------------------
// The persistent decode kernel.
//
// A wave walks the flat blocks [F0, F1) of its range as one continuous
// stream.  Per chunk of 64 flat blocks each lane resolves one block: its unit
// (binary search over the starts of a window of 64 consecutive non-empty
// units), its physical id (table gather) and whether a unit starts or ends
// there.  The next chunk is resolved while the current one is processed, the
// descriptor and query of the next unit are loaded while the current unit
// runs, and the K/V prefetch runs across unit and chunk boundaries, so the
// memory pipeline only drains at the end of the range.
// ---------------------------------------------------------------------------
constexpr int kResolveAt = 4;   // step of a full chunk at which the next chunk is resolved

// The chunk loop is laid out so that every value loaded ahead is consumed at
// a fixed distance (in issued loads) from its load: the first kResolveAt steps
// of a full chunk are unrolled before the next chunk is resolved, the middle
// steps run a loop of constant trip count and the last PD steps, which
// prefetch from the next chunk, are unrolled after it.  The compiler's wait
// counts are then exact instead of draining the prefetch queue.
// Log-sum-exp merge of the pieces of one unit cut by range boundaries, for
// the four heads of head group u, by one wave: lanes 16h .. 16h+15 hold head
// h, D/16 elements each.  Pieces come from the partial slots of ranges w0 .. w1
// (slot of range w: w + tb), loaded in batches of BATCH with all loads issued
// together and merged online (running max, rescaled sum and accumulator).
template <typename ET, int D, int BATCH>
__device__ __forceinline__ void merge_pieces(const DecodeArgs& a, const float* part, int tb, int u, int w0, int w1,
                                             int lane) {
  constexpr int EPL = D / 16;
  using OT = typename Storage<ET>::T;
  const int t = tb / a.B, b = tb - t * a.B;
  const int h = lane >> 4, d0 = (lane & 15) * EPL;
  const size_t orow = (((size_t)b * a.T + t) * a.Hq + u * kHPW + h) * D + d0;
  OT* out = static_cast<OT*>(a.out) + orow;
  float* lse_out = a.lse_out ? a.lse_out + ((size_t)b * a.T + t) * a.Hq + u * kHPW + h : nullptr;
  float m = kNegInf, ssum = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  auto absorb = [&](float lv, const float* ov) {
    if (lv == kNegInf) return;   // absent or empty piece: its o is not read
    const float nm = fmaxf(m, lv);
    const float sa_ = __builtin_amdgcn_exp2f((m - nm) * kLog2e);
    const float sb = __builtin_amdgcn_exp2f((lv - nm) * kLog2e);
    ssum = ssum * sa_ + sb;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = acc[e] * sa_ + sb * ov[e];
    m = nm;
  };
  for (int w = w0; w <= w1; w += BATCH) {
    float lv[BATCH], ov[BATCH][EPL];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      lv[k] = kNegInf;
      if (w + k <= w1) {
        const float* slot = part + ((size_t)(w + k + tb) * a.Hq + u * kHPW + h) * (D + 1);
        lv[k] = slot[D];
#pragma unroll
        for (int e = 0; e < EPL; ++e) ov[k][e] = slot[d0 + e];
      }
    }
#pragma unroll
    for (int k = 0; k < BATCH; ++k) absorb(lv[k], ov[k]);
  }
  const float inv = ssum != 0.f ? 1.f / ssum : 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) store_out<ET>(out + e, acc[e] * inv);
  if (lse_out && (lane & 15) == 0) *lse_out = ssum != 0.f ? m + logf(ssum) : kNegInf;
}

constexpr int kStage = 8;   // units whose descriptors and queries are staged at a time

template <typename ET, int D, int GW>
struct StreamLds {
  static constexpr int QCH = SGeo<ET, D, GW>::NC * SGeo<ET, D, GW>::KW;   // distinct 16-byte query chunks per head
  static constexpr int QWAVE = kStage * GW * QCH * 16;                   // staged query bytes per wave
};

// INL: the plan is computed by the kernel itself (inline_plan) and the unit
// descriptors are read from LDS; otherwise the planning kernel wrote them to
// the workspace.  LDS: staged queries (QWAVE bytes per wave), then, with INL,
// the unit descriptors; dynamic, sized by the launch.
template <typename ET, int D, int GW, int PD, bool INL>
__global__ __launch_bounds__(64 * kMaxU) __attribute__((amdgpu_waves_per_eu(2)))
void stream_decode_kernel(StreamArgs sa, const int4* __restrict__ udesc, float scale_log2e) {
  using G = SGeo<ET, D, GW>;
  using ST = typename Storage<ET>::T;
  using LD = StreamLds<ET, D, GW>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const DecodeArgs& a = sa.a;
  const int lane = threadIdx.x & 63;
  const int U = a.Hq / kHPW;
  const int wpg = blockDim.x >> 6;                      // waves per workgroup
  int4* lud = reinterpret_cast<int4*>(lds + wpg * LD::QWAVE);   // INL: unit descriptors
  __shared__ int wsc[32];
  int total, per, nu;
  if constexpr (INL) {
    const InlinePlan ip = inline_plan(sa, lud, wsc);
    total = __builtin_amdgcn_readfirstlane(ip.total);
    per = __builtin_amdgcn_readfirstlane(ip.per);
    nu = __builtin_amdgcn_readfirstlane(ip.nu);
  } else {
    total = sa.hdr[0];
    per = sa.hdr[1];
    nu = sa.hdr[4];
  }
  // Workgroup -> range.  Workgroups go to the 8 XCDs round-robin; when the
  // ranges are longer than the minimum (the batch fills them all, but for
  // rounding at the end), each XCD takes a contiguous run of ranges instead,
  // so neighbouring sequences (where a batch shares a prompt prefix) re-read
  // their common blocks through one XCD's L2 rather than all eight (8B batch
  // with shared prefixes: 240 -> 232 us; the 1B batch, private blocks: +1 %).
  // Small batches keep the launch order, which spreads their few non-empty
  // ranges over every XCD.
  const bool contiguous = INL && gridDim.x % 8 == 0 && per > kMinBlocksPerRange;
  const int wid = __builtin_amdgcn_readfirstlane(contiguous ? (int)xcd_logical_id(blockIdx.x, gridDim.x / 8)
                                                            : (int)blockIdx.x);
  const int rng = wid / (U / wpg);               // block range of this workgroup
  const int u = (wid % (U / wpg)) * wpg + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // INL: units with nothing visible get out = 0 and lse = -inf, spread over
  // all waves of the grid (the planning kernel does this otherwise)
  auto finish_empty = [&]() {
    if constexpr (INL) {
      using OT = typename Storage<ET>::T;
      const int lane_ = threadIdx.x & 63;
      const int gw = wid * wpg + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), nwt = gridDim.x * wpg;
      for (int i = gw; i < sa.TB; i += nwt) {
        if (unit_visible(a.context_lens, i, a.B, a.T, a.max_blocks * kBS) > 0) continue;
        const int t = i / a.B, b = i - t * a.B;
        const size_t row = ((size_t)b * a.T + t) * a.Hq;
        OT* o = static_cast<OT*>(a.out) + row * D;
        for (int e = lane_; e < a.Hq * D; e += 64) store_out<ET>(o + e, 0.f);
        if (a.lse_out)
          for (int h = lane_; h < a.Hq; h += 64) a.lse_out[row + h] = kNegInf;
      }
    }
  };
  const int F0 = rng * per;
  const bool mwriter = INL && rng > 0 && threadIdx.x == 0 && wid % (U / wpg) == 0;
  if (F0 >= total) {
    if (mwriter) sa.mdesc[rng] = make_int4(-1, 0, 0, 0);
    finish_empty();
    return;
  }
  const int F1 = min(total, F0 + per);

  const int c = lane % G::NC;
  const int grp = lane / G::NC;
  const int kl = grp % G::KW;
  const int tg = grp / G::KW;
  const bool upper_half = (lane & 8) != 0;
  const int lc = c / GW;            // load index of this lane's score combo
  const int G_ratio = a.Hq / a.Hkv;
  const size_t block_bytes = (size_t)kBS * a.Hkv * G::RB;
  const uint32_t load_step = (uint32_t)(G::RPL * a.Hkv * G::RB);
  const int nmax = a.N_blocks - 1;
  const int h0 = u * kHPW;
  const int kv0 = h0 / G_ratio;
  const uint32_t lane_off = (uint32_t)(((tg * a.Hkv) + kv0 + kl) * G::RB + c * 16);
  const unsigned char* kpool = static_cast<const unsigned char*>(a.k_pool) + lane_off;
  const unsigned char* vpool = static_cast<const unsigned char*>(a.v_pool) + lane_off;

  // ---- chunk resolution ----
  auto desc = [&](int k) -> int4 {
    if constexpr (INL) return lud[k];
    else return udesc[k];
  };
  auto window = [&](int kc, int4& w, int& ue) {
    w = desc(min(kc + lane, nu));
    ue = desc(min(kc + lane + 1, nu)).y;
  };
  // Resolves flat blocks Fc + lane against the window of units starting at
  // wbase; returns the first unit of the following chunk.
  auto resolve = [&](int Fc, int wbase, const int4& w, int ue, int& phys, int& flags) {
    const int f = min(Fc + lane, F1 - 1);
    int pos = 0;
#pragma unroll
    for (int step = 32; step >= 1; step >>= 1) {
      const int cand = pos + step;
      if (__shfl(w.y, cand) <= f) pos = cand;
    }
    const int us = __shfl(w.y, pos), tofs = __shfl(w.z, pos), uen = __shfl(ue, pos);
    phys = a.block_tables[tofs + (f - us)];   // clamped where it is read
    flags = Fc + lane < F1 ? ((f == us || f == F0) ? 1 : 0) | ((f + 1 == uen || f + 1 == F1) ? 2 : 0) : 0;
    return wbase + __builtin_amdgcn_readlane(pos, 63) + ((__builtin_amdgcn_readlane(flags, 63) & 2) ? 1 : 0);
  };

  int Fc = F0;
  int kfirst;
  if constexpr (INL) {
    kfirst = __builtin_amdgcn_readfirstlane(find_unit(lud, nu, F0));
    if (mwriter) {   // the unit cut by this range's start is merged here if this is its first cut
      const int4 d = lud[kfirst];
      const int ue = lud[kfirst + 1].y;
      sa.mdesc[rng] = d.y < F0 && d.y >= F0 - per ? make_int4(d.x, rng - 1, (ue - 1) / per, 0) : make_int4(-1, 0, 0, 0);
    }
  } else {
    kfirst = sa.first[rng];
  }
  int4 wv; int wue;
  int cphys, cflags, nphys = 0, nflags = 0;
  window(kfirst, wv, wue);
  int wbase = resolve(Fc, kfirst, wv, wue, cphys, cflags);   // window base of the next chunk
  bool has_next = Fc + 64 < F1;
  if (has_next) window(wbase, wv, wue);

  // ---- unit staging ----
  // The descriptors and query chunks of the next kStage units are staged at
  // once: descriptors in registers (lane s holds unit kbase + s), queries in
  // LDS.  Beginning a unit then issues no memory operation, so the K/V
  // prefetch keeps running across unit boundaries; the stage itself waits for
  // its loads and is refilled every kStage units.
  constexpr int QCH = LD::QCH;
  static_assert(GW * QCH <= 64, "one staged chunk per lane");
  u32x4_t (*qlds)[kStage][GW][QCH] = reinterpret_cast<u32x4_t (*)[kStage][GW][QCH]>(lds);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sl = lane % (GW * QCH);             // lanes past GW * QCH repeat a chunk
  const int sg = sl / QCH, sr = sl % QCH;        // chunk this lane stages: head sg, chunk sr
  const int skl = sr / G::NC, sc = sr % G::NC;
  int kbase = 0;
  int4 sd;          // lane s: descriptor of unit kbase + s
  int se = 0;       // lane s: flat start of unit kbase + s + 1 (its end)
  auto stage = [&](int kb) {
    kbase = kb;
    sd = desc(min(kb + lane, nu));
    se = desc(min(kb + lane + 1, nu)).y;
    u32x4_t tmp[kStage];
#pragma unroll
    for (int s = 0; s < kStage; ++s) {
      const int tb_s = __builtin_amdgcn_readlane(sd.x, s);
      const int t = tb_s / a.B, b = tb_s - t * a.B;
      const unsigned char* qp = reinterpret_cast<const unsigned char*>(static_cast<const ST*>(a.q)) +
                                (((size_t)(b * a.T + t) * a.Hq + h0 + skl * GW + sg) * D) * G::EB + sc * 16;
      tmp[s] = load16(qp);
    }
    // consume every staged register here, so that no later use waits on these loads
    __asm__ volatile("" ::"v"(sd.y), "v"(sd.z), "v"(sd.w), "v"(se));
    if (lane < GW * QCH) {
#pragma unroll
      for (int s = 0; s < kStage; ++s) qlds[wave][s][sg][sr] = tmp[s];
    }
  };
  int knext = kfirst;               // unit that begins next
  stage(kfirst);
  u32x4_t qreg[GW];

  // current unit
  int tb = 0, kb_off = 0, hi = 0;
  bool direct = false;
  float m_lane = kNegInf, l_part = 0.f;
  float acc[GW][G::EC];

  auto begin_unit = [&]() {
    if (knext - kbase == kStage) stage(knext);
    const int s = knext - kbase;
    ++knext;
    tb = __builtin_amdgcn_readlane(sd.x, s);
    const int ustart = __builtin_amdgcn_readlane(sd.y, s);
    const int tofs = __builtin_amdgcn_readlane(sd.z, s);
    const int hv = __builtin_amdgcn_readlane(sd.w, s);
    const int uend = __builtin_amdgcn_readlane(se, s);
#pragma unroll
    for (int g = 0; g < GW; ++g) qreg[g] = qlds[wave][s][g][kl * G::NC + c];
    const int b = tb % a.B;
    kb_off = (tofs - b * a.max_blocks) - ustart;   // logical block = flat index + kb_off
    hi = hv;
    direct = ustart >= F0 && uend <= F1;
    m_lane = kNegInf;
    l_part = 0.f;
#pragma unroll
    for (int g = 0; g < GW; ++g)
#pragma unroll
      for (int e = 0; e < G::EC; ++e) acc[g][e] = 0.f;
  };

  auto end_unit = [&]() {
    // combine token groups and lanes of each head, then store
    const float l_head = head_reduce<G::NC, GW, G::KW, false>(l_part);
#pragma unroll
    for (int bit = 0; bit < 6; ++bit) {
      const int m = 1 << bit;
      if (m < G::NC * G::KW) continue;       // tg bits only
#pragma unroll
      for (int g = 0; g < GW; ++g)
#pragma unroll
        for (int e = 0; e < G::EC; ++e) acc[g][e] += __shfl_xor(acc[g][e], m);
    }
    if (tg == 0) {
      const int t = tb / a.B, b = tb - t * a.B;
      const size_t row0 = ((size_t)b * a.T + t) * a.Hq + h0;
      float* slot = sa.part + ((size_t)(rng + tb) * a.Hq + h0) * (D + 1);
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        const int hh = kl * GW + g;            // head within the unit
        const float lh = __shfl(l_head, grp * G::NC + g);
        const float mh = __shfl(m_lane, grp * G::NC + g);
        float o[G::EC];
#pragma unroll
        for (int e = 0; e < G::EC; ++e) o[e] = lh != 0.f ? acc[g][e] / lh : 0.f;
        const float lse = lh != 0.f ? (mh + log2f(lh)) * kLn2 : kNegInf;
        if (direct) {
          store_chunk<ET>(static_cast<unsigned char*>(a.out) + ((row0 + hh) * D + c * G::EC) * G::EB, o);
          if (c == 0 && a.lse_out) a.lse_out[row0 + hh] = lse;
        } else {
          float* od = slot + hh * (D + 1) + c * G::EC;
#pragma unroll
          for (int e = 0; e < G::EC; e += 4) store16(od + e, u32x4_t{__float_as_uint(o[e]), __float_as_uint(o[e + 1]),
                                                                      __float_as_uint(o[e + 2]), __float_as_uint(o[e + 3])});
          if (c == 0) slot[hh * (D + 1) + D] = lse;
        }
      }
    }
  };

  u32x4_t kbuf[PD][G::LOADS], vbuf[PD][G::LOADS];
  // Loads are fenced from the scheduler: left alone it sinks them next to
  // their use to shorten register live ranges, which undoes the prefetch.
  auto load_block = [&](u32x4_t (&dst)[G::LOADS], const unsigned char* pool, int ph) {
    const unsigned char* base = pool + (size_t)ph * block_bytes;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int l = 0; l < G::LOADS; ++l) dst[l] = load16(base + l * load_step);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto rl = [&](int v, int j) { return clampi(__builtin_amdgcn_readlane(v, j), 0, nmax); };

  auto body = [&](u32x4_t (&kcur)[G::LOADS], u32x4_t (&vcur)[G::LOADS], int kb, int ph_ahead) {
    // scores: partial dots of this lane's chunk, then reduce-scatter along the row
    float part[G::NCOMB];
#pragma unroll
    for (int l = 0; l < G::LOADS; ++l)
#pragma unroll
      for (int g = 0; g < GW; ++g) part[l * GW + g] = chunk_dot4<ET>(kcur[l], qreg[g], 0.f);
    load_block(kcur, kpool, ph_ahead);
    const float sc = reduce_scatter<G::NC>(part, c);
    const int tok = kb * kBS + lc * G::RPL + tg;
    const bool valid = tok < hi;
    const float s2 = valid ? sc * scale_log2e : kNegInf;
    if (__builtin_amdgcn_ballot_w64(s2 > m_lane + kSlack)) {
      const float m_new = fmaxf(m_lane, head_reduce<G::NC, GW, G::KW, true>(s2));
      // 1 while a head is still empty (both -inf), 0 on its first key
      const float alpha = m_lane == m_new ? 1.f : __builtin_amdgcn_exp2f(m_lane - m_new);
      l_part *= alpha;
      m_lane = m_new;
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        const float ag = __shfl(alpha, grp * G::NC + g);
#pragma unroll
        for (int e = 0; e < G::EC; ++e) acc[g][e] *= ag;
      }
    }
    const float p = valid ? __builtin_amdgcn_exp2f(s2 - m_lane) : 0.f;
    l_part += p;
    // acc += p * V; V of tokens past the end is zeroed (never multiply poison by 0)
#pragma unroll
    for (int l = 0; l < G::LOADS; ++l) {
      const bool vvalid = kb * kBS + l * G::RPL + tg < hi;
      const u32x4_t vz{0u, 0u, 0u, 0u};
      float vf[G::EC];
      widen<ET>(vvalid ? vcur[l] : vz, vf);
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        const float pb = group_bcast<G::NC>(p, l * GW + g, upper_half);
#pragma unroll
        for (int e = 0; e < G::EC; ++e) acc[g][e] = fmaf(pb, vf[e], acc[g][e]);
      }
    }
    load_block(vcur, vpool, ph_ahead);
  };

#pragma unroll
  for (int s = 0; s < PD; ++s) {
    const int ph = rl(cphys, s);
    load_block(kbuf[s], kpool, ph);
    load_block(vbuf[s], vpool, ph);
  }

  auto step = [&](u32x4_t (&kb)[G::LOADS], u32x4_t (&vb)[G::LOADS], int ii, int ph_ahead) {
    const int fl = __builtin_amdgcn_readlane(cflags, ii);
    if (fl & 1) begin_unit();
    body(kb, vb, Fc + ii + kb_off, ph_ahead);
    if (fl & 2) end_unit();
  };

  while (true) {
    if (has_next) {   // a full chunk of 64 blocks with another one after it
#pragma unroll
      for (int ii = 0; ii < kResolveAt; ii += PD)
#pragma unroll
        for (int s = 0; s < PD; ++s) step(kbuf[s], vbuf[s], ii + s, rl(cphys, ii + s + PD));
      const int wnext = resolve(Fc + 64, wbase, wv, wue, nphys, nflags);
      for (int ii = kResolveAt; ii < 64 - PD; ii += PD)
#pragma unroll
        for (int s = 0; s < PD; ++s) step(kbuf[s], vbuf[s], ii + s, rl(cphys, ii + s + PD));
#pragma unroll
      for (int s = 0; s < PD; ++s) step(kbuf[s], vbuf[s], 64 - PD + s, rl(nphys, s));
      Fc += 64;
      cphys = nphys;
      cflags = nflags;
      wbase = wnext;
      has_next = Fc + 64 < F1;
      if (has_next) window(wbase, wv, wue);
    } else {
      // The last chunk: 1 .. 64 blocks; lanes past the end repeat the last
      // block.  A pad step (cnt odd with PD = 2) has no unit events and runs
      // after the range's last unit has been stored, so it only touches dead
      // state; it keeps the load count per step constant.
      const int cnt = F1 - Fc;
      for (int i = 0; i < cnt; i += PD) {
#pragma unroll
        for (int s = 0; s < PD; ++s) step(kbuf[s], vbuf[s], i + s, rl(cphys, min(i + s + PD, 63)));
      }
      break;
    }
  }
  finish_empty();
}

// ---------------------------------------------------------------------------
// Merge the pieces of units cut by wave ranges.
// ---------------------------------------------------------------------------
// Only units cut by range boundaries need a merge, and each
// boundary cuts at most one unit: the one containing the boundary's first
// block.  Workgroup (r, j) merges that unit for head groups 4j .. 4j+3 when
// the unit begins in range r - 1 (its first cut), one wave per head group;
// the plan left that decision and the unit's ranges in mdesc[r].
// Units with nothing visible were written by the plan.
template <typename ET, int D>
__global__ __launch_bounds__(256) void boundary_merge_kernel(StreamArgs sa) {
  const DecodeArgs& a = sa.a;
  const int lane = threadIdx.x & 63;
  const int U = a.Hq / kHPW;
  const int nj = (U + 3) / 4;
  const int r = blockIdx.x / nj + 1;
  const int u = (blockIdx.x % nj) * 4 + (threadIdx.x >> 6);
  if (u >= U) return;
  const int4 md = sa.mdesc[r];   // {unit, first range, last range}; x < 0: nothing to merge here
  if (md.x < 0) return;
  merge_pieces<ET, D, 8>(a, sa.part, md.x, u, md.y, md.z, lane);
}

template <typename ET, int D, int GW>
hipError_t launch_s(StreamArgs sa, hipStream_t stream) {
  constexpr int LOADS = SGeo<ET, D, GW>::LOADS;
  // One block ahead per wave: with the block stream running across unit
  // boundaries this measured faster than two (8B- and 1B-shaped batches) and
  // needs 60 fewer VGPRs.
  constexpr int PD = 1;
  (void)LOADS;
  const float sl2 = sa.a.scale * kLog2e;
  const int U = sa.a.Hq / kHPW;
  const int wpg = U < kMaxU ? U : kMaxU;
  sa.stream_wgs = sa.ranges * (U / wpg);
  using LD = StreamLds<ET, D, GW>;
  const size_t qbytes = (size_t)wpg * LD::QWAVE;
  if (sa.inl)
    hipLaunchKernelGGL((stream_decode_kernel<ET, D, GW, PD, true>), dim3(sa.stream_wgs), dim3(64 * wpg),
                       qbytes + (size_t)kInlineUnitsPerWave * wpg * sizeof(int4), stream, sa, sa.udesc, sl2);
  else
    hipLaunchKernelGGL((stream_decode_kernel<ET, D, GW, PD, false>), dim3(sa.stream_wgs), dim3(64 * wpg), qbytes,
                       stream, sa, sa.udesc, sl2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (sa.ranges > 1) {
    hipLaunchKernelGGL((boundary_merge_kernel<ET, D>), dim3((sa.ranges - 1) * ((U + 3) / 4)), dim3(256), 0, stream, sa);
  }
  return hipGetLastError();
}

template <typename ET, int D>
hipError_t launch_sd(const StreamArgs& sa, hipStream_t stream) {
  const int G = sa.a.Hq / sa.a.Hkv;
  if (G >= 4) return launch_s<ET, D, 4>(sa, stream);
  if (G == 2) return launch_s<ET, D, 2>(sa, stream);
  return launch_s<ET, D, 1>(sa, stream);
}

hipError_t launch_main(const StreamArgs& sa, hipStream_t stream) {
  if (sa.a.bf16) return sa.a.D == 64 ? launch_sd<Bf16, 64>(sa, stream) : launch_sd<Bf16, 128>(sa, stream);
  return launch_sd<float, 64>(sa, stream);
}

}  // namespace

hipError_t launch_plan(const int32_t* lens, int B, int T, int ranges, int max_blocks, int* hdr, int* prefix, int* first,
                       int4* udesc, hipStream_t stream, const PlanFinish* fin, int4* mdesc) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, lens, B, T, ranges, max_blocks, B * T, hdr,
                     prefix, first, udesc, mdesc, fin ? *fin : PlanFinish{}, fin != nullptr);
  return hipGetLastError();
}

// LDS of the inline-plan decode launch: staged queries plus the unit list.
static size_t inline_lds_bytes(const DecodeArgs& a, int wpg) {
  const int G = a.Hq / a.Hkv;
  const int GW = G >= 4 ? 4 : (G == 2 ? 2 : 1);
  const int EB = a.bf16 ? 2 : 4;
  const int NC = a.D * EB / 16, KW = kHPW / GW;
  return (size_t)wpg * kStage * GW * NC * KW * 16 + (size_t)kInlineUnitsPerWave * wpg * sizeof(int4) + 256;
}

int stream_ranges(int Hq) { return kWaves / (Hq >= kHPW ? Hq / kHPW : 1); }

size_t stream_workspace_bytes(int B, int T, int Hq, int D) {
  const size_t TB = (size_t)B * T;
  const size_t R = (size_t)stream_ranges(Hq);
  size_t off = 256;                                       // header
  off += ((TB + 1) * 4 + 255) / 256 * 256;                // prefix
  off += (R * 4 + 255) / 256 * 256;                       // first unit per range
  off += R * 16;                                          // merge descriptor per boundary
  off += ((TB + 1) * 16 + 255) / 256 * 256;               // unit descriptors
  off += (R + TB) * Hq * (D + 1) * 4;                     // partial slots
  return (off + 255) / 256 * 256;
}

bool stream_supported(const DecodeArgs& a) {
  // rows of 8 or 16 lanes: bf16 D in {64,128}, fp32 D = 64
  const bool rows_ok = a.bf16 || a.D == 64;
  const int U = a.Hq / kHPW;
  return rows_ok && (U <= kMaxU || U % kMaxU == 0) && (long long)a.B * a.T <= kStreamMaxTB &&
         (long long)a.B * a.T * a.max_blocks < (1ll << 30);
}

hipError_t launch_decode_stream(const DecodeArgs& a, void* workspace, hipStream_t stream) {
  StreamArgs sa{};
  sa.a = a;
  sa.TB = a.B * a.T;
  sa.ranges = stream_ranges(a.Hq);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  int* hdr = reinterpret_cast<int*>(ws);
  int* prefix = reinterpret_cast<int*>(ws + 256);
  int* first = reinterpret_cast<int*>(ws + 256 + ((size_t)(sa.TB + 1) * 4 + 255) / 256 * 256);
  int4* mdesc = reinterpret_cast<int4*>(reinterpret_cast<unsigned char*>(first) +
                                        ((size_t)sa.ranges * 4 + 255) / 256 * 256);
  int4* udesc = mdesc + sa.ranges;
  float* part = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(udesc) +
                                         ((size_t)(sa.TB + 1) * 16 + 255) / 256 * 256);
  sa.hdr = hdr; sa.prefix = prefix; sa.first = first; sa.mdesc = mdesc; sa.udesc = udesc; sa.part = part;
  const int U = a.Hq / kHPW;
  const int wpg = U < kMaxU ? U : kMaxU;
  // the plan is computed inside the decode kernel when the unit list fits in
  // its LDS, else by a planning launch first
  sa.inl = sa.TB + 1 <= kInlineUnitsPerWave * wpg && inline_lds_bytes(a, wpg) <= (size_t)device_lds_per_block();
  const PlanFinish fin{a.out, a.lse_out, a.Hq, a.D, a.bf16};
  const hipError_t e = sa.inl ? hipSuccess
                              : launch_plan(a.context_lens, a.B, a.T, sa.ranges, a.max_blocks, hdr, prefix, first,
                                            udesc, stream, &fin, mdesc);
  if (e != hipSuccess) return e;
  return launch_main(sa, stream);
}

}  // namespace pkv
