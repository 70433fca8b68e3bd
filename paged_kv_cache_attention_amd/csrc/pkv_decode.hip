// Paged decode attention, VALU path (gfx950).
//
// One work item = (sequence b, query token t, group of 4 query heads u,
// split-KV partition p).  A workgroup of NW waves runs one work item; the
// partition's 16-token blocks are dealt round-robin to the waves.  Per block a
// wave:
//   1. gathers the block's K and V rows for its KV head(s) from the pool with
//      16-byte loads (the block's physical id comes from the block table;
//      "Inference From Scratch", ch. 10 paged attention),
//   2. stages K through LDS (XOR-swizzled rows) so that lane (head, token)
//      can dot its query row with one key row -- the key row is read once
//      and serves every query head of the KV group (GQA, "The Project", M2),
//   3. keeps an online softmax per query head ("Inference From Scratch",
//      ch. 8): a running maximum m (base-2 units, scale*log2(e) folded in),
//      a running denominator and accumulator; m is only raised when a block
//      maximum exceeds it by more than 8, so rescaling is rare and every
//      exponent stays <= 2^8,
//   4. accumulates p * V in fp32 straight from the V registers.
// At the end the waves' (m, l, acc) states are merged through LDS.  A work
// item whose sequence has a single partition writes the final output; other
// work items write a normalised partial and its log-sum-exp for lse_reduce.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kBS = 16;            // tokens per block (the only supported block size)
constexpr int kHeadsPerWave = 4;   // query heads handled by one wave
constexpr float kRescaleSlack = 8.0f;

template <typename ET, int D, int GW, int NW>
struct Geo {
  static constexpr int EB = Storage<ET>::bytes;
  static constexpr int EC = 16 / EB;               // elements per 16-byte chunk
  static constexpr int RB = D * EB;                // bytes of one (token, KV head) row
  static constexpr int NC = RB / 16;               // chunks per row
  static constexpr int KW = kHeadsPerWave / GW;    // KV heads read by one wave
  static constexpr int TILE = kBS * KW * RB;       // bytes of one block for those heads
  static constexpr int LOADS = TILE / (64 * 16);   // 16-byte loads per lane per block
  static constexpr int RPL = 64 / (NC * KW);       // tokens per wave load and KV head
  static constexpr int QW = D * EB / 4;            // 32-bit words of one query row
  static constexpr int ROWS_PER_LINE = RB >= 256 ? 1 : 256 / RB;
  static constexpr int WAVE_LDS = TILE + kBS * kHeadsPerWave * 4 + kHeadsPerWave * 4;
  static constexpr int MERGE_LDS = NW * 64 * GW * EC * 4 + NW * 2 * kHeadsPerWave * 4;
  static constexpr int LDS = WAVE_LDS * NW > MERGE_LDS ? WAVE_LDS * NW : MERGE_LDS;
  static_assert(NC * KW <= 64, "one wave load must cover whole rows");
  static_assert(LOADS * 64 * 16 == TILE, "a block must split evenly over the wave");
};

// Physical 16-byte chunk of logical chunk c in LDS row `row`: XOR with the
// row's position so that 16 lanes reading chunk c of 16 rows hit 16 banks.
template <int NC, int ROWS_PER_LINE>
__device__ __forceinline__ int swz(int c, int row) {
  return c ^ ((row / ROWS_PER_LINE) & (NC - 1));
}

__device__ __forceinline__ void lds_order() { __asm__ volatile("" ::: "memory"); }

// q . k over one 16-byte chunk.
template <typename ET> __device__ __forceinline__ float chunk_dot(u32x4_t k, const uint32_t* q, float acc);
template <> __device__ __forceinline__ float chunk_dot<Bf16>(u32x4_t k, const uint32_t* q, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(k.x), as_bf16x2(q[0]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(k.y), as_bf16x2(q[1]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(k.z), as_bf16x2(q[2]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(k.w), as_bf16x2(q[3]), acc, false);
  return acc;
}
template <> __device__ __forceinline__ float chunk_dot<float>(u32x4_t k, const uint32_t* q, float acc) {
  acc = fmaf(__uint_as_float(k.x), __uint_as_float(q[0]), acc);
  acc = fmaf(__uint_as_float(k.y), __uint_as_float(q[1]), acc);
  acc = fmaf(__uint_as_float(k.z), __uint_as_float(q[2]), acc);
  acc = fmaf(__uint_as_float(k.w), __uint_as_float(q[3]), acc);
  return acc;
}

// Widen one 16-byte chunk of V to fp32.
template <typename ET> __device__ __forceinline__ void chunk_widen(u32x4_t v, float* f);
template <> __device__ __forceinline__ void chunk_widen<Bf16>(u32x4_t v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}
template <> __device__ __forceinline__ void chunk_widen<float>(u32x4_t v, float* f) {
  f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y); f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}

constexpr int PD = 2;   // blocks in flight per wave

template <typename ET, int D, int GW, int NW>
__global__ __launch_bounds__(64 * NW) void decode_valu_kernel(DecodeArgs a, float scale_log2e, uint32_t n_items) {
  using G = Geo<ET, D, GW, NW>;
  using ST = typename Storage<ET>::T;
  __shared__ __attribute__((aligned(16))) unsigned char smem[G::LDS];

  const uint32_t lam = xcd_logical_id(blockIdx.x, 16);
  if (lam >= n_items) return;
  const int U = a.Hq / kHeadsPerWave;
  const int b = (int)(lam % (uint32_t)a.B);
  uint32_t r = lam / (uint32_t)a.B;
  const int u = (int)(r % (uint32_t)U);
  r /= (uint32_t)U;
  const int t = (int)(r % (uint32_t)a.T);
  const int p = (int)(r / (uint32_t)a.T);

  const int L = clampi(a.context_lens[b], 0, a.max_blocks * kBS);
  const int PT = a.part_tokens;
  const int Pb = L > PT ? (L + PT - 1) / PT : 1;
  if (p >= Pb) return;
  const int n_vis = L - a.T + t + 1;             // keys visible to query token t
  const int lo = p * PT;
  const int hi = min(lo + PT, n_vis);
  const int nblk = hi > lo ? (hi - lo + kBS - 1) / kBS : 0;
  const bool direct = (Pb == 1);

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index, uniform
  const int h0 = u * kHeadsPerWave;
  const int kv0 = h0 / (a.Hq / a.Hkv);

  // QK roles: lane = (hl, tq) -- query head hl of the group, token tq of the block.
  const int hl = lane >> 4, tq = lane & 15;
  const int q_row = tq * G::KW + hl / GW;
  // PV / load roles: lane = (token group tg, KV head kl, chunk c).
  const int c = lane % G::NC;
  const int grp = lane / G::NC;
  const int kl = grp % G::KW;
  const int tg = grp / G::KW;

  uint32_t qw[G::QW];
  {
    const unsigned char* qp = reinterpret_cast<const unsigned char*>(static_cast<const ST*>(a.q) +
                                                                     ((size_t)(b * a.T + t) * a.Hq + h0 + hl) * D);
#pragma unroll
    for (int i = 0; i < G::QW / 4; ++i) {
      const u32x4_t v = load16(qp + 16 * i);
      qw[4 * i + 0] = v.x; qw[4 * i + 1] = v.y; qw[4 * i + 2] = v.z; qw[4 * i + 3] = v.w;
    }
  }

  unsigned char* ktile = smem + wv * G::WAVE_LDS;
  float* pbuf = reinterpret_cast<float*>(ktile + G::TILE);   // [16 tokens][4 heads]
  float* abuf = pbuf + kBS * kHeadsPerWave;                   // [4 heads]

  const size_t block_bytes = (size_t)kBS * a.Hkv * G::RB;
  const uint32_t lane_off = (uint32_t)(((tg * a.Hkv) + kv0 + kl) * G::RB + c * 16);
  const uint32_t load_step = (uint32_t)(G::RPL * a.Hkv * G::RB);
  const unsigned char* kpool = static_cast<const unsigned char*>(a.k_pool) + lane_off;
  const unsigned char* vpool = static_cast<const unsigned char*>(a.v_pool) + lane_off;

  // This wave's blocks: j = wv + NW*i, i < nb, taken in chunks of 64 whose
  // table entries sit one per lane.
  const int nb = nblk > wv ? (nblk - wv + NW - 1) / NW : 0;
  const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks + lo / kBS + wv;
  const int nmax = a.N_blocks - 1;

  float m_run = kNegInf;   // per query head, base-2 units
  float l_part = 0.f;      // this lane's share of the denominator
  float acc[GW][G::EC];
#pragma unroll
  for (int g = 0; g < GW; ++g)
#pragma unroll
    for (int e = 0; e < G::EC; ++e) acc[g][e] = 0.f;

  // Software pipeline of depth PD: while block i is processed, K and V of
  // blocks i+1 .. i+PD are in flight in registers.  The loop is unrolled by
  // PD so the buffers rotate without copies; prefetches past the last block
  // re-read the current block (an L2 hit) so no load is conditional, and the
  // trip count is padded to a multiple of PD with fully masked steps.
  u32x4_t* ktile16 = reinterpret_cast<u32x4_t*>(ktile);
  u32x4_t kbuf[PD][G::LOADS], vbuf[PD][G::LOADS];
  int tbl = 0, cn = 0;
  auto load_block = [&](u32x4_t (&dst)[G::LOADS], const unsigned char* pool, int ph) {
    const unsigned char* base = pool + (size_t)ph * block_bytes;
#pragma unroll
    for (int l = 0; l < G::LOADS; ++l) dst[l] = load16(base + l * load_step);
  };
  auto phys = [&](int i) { return __builtin_amdgcn_readlane(tbl, i < cn ? i : cn - 1); };

  auto body = [&](u32x4_t (&kcur)[G::LOADS], u32x4_t (&vcur)[G::LOADS], int c0, int i) {
    const int kb = lo / kBS + wv + NW * (c0 + i);   // logical block
    const int ph_ahead = phys(i + PD);
    // 1. K rows of this block -> LDS, then refill the slot with block i+PD
#pragma unroll
    for (int l = 0; l < G::LOADS; ++l) {
      const int row = l * (64 / G::NC) + grp;
      ktile16[row * G::NC + swz<G::NC, G::ROWS_PER_LINE>(c, row)] = kcur[l];
    }
    load_block(kcur, kpool, ph_ahead);
    lds_order();
    // 2. scores: lane (hl, tq) dots its query row with key row tq
    float dot = 0.f;
#pragma unroll
    for (int cc = 0; cc < G::NC; ++cc)
      dot = chunk_dot<ET>(ktile16[q_row * G::NC + swz<G::NC, G::ROWS_PER_LINE>(cc, q_row)], qw + 4 * cc, dot);
    const int tok = kb * kBS + tq;
    const float s2 = tok < hi ? dot * scale_log2e : kNegInf;
    const float m_new = fmaxf(m_run, row16_max(s2));
    const bool need = m_new > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      m_run = need ? m_new : m_run;
      l_part *= alpha;
      if (tq == 0) abuf[hl] = alpha;
      lds_order();
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        const float al = abuf[kl * GW + g];
#pragma unroll
        for (int e = 0; e < G::EC; ++e) acc[g][e] *= al;
      }
    }
    const float pr = tok < hi ? __builtin_amdgcn_exp2f(s2 - m_run) : 0.f;
    l_part += pr;
    pbuf[tq * kHeadsPerWave + hl] = pr;
    lds_order();
    // 3. acc += p * V, then refill the V slot with block i+PD
    const bool partial = (kb + 1) * kBS > hi;
#pragma unroll
    for (int l = 0; l < G::LOADS; ++l) {
      const int tk = l * G::RPL + tg;
      u32x4_t vc = vcur[l];
      if (partial && kb * kBS + tk >= hi) vc = u32x4_t{0u, 0u, 0u, 0u};  // never multiply poison by 0
      float pv[GW];
#pragma unroll
      for (int g = 0; g < GW; ++g) pv[g] = pbuf[tk * kHeadsPerWave + kl * GW + g];
      float vf[G::EC];
      chunk_widen<ET>(vc, vf);
#pragma unroll
      for (int g = 0; g < GW; ++g)
#pragma unroll
        for (int e = 0; e < G::EC; ++e) acc[g][e] = fmaf(pv[g], vf[e], acc[g][e]);
    }
    load_block(vcur, vpool, ph_ahead);
    lds_order();
  };

  for (int c0 = 0; c0 < nb; c0 += 64) {
    cn = min(64, nb - c0);
    tbl = lane < cn ? clampi(trow[NW * (c0 + lane)], 0, nmax) : 0;
#pragma unroll
    for (int s = 0; s < PD; ++s) {
      load_block(kbuf[s], kpool, phys(s));
      load_block(vbuf[s], vpool, phys(s));
    }
    for (int i = 0; i < cn; i += PD) {
#pragma unroll
      for (int s = 0; s < PD; ++s) body(kbuf[s], vbuf[s], c0, i + s);
    }
  }

  // ---- merge the waves' softmax states and write ----
  const float l_row = row16_sum(l_part);
  __syncthreads();
  float* macc = reinterpret_cast<float*>(smem);                 // [NW][64][GW*EC]
  float* mstat = macc + NW * 64 * GW * G::EC;                    // [NW][2][4]
  {
    float* dst = macc + (wv * 64 + lane) * (GW * G::EC);
#pragma unroll
    for (int g = 0; g < GW; ++g)
#pragma unroll
      for (int e = 0; e < G::EC; e += 4)
        *reinterpret_cast<float4*>(dst + g * G::EC + e) = make_float4(acc[g][e], acc[g][e + 1], acc[g][e + 2], acc[g][e + 3]);
    if (tq == 0) {
      mstat[(wv * 2 + 0) * kHeadsPerWave + hl] = m_run;
      mstat[(wv * 2 + 1) * kHeadsPerWave + hl] = l_row;
    }
  }
  __syncthreads();
  using OT = typename Storage<ET>::T;
  for (int o = threadIdx.x; o < kHeadsPerWave * D; o += 64 * NW) {
    const int h2 = o / D, d = o % D;
    const int kl2 = h2 / GW, g2 = h2 % GW, c2 = d / G::EC, e2 = d % G::EC;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, mstat[(w * 2) * kHeadsPerWave + h2]);
    float lsum = 0.f, sum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = mstat[(w * 2) * kHeadsPerWave + h2];
      const float f = mw == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      lsum += f * mstat[(w * 2 + 1) * kHeadsPerWave + h2];
      float sw = 0.f;
#pragma unroll
      for (int rr = 0; rr < G::RPL; ++rr)
        sw += macc[(w * 64 + (rr * G::KW + kl2) * G::NC + c2) * (GW * G::EC) + g2 * G::EC + e2];
      sum += f * sw;
    }
    // lsum == 0 only when no key was visible; a NaN input stays NaN.
    const float ov = lsum != 0.f ? sum / lsum : 0.f;
    const float lse = lsum != 0.f ? (M + log2f(lsum)) * kLn2 : kNegInf;
    const size_t row = ((size_t)b * a.T + t) * a.Hq + h0 + h2;
    if (direct) {
      store_out<ET>(static_cast<OT*>(a.out) + row * D + d, ov);
      if (d == 0 && a.lse_out) a.lse_out[row] = lse;
    } else {
      a.part_out[(row * a.P_max + p) * D + d] = ov;
      if (d == 0) a.part_lse[row * a.P_max + p] = lse;
    }
  }
}

template <typename ET, int D, int GW>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  constexpr int NW = 4;
  const uint32_t n_items = (uint32_t)a.P_max * a.T * (a.Hq / kHeadsPerWave) * a.B;
  const uint32_t grid = (n_items + 127u) / 128u * 128u;
  const float sl2 = a.scale * kLog2e;
  hipLaunchKernelGGL((decode_valu_kernel<ET, D, GW, NW>), dim3(grid), dim3(64 * NW), 0, stream, a, sl2, n_items);
  return hipGetLastError();
}

template <typename ET, int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  if (G >= 4) return launch_t<ET, D, 4>(a, stream);
  if (G == 2) return launch_t<ET, D, 2>(a, stream);
  if constexpr (Storage<ET>::bytes * D <= 256) return launch_t<ET, D, 1>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_valu(const DecodeArgs& a, hipStream_t stream) {
  if (a.bf16) return a.D == 64 ? launch_d<Bf16, 64>(a, stream) : launch_d<Bf16, 128>(a, stream);
  return a.D == 64 ? launch_d<float, 64>(a, stream) : launch_d<float, 128>(a, stream);
}

}  // namespace pkv
