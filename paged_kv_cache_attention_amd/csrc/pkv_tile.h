// A 16-row attention tile on MFMA (gfx950), shared by the multi-query verify
// kernel and the shared-prefix group kernel.
//
// One wave owns up to 16 query rows that read the same KV head.  Per 16-token
// block of the cache:
//   S^T[token][row] = K[token][:] . Q[row][:]      v_mfma_f32_16x16x32_bf16
//     A = K straight from 16-byte global loads (lane: token lane%16, d chunk
//     32c + 8*(lane/16)); B = Q^T from registers (same chunking).  The result
//     leaves row lane%16 and tokens 4*(lane/16) .. +3 in each lane.
//   online softmax per row (running max in base-2 units, raised lazily)
//   O[row][d] += P[row][token] . V[token][d]       v_mfma_f32_16x16x16_bf16
//     A = P in exactly the S^T layout, split into bf16 hi + lo parts so the
//     product keeps about 16 bits of P; B = V, loaded straight into an LDS
//     tile of the wave (global_load_lds_dwordx4, rows XOR-swizzled) and read
//     back transposed (ds_read_b64_tr_b16).
// K and V of the next PD blocks are in flight while a block is processed
// (K in registers, V in PD + 1 LDS tiles per wave).
#pragma once

#include "pkv_device.h"

namespace pkv {
namespace tile {

constexpr int kBS = 16;
// LDS bytes of the V tiles of one wave in run<D, PD>.
template <int D, int PD>
constexpr int run_tile_bytes() { return (PD + 1) * kBS * 2 * D; }
constexpr float kSlack = 8.f;

typedef __bf16 bf16x4_v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8_v as_bf16x8(u32x4_t v) {
  bf16x8_v r;
  __builtin_memcpy(&r, &v, sizeof(r));
  return r;
}
__device__ __forceinline__ uint32_t pack_bf16(uint16_t lo, uint16_t hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

// B operand of v_mfma_f32_16x16x16bf16_1k for column tile d of V (lane
// (row, quad) gets V[4 quad + k][16 d + row], k = 0..3) from a row-major LDS
// tile of 16 tokens, ROW bytes apart, with one ds_read_b64_tr_b16.  That
// read works on groups of 16 lanes: lane i of a group receives element i % 4
// of the 8-byte chunk addressed by lane 4 k + i / 4 of the group, for
// k = 0..3 (measured on gfx950 with an index-coded LDS tile).  So lane j of
// group quad addresses token 4 quad + j / 4, columns 16 d + 4 (j % 4) .. +3.
typedef short i16x4_v __attribute__((ext_vector_type(4)));
template <int ROW>
__device__ __forceinline__ bf16x4_v vt_operand(const unsigned char* tile, int d, int row, int quad) {
  const unsigned char* p = tile + (4 * quad + (row >> 2)) * ROW + (16 * d + 4 * (row & 3)) * 2;
  const i16x4_v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_v*)(const_cast<unsigned char*>(p)));
  bf16x4_v v;
  __builtin_memcpy(&v, &r, 8);
  return v;
}

// V tiles of run<D, PD>: 16 unpadded token rows of 2 D bytes, 16-byte chunk c
// of row r in slot c ^ vswz(r), so that the 4 rows x 2 chunks of one
// transposing read of a 16-lane group sit on 8 distinct 4-bank slots (at
// D = 64 a row covers half the banks and its parity picks the half).
template <int D>
__device__ __forceinline__ int vswz(int r) { return D == 128 ? 2 * (r & 3) : 2 * ((r >> 1) & 1); }

template <int D>
__device__ __forceinline__ bf16x4_v vt_operand_swz(const unsigned char* tile, int d, int row, int quad) {
  const int r = 4 * quad + (row >> 2);
  const unsigned char* p = tile + r * (2 * D) + (((2 * d + ((row & 3) >> 1)) ^ vswz<D>(r)) * 16) + 8 * (row & 1);
  const i16x4_v x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_v*)(const_cast<unsigned char*>(p)));
  bf16x4_v v;
  __builtin_memcpy(&v, &x, 8);
  return v;
}

// 16 bytes from global memory straight to LDS (global_load_lds_dwordx4):
// lane l of the wave writes lds_run + 16 l, lds_run being wave-uniform.
__device__ __forceinline__ void load_lds16(const void* g, unsigned char* lds_run) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_run, 16, 0, 0);
}

// s_waitcnt vmcnt(N) (no wait on the other counters): N of the wave's latest
// memory loads may still be in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | 0x0F70 | (N & 15));
}

template <int D>
struct State {
  floatx4_t acc[D / 16];   // O rows 4*(lane/16) + k, column 16*d + lane%16
  float m_row;             // running max of row lane%16 (base 2)
  float l_part;            // this lane's share of row lane%16's denominator
};

template <int D>
__device__ __forceinline__ void init(State<D>& st) {
#pragma unroll
  for (int d = 0; d < D / 16; ++d) st.acc[d] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  st.m_row = kNegInf;
  st.l_part = 0.f;
}

// Q^T operand of this lane's row: 16 bytes per MFMA step; rows outside the
// tile (row_ok false) read a safe row and are zeroed.
template <int D>
__device__ __forceinline__ void load_q(u32x4_t (&qreg)[D / 32], const uint16_t* qrow, bool row_ok, int lane) {
  const unsigned char* qp = reinterpret_cast<const unsigned char*>(qrow) + (lane >> 4) * 16;
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    const u32x4_t v = load16(qp + c * 64);
    qreg[c] = row_ok ? v : u32x4_t{0u, 0u, 0u, 0u};
  }
}

// Process logical blocks [kb0, kb0 + nb) whose physical ids are trow[0 .. nb).
// hi_row: keys of this lane's row with position < hi_row are visible.
// vlimit: V rows at positions >= vlimit are zeroed before use (they may hold
// poison, and p = 0 there).  kpool/vpool point at this lane's 16-byte chunk
// of token 0 of physical block 0 of the KV head.
template <int D, int PD>
__device__ __forceinline__ void run(State<D>& st, const u32x4_t (&qreg)[D / 32], int hi_row, int vlimit,
                                    const int32_t* trow, int kb0, int nb, int nmax, const unsigned char* kpool,
                                    const unsigned char* vhead, size_t kv_row_bytes, size_t block_bytes,
                                    unsigned char* vtiles, float scale_log2e, int lane) {
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int TILE = kBS * 2 * D;
  const int row = lane & 15, quad = lane >> 4;
  hi_row = min(hi_row, (kb0 + nb) * kBS);   // pad steps past the range stay masked
  u32x4_t kbuf[PD][KS];
  int tbl = 0, cn = 0;
  // V load c of a block: lane -> tile byte 1024 c + 16 lane = token row vr[c],
  // slot (chunk ^ vswz(row)); voff: that chunk's offset in a physical block
  int vr[KS];
  uint32_t voff[KS];
#pragma unroll
  for (int c = 0; c < KS; ++c) {
    const int pos = 1024 * c + 16 * lane;
    vr[c] = pos / (2 * D);
    voff[c] = (uint32_t)(vr[c] * kv_row_bytes + (((pos % (2 * D)) / 16) ^ vswz<D>(vr[c])) * 16);
  }
  auto load_v = [&](int t, int ph) {
    const unsigned char* base = vhead + (size_t)ph * block_bytes;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < KS; ++c) load_lds16(base + voff[c], vtiles + t * TILE + 1024 * c);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto load_block = [&](u32x4_t (&dst)[KS], const unsigned char* pool, int ph) {
    const unsigned char* base = pool + (size_t)ph * block_bytes;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < KS; ++c) dst[c] = load16(base + c * 64);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto phys = [&](int i) { return __builtin_amdgcn_readlane(tbl, i < cn ? i : cn - 1); };

  auto body = [&](u32x4_t (&kcur)[KS], int kb, int i) {
    const int ph_ahead = phys(i + PD);
    unsigned char* vtile = vtiles + (i % (PD + 1)) * TILE;
    floatx4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KS; ++c) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kcur[c]), as_bf16x8(qreg[c]), s, 0, 0, 0);
    load_block(kcur, kpool, ph_ahead);
    load_v((i + PD) % (PD + 1), ph_ahead);
    const int tok0 = kb * kBS + 4 * quad;
    float sv[4];
    bool need = false;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      sv[k] = tok0 + k < hi_row ? s[k] * scale_log2e : kNegInf;
      need |= sv[k] > st.m_row + kSlack;
    }
    if (__builtin_amdgcn_ballot_w64(need)) {
      float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(st.m_row, mx);
      // 1 for rows that are still empty (both -inf), 0 on a row's first key
      const float alpha = st.m_row == m_new ? 1.f : __builtin_amdgcn_exp2f(st.m_row - m_new);
      st.l_part *= alpha;
      st.m_row = m_new;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float ak = __shfl(alpha, 4 * quad + k);
#pragma unroll
        for (int d = 0; d < DT; ++d) st.acc[d][k] *= ak;
      }
    }
    uint16_t ph[4], pl[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float p = sv[k] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(sv[k] - st.m_row);
      st.l_part += p;
      ph[k] = f32_to_bf16_rne(p);
      pl[k] = f32_to_bf16_rne(p - __uint_as_float((uint32_t)ph[k] << 16));
    }
    bf16x4_v phi, plo;
    {
      const uint32_t h2[2] = {pack_bf16(ph[0], ph[1]), pack_bf16(ph[2], ph[3])};
      const uint32_t l2[2] = {pack_bf16(pl[0], pl[1]), pack_bf16(pl[2], pl[3])};
      __builtin_memcpy(&phi, h2, 8);
      __builtin_memcpy(&plo, l2, 8);
    }
    // this block's V has landed once the 2 KS PD loads issued after it are
    // all that may be in flight; rows at or past the length are then zeroed
    // (each lane the chunks it loaded: they may hold anything)
    wait_vmcnt<2 * KS * PD>();
    if ((kb + 1) * kBS > vlimit) {
#pragma unroll
      for (int c = 0; c < KS; ++c)
        if (kb * kBS + vr[c] >= vlimit) store16(vtile + 1024 * c + 16 * lane, u32x4_t{0u, 0u, 0u, 0u});
    }
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      const bf16x4_v bv = vt_operand_swz<D>(vtile, d, row, quad);
      st.acc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, bv, st.acc[d], 0, 0, 0);
      st.acc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, bv, st.acc[d], 0, 0, 0);
    }
    __asm__ volatile("" ::: "memory");
  };

  for (int c0 = 0; c0 < nb; c0 += 64) {
    cn = min(64, nb - c0);
    tbl = lane < cn ? clampi(trow[c0 + lane], 0, nmax) : 0;
    // the previous chunk's last steps prefetched pad blocks into the tiles:
    // let them land before the tiles are loaded again
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int s = 0; s < PD; ++s) {
      load_block(kbuf[s], kpool, phys(s));
      load_v(s, phys(s));
    }
    for (int i = 0; i < cn; i += PD) {
#pragma unroll
      for (int s = 0; s < PD; ++s) body(kbuf[s], kb0 + c0 + i + s, i + s);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // no load into the tiles outlives the call
}

// Same tile step with K and V already staged in LDS by the workgroup:
// nblk blocks, token row r (0 .. 16*nblk) at ks + r * ROW (K) and
// vs + r * ROW (V; rows past the last visible position zeroed by the
// stager).  kb0 is the logical index of the first staged block.  ROW = 2D + 16
// bytes keeps the row reads bank-conflict free.
template <int D, int ROW = 2 * D + 16>
__device__ __forceinline__ void run_lds(State<D>& st, const u32x4_t (&qreg)[D / 32], int hi_row, int kb0, int nblk,
                                        const unsigned char* ks, const unsigned char* vs, float scale_log2e,
                                        int lane) {
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  const int row = lane & 15, quad = lane >> 4;
  for (int j = 0; j < nblk; ++j) {
    const unsigned char* kr = ks + (j * kBS + row) * ROW + quad * 16;
    floatx4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KS; ++c) {
      const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(kr + c * 64);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kv), as_bf16x8(qreg[c]), s, 0, 0, 0);
    }
    const int tok0 = (kb0 + j) * kBS + 4 * quad;
    float sv[4];
    bool need = false;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      sv[k] = tok0 + k < hi_row ? s[k] * scale_log2e : kNegInf;
      need |= sv[k] > st.m_row + kSlack;
    }
    if (__builtin_amdgcn_ballot_w64(need)) {
      float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(st.m_row, mx);
      const float alpha = st.m_row == m_new ? 1.f : __builtin_amdgcn_exp2f(st.m_row - m_new);
      st.l_part *= alpha;
      st.m_row = m_new;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float ak = __shfl(alpha, 4 * quad + k);
#pragma unroll
        for (int d = 0; d < DT; ++d) st.acc[d][k] *= ak;
      }
    }
    uint16_t ph[4], pl[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float p = sv[k] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(sv[k] - st.m_row);
      st.l_part += p;
      ph[k] = f32_to_bf16_rne(p);
      pl[k] = f32_to_bf16_rne(p - __uint_as_float((uint32_t)ph[k] << 16));
    }
    bf16x4_v phi, plo;
    {
      const uint32_t h2[2] = {pack_bf16(ph[0], ph[1]), pack_bf16(ph[2], ph[3])};
      const uint32_t l2[2] = {pack_bf16(pl[0], pl[1]), pack_bf16(pl[2], pl[3])};
      __builtin_memcpy(&phi, h2, 8);
      __builtin_memcpy(&plo, l2, 8);
    }
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      const bf16x4_v bv = vt_operand<ROW>(vs + j * kBS * ROW, d, row, quad);
      st.acc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, bv, st.acc[d], 0, 0, 0);
      st.acc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, bv, st.acc[d], 0, 0, 0);
    }
  }
}

// Row totals after the range: l summed over the 4 lanes of each row.
template <int D>
__device__ __forceinline__ float row_sum(const State<D>& st) {
  float l = st.l_part + __shfl_xor(st.l_part, 16);
  return l + __shfl_xor(l, 32);
}

}  // namespace tile
}  // namespace pkv
