// A 16-row attention tile on MFMA (gfx950): the multi-query verify kernel's
// walk over the cache blocks of one KV head.
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
//     product keeps about 16 bits of P; B = V, loaded into registers, written
//     to an LDS tile of the wave (rows XOR-swizzled) and read back transposed
//     (ds_read_b64_tr_b16).
// K and V of the next PD blocks are in flight while a block is processed.
#pragma once

#include "pkv_device.h"

namespace pkv {
namespace tile {

constexpr int kBS = 16;
constexpr float kSlack = 8.f;

typedef __bf16 bf16x4_v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef short i16x4_v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_v as_bf16x8(u32x4_t v) {
  bf16x8_v r;
  __builtin_memcpy(&r, &v, sizeof(r));
  return r;
}
__device__ __forceinline__ uint32_t pack_bf16(uint16_t lo, uint16_t hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

// B operand of v_mfma_f32_16x16x16bf16_1k for column tile d of V (lane
// (row, quad) gets V[4 quad + k][16 d + row], k = 0..3) from a row-major LDS
// tile of 16 tokens with one ds_read_b64_tr_b16.  That read works on groups
// of 16 lanes: lane i of a group receives element i % 4 of the 8-byte chunk
// addressed by lane 4 k + i / 4 of the group, for k = 0..3 (measured on
// gfx950 with an index-coded LDS tile).  So lane j of group quad addresses
// token 4 quad + j / 4, columns 16 d + 4 (j % 4) .. +3.
//
// LDS bytes of the wave's V tile in run<D, PD>.
template <int D>
constexpr int run_tile_bytes() { return kBS * 2 * D; }

// The V tile: 16 unpadded token rows of 2 D bytes, 16-byte chunk c
// of row r in slot c ^ vswz(r), so that the 4 rows x 2 chunks of one
// transposing read of a 16-lane group sit on 8 distinct 4-bank slots, and at
// D = 128 (a row is exactly the 64 banks) the neighbouring group, 4 rows
// further, on the other half of the banks (8B decode batch: 3.04 M LDS bank
// conflict cycles per call without that bit, 0.01 M with it; the call time
// is set by memory and did not move).  At D = 64 a row covers half the banks
// and its parity picks the half.
template <int D>
__device__ __forceinline__ int vswz(int r) {
  return D == 128 ? (2 * (r & 3)) | (8 * ((r >> 2) & 1)) : 2 * ((r >> 1) & 1);
}

// All D/16 V operands of one block (column tiles d = 0 .. D/16 - 1), read
// back to back in one asm block that also waits for them (lgkmcnt(0)) before
// it ends.  Issued as builtins, the compiler sent them one at a time, each
// waiting for the last, when registers ran short.
template <int D>
__device__ __forceinline__ void vt_operands_swz(bf16x4_v (&bv)[D / 16], const unsigned char* tile, int row,
                                                int quad) {
  constexpr int DT = D / 16;
  static_assert(DT == 4 || DT == 8, "D = 64 or 128");
  const int r = 4 * quad + (row >> 2);
  uint32_t ad[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d) {
    const unsigned char* p = tile + r * (2 * D) + (((2 * d + ((row & 3) >> 1)) ^ vswz<D>(r)) * 16) + 8 * (row & 1);
    ad[d] = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)(const_cast<unsigned char*>(p));
  }
  typedef uint32_t u32x2_v __attribute__((ext_vector_type(2)));
  u32x2_v x[DT];
  if constexpr (DT == 4) {
    __asm__ volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %5\n\t"
        "ds_read_b64_tr_b16 %2, %6\n\t"
        "ds_read_b64_tr_b16 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
        : "memory");
  } else {
    __asm__ volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\t"
        "ds_read_b64_tr_b16 %3, %11\n\t"
        "ds_read_b64_tr_b16 %4, %12\n\t"
        "ds_read_b64_tr_b16 %5, %13\n\t"
        "ds_read_b64_tr_b16 %6, %14\n\t"
        "ds_read_b64_tr_b16 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7])
        : "memory");
  }
#pragma unroll
  for (int d = 0; d < DT; ++d) __builtin_memcpy(&bv[d], &x[d], 8);
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
// poison, and p = 0 there).  kpool points at this lane's 16-byte chunk of
// token 0 of physical block 0 of the KV head, vhead at that block's head.
//
// V goes through registers and is written to the wave's one LDS tile
// (run_tile_bytes) by the wave itself, just before its block's P.V step.
// Loading it with global_load_lds instead measured no faster, and with LDS
// DMA in flight the compiler waits for every outstanding load before it uses
// any loaded register; through registers it counts the loads exactly.  One
// block ahead (PD = 1) measured faster than two: 216.5 against 219.0 us on
// the 8B shared-prefix decode batch, 431.6 against 441.3 us on the
// long-context verify batch.
//
// stream_v: V of a block is loaded with the non-temporal hint unless one of
// the neighbouring sequences in the batch (tables tprev, tnext: their rows at
// the same logical block, or nullptr) lists the same physical block.  K
// keeps the default policy.  Measured (interleaved A/B, us per call): 8B
// shared-prefix batch 215.8 -> 211.3, long-context verify 431.1 -> 386.0, a
// D = 64 batch of 64 sequences of 4000-8000 tokens 153.0 -> 136.5; the
// hint on every block instead cost the 8B batch its cached prefix re-reads
// (216.9 -> 248.6), and on K as well as V it was slower there (224.4).
// With pblocks > 0 the walk also cuts at every multiple of pblocks logical
// blocks: after the block that ends such a partition (if more blocks of the
// walk follow) it calls flush(st, kb_end), kb_end being the logical block the
// partition ends before; flush consumes st and leaves it initialised.  The
// loads of the next block are already in flight then.  The caller flushes
// the last partition after the walk.
struct NoFlush {
  template <typename S>
  __device__ void operator()(S&, int) const {}
};

template <int D, int PD, typename Flush = NoFlush>
__device__ __forceinline__ void run(State<D>& st, const u32x4_t (&qreg)[D / 32], int hi_row, int vlimit,
                                         const int32_t* trow, int kb0, int nb, int nmax, const unsigned char* kpool,
                                         const unsigned char* vhead, size_t kv_row_bytes, size_t block_bytes,
                                         unsigned char* vtile, float scale_log2e, int lane, int pblocks = 0,
                                         Flush flush = Flush(), bool stream_v = false,
                                         const int32_t* tprev = nullptr, const int32_t* tnext = nullptr) {
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  const int row = lane & 15, quad = lane >> 4;
  hi_row = min(hi_row, (kb0 + nb) * kBS);
  u32x4_t kbuf[PD][KS], vbuf[PD][KS];
  int tbl = 0, cn = 0;
  // V chunk c of a block: this lane's 16 bytes land at tile byte 1024 c + 16
  // lane = token row vr[c], slot (chunk ^ vswz(row)); voff: the chunk's
  // offset in a physical block
  int vr[KS];
  uint32_t voff[KS];
#pragma unroll
  for (int c = 0; c < KS; ++c) {
    const int pos = 1024 * c + 16 * lane;
    vr[c] = pos / (2 * D);
    voff[c] = (uint32_t)(vr[c] * kv_row_bytes + (((pos % (2 * D)) / 16) ^ vswz<D>(vr[c])) * 16);
  }
  uint64_t keep = 0;   // blocks of the table chunk whose V keeps the default cache policy
  // the loads of entry i of the table chunk (the last one past its end)
  auto load_kv = [&](u32x4_t (&kd)[KS], u32x4_t (&vd)[KS], int i) {
    const int e = i < cn ? i : cn - 1;
    const int ph = __builtin_amdgcn_readlane(tbl, e);
    const unsigned char* kb = kpool + (size_t)ph * block_bytes;
    const unsigned char* vb = vhead + (size_t)ph * block_bytes;
    __builtin_amdgcn_sched_barrier(0);
    if ((keep >> e) & 1) {
#pragma unroll
      for (int c = 0; c < KS; ++c) kd[c] = load16(kb + c * 64);
#pragma unroll
      for (int c = 0; c < KS; ++c) vd[c] = load16(vb + voff[c]);
    } else {
      // the empty asm keeps the two arms apart: merged, the loads lost the
      // non-temporal hint
      __asm__ volatile("" ::: "memory");
#pragma unroll
      for (int c = 0; c < KS; ++c) kd[c] = load16(kb + c * 64);
#pragma unroll
      for (int c = 0; c < KS; ++c) vd[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vb + voff[c]));
      __asm__ volatile("" ::: "memory");
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  auto body = [&](u32x4_t (&kcur)[KS], u32x4_t (&vcur)[KS], int kb, int i) {
    floatx4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KS; ++c) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kcur[c]), as_bf16x8(qreg[c]), s, 0, 0, 0);
    // this block's V into the tile; rows at or past the length zeroed (they
    // may hold anything, and p = 0 there).  The previous block's reads of
    // the tile came earlier in program order, and one wave's LDS operations
    // complete in order.
#pragma unroll
    for (int c = 0; c < KS; ++c) {
      const bool dead = kb * kBS + vr[c] >= vlimit;
      store16(vtile + 1024 * c + 16 * lane, dead ? u32x4_t{0u, 0u, 0u, 0u} : vcur[c]);
    }
    load_kv(kcur, vcur, i + PD);
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
    bf16x4_v bv[DT];
    vt_operands_swz<D>(bv, vtile, row, quad);
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      st.acc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, bv[d], st.acc[d], 0, 0, 0);
      st.acc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, bv[d], st.acc[d], 0, 0, 0);
    }
    if (pblocks > 0 && (kb + 1) % pblocks == 0 && kb + 1 < kb0 + nb) flush(st, kb + 1);
  };

  for (int c0 = 0; c0 < nb; c0 += 64) {
    cn = min(64, nb - c0);
    const int raw = lane < cn ? trow[c0 + lane] : -1;
    tbl = lane < cn ? clampi(raw, 0, nmax) : 0;
    bool kp = true;
    if (stream_v) {
      kp = (tprev && lane < cn && tprev[c0 + lane] == raw) || (tnext && lane < cn && tnext[c0 + lane] == raw);
    }
    keep = __builtin_amdgcn_ballot_w64(kp);
#pragma unroll
    for (int s = 0; s < PD; ++s) load_kv(kbuf[s], vbuf[s], s);
    for (int i = 0; i < cn; i += PD) {
#pragma unroll
      for (int s = 0; s < PD; ++s) body(kbuf[s], vbuf[s], kb0 + c0 + i + s, i + s);
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
