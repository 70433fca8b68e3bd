// Internal launcher interface between the C ABI (pkv_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Arguments of one paged-attention launch, already validated by the host.
struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  float* lse_out;
  float* part_out;  // [B, T, Hq, P_max, D] or nullptr when not split
  float* part_lse;  // [B, T, Hq, P_max]
  int B, T, Hq, Hkv, D, block_size, max_blocks, N_blocks;
  int part_tokens;  // tokens per partition (max_blocks * block_size when not split)
  int P_max;        // partitions per sequence upper bound (1 when not split)
  float scale;
  bool bf16;
};

// Balanced persistent VALU path: a fixed grid of kStreamWaves waves splits
// the flattened block list of all (head group, query token, sequence) units
// evenly; pieces of units cut by wave ranges are merged by a second kernel.
constexpr int kStreamWaves = 2048;   // 8 waves per CU of a 256-CU device
constexpr int kStreamMaxTB = 8192;   // B * T limit of the planning kernel
bool stream_supported(const DecodeArgs& a);
size_t stream_workspace_bytes(int B, int T, int Hq, int D);
hipError_t launch_decode_stream(const DecodeArgs& a, void* workspace, hipStream_t stream);

// Chunked-prefill attention (T up to kPrefillMaxT causal query rows per
// sequence, bf16) on MFMA tiles with LDS-staged keys and values.
constexpr int kPrefillMaxT = 8192;
constexpr int kPrefillTPW = 2;                  // 16-row MFMA tiles per wave
constexpr int kPrefillRows = 16 * kPrefillTPW * 4;   // query rows per work item (4 waves)
constexpr int kPrefillRowsWide = 16 * kPrefillTPW * 8;   // with key pieces at D = 128 (8 waves)
constexpr int kPrefillStep = 32;                // keys per staged step; pieces are multiples of it
constexpr int kPrefillMinPiece = 512;           // smallest piece the policy picks
// Key pieces per item for piece_tokens (1: no split).
int prefill_pieces(int max_blocks, int piece_tokens);
// Workspace for the partials of split items (0 when nothing splits).
size_t prefill_workspace_bytes(int B, int T, int Hq, int Hkv, int D, int max_blocks, int piece_tokens);
// Piece length the library suggests: 0 when the items already give every
// workgroup slot of the chip one, else the table's key bound cut into enough
// pieces for that.
int prefill_piece_tokens(int B, int T, int Hq, int Hkv, int D, int max_blocks, int cus);
// piece_tokens: 0 or a positive multiple of kPrefillStep; workspace holds
// prefill_workspace_bytes(...) bytes when that is nonzero.
hipError_t launch_prefill(const DecodeArgs& a, int piece_tokens, float* workspace, hipStream_t stream);

int device_lds_per_block();   // LDS bytes a workgroup may use on the current device (cached)
int device_cus();             // compute units of the current device (cached)

// VALU decode kernel: any T (one query token per work item), Hq/Hkv in {1,2,4,8}.
hipError_t launch_decode_valu(const DecodeArgs& a, hipStream_t stream);

// Planning kernel shared by the balanced paths: blocks per (t, b) pair with
// the causal limit of query token t, their prefix sums, the range length, the
// compact list of non-empty pairs (udesc, nu + 1 entries with a sentinel) and
// each range's first non-empty pair as an index into that list
// (B*T <= kStreamMaxTB).  hdr = {total, per range, total, 0, nu}.
// With `fin` the planning kernel also writes the result of every unit with
// no visible token (out = 0, lse = -inf), which no decode wave visits.
struct PlanFinish {
  void* out;         // [B, T, Hq, D]
  float* lse_out;    // [B, T, Hq] or null
  int Hq, D;
  bool bf16;
};
hipError_t launch_plan(const int32_t* lens, int B, int T, int ranges, int max_blocks, int* hdr, int* prefix, int* first,
                       int4* udesc, hipStream_t stream, const PlanFinish* fin = nullptr, int4* mdesc = nullptr);

// MFMA tile for bf16 with T * (Hq/Hkv) <= 16 query rows per KV head (the
// verify step, and single-token decode when verify_tile_for says so);
// balanced like the VALU path, with its own workspace layout.
bool verify_mfma_supported(const DecodeArgs& a);
// Whether paged_attention_decode (single pass) runs the MFMA tile for a.
bool verify_tile_for(const DecodeArgs& a);
size_t verify_workspace_bytes(int B, int T, int Hq, int D);
// Split-KV partitions on the tile (a.part_tokens > 0): bytes the workspace
// needs beyond the documented partials (plan and piece slots).
size_t verify_partition_extra_bytes(int B, int T, int Hq, int D);
// Single pass (a.part_tokens == 0) or split-KV partitions of a.part_tokens
// tokens (a.P_max per sequence): the workspace then starts with the partials
// [B, T, Hq, P_max, D] and [B, T, Hq, P_max].
hipError_t launch_verify_mfma(const DecodeArgs& a, void* workspace, hipStream_t stream);

// Log-sum-exp merge of split partials.  When `lens` is given, rows whose
// sequence has a single partition are skipped (the decode kernel wrote them).
hipError_t launch_lse_reduce(const float* part_out, const float* part_lse, void* out, float* lse_out,
                             int B, int T, int Hq, int D, int P_max, bool bf16, const int32_t* lens,
                             int part_tokens, hipStream_t stream);

hipError_t launch_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                         const int32_t* block_tables, const int32_t* lens_pre, int B, int T, int Hkv, int D,
                         int block_size, int max_blocks, int N_blocks, int elem_bytes, hipStream_t stream);
// KV append with RoPE fused in: rotates k_new (and q in place when given) at
// position lens_pre[b] + t, writes the rotated key and the value row.
hipError_t launch_copy_blocks(void* k_pool, void* v_pool, const int32_t* src, const int32_t* dst, int n, int Hkv,
                              int D, int block_size, int N_blocks, int elem_bytes, hipStream_t stream);
hipError_t launch_append_rope(void* q, int Hq, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                              const int32_t* block_tables, const int32_t* lens_pre, int B, int T, int Hkv, int D,
                              int block_size, int max_blocks, int N_blocks, double theta, bool bf16,
                              hipStream_t stream);

hipError_t launch_gather(const void* k_pool, const void* v_pool, const int32_t* block_tables,
                         const int32_t* lens, void* k_out, void* v_out, int B, int max_len, int Hkv, int D,
                         int block_size, int max_blocks, int N_blocks, int elem_bytes, hipStream_t stream);

// Device-side contract check (PKV_DEBUG): with L = lens[b] + len_add, sets
// *bad = 1 unless T <= L <= max_blocks*block_size and every table entry of the
// first ceil(L/block_size) blocks lies in [0, N_blocks).
hipError_t launch_validate(const int32_t* block_tables, const int32_t* lens, int B, int T, int len_add,
                           int block_size, int max_blocks, int N_blocks, int* bad, hipStream_t stream);

}  // namespace pkv
