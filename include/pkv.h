/*
 * pkv.h -- C ABI of the paged KV-cache decode-attention library (libpkv.so).
 *
 * One decode step of causal attention over a paged KV cache on an AMD
 * Instinct MI355X (gfx950).  Each sequence's new query token(s) attend to
 * every cached key/value row of that sequence.  The cache lives in a pool
 * of fixed-size physical blocks; a per-sequence block table maps logical
 * block i of a sequence to a physical block of the pool ("Inference From
 * Scratch", chapter table, ch. 10 "Paged attention, block tables"; "The
 * Project: Serve Your Own LLM", M13, mini-vLLM with a paged KV cache).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every array argument is a DEVICE pointer to dense, row-major memory
 *    owned by the caller.  The library never allocates, frees or keeps any
 *    caller memory.  Scalars are passed by value.
 *  - q, out, k_pool, v_pool, k_new, v_new and the gather outputs are read
 *    and written with 16-byte vector accesses: each must be 16-byte aligned
 *    (device allocations are), else the call returns PKV_EINVAL.
 *  - Layouts (element type given by `dtype`):
 *      q, out         [B, T, Hq, D]
 *      k_pool, v_pool [N_blocks, block_size, Hkv, D]
 *      k_new, v_new   [B, T, Hkv, D]
 *      block_tables   int32 [B, max_blocks]
 *      context_lens   int32 [B]
 *      lse_out        float32 [B, T, Hq] (natural log), optional (NULL)
 *    Logical token j of sequence b is slot j % block_size of physical block
 *    block_tables[b][j / block_size].  Table entries past the last block a
 *    sequence needs are never read.
 *  - Grouped-query attention: query head h reads KV head h / (Hq / Hkv)
 *    ("The Project", M2: MHA/GQA/MQA chosen from the KV-cache budget).
 *  - Query token t of T sits at position L - T + t of its sequence (L =
 *    context_lens[b], which counts the T query tokens) and attends to
 *    positions 0 .. L - T + t: T = 1 is plain decode, T > 1 is the
 *    speculative-decoding verify step ("LLM Inference from Scratch", M7).
 *  - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *    Every launch is asynchronous on that stream; no call synchronises,
 *    except that PKV_DEBUG=1 in the environment (read once, at the first
 *    call) adds a device-side check of table entries and lengths, followed by
 *    a stream synchronisation.  No other environment variable is read: which
 *    kernels a call runs depends only on its arguments and the device.
 *  - Errors: argument errors are detected on the host before any launch and
 *    return a status; nothing is launched then.  Launch failures return
 *    PKV_EHIP.  pkv_last_error() gives a message for the last non-OK status
 *    of the calling thread.  No C++ exception crosses this interface.
 *  - Device-side contract, not checked unless PKV_DEBUG=1: T <= L <=
 *    max_blocks * block_size for every sequence and every table entry a
 *    sequence needs lies in [0, N_blocks).  Violations read or write outside
 *    the pool.
 *  - Supported shapes: block_size 16; D 64 or 128; Hq a multiple of Hkv and
 *    of 4; Hq / Hkv in {1, 2, 4, 8}; 1 <= T <= 16.  Others return
 *    PKV_EUNSUPPORTED rather than taking a slow path.  B = 0 is a no-op.
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = 1,        /* bad argument (null pointer, bad size, workspace too small) */
  PKV_EUNSUPPORTED = 2,  /* valid but outside the supported shape set */
  PKV_EWORKSPACE = 3,    /* workspace missing or smaller than pkv_decode_workspace_bytes */
  PKV_EHIP = 4           /* a HIP runtime call or kernel launch failed */
} pkv_status;

typedef enum {
  PKV_FP32 = 0, /* float32 storage; accumulation in float32 */
  PKV_BF16 = 1, /* bfloat16 storage; accumulation in float32, output rounded to nearest even */
  /* Not a dtype: makes every int value representable in a pkv_dtype, so that
   * the library can reject an unknown value (PKV_EINVAL) instead of receiving
   * a value outside the enumeration's range. */
  PKV_DTYPE_INT_RANGE_ = 0x7fffffff
} pkv_dtype;

/*
 * paged_kv_append -- write this step's new key/value rows into the cache.
 *
 * For every sequence b and t < T the row k_new[b][t] (and v_new[b][t]) is
 * copied to position p = context_lens_pre[b] + t, i.e. to slot p % block_size
 * of physical block block_tables[b][p / block_size].  This is the KV-cache
 * update of a decode step ("LLM Inference from Scratch", M1: past keys and
 * values are kept so decode only adds the new token's rows).  Only those
 * slots are written; the copy is exact (bytes are moved, not converted).
 *
 * context_lens_pre counts the tokens cached BEFORE the append; the library
 * does not update it (the caller passes context_lens_pre + T to attention).
 * The caller's allocator must already have put the target blocks in the
 * table.  Two (b, t) pairs must not address the same slot.
 */
pkv_status paged_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                           const int32_t* block_tables, const int32_t* context_lens_pre,
                           int B, int T, int Hkv, int D, int block_size, int max_blocks, int N_blocks,
                           pkv_dtype dtype, void* stream);

/*
 * paged_kv_gather -- diagnostic copy of each sequence's cached rows into a
 * contiguous buffer: out[b][j] = pool row of logical token j for j <
 * context_lens[b], zero for context_lens[b] <= j < max_len.  out is
 * [B, max_len, Hkv, D] for K and V each (k_out, v_out); the copy is exact.
 * This is the block-table gather that attention performs internally, exposed
 * so that its indexing can be checked bit for bit ("The Project", M10: a
 * paged_gather kernel).  Requires context_lens[b] <= max_len.
 */
pkv_status paged_kv_gather(const void* k_pool, const void* v_pool, const int32_t* block_tables,
                           const int32_t* context_lens, void* k_out, void* v_out,
                           int B, int max_len, int Hkv, int D, int block_size, int max_blocks, int N_blocks,
                           pkv_dtype dtype, void* stream);

/*
 * paged_kv_append_rope -- paged_kv_append with rotary position embedding
 * fused in ("LLM Inference from Scratch", Architecture overview: the decoder
 * is Llama-style with RoPE; "warpllama", Milestones: fused RoPE kernel).
 * New key t of sequence b is written to position p = context_lens_pre[b] + t
 * (same slot rule as paged_kv_append) rotated by its position: for each KV
 * head and i < D/2, with w_i = rope_theta^(-2i/D),
 *   k'[i]       = k[i] cos(p w_i) - k[i + D/2] sin(p w_i)
 *   k'[i + D/2] = k[i + D/2] cos(p w_i) + k[i] sin(p w_i)
 * (Llama's pairing of dimension i with i + D/2).  The value row is written
 * unchanged.  When q (the step's queries, [B, T, Hq, D], same dtype) is not
 * NULL it is rotated in place at the same positions; Hq is ignored otherwise.
 * Angles and rotations are computed in float64 and rounded once to the
 * storage type (round to nearest even).  k_new and v_new are not modified;
 * the target blocks must already be in the table.  rope_theta must be
 * finite and > 0 (PKV_EINVAL otherwise).
 */
pkv_status paged_kv_append_rope(void* q, int Hq, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                const int32_t* block_tables, const int32_t* context_lens_pre,
                                int B, int T, int Hkv, int D, int block_size, int max_blocks, int N_blocks,
                                float rope_theta, pkv_dtype dtype, void* stream);

/*
 * paged_kv_copy_blocks -- copy-on-write support for prefix caching
 * ("Inference From Scratch", Chapters table, ch. 10-11: block tables, and
 * prefix caching by hash-based block reuse across requests).  A sequence that
 * appends into a block other sequences also reference writes to a private
 * copy of it (this library's rule for reused, partly filled blocks): for
 * i < n, block dst[i] of both pools
 * becomes a byte copy of block src[i].  src and dst are device arrays of n
 * block ids; pairs with an id outside [0, N_blocks) are skipped; no id may be
 * both a source and a destination in one call.  n = 0 is a no-op.
 */
pkv_status paged_kv_copy_blocks(void* k_pool, void* v_pool, const int32_t* src, const int32_t* dst, int n,
                                int Hkv, int D, int block_size, int N_blocks, pkv_dtype dtype, void* stream);

/*
 * pkv_decode_workspace_bytes -- bytes of device workspace paged_attention_decode
 * needs for these sizes and this partition size.  With partition_size > 0 the
 * workspace starts with the split-KV partials, B*T*Hq*P_max*(D+1) float32
 * values where P_max = ceil(max_blocks * block_size / partition_size); the
 * MFMA tile adds its plan (a header and per-sequence prefix sums), one
 * normalised slot per (range, sequence) piece, at most
 * (2048*min(16, T*Hq) + B*T*Hq)*(D+1) float32 values, and two slots per range
 * for the pieces of partitions cut by range boundaries, at most
 * 2*2048*min(16, T*Hq)*(D+1) float32 values.  With partition_size = 0 the workspace holds the plan of the
 * balanced split (a header, per-unit prefix sums and descriptors) and one
 * normalised partial per (range, unit) piece: (ranges + B*T) * Hq * (D+1)
 * float32 values, where ranges = 2048 / (Hq/4) (256 at Hq = 32).  Returns 0
 * for invalid sizes.
 */
size_t pkv_decode_workspace_bytes(int B, int T, int Hq, int D, int max_blocks, int block_size,
                                  int partition_size);

/*
 * paged_attention_decode -- out = softmax(scale * q K^T + causal mask) V per
 * (sequence, query token, query head), with K and V read through the block
 * table ("Inference From Scratch", ch. 8 online softmax / flash attention and
 * ch. 10 paged attention; the result equals recomputing attention over the
 * full contiguous prefix).
 *
 * scale is normally 1/sqrt(D).  lse_out, when not NULL, receives the natural
 * log of the softmax denominator, log sum_j exp(scale * q.k_j).
 *
 * partition_size = 0 (the fast path) splits the whole batch evenly: the 16-token
 * blocks of all (sequence, query token) units are laid end to end and cut into
 * equal ranges, one per persistent workgroup, whatever the length mix.  A unit
 * inside one range is written straight to `out`; a unit cut by range
 * boundaries leaves one normalised partial per piece and a merge kernel
 * combines them by log-sum-exp weights.  Shapes: bf16 with D in {64, 128} or
 * fp32 with D = 64, Hq a multiple of 4 with Hq/4 <= 8 or a multiple of 8,
 * Hq/Hkv in {1, 2, 4, 8}, B*T <= 8192.  bf16 with D in {64, 128} and
 * T*Hq/Hkv <= 16 (with Hkv <= 8 or a multiple of 8) runs 16-row MFMA tiles
 * instead (the T*Hq/Hkv query rows of a KV head), split the same way, for
 * single-token decode and multi-query verify alike.  Other shapes run the
 * partitioned kernel below with one partition.
 * The partitioned path and the balanced path give results that agree within
 * rounding; each is deterministic: equal inputs give equal bits.
 * partition_size > 0 (a multiple of block_size) splits every sequence into
 * partitions of that many tokens starting at position 0; each partition
 * emits a normalised partial output and its log-sum-exp into `workspace`,
 * and a second kernel merges them as lse_reduce does ("Inference From
 * Scratch", Chapters table, ch. 8: softmax over pieces combines through the
 * running max and sum).  On the MFMA tile shapes the partitions are spread
 * over the balanced ranges above (a partition cut by a range boundary is
 * rebuilt from its pieces by the merge kernel); other shapes run one
 * workgroup per partition.  Sequences with one partition are written
 * straight to `out`.  After a split call, the workspace holds, for every
 * (b, t, h) whose sequence has P_b = ceil(L / partition_size) > 1
 * partitions, part_out [B, T, Hq, P_max, D] float32 at offset 0 followed by
 * part_lse [B, T, Hq, P_max] float32, valid for p < P_b; everything else in it
 * is unspecified.  A partition with no visible token for a query row has
 * part_lse = -inf and part_out = 0.
 *
 * out must not alias any input.  The workspace must be at least
 * pkv_decode_workspace_bytes(...) bytes of device memory (else PKV_EWORKSPACE);
 * it is overwritten by every call and two calls in flight at once need two
 * workspaces.
 */
pkv_status paged_attention_decode(const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  void* out, float* lse_out,
                                  int B, int T, int Hq, int Hkv, int D, int block_size, int max_blocks,
                                  int N_blocks, float scale, int partition_size,
                                  void* workspace, size_t workspace_bytes, pkv_dtype dtype, void* stream);

/*
 * paged_attention_decode_noalloc -- paged_attention_decode for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, layouts, kernels
 * and results as paged_attention_decode, without the workspace arguments: the
 * library works in a static device scratch of PKV_NOALLOC_SCRATCH_BYTES (plus
 * 256 bytes) that each GPU it runs on holds until the process ends.  Calls
 * whose pkv_decode_workspace_bytes(...) exceeds that return PKV_EWORKSPACE
 * before anything runs.  Nothing is allocated or freed, by the library or on
 * its behalf; the scratch's device address is looked up once per device, at
 * the first call on it.  Every call on one GPU shares that GPU's scratch, and
 * nothing in it needs clearing between calls (each call writes what it later
 * reads): two calls in flight at once on one GPU (other streams, other host
 * threads) race on it and give undefined results.  The partial layout that a
 * split call leaves at offset 0 of the workspace is not exposed here.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (64u << 20)
pkv_status paged_attention_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                          const int32_t* block_tables, const int32_t* context_lens,
                                          void* out, float* lse_out,
                                          int B, int T, int Hq, int Hkv, int D, int block_size, int max_blocks,
                                          int N_blocks, float scale, int partition_size, pkv_dtype dtype,
                                          void* stream);

/*
 * paged_attention_prefill -- chunked-prefill attention over the paged cache
 * ("Efficient LLM Inference", KV Caching: Verify Reuse, Positions and
 * Windows: attending a prompt chunk by chunk against the cached prefix equals
 * one pass over the whole prefix; "LLM Inference from Scratch", Architecture
 * overview, M1).  The T chunk tokens of sequence b have already been appended
 * (paged_kv_append), so context_lens[b] = L counts them; query t sits at
 * position L - T + t and attends causally to keys 0 .. L - T + t:
 *   out[b, t, h, :] = softmax_j(scale * q[b, t, h, :] . K_b[j, h / G, :]) V_b[j, h / G, :]
 * with G = Hq / Hkv.  Same layouts, ownership, lse_out and stream semantics as
 * paged_attention_decode.
 * Supported: bf16 only (PKV_EUNSUPPORTED for fp32), D in {64, 128},
 * Hq / Hkv in {1, 2, 4, 8}, 1 <= T <= 8192, block_size 16.  The device-side
 * contract T <= L <= max_blocks * block_size is the decode one (checked under
 * PKV_DEBUG=1).  Work is split into items of 128 query rows of one KV head
 * (256 at D = 128 when keys are split into pieces); K and V of the item's
 * visible keys are read once per item.
 *
 * piece_tokens = 0: every item is finished by the workgroup that owns it; the
 * workspace is not used (may be NULL).  piece_tokens > 0 (a multiple of 32)
 * also splits each item's keys into pieces of that many tokens from position
 * 0, one workgroup per piece, so that batches with few items (one sequence,
 * a long cached prefix) occupy the whole device.  Each piece of an item with
 * more than one leaves a normalised partial and its log-sum-exp in the
 * workspace, and a second kernel merges them as lse_reduce does; items that
 * fit in one piece are written directly.  The workspace must then hold
 * pkv_prefill_workspace_bytes(...) bytes (else PKV_EWORKSPACE), be 16-byte
 * aligned, and not overlap any other argument; its contents after the call
 * are unspecified, and two calls in flight need two workspaces.  Results with
 * and without pieces agree within rounding; each is deterministic.
 */
pkv_status paged_attention_prefill(const void* q, const void* k_pool, const void* v_pool,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   void* out, float* lse_out,
                                   int B, int T, int Hq, int Hkv, int D, int block_size, int max_blocks,
                                   int N_blocks, float scale, int piece_tokens,
                                   void* workspace, size_t workspace_bytes, pkv_dtype dtype, void* stream);

/* Workspace bytes paged_attention_prefill needs for these arguments (0 when
 * piece_tokens = 0 or no item can have more than one piece, and for
 * arguments it rejects). */
size_t pkv_prefill_workspace_bytes(int B, int T, int Hq, int Hkv, int D, int block_size, int max_blocks,
                                   int piece_tokens);

/* A piece length for paged_attention_prefill on the current device: 0 when
 * the B * ceil(T * Hq / Hkv / 128) * Hkv items already give every workgroup
 * slot one (two slots per CU at D = 128, four at D = 64), else the key bound
 * max_blocks * block_size cut into enough pieces for that (rounded up to a
 * multiple of 32, at least 512 tokens).  0 for arguments the prefill
 * rejects. */
int pkv_prefill_piece_tokens(int B, int T, int Hq, int Hkv, int D, int block_size, int max_blocks);

/*
 * lse_reduce -- merge P_max normalised partial attention results per row by
 * their log-sum-exp ("Inference From Scratch", ch. 8: softmax pieces over
 * disjoint key ranges combine through their running max and sum):
 *   M = max_p lse_p,  w_p = exp(lse_p - M),
 *   out = sum_p w_p part_out_p / sum_p w_p,  lse = M + log sum_p w_p.
 * part_out is float32 [B, T, Hq, P_max, D], part_lse float32 [B, T, Hq, P_max];
 * a partition with part_lse = -inf is empty and its part_out is never read.
 * A row whose partitions are all empty gets out = 0 and lse = -inf.  The
 * order of the sum over p is fixed, so results are deterministic.
 * out is [B, T, Hq, D] in out_dtype; lse_out (float32 [B, T, Hq]) may be NULL.
 */
pkv_status lse_reduce(const float* part_out, const float* part_lse, void* out, float* lse_out,
                      int B, int T, int Hq, int D, int P_max, pkv_dtype out_dtype, void* stream);

/* Message for the calling thread's last non-OK status ("" if none). */
const char* pkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
