/*
 * pkv_engine -- host-side serving runtime over the paged cache: a block
 * manager with prefix caching and copy-on-write, and a continuous-batching
 * scheduler with recompute preemption ("Inference From Scratch", ch. 9
 * continuous batching, ch. 10 block tables, ch. 11 hash-based block reuse;
 * "The Project: Serve Your Own LLM", M13c: 16 requests, continuous batching,
 * a block pool smaller than the worst case so that preemption fires).
 *
 * The engine plans; the caller executes.  Each iteration:
 *   pkv_engine_schedule() returns a plan; the caller then, on the device,
 *     1. copies every block copy_src[i] -> copy_dst[i] (paged_kv_copy_blocks),
 *     2. for every planned request, appends the K/V of its `count` tokens at
 *        positions start .. start+count-1 (paged_kv_append or
 *        paged_kv_append_rope, lengths before the append = start),
 *     3. attends: prefill entries with paged_attention_prefill (T = count),
 *        decode entries with paged_attention_decode (T = 1), using the plan's
 *        block tables and context lengths (start + count),
 *     4. samples one next token per planned request from the output of its
 *        last position;
 *   pkv_engine_commit() takes those tokens in plan order.
 * A request finishes after max_new_tokens sampled tokens.  All pointers in a
 * plan stay valid until the next schedule call.  Host memory only; nothing
 * here touches a GPU.  The engine is not thread-safe.
 */
#ifndef PKV_ENGINE_H_
#define PKV_ENGINE_H_

#include <stdint.h>

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_engine pkv_engine;

typedef struct {
  int num_blocks;           /* physical blocks in the pool */
  int block_size;           /* tokens per block */
  int max_blocks_per_seq;   /* width of the plan's block tables */
  int max_running;          /* requests decoding at once */
  int max_prefill_tokens;   /* prefill tokens per iteration (the first admission may exceed it) */
  int enable_prefix_cache;  /* 0 or 1 */
  int pad_block;            /* table entry written past a request's blocks */
} pkv_engine_config;

enum { PKV_ENGINE_PREFILL = 0, PKV_ENGINE_DECODE = 1 };

typedef struct {
  int n;                        /* planned requests */
  const int64_t* request_id;    /* [n] */
  const int32_t* kind;          /* [n] PKV_ENGINE_PREFILL or PKV_ENGINE_DECODE */
  const int32_t* start;         /* [n] tokens already in the cache = first position to compute */
  const int32_t* count;         /* [n] tokens to compute (1 for decode) */
  const int32_t* token_offset;  /* [n + 1] offsets into tokens */
  const int32_t* tokens;        /* the token ids to compute, request after request */
  const int32_t* block_tables;  /* [n, max_blocks_per_seq] */
  const int32_t* context_lens;  /* [n] start + count */
  int max_blocks_per_seq;
  int n_copies;                 /* copy-on-write: block copies to run before the appends */
  const int32_t* copy_src;      /* [n_copies] */
  const int32_t* copy_dst;      /* [n_copies] */
  int n_preempted;              /* requests preempted by this plan (recomputed later) */
  const int64_t* preempted;     /* [n_preempted] */
} pkv_engine_plan;

typedef struct {
  int64_t iterations, preemptions, cow_copies, prefix_hit_tokens, computed_tokens, finished;
  int waiting, running, free_blocks, cached_blocks, cache_entries;
} pkv_engine_stats;

/* NULL when the configuration is invalid (a count below 1). */
pkv_engine* pkv_engine_create(const pkv_engine_config* config);
void pkv_engine_destroy(pkv_engine* engine);
/* Message for the last non-OK status of this engine. */
const char* pkv_engine_last_error(const pkv_engine* engine);
/* Queue a request (arrival order = call order).  PKV_EINVAL for a reused id,
 * an empty prompt, max_new_tokens < 1, or prompt_len + max_new_tokens beyond
 * max_blocks_per_seq * block_size. */
pkv_status pkv_engine_add_request(pkv_engine* engine, int64_t request_id, const int32_t* prompt, int prompt_len,
                                  int max_new_tokens);
/* Plan the next iteration (plan->n = 0 when nothing is left).  PKV_EINVAL if
 * the previous plan was not committed, or if a waiting request cannot fit in
 * the pool even alone. */
pkv_status pkv_engine_schedule(pkv_engine* engine, pkv_engine_plan* plan);
/* Commit the current plan with one sampled token per planned request. */
pkv_status pkv_engine_commit(pkv_engine* engine, const int32_t* next_tokens);
pkv_status pkv_engine_get_stats(const pkv_engine* engine, pkv_engine_stats* stats);
/* All tokens of a request (prompt, then generated); returns their number
 * (copies at most cap), -1 for an unknown id. */
int pkv_engine_request_tokens(const pkv_engine* engine, int64_t request_id, int32_t* tokens, int cap);
/* Reference count of a physical block (-1 when out of range). */
int pkv_engine_block_ref(const pkv_engine* engine, int block);

#ifdef __cplusplus
}
#endif

#endif /* PKV_ENGINE_H_ */
