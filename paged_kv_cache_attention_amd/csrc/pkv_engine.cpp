// Host-side serving runtime above the paged-attention kernels: a block
// manager with prefix caching and copy-on-write, and a continuous-batching
// scheduler with recompute preemption.
//
// Block manager ("Inference From Scratch", Chapters table, ch. 10 and ch. 11:
// block tables, prefix caching by hash-based block reuse across requests; the
// copy-on-write rule for shared, partly filled blocks is this library's own):
//   * a pool of num_blocks physical blocks, each with a reference count;
//   * a prefix cache mapping a block's content key to its physical block.
//     The key of logical block j of a sequence chains the key of block j - 1
//     with the token ids in block j (and their count, so a partly filled block
//     has a key of its own).  Slots are written once, in order, so a block
//     that once held n tokens keeps serving the key for those n tokens while
//     it stays allocated or cached;
//   * blocks whose count drops to zero stay cached (evictable, least recently
//     freed first) until a new allocation needs them;
//   * appending into a block that another sequence also references copies the
//     block first (the copy is part of the iteration plan: the caller runs it
//     on the device before the appends).
//
// Scheduler ("Inference From Scratch", ch. 9: iteration-level scheduling;
// "The Project", M13c: 16 requests, continuous batching, a block pool smaller
// than the worst case so that preemption fires):
//   * every iteration, each running request decodes one token; if the pool
//     cannot hold all of their next slots, the most recently arrived running
//     requests are preempted (blocks released, request back to the head of
//     the queue; it is recomputed from its known tokens on re-admission);
//   * waiting requests are then admitted in arrival order while blocks, the
//     running-request limit and the per-iteration prefill-token budget allow
//     (a request preempted in this iteration waits for the next one);
//     an admitted request prefills every token not served by the prefix cache
//     (at least its last token, whose output samples the next token).
#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <deque>
#include <list>
#include <memory>
#include <string>
#include <unordered_map>
#include <vector>

#include "pkv_engine.h"

namespace {

uint64_t mix64(uint64_t x) {   // splitmix64 finaliser
  x += 0x9e3779b97f4a7c15ull;
  x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
  x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
  return x ^ (x >> 31);
}

uint64_t block_key(uint64_t parent, const int32_t* tok, int n) {
  uint64_t h = mix64(parent ^ 0x51ed270b27b3c5a9ull) ^ (uint64_t)n;
  for (int i = 0; i < n; ++i) h = mix64(h ^ (uint32_t)tok[i]);
  return h;
}

constexpr uint64_t kRootKey = 0x243f6a8885a308d3ull;

class BlockManager {
 public:
  BlockManager(int num_blocks, int block_size, bool prefix_cache)
      : bs_(block_size), cache_on_(prefix_cache), ref_(num_blocks, 0), info_(num_blocks), in_lru_(num_blocks, false),
        lru_it_(num_blocks) {
    for (int b = num_blocks - 1; b >= 0; --b) free_.push_back(b);
  }

  int block_size() const { return bs_; }
  int num_blocks() const { return (int)ref_.size(); }
  int available() const { return (int)free_.size() + (int)lru_.size(); }
  int free_count() const { return (int)free_.size(); }
  int cached_count() const { return (int)lru_.size(); }
  int ref(int b) const { return ref_[b]; }
  int cache_entries() const { return indexed_; }

  // A new block for exclusive use (reference count 1); -1 when none is left.
  int allocate() {
    int b;
    if (!free_.empty()) {
      b = free_.back();
      free_.pop_back();
    } else if (!lru_.empty()) {   // evict the least recently freed cached block
      b = lru_.front();
      lru_.pop_front();
      in_lru_[b] = false;
      unindex(b);
    } else {
      return -1;
    }
    ref_[b] = 1;
    return b;
  }

  void retain(int b) {
    if (ref_[b] == 0 && in_lru_[b]) {
      lru_.erase(lru_it_[b]);
      in_lru_[b] = false;
    }
    ++ref_[b];
  }

  void release(int b) {
    if (--ref_[b] > 0) return;
    if (cache_on_ && info_[b].indexed) {
      lru_it_[b] = lru_.insert(lru_.end(), b);
      in_lru_[b] = true;
    } else {
      unindex(b);
      free_.push_back(b);
    }
  }

  // Cached block whose first n tokens are tok[0..n) after the chain key
  // `parent`, or -1.  Full blocks are found by their chained key, partly
  // used prefixes by (parent, first token) and a comparison of the contents.
  int lookup(uint64_t parent, const int32_t* tok, int n) const {
    if (!cache_on_ || n < 1) return -1;
    if (n == bs_) {
      auto it = full_.find(block_key(parent, tok, n));
      if (it == full_.end()) return -1;
      const Info& f = info_[it->second];
      return f.parent == parent && (int)f.content.size() == bs_ && std::equal(tok, tok + n, f.content.begin())
                 ? it->second : -1;
    }
    auto range = part_.equal_range(head_key(parent, tok[0]));
    for (auto it = range.first; it != range.second; ++it) {
      const Info& f = info_[it->second];
      if (f.parent == parent && (int)f.content.size() >= n && std::equal(tok, tok + n, f.content.begin()))
        return it->second;
    }
    return -1;
  }

  // Block b now holds tokens tok[0..n) after `parent` (n grows as the owner
  // appends; the first tokens never change while the block is allocated or
  // cached).
  void record(int b, uint64_t parent, const int32_t* tok, int n) {
    if (!cache_on_ || n < 1) return;
    Info& f = info_[b];
    if (!f.indexed) {
      f.parent = parent;
      f.content.clear();
      f.content.reserve(bs_);
      f.head = head_key(parent, tok[0]);
      part_.emplace(f.head, b);
      f.indexed = true;
      ++indexed_;
    }
    f.content.assign(tok, tok + n);
    if (n == bs_ && !f.full) {
      const uint64_t k = block_key(parent, tok, n);
      if (!full_.count(k)) {   // the first block with this content stays the cached one
        full_.emplace(k, b);
        f.full = true;
        f.full_key = k;
      }
    }
  }

 private:
  struct Info {
    bool indexed = false, full = false;
    uint64_t parent = 0, head = 0, full_key = 0;
    std::vector<int32_t> content;   // tokens in the block, in slot order
  };

  static uint64_t head_key(uint64_t parent, int32_t first) { return mix64(parent ^ ((uint64_t)(uint32_t)first << 1)); }

  void unindex(int b) {
    Info& f = info_[b];
    if (!f.indexed) return;
    auto range = part_.equal_range(f.head);
    for (auto it = range.first; it != range.second; ++it)
      if (it->second == b) {
        part_.erase(it);
        break;
      }
    if (f.full) full_.erase(f.full_key);
    f = Info{};
    --indexed_;
  }

  int bs_;
  bool cache_on_;
  std::vector<int> ref_;
  std::vector<Info> info_;
  std::vector<int> free_;
  std::list<int> lru_;
  std::vector<bool> in_lru_;
  std::vector<std::list<int>::iterator> lru_it_;
  std::unordered_map<uint64_t, int> full_;        // chained key of a full block -> block
  std::unordered_multimap<uint64_t, int> part_;   // (parent, first token) -> blocks
  int indexed_ = 0;
};

enum class State { kWaiting, kRunning, kFinished };

struct Request {
  int64_t id;
  int64_t arrival;
  std::vector<int32_t> tokens;   // prompt, then generated tokens
  int prompt_len;
  int max_new;
  int generated = 0;
  int computed = 0;              // tokens whose K/V are in the cache
  std::vector<int32_t> table;    // physical block per logical block
  std::vector<uint64_t> chain;   // key after each full block: chain[j] = key of blocks 0..j
  State state = State::kWaiting;
  int preemptions = 0;
};

}  // namespace

struct pkv_engine {
  pkv_engine(const pkv_engine_config& c) : cfg(c), bm(c.num_blocks, c.block_size, c.enable_prefix_cache != 0) {}

  pkv_engine_config cfg;
  BlockManager bm;
  std::vector<std::unique_ptr<Request>> all;
  std::unordered_map<int64_t, Request*> by_id;
  std::deque<Request*> waiting;    // arrival order (preempted requests go back in that order)
  std::vector<Request*> running;   // arrival order
  int64_t next_arrival = 0;
  std::string error;

  // the current plan
  std::vector<Request*> planned;
  std::vector<int64_t> p_id;
  std::vector<int32_t> p_kind, p_start, p_count, p_tok_off, p_tokens, p_tables, p_lens, p_src, p_dst;
  std::vector<int64_t> p_preempted;
  // Sources of this plan's block copies, released only once the plan is
  // complete: a source that dropped to no users mid-plan would be evictable,
  // and a later allocation of the same plan could take it as a copy
  // destination (the plan would then copy into a block it also copies from).
  std::vector<int> p_release;
  bool plan_open = false;
  pkv_engine_stats stats{};

  uint64_t parent_key(const Request& r, int j) const { return j == 0 ? kRootKey : r.chain[j - 1]; }

  void release_all(Request& r) {
    for (int b : r.table) bm.release(b);
    r.table.clear();
    r.chain.clear();
    r.computed = 0;
  }

  // Record the contents of the blocks that tokens [from_token, computed)
  // were written to, so later prompts can find them (a prompt ending
  // anywhere inside a block matches its first tokens).
  void register_blocks(Request& r, int from_token) {
    const int bs = bm.block_size();
    const int last = r.computed;   // tokens [0, last) are in the cache
    for (int j = from_token / bs; j * bs < last; ++j) {
      const int n = std::min(bs, last - j * bs);
      const uint64_t parent = parent_key(r, j);
      bm.record(r.table[j], parent, r.tokens.data() + j * bs, n);
      if (n == bs && (int)r.chain.size() == j) r.chain.push_back(block_key(parent, r.tokens.data() + j * bs, bs));
    }
  }

  // Slot for the token at position r.computed: a new block at a block
  // boundary, a private copy of a shared last block, or nothing.  Returns the
  // blocks it takes from the pool (0 or 1); with do_it false only counts.
  int prepare_slot(Request& r, bool do_it) {
    const int bs = bm.block_size();
    const int p = r.computed;
    if (p % bs == 0) {
      if (!do_it) return 1;
      const int b = bm.allocate();
      r.table.push_back(b);
      return 1;
    }
    const int last = r.table[p / bs];
    if (bm.ref(last) <= 1) return 0;
    if (!do_it) return 1;
    const int b = bm.allocate();
    p_src.push_back(last);
    p_dst.push_back(b);
    p_release.push_back(last);
    r.table[p / bs] = b;
    ++stats.cow_copies;
    return 1;
  }

  // Admission of r: reuse cached blocks for its known tokens (all but the
  // last, which is always computed), allocate the rest.  Returns false (and
  // changes nothing) when the pool cannot hold it.
  bool try_admit(Request& r, int budget_left, bool first) {
    const int bs = bm.block_size();
    const int len = (int)r.tokens.size();
    // longest cached prefix, block by block
    std::vector<int> hit;
    std::vector<uint64_t> chain;
    int cached = 0;
    uint64_t parent = kRootKey;
    while (cached < len - 1) {
      const int n = std::min(bs, len - 1 - cached);
      const int b = bm.lookup(parent, r.tokens.data() + cached, n);
      if (b < 0) break;
      hit.push_back(b);
      cached += n;
      if (n < bs) break;
      parent = block_key(parent, r.tokens.data() + cached - bs, bs);
      chain.push_back(parent);
    }
    const int todo = len - cached;
    if (!first && todo > budget_left) return false;
    const int nblocks = (len + bs - 1) / bs;
    // blocks from the pool: the missing ones, plus a private copy when the
    // first computed token lands in a shared (cached) partly used block
    int need = nblocks - (int)hit.size();
    const bool copy_partial = cached % bs != 0;
    if (copy_partial) ++need;
    // cached hits that sit in the evictable list stop being available
    int hits_evictable = 0;
    for (int b : hit)
      if (bm.ref(b) == 0) ++hits_evictable;
    if (bm.available() - hits_evictable < need) return false;
    for (int b : hit) bm.retain(b);
    r.table = hit;
    r.chain = chain;
    r.computed = cached;
    stats.prefix_hit_tokens += cached;
    if (copy_partial) {   // the shared block's first cached % bs slots are ours: copy, then write after them
      const int j = cached / bs;
      const int b = bm.allocate();
      p_src.push_back(r.table[j]);
      p_dst.push_back(b);
      p_release.push_back(r.table[j]);
      r.table[j] = b;
      ++stats.cow_copies;
    }
    while ((int)r.table.size() < nblocks) r.table.push_back(bm.allocate());
    return true;
  }

  void emit(Request& r, int kind, int start, int count) {
    planned.push_back(&r);
    p_id.push_back(r.id);
    p_kind.push_back(kind);
    p_start.push_back(start);
    p_count.push_back(count);
    p_tok_off.push_back((int32_t)p_tokens.size());
    p_tokens.insert(p_tokens.end(), r.tokens.begin() + start, r.tokens.begin() + start + count);
    p_lens.push_back(start + count);
    const size_t row = p_tables.size();
    p_tables.resize(row + cfg.max_blocks_per_seq, cfg.pad_block);
    std::copy(r.table.begin(), r.table.end(), p_tables.begin() + row);
  }

  pkv_status schedule(pkv_engine_plan* out) {
    if (plan_open) return set_error(PKV_EINVAL, "the previous plan has not been committed");
    planned.clear();
    p_id.clear(); p_kind.clear(); p_start.clear(); p_count.clear(); p_tok_off.clear(); p_tokens.clear();
    p_tables.clear(); p_lens.clear(); p_src.clear(); p_dst.clear(); p_preempted.clear(); p_release.clear();

    // 1. decode slots for the running requests; preempt the latest arrivals until they fit
    while (!running.empty()) {
      int need = 0;
      for (Request* r : running) need += prepare_slot(*r, false);
      if (need <= bm.available()) break;
      Request* victim = running.back();
      running.pop_back();
      release_all(*victim);
      victim->state = State::kWaiting;
      ++victim->preemptions;
      ++stats.preemptions;
      p_preempted.push_back(victim->id);
      auto pos = std::find_if(waiting.begin(), waiting.end(), [&](Request* w) { return w->arrival > victim->arrival; });
      waiting.insert(pos, victim);
    }
    for (Request* r : running) {
      prepare_slot(*r, true);
      emit(*r, PKV_ENGINE_DECODE, r->computed, 1);
    }
    // 2. admissions in arrival order; a request preempted by this plan waits
    //    for the next iteration (re-admitting it now would recompute it to
    //    stand where it was)
    int budget = cfg.max_prefill_tokens;
    bool first = true;
    while (!waiting.empty() && (int)running.size() < cfg.max_running) {
      Request* r = waiting.front();
      if (std::find(p_preempted.begin(), p_preempted.end(), r->id) != p_preempted.end()) break;
      if (!try_admit(*r, budget, first)) break;
      waiting.pop_front();
      r->state = State::kRunning;
      auto pos = std::find_if(running.begin(), running.end(), [&](Request* x) { return x->arrival > r->arrival; });
      running.insert(pos, r);
      const int count = (int)r->tokens.size() - r->computed;
      budget -= count;
      first = false;
      emit(*r, PKV_ENGINE_PREFILL, r->computed, count);
    }
    for (int b : p_release) bm.release(b);
    p_release.clear();
    plan_open = !planned.empty();
    if (!plan_open && !waiting.empty())
      return set_error(PKV_EINVAL, "request %lld cannot be admitted: the pool is too small for it alone",
                       (long long)waiting.front()->id);
    fill(out);
    ++stats.iterations;
    return PKV_OK;
  }

  void fill(pkv_engine_plan* o) {
    o->n = (int)planned.size();
    o->request_id = p_id.data();
    o->kind = p_kind.data();
    o->start = p_start.data();
    o->count = p_count.data();
    p_tok_off.push_back((int32_t)p_tokens.size());
    o->token_offset = p_tok_off.data();
    o->tokens = p_tokens.data();
    o->block_tables = p_tables.data();
    o->context_lens = p_lens.data();
    o->max_blocks_per_seq = cfg.max_blocks_per_seq;
    o->n_copies = (int)p_src.size();
    o->copy_src = p_src.data();
    o->copy_dst = p_dst.data();
    o->n_preempted = (int)p_preempted.size();
    o->preempted = p_preempted.data();
  }

  pkv_status commit(const int32_t* next_tokens) {
    if (!plan_open) return set_error(PKV_EINVAL, "no plan to commit");
    for (size_t i = 0; i < planned.size(); ++i) {
      Request& r = *planned[i];
      const int from = r.computed;
      r.computed += p_count[i];
      register_blocks(r, from);
      stats.computed_tokens += p_count[i];
      r.tokens.push_back(next_tokens[i]);
      ++r.generated;
      if (r.generated >= r.max_new) {
        r.state = State::kFinished;
        running.erase(std::find(running.begin(), running.end(), &r));
        release_all(r);
        ++stats.finished;
      }
    }
    plan_open = false;
    return PKV_OK;
  }

  pkv_status set_error(pkv_status st, const char* fmt, ...) {
    char buf[256];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    error = buf;
    return st;
  }
};

extern "C" {

pkv_engine* pkv_engine_create(const pkv_engine_config* cfg) {
  if (!cfg || cfg->num_blocks < 1 || cfg->block_size < 1 || cfg->max_blocks_per_seq < 1 || cfg->max_running < 1 ||
      cfg->max_prefill_tokens < 1)
    return nullptr;
  return new pkv_engine(*cfg);
}

void pkv_engine_destroy(pkv_engine* e) { delete e; }

const char* pkv_engine_last_error(const pkv_engine* e) { return e ? e->error.c_str() : "null engine"; }

pkv_status pkv_engine_add_request(pkv_engine* e, int64_t request_id, const int32_t* prompt, int prompt_len,
                                  int max_new_tokens) {
  if (!e) return PKV_EINVAL;
  if (!prompt || prompt_len < 1 || max_new_tokens < 1)
    return e->set_error(PKV_EINVAL, "a request needs a prompt and at least one new token");
  if (e->by_id.count(request_id)) return e->set_error(PKV_EINVAL, "request id %lld already used", (long long)request_id);
  const long long worst = (long long)prompt_len + max_new_tokens;
  if (worst > (long long)e->cfg.max_blocks_per_seq * e->cfg.block_size)
    return e->set_error(PKV_EINVAL, "request %lld needs %lld tokens, more than a block table holds",
                        (long long)request_id, worst);
  auto r = std::make_unique<Request>();
  r->id = request_id;
  r->arrival = e->next_arrival++;
  r->tokens.assign(prompt, prompt + prompt_len);
  r->prompt_len = prompt_len;
  r->max_new = max_new_tokens;
  e->waiting.push_back(r.get());
  e->by_id[request_id] = r.get();
  e->all.push_back(std::move(r));
  return PKV_OK;
}

pkv_status pkv_engine_schedule(pkv_engine* e, pkv_engine_plan* plan) {
  if (!e || !plan) return PKV_EINVAL;
  return e->schedule(plan);
}

pkv_status pkv_engine_commit(pkv_engine* e, const int32_t* next_tokens) {
  if (!e) return PKV_EINVAL;
  if (!next_tokens && e->plan_open) return e->set_error(PKV_EINVAL, "next_tokens missing");
  return e->commit(next_tokens);
}

pkv_status pkv_engine_get_stats(const pkv_engine* e, pkv_engine_stats* out) {
  if (!e || !out) return PKV_EINVAL;
  *out = e->stats;
  out->waiting = (int)e->waiting.size();
  out->running = (int)e->running.size();
  out->free_blocks = e->bm.free_count();
  out->cached_blocks = e->bm.cached_count();
  out->cache_entries = e->bm.cache_entries();
  return PKV_OK;
}

int pkv_engine_request_tokens(const pkv_engine* e, int64_t request_id, int32_t* tokens, int cap) {
  if (!e) return -1;
  auto it = e->by_id.find(request_id);
  if (it == e->by_id.end()) return -1;
  const Request& r = *it->second;
  const int n = (int)r.tokens.size();
  if (tokens)
    for (int i = 0; i < n && i < cap; ++i) tokens[i] = r.tokens[i];
  return n;
}

int pkv_engine_block_ref(const pkv_engine* e, int block) {
  if (!e || block < 0 || block >= e->bm.num_blocks()) return -1;
  return e->bm.ref(block);
}

}  // extern "C"
