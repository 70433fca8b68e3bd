"""The host runtime (block manager, prefix cache, copy-on-write, continuous
batching with preemption) driven by a CPU stand-in for the device (CPU only).

The stand-in holds a pool of (token, position) pairs instead of K/V rows and
executes each plan in the documented order: block copies, then appends, then
"attention", which here checks that every planned request's block table yields
exactly its own token history at every position it may read.  Any wrong
table entry, missed or misordered copy, block freed while still read, or
prefix-cache hit on the wrong content shows up as a mismatch.  Next tokens are
a fixed function of (request, tokens so far), so runs with different pool
sizes, cache settings and preemptions must produce the same token streams."""
import numpy as np
import pytest

import paged_kv_cache_attention_amd as pkv


def next_token(rid, n_tokens):
    return int((rid * 2654435761 + n_tokens * 40503) % 997)


class FakeDevice:
    def __init__(self, num_blocks, bs):
        self.bs = bs
        self.pool = np.full((num_blocks, bs, 2), -1, dtype=np.int64)   # (token, position); -1 = never written

    def execute(self, eng, plan):
        assert len(set(plan.copy_dst.tolist()) & set(plan.copy_src.tolist())) == 0
        for s, d in zip(plan.copy_src, plan.copy_dst):
            self.pool[d] = self.pool[s]
        written = set()
        for i in range(plan.n):
            tab = plan.block_tables[i]
            for j, tok in enumerate(plan.tokens_of(i)):
                pos = int(plan.start[i]) + j
                slot = (int(tab[pos // self.bs]), pos % self.bs)
                assert slot not in written, "two requests write one slot in one iteration"
                written.add(slot)
                self.pool[slot] = (tok, pos)
        out = []
        for i in range(plan.n):
            rid = int(plan.request_id[i])
            hist = eng.request_tokens(rid)
            L = int(plan.context_lens[i])
            tab = plan.block_tables[i]
            got = np.array([self.pool[tab[p // self.bs], p % self.bs] for p in range(L)])
            want = np.stack([hist[:L], np.arange(L)], axis=1)
            assert np.array_equal(got, want), f"request {rid}: cache content differs from its history"
            out.append(next_token(rid, len(hist)))
        return np.array(out, dtype=np.int32)


def make_requests(seed, n=16, shared=0, shared_len=40):
    rng = np.random.default_rng(seed)
    common = rng.integers(0, 997, size=shared_len)
    reqs = []
    for r in range(n):
        L = int(rng.integers(5, 120))
        p = rng.integers(0, 997, size=L)
        if r < shared:   # these share a prefix (and some the whole prompt)
            p = np.concatenate([common, p[: L // 3]]) if r % 2 else common[: shared_len - (r % 3)].copy()
        reqs.append((100 + r, p.astype(np.int32), int(rng.integers(3, 40))))
    return reqs


def run(reqs, num_blocks, bs=16, prefix_cache=True, max_running=8, max_prefill=256, check_each_step=None):
    eng = pkv.Engine(num_blocks, bs, max_blocks_per_seq=512 // bs, max_running=max_running,
                     max_prefill_tokens=max_prefill, prefix_cache=prefix_cache)
    dev = FakeDevice(num_blocks, bs)
    for rid, p, m in reqs:
        eng.add_request(rid, p, m)
    for _ in range(10000):
        plan = eng.schedule()
        if plan.n == 0:
            break
        assert len(plan.preempted) == 0 or all(rid not in plan.request_id for rid in plan.preempted)
        toks = dev.execute(eng, plan)
        eng.commit(toks)
        if check_each_step:
            check_each_step(eng, plan)
    st = eng.stats()
    streams = {rid: eng.request_tokens(rid) for rid, _, _ in reqs}
    refs = [eng.block_ref(b) for b in range(num_blocks)]
    eng.close()
    return st, streams, refs


def expected_stream(rid, prompt, max_new):
    toks = list(prompt)
    for _ in range(max_new):
        toks.append(next_token(rid, len(toks)))
    return np.array(toks)


@pytest.mark.parametrize("bs", [4, 16])
def test_large_pool_no_preemption(bs):
    reqs = make_requests(1)
    st, streams, refs = run(reqs, num_blocks=2000, bs=bs, prefix_cache=False)
    assert st["preemptions"] == 0 and st["finished"] == 16 and st["waiting"] == st["running"] == 0
    for rid, p, m in reqs:
        assert np.array_equal(streams[rid], expected_stream(rid, p, m))
    assert all(r == 0 for r in refs) and st["free_blocks"] == 2000


@pytest.mark.parametrize("prefix_cache", [False, True])
def test_small_pool_forces_preemption(prefix_cache):
    """16 requests, a pool well below their worst case: preemption fires, the
    preempted requests are recomputed, every stream is the one it would have
    been alone, and every block comes back."""
    reqs = make_requests(2)
    worst = sum(-(-(len(p) + m) // 16) for _, p, m in reqs)
    pool = worst // 3
    st, streams, refs = run(reqs, num_blocks=pool, prefix_cache=prefix_cache)
    assert st["preemptions"] >= 1
    assert st["finished"] == 16
    for rid, p, m in reqs:
        assert np.array_equal(streams[rid], expected_stream(rid, p, m))
    assert all(r == 0 for r in refs)
    assert st["free_blocks"] + st["cached_blocks"] == pool


def test_prefix_cache_shares_blocks_and_copies_on_write():
    """Requests with a common prompt prefix (some with the whole prompt in
    common, ending inside a block) reuse the cached blocks; the ones whose
    first computed token lands in a shared, partly filled block get a private
    copy first."""
    reqs = make_requests(3, shared=8)
    st, streams, refs = run(reqs, num_blocks=400, prefix_cache=True, max_running=4)
    assert st["prefix_hit_tokens"] > 0
    assert st["cow_copies"] > 0
    st_off, streams_off, _ = run(reqs, num_blocks=400, prefix_cache=False, max_running=4)
    assert st["computed_tokens"] < st_off["computed_tokens"]
    for rid, _, _ in reqs:
        assert np.array_equal(streams[rid], streams_off[rid])
    assert all(r == 0 for r in refs)


def test_budget_and_running_limits():
    """At most max_running requests decode at once and the prefill tokens of an
    iteration stay within the budget unless a single admission exceeds it."""
    reqs = make_requests(4)
    seen = []

    def check(eng, plan):
        seen.append(plan)
    run(reqs, num_blocks=600, max_running=3, max_prefill=64, check_each_step=check)
    for plan in seen:
        assert plan.n <= 3
        pre = plan.count[plan.kind == pkv.PKV_ENGINE_PREFILL]
        assert len(pre) <= 1 or pre.sum() <= 64


def test_engine_errors():
    eng = pkv.Engine(8, 16, max_blocks_per_seq=4, max_running=2, max_prefill_tokens=64)
    eng.add_request(1, [1, 2, 3], 2)
    with pytest.raises(pkv.PkvError, match="already used"):
        eng.add_request(1, [4], 1)
    with pytest.raises(pkv.PkvError, match="more than a block table holds"):
        eng.add_request(2, list(range(60)), 5)
    with pytest.raises(pkv.PkvError):
        eng.add_request(3, [], 1)
    with pytest.raises(pkv.PkvError, match="no plan"):
        eng.commit([0])
    eng.schedule()
    with pytest.raises(pkv.PkvError, match="not been committed"):
        eng.schedule()
    eng.close()
    tiny = pkv.Engine(2, 16, max_blocks_per_seq=8, max_running=2, max_prefill_tokens=512)
    tiny.add_request(1, list(range(40)), 2)   # needs 3 blocks, the pool has 2
    with pytest.raises(pkv.PkvError, match="too small"):
        tiny.schedule()
    tiny.close()
    with pytest.raises(pkv.PkvError):
        pkv.Engine(0, 16, 4, 1, 1)


@pytest.mark.parametrize("seed", range(6))
def test_randomised_workloads_keep_every_invariant(seed):
    """Random request mixes, block sizes, pool sizes, limits and cache
    settings: every cache read matches its history, streams equal the solo
    streams, and all blocks come back."""
    rng = np.random.default_rng(1000 + seed)
    bs = int(rng.choice([4, 8, 16]))
    n = int(rng.integers(4, 24))
    common = rng.integers(0, 997, size=int(rng.integers(1, 60)))
    reqs = []
    for r in range(n):
        if rng.random() < 0.4:   # share a prefix of the common prompt, possibly all of it
            p = np.concatenate([common[: int(rng.integers(1, len(common) + 1))],
                                rng.integers(0, 997, size=int(rng.integers(0, 30)))])
        else:
            p = rng.integers(0, 997, size=int(rng.integers(1, 100)))
        reqs.append((r, p.astype(np.int32), int(rng.integers(1, 25))))
    need_max = max(-(-(len(p) + m) // bs) for _, p, m in reqs)
    worst = sum(-(-(len(p) + m) // bs) for _, p, m in reqs)
    pool = int(rng.integers(need_max + 1, max(need_max + 2, worst + 1)))
    st, streams, refs = run(reqs, num_blocks=pool, bs=bs, prefix_cache=bool(rng.random() < 0.7),
                            max_running=int(rng.integers(1, 9)), max_prefill=int(rng.integers(8, 300)))
    assert st["finished"] == n
    for rid, p, m in reqs:
        assert np.array_equal(streams[rid], expected_stream(rid, p, m))
    assert all(r == 0 for r in refs)
    assert st["free_blocks"] + st["cached_blocks"] == pool


def test_copy_sources_never_reused_as_destinations_in_one_plan():
    """A partly filled cached block that an admission copies from must not be
    handed out again in the same plan.  Pool of 4 blocks of 4 tokens: A
    [1..6] and B [21..23] finish and stay cached; then C [1..7] reuses A's
    blocks (copying A's partly filled second block) and D [21..24] reuses B's
    partly filled block.  Had C's copy source gone back to the evictable list
    at once, D's copy would have taken it as its destination in the same plan
    (sources {a1, b0}, destinations {free, a1})."""
    eng = pkv.Engine(4, 4, max_blocks_per_seq=4, max_running=4, max_prefill_tokens=64, prefix_cache=True)
    dev = FakeDevice(4, 4)
    plans = []

    def drain():
        for _ in range(100):
            plan = eng.schedule()
            if plan.n == 0:
                return
            plans.append(plan)
            src, dst = set(plan.copy_src.tolist()), set(plan.copy_dst.tolist())
            assert not src & dst, f"plan copies {plan.copy_src} -> {plan.copy_dst}"
            eng.commit(dev.execute(eng, plan))

    eng.add_request(1, [1, 2, 3, 4, 5, 6], 1)
    eng.add_request(2, [21, 22, 23], 1)
    drain()
    eng.add_request(3, [1, 2, 3, 4, 5, 6, 7], 1)
    eng.add_request(4, [21, 22, 23, 24], 1)
    drain()
    st = eng.stats()
    assert st["finished"] == 4 and st["cow_copies"] >= 2 and st["prefix_hit_tokens"] >= 9
    for rid, p in ((3, [1, 2, 3, 4, 5, 6, 7]), (4, [21, 22, 23, 24])):
        assert np.array_equal(eng.request_tokens(rid), expected_stream(rid, p, 1))
    assert all(eng.block_ref(b) == 0 for b in range(4))
    eng.close()
