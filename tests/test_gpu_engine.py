"""The host engine driving the kernels end to end on the device: 16 requests,
continuous batching, a block pool a third of their worst case (preemption and
recompute), a shared prompt that ends inside a block (prefix-cache hits and
copy-on-write block copies), RoPE append, chunked prefill for admissions and batched decode.

The model around attention is a stand-in: seeded bf16 embedding tables give
each token its q, k and v (k and q rotated by position in the append), and the
next token is a fixed function of (request, tokens so far), so every run has
the same token streams.  Every attention output row of every iteration is
checked against the oracle on that request's contiguous history (paged with
preemption and sharing == each request computed alone, in fp64)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_attention_amd as pkv
from paged_kv_cache_attention_amd.serve import PagedExecutor
from gpu_util import check_attention, check_attention_pbf16, host

pytestmark = pytest.mark.gpu

V, HQ, HKV, D, BS, THETA = 997, 8, 2, 64, 16, 10000.0


def next_token(rid, n_tokens):
    return int((rid * 2654435761 + n_tokens * 40503) % V)


def requests(seed, n=16, shared_len=37):
    """Random prompts, except one shared 37-token prompt (ending inside a
    block) for requests 0, 5, 9 and 13 and two longer prompts that start with
    it; request 0 runs long enough that the later ones find its blocks."""
    rng = np.random.default_rng(seed)
    common = rng.integers(0, V, size=shared_len)
    out = []
    for r in range(n):
        L = int(rng.integers(5, 150))
        p = rng.integers(0, V, size=L).astype(np.int32)
        m = int(rng.integers(3, 30))
        if r in (0, 5, 9, 13):
            p = common.astype(np.int32).copy()
        if r in (2, 7):
            p = np.concatenate([common, p[: L // 3]]).astype(np.int32)
        if r == 0:
            m = 40
        out.append((200 + r, p, m))
    return out


@pytest.mark.parametrize("prefix_cache", [True, False])
def test_engine_serves_16_requests_with_preemption(prefix_cache):
    torch.manual_seed(0)
    g = torch.Generator().manual_seed(1234)
    tables = {name: (torch.randn(V, h, D, generator=g)).to(torch.bfloat16).cuda() for name, h in
              (("q", HQ), ("k", HKV), ("v", HKV))}
    Eq, Ek, Ev = (tables[n].float().cpu().numpy().astype(np.float64) for n in ("q", "k", "v"))

    def qkv(tok):
        t = tok.long()
        return tables["q"][t], tables["k"][t], tables["v"][t]

    reqs = requests(7)
    worst = sum(-(-(len(p) + m) // BS) for _, p, m in reqs)
    nblocks = worst // 3
    eng = pkv.Engine(nblocks, BS, max_blocks_per_seq=16, max_running=8, max_prefill_tokens=256,
                     prefix_cache=prefix_cache, pad_block=0)
    for rid, p, m in reqs:
        eng.add_request(rid, p, m)
    k_pool = torch.zeros(nblocks, BS, HKV, D, dtype=torch.bfloat16, device="cuda")
    v_pool = torch.zeros_like(k_pool)
    checked = {"rows": 0}

    def sample(plan, outputs):
        torch.cuda.synchronize()
        toks = []
        for i in range(plan.n):
            rid = int(plan.request_id[i])
            hist = eng.request_tokens(rid)
            L, s = int(plan.context_lens[i]), int(plan.start[i])
            pos = np.arange(L)
            K = oracle.round_to_bf16(oracle.rope_rotate(Ek[hist[:L]], pos, THETA))
            Vv = Ev[hist[:L]]
            Q = oracle.round_to_bf16(oracle.rope_rotate(Eq[hist[s:L]], pos[s:], THETA))
            got = host(outputs[i]).reshape(L - s, HQ, D)
            ref = np.zeros_like(got)
            abs_ref = np.zeros_like(got)
            for r in range(L - s):
                for h in range(HQ):
                    kh = h // (HQ // HKV)
                    ref[r, h], _ = oracle.softmax_attention_row(Q[r, h], K[: s + r + 1, kh], Vv[: s + r + 1, kh],
                                                                1.0 / D ** 0.5)
                    abs_ref[r, h], _ = oracle.softmax_attention_row(Q[r, h], K[: s + r + 1, kh],
                                                                    np.abs(Vv[: s + r + 1, kh]), 1.0 / D ** 0.5)
            kind = "prefill" if plan.kind[i] == pkv.PKV_ENGINE_PREFILL else "decode"
            if kind == "prefill":   # the prefill tile rounds P to bf16 once
                check_attention_pbf16(got, ref, abs_ref, f"request {rid} prefill at {s}..{L}")
            else:
                check_attention(got, ref, "bf16", f"request {rid} decode at {s}..{L}")
            checked["rows"] += L - s
            toks.append(next_token(rid, len(hist)))
        return np.array(toks, dtype=np.int32)

    ex = PagedExecutor(eng, k_pool, v_pool, HQ, THETA, qkv, sample)
    it = 0
    while ex.step() is not None:
        it += 1
        assert it < 2000
    st = eng.stats()
    print("engine", st, "rows checked", checked["rows"], flush=True)
    assert st["finished"] == 16 and st["preemptions"] >= 1
    if prefix_cache:
        assert st["prefix_hit_tokens"] > 0 and st["cow_copies"] > 0
    for rid, p, m in reqs:
        want = list(p)
        for _ in range(m):
            want.append(next_token(rid, len(want)))
        assert np.array_equal(eng.request_tokens(rid), want)
    eng.close()
