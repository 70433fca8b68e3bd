"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin raises AssertionError when the oracle disagrees with a fixed fact:
hand-derived golden values, a library routine (torch's scaled_dot_product_attention
in float64), an independent brute-force evaluation with ``math.fsum``, closed
forms, or an invariant the pages state (paged == contiguous recompute, cached
decode == full-prefix forward).  ``ALL_PINS`` lists them so the mutation tests
can show that planted mistakes in the oracle are caught.
"""
from __future__ import annotations

import json
import math
import pathlib

import numpy as np
import torch

import oracle
import workload

GOLDEN = pathlib.Path(__file__).parent / "golden"


def _arr(x):
    def conv(v):
        if v is None:
            return float("nan")
        if isinstance(v, str):
            return float(v)
        if isinstance(v, list):
            return [conv(e) for e in v]
        return float(v)
    return np.array(conv(x), dtype=np.float64)


def _golden_attention(name):
    g = json.loads((GOLDEN / name).read_text())
    out, lse = oracle.paged_attention(_arr(g["q"]), _arr(g["k_pool"]), _arr(g["v_pool"]),
                                      np.array(g["block_tables"]), np.array(g["context_lens"]),
                                      g["scale"], g["block_size"])
    np.testing.assert_allclose(out, _arr(g["expected_out"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, _arr(g["expected_lse"]), rtol=0, atol=1e-12)


def pin_golden_two_token():
    _golden_attention("two_token_softmax.json")


def pin_golden_gqa_causal_verify():
    _golden_attention("gqa_causal_verify.json")


def pin_golden_gqa_head_mapping():
    _golden_attention("gqa_head_mapping.json")


def pin_golden_lse_merge():
    g = json.loads((GOLDEN / "lse_merge.json").read_text())
    out, lse = oracle.lse_combine(_arr(g["o_parts"]), _arr(g["lse_parts"]))
    np.testing.assert_allclose(out, _arr(g["expected_out"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, _arr(g["expected_lse"]), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Small random problems built here (never by the oracle).
# ---------------------------------------------------------------------------

def random_problem(seed, B=3, T=1, Hq=8, Hkv=2, D=16, bs=4, lens=(5, 13, 8), spare=3):
    """Random logical K/V per sequence, scattered into a shuffled pool.

    The scatter walks the physical blocks and looks up which (sequence,
    logical block) owns each one, the inverse of the block-table lookup."""
    rng = np.random.default_rng(seed)
    lens = list(lens)
    nblk = [-(-L // bs) for L in lens]
    N = sum(nblk) + spare
    perm = rng.permutation(N)
    owner = {}
    tables = np.full((B, max(nblk)), perm[-1], dtype=np.int64)  # padding -> an unused (NaN) block
    nxt = 0
    for b in range(B):
        for i in range(nblk[b]):
            tables[b, i] = perm[nxt]
            owner[int(perm[nxt])] = (b, i)
            nxt += 1
    Klog = [rng.standard_normal((L, Hkv, D)) for L in lens]
    Vlog = [rng.standard_normal((L, Hkv, D)) for L in lens]
    kp = np.full((N, bs, Hkv, D), np.nan)
    vp = np.full((N, bs, Hkv, D), np.nan)
    for phys in range(N):
        if phys not in owner:
            continue
        b, i = owner[phys]
        rows = range(i * bs, min((i + 1) * bs, lens[b]))
        for s, j in enumerate(rows):
            kp[phys, s] = Klog[b][j]
            vp[phys, s] = Vlog[b][j]
    q = rng.standard_normal((B, T, Hq, D))
    return dict(q=q, k_pool=kp, v_pool=vp, tables=tables, lens=np.array(lens), bs=bs,
                Klog=Klog, Vlog=Vlog, scale=1.0 / math.sqrt(D))


def _run(p, q=None, lens=None):
    return oracle.paged_attention(p["q"] if q is None else q, p["k_pool"], p["v_pool"], p["tables"],
                                  p["lens"] if lens is None else lens, p["scale"], p["bs"])


def pin_gather_inverse_scatter():
    """Gather returns the logical rows that were scattered by the inverse map."""
    p = random_problem(11)
    for b, L in enumerate(p["lens"]):
        got = oracle.gather_sequence(p["k_pool"], p["tables"][b], int(L), p["bs"])
        np.testing.assert_array_equal(got, p["Klog"][b])


def pin_append_then_gather():
    """Appending T rows then gathering returns them at the end; every other byte is unchanged."""
    rng = np.random.default_rng(12)
    bs, Hkv, D, T = 4, 2, 8, 3
    lens_pre = np.array([3, 4, 9])          # crossings: 3->6 (within/into block 1), 4->7, 9->12
    B = len(lens_pre)
    nblk = [-(-(L + T) // bs) for L in lens_pre]
    N = sum(nblk) + 2
    ids = rng.permutation(N)
    tables = np.zeros((B, max(nblk)), dtype=np.int64)
    c = 0
    for b in range(B):
        tables[b, :nblk[b]] = ids[c:c + nblk[b]]
        c += nblk[b]
    kp = rng.standard_normal((N, bs, Hkv, D))
    vp = rng.standard_normal((N, bs, Hkv, D))
    k_new = rng.standard_normal((B, T, Hkv, D))
    v_new = rng.standard_normal((B, T, Hkv, D))
    k2, v2 = oracle.kv_append(kp, vp, tables, lens_pre, k_new, v_new, bs)
    changed_k = np.zeros(kp.shape[:2], dtype=bool)
    for b in range(B):
        L = int(lens_pre[b])
        gk = oracle.gather_sequence(k2, tables[b], L + T, bs)
        gv = oracle.gather_sequence(v2, tables[b], L + T, bs)
        np.testing.assert_array_equal(gk[L:], k_new[b])
        np.testing.assert_array_equal(gv[L:], v_new[b])
        np.testing.assert_array_equal(gk[:L], oracle.gather_sequence(kp, tables[b], L, bs))
        for t in range(T):
            pos = L + t
            changed_k[tables[b, pos // bs], pos % bs] = True
    np.testing.assert_array_equal(k2[~changed_k], kp[~changed_k])
    np.testing.assert_array_equal(v2[~changed_k], vp[~changed_k])


def pin_torch_sdpa_decode():
    """T=1 GQA decode equals torch SDPA (float64, CPU) on the contiguous, head-repeated K/V."""
    p = random_problem(13, Hq=8, Hkv=2)
    out, lse = _run(p)
    g = 8 // 2
    for b, L in enumerate(p["lens"]):
        K = torch.from_numpy(np.repeat(p["Klog"][b], g, axis=1)).permute(1, 0, 2)  # [Hq, L, D]
        V = torch.from_numpy(np.repeat(p["Vlog"][b], g, axis=1)).permute(1, 0, 2)
        Q = torch.from_numpy(p["q"][b, 0])[:, None, :]                               # [Hq, 1, D]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=p["scale"])[:, 0, :]
        np.testing.assert_allclose(out[b, 0], ref.numpy(), rtol=0, atol=1e-12)
        s = p["scale"] * torch.einsum("hd,hld->hl", Q[:, 0, :], K)
        np.testing.assert_allclose(lse[b, 0], torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


def pin_torch_sdpa_causal_verify():
    """T=4 verify equals the last 4 rows of a causal full-prefix forward (torch SDPA, is_causal)."""
    T = 4
    p = random_problem(14, T=T, Hq=8, Hkv=2, lens=(4, 9, 17))
    out, _ = _run(p)
    g = 4
    rng = np.random.default_rng(99)
    for b, L in enumerate(p["lens"]):
        K = torch.from_numpy(np.repeat(p["Klog"][b], g, axis=1)).permute(1, 0, 2)
        V = torch.from_numpy(np.repeat(p["Vlog"][b], g, axis=1)).permute(1, 0, 2)
        Qfull = rng.standard_normal((8, int(L), K.shape[-1]))
        Qfull[:, L - T:, :] = p["q"][b].transpose(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(Qfull), K, V, is_causal=True,
                                                               scale=p["scale"])
        np.testing.assert_allclose(out[b], ref[:, L - T:, :].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def pin_torch_sdpa_chunked_prefill():
    """A chunk of T = 37 query tokens (chunked prefill) equals the last 37 rows of
    a causal full-prefix forward (torch SDPA, is_causal), for GQA 8/2; one
    sequence is the chunk alone (L = T), the others have a cached prefix."""
    T = 37
    p = random_problem(15, T=T, Hq=8, Hkv=2, lens=(37, 52, 90))
    out, lse = _run(p)
    g = 4
    rng = np.random.default_rng(98)
    for b, L in enumerate(p["lens"]):
        K = torch.from_numpy(np.repeat(p["Klog"][b], g, axis=1)).permute(1, 0, 2)
        V = torch.from_numpy(np.repeat(p["Vlog"][b], g, axis=1)).permute(1, 0, 2)
        Qfull = rng.standard_normal((8, int(L), K.shape[-1]))
        Qfull[:, L - T:, :] = p["q"][b].transpose(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(Qfull), K, V, is_causal=True,
                                                               scale=p["scale"])
        np.testing.assert_allclose(out[b], ref[:, L - T:, :].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
        # lse of row t: log-sum-exp over the keys it sees
        s = p["scale"] * torch.einsum("hld,hmd->hlm", torch.from_numpy(Qfull), K)
        mask = torch.ones(int(L), int(L), dtype=torch.bool).tril()
        ref_lse = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=-1)[:, L - T:]
        np.testing.assert_allclose(lse[b], ref_lse.permute(1, 0).numpy(), rtol=0, atol=1e-12)


def pin_rope_hand_values():
    """D = 4, theta = 10000: w = (1, 0.01).  A unit vector in dimension 0 at
    position 1 turns into dimension 2 (its pair partner is i + D/2) by 1 rad;
    one in dimension 1 turns into dimension 3 by 0.01 rad; position 0 is the
    identity."""
    y = oracle.rope_rotate(np.array([[1.0, 0.0, 0.0, 0.0], [0.0, 1.0, 0.0, 0.0]]), np.array(1), 10000.0)
    np.testing.assert_allclose(y[0], [math.cos(1.0), 0.0, math.sin(1.0), 0.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(y[1], [0.0, math.cos(0.01), 0.0, math.sin(0.01)], rtol=0, atol=1e-15)
    x = np.random.default_rng(3).standard_normal((5, 3, 64))
    np.testing.assert_array_equal(oracle.rope_rotate(x, np.zeros(5), 500000.0), x)


def pin_rope_relative_position():
    """<R(q, m), R(k, n)> depends only on m - n (shifting both positions keeps
    every pair's dot product), each pair keeps its length, and R(R(x, a), b) =
    R(x, a + b)."""
    rng = np.random.default_rng(4)
    D, theta = 128, 10000.0
    q, k = rng.standard_normal((2, 7, 1, D))
    m, n = rng.integers(0, 5000, size=(2, 7))
    shift = 1234
    d1 = np.sum(oracle.rope_rotate(q, m, theta) * oracle.rope_rotate(k, n, theta), axis=-1)
    d2 = np.sum(oracle.rope_rotate(q, m + shift, theta) * oracle.rope_rotate(k, n + shift, theta), axis=-1)
    np.testing.assert_allclose(d1, d2, rtol=1e-9, atol=1e-9)
    y = oracle.rope_rotate(q, m, theta)
    np.testing.assert_allclose(y[..., :D // 2] ** 2 + y[..., D // 2:] ** 2,
                               q[..., :D // 2] ** 2 + q[..., D // 2:] ** 2, rtol=1e-12)
    np.testing.assert_allclose(oracle.rope_rotate(oracle.rope_rotate(q, m, theta), n, theta),
                               oracle.rope_rotate(q, m + n, theta), rtol=0, atol=1e-9)


def pin_rope_append_positions():
    """The fused append writes R(k_new[b, t], lens_pre[b] + t) into that
    position's slot and v_new unchanged; every other slot keeps its bytes."""
    rng = np.random.default_rng(5)
    B, T, Hkv, D, bs, N = 3, 5, 2, 8, 4, 12
    lens_pre = np.array([0, 3, 9])
    tables = rng.permutation(N)[: B * 4].reshape(B, 4)
    kp, vp = rng.standard_normal((2, N, bs, Hkv, D))
    k_new, v_new = rng.standard_normal((2, B, T, Hkv, D))
    k2, v2 = oracle.kv_append_rope(kp, vp, tables, lens_pre, k_new, v_new, bs, 10000.0)
    touched = np.zeros((N, bs), dtype=bool)
    for b in range(B):
        for t in range(T):
            pos = int(lens_pre[b]) + t
            blk, slot = tables[b, pos // bs], pos % bs
            touched[blk, slot] = True
            np.testing.assert_allclose(k2[blk, slot], oracle.rope_rotate(k_new[b, t], np.array(pos), 10000.0),
                                       rtol=0, atol=1e-15)
            np.testing.assert_array_equal(v2[blk, slot], v_new[b, t])
    np.testing.assert_array_equal(k2[~touched], kp[~touched])
    np.testing.assert_array_equal(v2[~touched], vp[~touched])


def pin_brute_force_fsum():
    """Tiny fp32 workload: every output recomputed with scalar loops and math.fsum."""
    w = workload.tiny_fp32()
    q, kp, vp = w.values(w.q), w.values(w.k_pool), w.values(w.v_pool)
    out, lse = oracle.paged_attention(q, kp, vp, w.block_tables, w.context_lens, w.scale, w.block_size)
    bs = w.block_size
    for b in range(w.B):
        L = int(w.context_lens[b])
        for h in range(w.Hq):
            scores = []
            for j in range(L):
                blk = int(w.block_tables[b][j // bs])
                scores.append(float(w.scale) * math.fsum(float(q[b, 0, h, d]) * float(kp[blk, j % bs, h, d])
                                                         for d in range(w.D)))
            mx = max(scores)
            ex = [math.exp(s - mx) for s in scores]
            z = math.fsum(ex)
            for d in range(0, w.D, 7):
                num = math.fsum(ex[j] * float(vp[int(w.block_tables[b][j // bs]), j % bs, h, d]) for j in range(L))
                assert abs(out[b, 0, h, d] - num / z) < 1e-13
            assert abs(lse[b, 0, h] - (mx + math.log(z))) < 1e-12


def pin_closed_forms():
    p = random_problem(15, lens=(1, 2, 6))
    out, lse = _run(p)
    g = 4
    # L = 1: the single visible row, whatever q is
    for h in range(8):
        np.testing.assert_allclose(out[0, 0, h], p["Vlog"][0][0, h // g], rtol=0, atol=1e-15)
    # L = 2: sigma(s0 - s1) v0 + sigma(s1 - s0) v1
    for h in range(8):
        kh = h // g
        s = [p["scale"] * p["q"][1, 0, h] @ p["Klog"][1][j, kh] for j in range(2)]
        w0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
        np.testing.assert_allclose(out[1, 0, h], w0 * p["Vlog"][1][0, kh] + (1 - w0) * p["Vlog"][1][1, kh],
                                   rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[1, 0, h], math.log(math.exp(s[0]) + math.exp(s[1])), rtol=0, atol=1e-13)
    # q = 0: the mean of the visible values, lse = log L
    q0 = np.zeros_like(p["q"])
    out0, lse0 = _run(p, q=q0)
    for h in range(8):
        np.testing.assert_allclose(out0[2, 0, h], p["Vlog"][2][:, h // g].mean(axis=0), rtol=0, atol=1e-14)
        assert abs(lse0[2, 0, h] - math.log(6)) < 1e-14


def pin_dominant_score():
    """A score gap far beyond fp64's exp range: output is exactly the winning row."""
    p = random_problem(16, lens=(6, 6, 6))
    q = p["q"].copy()
    b, kh = 2, 1
    k_star = p["Klog"][b][3, kh]
    q[b, 0, 4] = 5000.0 * k_star / np.linalg.norm(k_star)
    others = [p["scale"] * q[b, 0, 4] @ p["Klog"][b][j, kh] for j in range(6)]
    assert others[3] - max(others[:3] + others[4:]) > 800
    out, lse = _run(p, q=q)
    np.testing.assert_array_equal(out[b, 0, 4], p["Vlog"][b][3, kh])
    assert abs(lse[b, 0, 4] - others[3]) < 1e-9 * abs(others[3])


def pin_key_shift_invariance():
    """Adding one vector a to every key shifts all scores of a query by scale*q.a:
    outputs are unchanged and lse moves by exactly that amount."""
    p = random_problem(17)
    out, lse = _run(p)
    a = np.random.default_rng(5).standard_normal(p["k_pool"].shape[-1])
    p2 = dict(p, k_pool=p["k_pool"] + a)
    out2, lse2 = _run(p2)
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-12)
    shift = p["scale"] * np.einsum("bthd,d->bth", p["q"], a)
    np.testing.assert_allclose(lse2 - lse, shift, rtol=0, atol=1e-12)


def pin_physical_permutation():
    """Relabelling physical blocks (pool and tables together) changes nothing, bit for bit."""
    w = workload.tinylm_mha_bf16()
    w2 = workload.relabel_physical(w, seed=123)
    args = lambda x: (x.values(x.q), x.values(x.k_pool), x.values(x.v_pool), x.block_tables, x.context_lens,
                      x.scale, x.block_size)
    o1, l1 = oracle.paged_attention(*args(w))
    o2, l2 = oracle.paged_attention(*args(w2))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    assert np.isfinite(o1).all()


def pin_gqa_equals_repeated_mha():
    """GQA with g = Hq/Hkv equals MHA over KV heads repeated g times."""
    p = random_problem(18, Hq=8, Hkv=2)
    out, lse = _run(p)
    pr = dict(p, k_pool=np.repeat(p["k_pool"], 4, axis=2), v_pool=np.repeat(p["v_pool"], 4, axis=2))
    out2, lse2 = _run(pr)
    np.testing.assert_allclose(out, out2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-14)


def pin_verify_equals_decode_chain():
    """Cached decode == full-prefix forward: verify row t at length L equals a T=1 decode
    at length L-T+1+t with that row's query."""
    T = 4
    p = random_problem(19, T=T, lens=(4, 11, 16))
    out, lse = _run(p)
    for t in range(T):
        lens_t = p["lens"] - T + 1 + t
        o1, l1 = _run(p, q=p["q"][:, t:t + 1], lens=lens_t)
        np.testing.assert_allclose(out[:, t], o1[:, 0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[:, t], l1[:, 0], rtol=0, atol=1e-13)


def pin_split_equals_full():
    """Partition + log-sum-exp merge equals unsplit attention for several partition sizes."""
    T = 2
    p = random_problem(20, T=T, lens=(9, 17, 25), bs=4)
    out, lse = _run(p)
    for P in (4, 8, 12, 100):
        o_p, l_p = oracle.partition_attention(p["q"], p["k_pool"], p["v_pool"], p["tables"], p["lens"],
                                              p["scale"], p["bs"], P)
        o, l = oracle.lse_combine(o_p, l_p)
        np.testing.assert_allclose(o, out, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l, lse, rtol=0, atol=1e-13)
    # a partition that is empty for the first query row (L mod P == 1) yields (0, -inf)
    o_p, l_p = oracle.partition_attention(p["q"], p["k_pool"], p["v_pool"], p["tables"], p["lens"],
                                          p["scale"], p["bs"], 8)
    assert l_p[0, 0, 0, 1] == -np.inf and not o_p[0, 0, 0, 1].any()
    assert np.isfinite(l_p[0, 1, 0, 1])


def pin_lse_merge_algebra():
    """One partition is the identity; merging is associative."""
    rng = np.random.default_rng(21)
    o = rng.standard_normal((5, 3, 6))
    l = rng.standard_normal((5, 3)) * 4
    o1, l1 = oracle.lse_combine(o[:, :1], l[:, :1])
    np.testing.assert_array_equal(o1, o[:, 0])
    np.testing.assert_array_equal(l1, l[:, 0])
    full_o, full_l = oracle.lse_combine(o, l)
    ab_o, ab_l = oracle.lse_combine(o[:, :2], l[:, :2])
    o2 = np.stack([ab_o, o[:, 2]], axis=1)
    l2 = np.stack([ab_l, l[:, 2]], axis=1)
    re_o, re_l = oracle.lse_combine(o2, l2)
    np.testing.assert_allclose(re_o, full_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(re_l, full_l, rtol=0, atol=1e-13)


def pin_bf16_rounding():
    """The epilogue rounding agrees with two independent RNE implementations:
    torch's float32 -> bfloat16 cast and the generator's bit arithmetic."""
    rng = np.random.default_rng(22)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-3).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, 2.0 ** -126], np.float32)])
    mine = oracle.round_to_bf16(x.astype(np.float64))
    lib = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    gen = workload.bf16_bits_to_f32(workload.f32_to_bf16_bits(x)).astype(np.float64)
    np.testing.assert_array_equal(mine, lib)
    np.testing.assert_array_equal(mine, gen)
    assert oracle.round_to_bf16(np.array([1.0 + 2 ** -8]))[0] == 1.0          # tie -> even
    assert oracle.round_to_bf16(np.array([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6


def pin_bf16_ulp():
    """The spacing of bf16 values, which sets every bf16 gate of the GPU tests.

    Hand values: bf16 keeps 8 significant bits, so the spacing in the binade
    [2^k, 2^(k+1)) is 2^(k-7): 1.0 -> 2^-7, 0.75 -> 2^-8, 3.0 -> 2^-6,
    1e-3 (in [2^-10, 2^-9)) -> 2^-17, and the sign does not matter.  Then, for
    every positive normal bf16 value below the largest, the spacing equals the
    gap to the next bf16 value, taken from the generator's bit arithmetic
    (the value of bit pattern u + 1 minus that of u)."""
    hand = {1.0: 2.0 ** -7, 0.75: 2.0 ** -8, 3.0: 2.0 ** -6, 1e-3: 2.0 ** -17, -1.5: 2.0 ** -7,
            2.0 ** -126: 2.0 ** -133, 255.0: 1.0, 256.0: 2.0}
    for x, want in hand.items():
        assert oracle.bf16_ulp(np.array([x]))[0] == want, (x, want)
    bits = np.arange(0x0080, 0x7F7F, dtype=np.uint32)           # positive normal, below the largest finite
    vals = workload.bf16_bits_to_f32(bits.astype(np.uint16)).astype(np.float64)
    nxt = workload.bf16_bits_to_f32((bits + 1).astype(np.uint16)).astype(np.float64)
    np.testing.assert_array_equal(oracle.bf16_ulp(vals), nxt - vals)
    np.testing.assert_array_equal(oracle.bf16_ulp(-vals), nxt - vals)


ALL_PINS = [
    pin_golden_two_token, pin_golden_gqa_causal_verify, pin_golden_gqa_head_mapping, pin_golden_lse_merge,
    pin_gather_inverse_scatter, pin_append_then_gather, pin_torch_sdpa_decode, pin_torch_sdpa_causal_verify,
    pin_torch_sdpa_chunked_prefill, pin_rope_hand_values, pin_rope_relative_position, pin_rope_append_positions,
    pin_brute_force_fsum, pin_closed_forms, pin_dominant_score, pin_key_shift_invariance,
    pin_physical_permutation, pin_gqa_equals_repeated_mha, pin_verify_equals_decode_chain,
    pin_split_equals_full, pin_lse_merge_algebra, pin_bf16_rounding, pin_bf16_ulp,
]
