"""Fused RoPE + KV append (paged_kv_append_rope) against the oracle.

Both sides rotate in float64 and round once to the storage type, so the cache
must match the oracle's correctly rounded values bit for bit except where the
two float64 sin/cos implementations differ in their last bit right at a
rounding boundary: those elements may differ by one ulp (at most 1 in 1000).
Value rows are copied bit-exact, every other pool byte (NaN poison included)
is unchanged, and the queries, when given, are rotated in place by the same
rule.  Positions reach 131000 so the float64 angle path is exercised where a
float32 angle would have lost the phase."""
import numpy as np
import pytest
import torch

import oracle
import workload
import paged_kv_cache_attention_amd as pkv
from gpu_util import check_attention, check_lse, host, upload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def bits(t, dtype):
    """Raw storage bits of a device tensor as a numpy array."""
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy().view(np.uint32)


def storage_bits(values, dtype):
    """Storage bits of float64 values that are already representable."""
    if dtype == "bf16":
        return workload.f32_to_bf16_bits(values.astype(np.float32))
    return values.astype(np.float32).view(np.uint32)


def rounded(x, dtype):
    return oracle.round_to_bf16(x) if dtype == "bf16" else x.astype(np.float32).astype(np.float64)


def ulp(x, dtype):
    if dtype == "bf16":
        return oracle.bf16_ulp(x)
    return np.spacing(np.abs(x).astype(np.float32)).astype(np.float64)


def assert_rounded_match(got_vals, ref, dtype, where):
    want = rounded(ref, dtype)
    diff = np.abs(got_vals - want)
    off = diff > 0
    assert (diff <= ulp(want, dtype) * 1.0000001).all(), f"{where}: max diff {diff.max():.3e}"
    assert off.mean() <= 1e-3, f"{where}: {int(off.sum())} of {off.size} elements not bit-exact"


CASES = [  # (dtype, D, Hkv, Hq, T, lens_pre, theta)
    ("bf16", 128, 8, 32, 1, [0, 15, 16, 31, 1000], 500000.0),
    ("bf16", 64, 2, 8, 3, [5, 14, 100], 10000.0),
    ("fp32", 64, 4, 8, 2, [0, 17, 63], 10000.0),
    ("fp32", 128, 2, 16, 1, [7, 300], 1.0e6),
    ("bf16", 64, 1, 4, 2, [65000, 99990], 10000.0),
    ("fp32", 64, 1, 4, 1, [131000], 500000.0),
]


@pytest.mark.parametrize("dtype,D,Hkv,Hq,T,lens_pre,theta", CASES)
@pytest.mark.parametrize("with_q", [True, False])
def test_append_rope_matches_oracle(dtype, D, Hkv, Hq, T, lens_pre, theta, with_q):
    lens = np.asarray(lens_pre) + T
    w = workload.uniform_batch("rope", seed=101 + T, B=len(lens), T=T, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype,
                               lens=lens, append=True)
    say("rope", dtype, D, Hkv, Hq, T, lens_pre, theta, "q" if with_q else "no q")
    d = upload(w)
    k_before, v_before = bits(d["k"], dtype), bits(d["v"], dtype)
    q_before = bits(d["q"], dtype)
    pkv.paged_kv_append_rope(d["k_new"], d["v_new"], d["k"], d["v"], d["tables"], d["lens_pre"], theta,
                             q=d["q"] if with_q else None)
    torch.cuda.synchronize()
    k_after, v_after = bits(d["k"], dtype), bits(d["v"], dtype)

    kp_ref, vp_ref = oracle.kv_append_rope(w.values(w.k_pool), w.values(w.v_pool), w.block_tables, w.lens_pre,
                                           w.values(w.k_new), w.values(w.v_new), w.block_size, theta)
    written = np.zeros((w.N_blocks, w.block_size), dtype=bool)
    for b in range(w.B):
        for t in range(T):
            pos = int(w.lens_pre[b]) + t
            written[w.block_tables[b, pos // w.block_size], pos % w.block_size] = True
    # untouched slots keep their exact bits (poison included); values are copied exactly
    assert np.array_equal(k_after[~written], k_before[~written]), "key slots outside the append changed"
    assert np.array_equal(v_after[~written], v_before[~written]), "value slots outside the append changed"
    assert np.array_equal(v_after[written], storage_bits(vp_ref[written], dtype)), "value rows not copied exactly"
    got_k = w.values(k_after.view(np.float32) if dtype == "fp32" else k_after).astype(np.float64)
    assert_rounded_match(got_k[written], kp_ref[written], dtype, "rotated keys")

    q_after = bits(d["q"], dtype)
    if with_q:
        q_ref = oracle.rope_rotate(w.values(w.q), oracle.token_positions(w.lens_pre, T), theta)
        got_q = w.values(q_after.view(np.float32) if dtype == "fp32" else q_after).astype(np.float64)
        assert_rounded_match(got_q, q_ref, dtype, "rotated queries")
    else:
        assert np.array_equal(q_after, q_before), "queries changed without being passed"


def test_append_rope_then_decode():
    """Rotate and append, then decode: attention over the rotated cache with the
    rotated queries, against the oracle on the oracle's rotated inputs."""
    theta = 500000.0
    w = workload.uniform_batch("rope-decode", seed=111, B=4, T=1, Hq=32, Hkv=8, D=128, dtype="bf16",
                               lens=[1, 17, 300, 2049], append=True)
    say("rope then decode")
    d = upload(w)
    pkv.paged_kv_append_rope(d["k_new"], d["v_new"], d["k"], d["v"], d["tables"], d["lens_pre"], theta, q=d["q"])
    lse = torch.full((w.B, w.T, w.Hq), float("nan"), device="cuda")
    out = pkv.paged_attention_decode(d["q"], d["k"], d["v"], d["tables"], d["lens"], lse_out=lse,
                                     scale=float(w.scale))
    torch.cuda.synchronize()
    kp, vp = oracle.kv_append_rope(w.values(w.k_pool), w.values(w.v_pool), w.block_tables, w.lens_pre,
                                   w.values(w.k_new), w.values(w.v_new), w.block_size, theta)
    q = oracle.rope_rotate(w.values(w.q), oracle.token_positions(w.lens_pre, 1), theta)
    # the kernel stores keys and queries in bf16: attention runs on the rounded values
    kp = oracle.round_to_bf16(kp)
    q = oracle.round_to_bf16(q)
    ref, ref_lse = oracle.paged_attention(q, kp, vp, w.block_tables, w.context_lens, w.scale, w.block_size)
    check_attention(host(out), ref, "bf16", "rope then decode")
    check_lse(host(lse), ref_lse, "rope then decode")
