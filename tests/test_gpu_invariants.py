"""GPU invariants and edge cases, each also checked against the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import workload
import paged_kv_cache_attention_amd as pkv
from gpu_util import (assert_within_bf16_ulp, check_attention, check_lse, check_partials, dev, host, max_abs_finite,
                      mfma_floor, oracle_inputs, upload)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def decode(w, d, part, lse=True):
    lse_t = torch.full((w.B, w.T, w.Hq), float("nan"), device="cuda") if lse else None
    out = pkv.paged_attention_decode(d["q"], d["k"], d["v"], d["tables"], d["lens"], lse_out=lse_t,
                                     scale=float(w.scale), partition_size=part)
    torch.cuda.synchronize()
    return out, lse_t


def oracle_check(w, out, lse, where):
    ref, ref_lse = oracle.paged_attention(*oracle_inputs(w), w.scale, w.block_size)
    check_attention(host(out), ref, w.dtype, where)
    if lse is not None:
        check_lse(host(lse), ref_lse, where)


SHAPES = [  # (dtype, D, Hq, Hkv, T)
    ("fp32", 64, 4, 4, 1), ("fp32", 64, 8, 2, 1), ("fp32", 128, 8, 2, 1), ("fp32", 128, 16, 4, 3),
    ("bf16", 64, 8, 8, 1), ("bf16", 64, 8, 4, 2), ("bf16", 64, 16, 4, 1), ("bf16", 64, 16, 2, 5),
    ("bf16", 128, 8, 8, 1), ("bf16", 128, 8, 4, 1), ("bf16", 128, 32, 8, 1), ("bf16", 128, 32, 8, 4),
    ("bf16", 128, 16, 4, 16), ("bf16", 128, 32, 4, 1), ("bf16", 128, 32, 4, 2), ("fp32", 64, 16, 4, 4),
]


@pytest.mark.parametrize("dtype,D,Hq,Hkv,T", SHAPES)
@pytest.mark.parametrize("part", [0, 32])
def test_shapes_and_edge_lengths(dtype, D, Hq, Hkv, T, part):
    """Lengths at block edges (1, 15, 16, 17, 33) and a ragged mix, several GQA ratios and T."""
    lens = [max(T, L) for L in (1, 15, 16, 17, 33, 70, 129)]
    w = workload.uniform_batch("shape", seed=7, B=len(lens), T=T, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, lens=lens)
    say("shape", dtype, D, Hq, Hkv, T, "part", part)
    d = upload(w)
    out, lse = decode(w, d, part)
    oracle_check(w, out, lse, f"{dtype} D={D} Hq={Hq} Hkv={Hkv} T={T} part={part}")


@pytest.mark.parametrize("factor", [4.0, 64.0])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_sharp_and_overflowing_scores(factor, dtype):
    """q x4 sharpens the softmax; q x64 pushes scores past the exp range without max subtraction."""
    w = workload.uniform_batch("sharp", seed=8, B=5, T=1, Hq=8, Hkv=2, D=64, dtype=dtype,
                               lens=[3, 40, 300, 1000, 17])
    w = workload.scaled_queries(w, factor)
    say("sharp", dtype, factor)
    d = upload(w)
    for part in (0, 64):
        out, lse = decode(w, d, part)
        ref, ref_lse = oracle.paged_attention(*oracle_inputs(w), w.scale, w.block_size)
        got = host(out)
        assert np.isfinite(got).all()
        if dtype == "bf16":
            check_attention(got, ref, "bf16", f"sharp x{factor} part={part}")
        else:
            # fp32 score error grows with |score| (~|s| * 2^-24 * sqrt(D)); the gate scales with the largest score
            smax = np.abs(ref_lse).max()
            assert np.abs(got - ref).max() <= 1e-5 * max(1.0, smax / 4), f"x{factor}"
        check_lse(host(lse), ref_lse, f"sharp x{factor}")


@pytest.mark.parametrize("factor", [4.0, 64.0])
def test_verify_tile_sharp_and_overflowing_scores(factor):
    """The same two variants through the MFMA verify tile (T*G = 16 rows)."""
    w = workload.uniform_batch("vsharp", seed=9, B=4, T=4, Hq=16, Hkv=4, D=128, dtype="bf16",
                               lens=[4, 40, 300, 1000])
    w = workload.scaled_queries(w, factor)
    say("verify sharp", factor)
    out, lse = decode(w, upload(w), 0)
    ref, ref_lse = oracle.paged_attention(*oracle_inputs(w), w.scale, w.block_size)
    check_attention(host(out), ref, "bf16", f"verify q x{factor}", floor=mfma_floor(w))
    check_lse(host(lse), ref_lse, f"verify q x{factor}")


def test_split_sizes_agree_and_runs_are_deterministic():
    w = workload.llama1b_gqa_append(partition_size=512)
    say("split sizes", w.name)
    d = upload(w)
    pkv.paged_kv_append(d["k_new"], d["v_new"], d["k"], d["v"], d["tables"], d["lens_pre"])
    outs = {}
    for part in (0, 16, 256, 512, 4096):
        o1, l1 = decode(w, d, part)
        o2, l2 = decode(w, d, part)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"part={part} not deterministic"
        outs[part] = (host(o1), host(l1))
    base_o, base_l = outs[0]
    for part, (o, l) in outs.items():
        assert_within_bf16_ulp(o, base_o, f"part={part} vs unsplit", floor=2 * mfma_floor(w))
        np.testing.assert_allclose(l, base_l, rtol=0, atol=1e-4)


def test_physical_permutation_bit_identical():
    w = workload.tinylm_mha_bf16()
    w2 = workload.relabel_physical(w, seed=77)
    say("permutation")
    for part in (0, 64):
        o1, l1 = decode(w, upload(w), part)
        o2, l2 = decode(w2, upload(w2), part)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_verify_rows_equal_decode_chain():
    """T=4 verify row t at length L equals a T=1 decode at length L-3+t (cached decode == full prefix)."""
    T = 4
    lens = [16, 17, 18, 19, 515, 516, 1027]
    w = workload.uniform_batch("chain", seed=9, B=len(lens), T=T, Hq=32, Hkv=8, D=128, dtype="bf16", lens=lens)
    d = upload(w)
    say("verify chain")
    for part in (0, 512):
        o4, l4 = decode(w, d, part)
        for t in range(T):
            qt = d["q"][:, t:t + 1].contiguous()
            lens_t = (d["lens"] - (T - 1 - t)).contiguous()
            lse1 = torch.empty((w.B, 1, w.Hq), device="cuda")
            o1 = pkv.paged_attention_decode(qt, d["k"], d["v"], d["tables"], lens_t, lse_out=lse1,
                                            scale=float(w.scale), partition_size=part)
            torch.cuda.synchronize()
            assert_within_bf16_ulp(host(o1)[:, 0], host(o4)[:, t], f"verify row {t} vs decode",
                                   floor=2 * mfma_floor(w))
            np.testing.assert_allclose(host(lse1)[:, 0], host(l4)[:, t], rtol=0, atol=1e-4)
        oracle_check(w, o4, l4, f"verify part={part}")


@pytest.mark.parametrize("D", [64, 128])
def test_verify_piece_visible_only_to_later_rows(D):
    """Balanced split with pieces of 16 blocks: a piece that is the last block alone, visible only to the
    later query tokens (L in 257..259, T=4), must leave the earlier rows empty, not NaN."""
    T = 4
    lens = [257, 258, 259, 300, 16 * 33 + 2]
    w = workload.uniform_batch("late_rows", seed=12, B=len(lens), T=T, Hq=16, Hkv=4, D=D, dtype="bf16", lens=lens)
    d = upload(w)
    say("late rows", D)
    out, lse = decode(w, d, 0)
    oracle_check(w, out, lse, f"late rows D={D}")


def test_fully_masked_partition_rows():
    """T=4 and L mod 512 in {1,2,3}: the last partition is empty for the first rows (lse -inf, o 0)."""
    T = 4
    lens = [513, 514, 515, 1025, 2050]
    w = workload.uniform_batch("masked", seed=10, B=len(lens), T=T, Hq=32, Hkv=8, D=128, dtype="bf16", lens=lens)
    d = upload(w)
    say("masked partitions")
    part = 512
    ws_bytes = pkv.pkv_decode_workspace_bytes(w.B, T, w.Hq, w.D, w.max_blocks, 16, part)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    lse = torch.empty((w.B, T, w.Hq), device="cuda")
    out = pkv.paged_attention_decode(d["q"], d["k"], d["v"], d["tables"], d["lens"], lse_out=lse,
                                     scale=float(w.scale), partition_size=part, workspace=ws)
    torch.cuda.synchronize()
    oracle_check(w, out, lse, "masked")
    P_max = math.ceil(w.max_blocks * 16 / part)
    rows = w.B * T * w.Hq
    po = ws[: rows * P_max * w.D * 4].view(torch.float32).view(w.B, T, w.Hq, P_max, w.D)
    pl = ws[rows * P_max * w.D * 4: rows * P_max * (w.D + 1) * 4].view(torch.float32).view(w.B, T, w.Hq, P_max)
    ref_o, ref_l = oracle.partition_attention(*oracle_inputs(w), w.scale, w.block_size, part, num_parts=P_max)
    got_o, got_l = host(po), host(pl)
    vmax = max_abs_finite(w, w.v_pool)
    for b, L in enumerate(lens):
        Pb = math.ceil(L / part)
        check_partials(got_o[b, :, :, :Pb], got_l[b, :, :, :Pb], ref_o[b, :, :, :Pb], ref_l[b, :, :, :Pb], vmax,
                       f"partials b={b}")
    assert np.isneginf(got_l[0, 0, :, 1]).all() and not got_o[0, 0, :, 1].any()


@pytest.mark.parametrize("T,Hq,Hkv,D,part", [(1, 32, 8, 128, 512), (4, 32, 8, 128, 512), (2, 16, 4, 64, 1024),
                                             (1, 8, 8, 64, 256)])
def test_tile_partitions_span_several_ranges(T, Hq, Hkv, D, part):
    """A batch small enough that the balanced ranges (16 blocks at least) are
    shorter than a partition, so most partitions are cut by one or more range
    boundaries and rebuilt from pieces by the merge.  Output, lse and every
    partition's partial against the oracle."""
    lens = [max(T, L) for L in (1500, 2049, 700, 3333, 15, 512 + 2, 4096)]
    w = workload.uniform_batch("span", seed=60 + T, B=len(lens), T=T, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16", lens=lens)
    say("tile partitions across ranges", T, Hq, Hkv, D, part)
    d = upload(w)
    ws = torch.empty(pkv.pkv_decode_workspace_bytes(w.B, T, Hq, D, w.max_blocks, 16, part), dtype=torch.uint8,
                     device="cuda")
    lse = torch.full((w.B, T, Hq), float("nan"), device="cuda")
    out = pkv.paged_attention_decode(d["q"], d["k"], d["v"], d["tables"], d["lens"], lse_out=lse,
                                     scale=float(w.scale), partition_size=part, workspace=ws)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.paged_attention(*oracle_inputs(w), w.scale, w.block_size)
    check_attention(host(out), ref, "bf16", f"span T={T} part={part}", floor=mfma_floor(w))
    check_lse(host(lse), ref_lse, f"span T={T} part={part}")
    P_max = math.ceil(w.max_blocks * 16 / part)
    rows = w.B * T * Hq
    po = ws[: rows * P_max * D * 4].view(torch.float32).view(w.B, T, Hq, P_max, D)
    pl = ws[rows * P_max * D * 4: rows * P_max * (D + 1) * 4].view(torch.float32).view(w.B, T, Hq, P_max)
    ref_o, ref_l = oracle.partition_attention(*oracle_inputs(w), w.scale, w.block_size, part, num_parts=P_max)
    got_o, got_l = host(po), host(pl)
    vmax = max_abs_finite(w, w.v_pool)
    for b, L in enumerate(lens):
        Pb = math.ceil(L / part)
        if Pb > 1:   # single-partition sequences go straight to out
            check_partials(got_o[b, :, :, :Pb], got_l[b, :, :, :Pb], ref_o[b, :, :, :Pb], ref_l[b, :, :, :Pb],
                           vmax, f"span partials b={b}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_lse_reduce_abi(dtype, D):
    """lse_reduce on oracle partials (with empty -inf partitions holding NaN) vs the oracle merge."""
    rng = np.random.default_rng(40)
    B, T, Hq, P = 3, 2, 4, 7
    o = rng.standard_normal((B, T, Hq, P, D)).astype(np.float32)
    l = (rng.standard_normal((B, T, Hq, P)) * 6).astype(np.float32)
    l[0, 0, 0, 2:] = -np.inf
    o[0, 0, 0, 2:] = np.nan
    l[1, 1, 3, :] = -np.inf
    o[1, 1, 3, :] = np.nan
    ref_o, ref_l = oracle.lse_combine(o, l)
    out = torch.empty((B, T, Hq, D), dtype=torch.float32 if dtype == "fp32" else torch.bfloat16, device="cuda")
    lse = torch.empty((B, T, Hq), device="cuda")
    say("lse_reduce", dtype, D)
    pkv.lse_reduce(torch.from_numpy(o).cuda(), torch.from_numpy(l).cuda(), out, lse)
    torch.cuda.synchronize()
    got = host(out)
    assert np.isfinite(got).all()
    assert not got[1, 1, 3].any() and np.isneginf(host(lse)[1, 1, 3])
    if dtype == "fp32":
        np.testing.assert_allclose(got, ref_o, rtol=0, atol=2e-6)
    else:
        check_attention(got, ref_o, "bf16", "lse_reduce")
    check_lse(host(lse), ref_l, "lse_reduce")


def test_empty_batch_and_single_partition_identity():
    B, T, Hq, D, P = 2, 1, 4, 64, 1
    o = torch.randn(B, T, Hq, P, D, device="cuda")
    l = torch.randn(B, T, Hq, P, device="cuda")
    out = torch.empty(B, T, Hq, D, device="cuda")
    lse = torch.empty(B, T, Hq, device="cuda")
    pkv.lse_reduce(o, l, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out, o[:, :, :, 0]) and torch.equal(lse, l[..., 0])
    lib = pkv.load_library()
    assert lib.paged_attention_decode(None, None, None, None, None, None, None, 0, 1, 4, 4, 64, 16, 1, 1, 0.125, 0,
                                      None, 0, 0, None) == 0


@pytest.mark.parametrize("T", [1, 2])
def test_many_heads_long_batch(T):
    """64 query heads (two decode workgroups per range) over a batch long
    enough that ranges exceed their minimum length, so each XCD takes a
    contiguous run of ranges: every row against the oracle."""
    rng = np.random.default_rng(17)
    lens = rng.integers(2000, 4000, size=16).tolist()
    w = workload.uniform_batch("many-heads", seed=19 + T, B=16, T=T, Hq=64, Hkv=8, D=128, dtype="bf16", lens=lens)
    say("many heads long batch", T)
    d = upload(w)
    out, lse = decode(w, d, 0)
    oracle_check(w, out, lse, f"Hq=64 long batch T={T}")
