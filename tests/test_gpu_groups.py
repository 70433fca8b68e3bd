"""Batches whose block tables share leading physical blocks (common prompt
prefixes, "vLLM and PagedAttention", memory sharing), against the oracle.

Adjacent sequences that start with the same physical block are attended as a
group over their common blocks; these cases cover the group boundaries: short
members that stop inside the shared prefix, a shared partial last block,
runs that cross the 16-sequence windows, runs longer than a group, sharing
between non-adjacent sequences, too-short shares and several GQA ratios."""
import numpy as np
import pytest
import torch

import oracle
import workload
import paged_kv_cache_attention_amd as pkv
from gpu_util import check_attention, check_lse, host, oracle_inputs, upload

pytestmark = pytest.mark.gpu
BS = workload.BLOCK_SIZE


@pytest.fixture(autouse=True, params=["groups", "plain"])
def group_switch(request, monkeypatch):
    """Every case runs with the shared-prefix group path switched on
    (PKV_PREFIX_GROUPS=1, read by the library on each call) and off."""
    monkeypatch.setenv("PKV_PREFIX_GROUPS", "1" if request.param == "groups" else "0")
    return request.param


def cdiv(a, b):
    return -(-a // b)


def build_lists(spec):
    """spec: list of (L, prefix_key or None, shared_blocks).  A sequence with a
    prefix key takes min(shared_blocks, its block count) blocks of that prefix,
    then private blocks."""
    per_seq = []
    for b, (L, key, nshare) in enumerate(spec):
        n = cdiv(L, BS)
        per_seq.append([(key, i) if key is not None and i < nshare else (b, i) for i in range(n)])
    return [L for L, _, _ in spec], per_seq


def mixed_spec(rng):
    spec = []
    # 0..15: one 20-block prefix; members stop before, at and after its end
    for L in (5, 17, 100, 319, 320, 321, 333, 640, 1000, 1500, 2000, 48, 800, 700, 401, 999):
        spec.append((L, "p0", 20))
    # 16..20: identical tables, lengths inside the same last block (shared partial block)
    for L in (200, 203, 207, 208, 150):
        spec.append((L, "p1", cdiv(208, BS)))
    # 21..52: a 32-sequence run crossing windows at 32 and 48
    for _ in range(32):
        spec.append((int(rng.integers(100, 1500)), "p2", 9))
    # 53, 55 share, 54 in between does not (not adjacent)
    spec.append((600, "p3", 12))
    spec.append((600, None, 0))
    spec.append((600, "p3", 12))
    # 56, 57: only 2 shared blocks (dissolved group)
    spec.append((300, "p4", 2))
    spec.append((310, "p4", 2))
    # 58: alone; 59..63: share exactly kGroupMinShare blocks
    spec.append((77, None, 0))
    for L in (64, 65, 90, 400, 64):
        spec.append((L, "p5", 4))
    return spec


def run(w, part=0):
    d = upload(w)
    lse = torch.full((w.B, w.T, w.Hq), float("nan"), device="cuda")
    out = pkv.paged_attention_decode(d["q"], d["k"], d["v"], d["tables"], d["lens"], lse_out=lse,
                                     scale=float(w.scale), partition_size=part)
    torch.cuda.synchronize()
    return host(out), host(lse)


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (32, 8, 64), (8, 8, 64), (64, 8, 128), (16, 8, 128)])
def test_shared_prefix_groups_match_oracle(Hq, Hkv, D):
    rng = np.random.Generator(np.random.PCG64(90))
    lens, per_seq = build_lists(mixed_spec(rng))
    w = workload.batch_from_block_lists("groups", seed=91, T=1, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16", lens=lens,
                                        per_seq_blocks=per_seq)
    print("groups", Hq, Hkv, D, "B", w.B, flush=True)
    out, lse = run(w)
    ref, ref_lse = oracle.paged_attention(*oracle_inputs(w), w.scale, w.block_size)
    check_attention(out, ref, "bf16", f"groups Hq={Hq} Hkv={Hkv} D={D}")
    check_lse(lse, ref_lse, "groups lse")


def test_whole_batch_one_table():
    """Every sequence uses the same table; lengths differ (beam-like fan-out)."""
    rng = np.random.Generator(np.random.PCG64(92))
    lens = [int(x) for x in rng.integers(1, 1200, size=40)]
    nmax = cdiv(max(lens), BS)
    per_seq = [[("s", i) for i in range(cdiv(L, BS))] for L in lens]
    w = workload.batch_from_block_lists("one_table", seed=93, T=1, Hq=32, Hkv=8, D=128, dtype="bf16", lens=lens,
                                        per_seq_blocks=per_seq, max_blocks=nmax)
    print("one table B", w.B, flush=True)
    out, lse = run(w)
    ref, ref_lse = oracle.paged_attention(*oracle_inputs(w), w.scale, w.block_size)
    check_attention(out, ref, "bf16", "one table")
    check_lse(lse, ref_lse, "one table lse")


def test_groups_invariant_under_physical_relabel():
    """Relabelling physical ids keeps the sharing structure: identical bits."""
    rng = np.random.Generator(np.random.PCG64(94))
    lens, per_seq = build_lists(mixed_spec(rng))
    w = workload.batch_from_block_lists("groups", seed=95, T=1, Hq=32, Hkv=8, D=128, dtype="bf16", lens=lens,
                                        per_seq_blocks=per_seq)
    print("relabel B", w.B, flush=True)
    out_a, lse_a = run(w)
    out_b, lse_b = run(workload.relabel_physical(w, 96))
    assert np.array_equal(out_a, out_b)
    assert np.array_equal(lse_a, lse_b)


def test_prefix_share_workload_repeatable():
    """The prefix-sharing 8B batch twice in a row: identical bits (no state kept between calls)."""
    w = workload.llama8b_prefix_share()
    d = upload(w)
    outs = []
    for _ in range(2):
        out = pkv.paged_attention_decode(d["q"], d["k"], d["v"], d["tables"], d["lens"], scale=float(w.scale),
                                         partition_size=0)
        torch.cuda.synchronize()
        outs.append(host(out))
    assert np.array_equal(outs[0], outs[1])
    sel = list(range(0, 256, 17))
    ref, _ = oracle.paged_attention(*oracle_inputs(w, sel), w.scale, w.block_size)
    check_attention(outs[0][sel], ref, "bf16", "8B prefix share sample")
