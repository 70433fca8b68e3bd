"""Block tables that share physical blocks, as prefix caching leaves them
("Inference From Scratch", What you will build and Chapters table, ch. 11:
prefix caching reuses KV blocks across requests): groups of sequences whose
tables start with the same physical blocks for different lengths, trees of
shared prefixes, groups that straddle each other in the batch, members
shorter than the shared prefix or ending inside a shared block, every query
rows per KV head ratio.  Each case is checked against the oracle, for
determinism, and against the same logical data with every block copied to a
private physical block: the result may not depend on which blocks are
shared."""
import dataclasses

import numpy as np
import pytest
import torch

import workload
import paged_kv_cache_attention_amd as pkv
from gpu_util import (assert_within_bf16_ulp, check_attention, check_lse, host, mfma_floor, oracle_by_sequence,
                      upload)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def shared_batch(name, seed, T, Hq, Hkv, D, lens, share):
    """share[b] = (group, blocks of the group's prefix chain sequence b uses);
    its remaining blocks are its own."""
    per_seq = []
    for b, L in enumerate(lens):
        n = -(-L // 16)
        g, s = share[b]
        s = min(s, n)
        per_seq.append([("p", g, i) for i in range(s)] + [(b, i) for i in range(s, n)])
    return workload.batch_from_block_lists(name, seed=seed, T=T, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16", lens=lens,
                                           per_seq_blocks=per_seq)


def privatised(w):
    """The same logical K/V with every sequence's blocks copied to blocks of
    its own (tables 0 .. n-1 after the previous sequence's), poison kept."""
    nbs = [-(-int(L) // 16) for L in w.context_lens]
    ids = np.concatenate([w.block_tables[b, :n] for b, n in enumerate(nbs)] + [[w.poison_block]])
    tables = np.full_like(w.block_tables, len(ids) - 1)
    off = 0
    for b, n in enumerate(nbs):
        tables[b, :n] = np.arange(off, off + n)
        off += n
    return dataclasses.replace(w, k_pool=w.k_pool[ids], v_pool=w.v_pool[ids], block_tables=tables,
                                        N_blocks=len(ids), poison_block=len(ids) - 1)


def run(w, d):
    lse = torch.full((w.B, w.T, w.Hq), float("nan"), device="cuda")
    out = pkv.paged_attention_decode(d["q"], d["k"], d["v"], d["tables"], d["lens"], lse_out=lse,
                                     scale=float(w.scale), partition_size=0)
    torch.cuda.synchronize()
    return out, lse


def check_case(w, where):
    d = upload(w)
    o1, l1 = run(w, d)
    o2, l2 = run(w, d)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2), f"{where}: not deterministic"
    ref, ref_lse = oracle_by_sequence(w)
    floor = mfma_floor(w)
    check_attention(host(o1), ref, "bf16", where, floor=floor)
    check_lse(host(l1), ref_lse, where)
    wp = privatised(w)
    op, lp = run(wp, upload(wp))
    assert_within_bf16_ulp(host(o1), host(op), f"{where}: shared vs private blocks", floor=2 * floor)
    np.testing.assert_allclose(host(l1), host(lp), rtol=0, atol=1e-4)


def test_groups_with_short_and_ragged_members():
    """Groups of 8 sequences sharing 40 blocks: members shorter than the
    prefix (1, 15, 200 tokens), members ending inside the last shared block,
    one longer than the longest other member inside its last block."""
    lens, share = [], []
    for g in range(3):
        for L in (1, 15, 200, 640, 641, 700, 3000, 40 * 16 - 3):
            lens.append(L + g)
            share.append((g, 40))
    w = shared_batch("groups", 70, 1, 32, 8, 128, lens, share)
    say("groups", lens)
    check_case(w, "groups")


def test_windows_across_group_boundaries():
    """Groups of 3, 5, 2 and 6 adjacent sequences sharing 20 blocks each."""
    sizes = [3, 5, 2, 6]
    rng = np.random.default_rng(71)
    lens, share = [], []
    for g, n in enumerate(sizes):
        for _ in range(n):
            lens.append(int(rng.integers(100, 2500)))
            share.append((g, 20))
    w = shared_batch("straddle", 71, 1, 32, 8, 128, lens, share)
    say("straddle", lens)
    check_case(w, "straddle")


def test_tree_of_prefixes_and_long_chain():
    """G = 4, D = 64: members sharing 150, 90 and 150 blocks of one chain
    whose longest member has 188; a tree of members sharing 10, 5 and 90
    blocks of the same chain; two members of another chain and one of a
    third."""
    lens = [2400, 3000, 2400, 2560, 2400, 1000, 160, 2400, 1600, 2000, 77]
    share = [(0, 150), (0, 150), (0, 90), (0, 150), (0, 10), (0, 5), (0, 10), (0, 90), (1, 64), (1, 64), (2, 5)]
    w = shared_batch("tree", 72, 1, 16, 4, 64, lens, share)
    say("tree", lens)
    check_case(w, "tree")


@pytest.mark.parametrize("T,Hq,Hkv,D", [(2, 32, 8, 128), (1, 8, 8, 64), (1, 64, 8, 128), (4, 8, 8, 128),
                                        (1, 16, 8, 64)])
def test_window_sizes(T, Hq, Hkv, D):
    """T G = 8, 1, 8, 4 and 2 query rows per KV head, groups of 7 sequences
    sharing 1 to 33 blocks."""
    rng = np.random.default_rng(73 + T + Hq)
    lens, share = [], []
    for b in range(21):
        lens.append(int(rng.integers(T, 1200)))
        share.append((b // 7, int(rng.integers(1, 34))))
    w = shared_batch("wsize", 73, T, Hq, Hkv, D, lens, share)
    say("window sizes", T, Hq, Hkv, D)
    check_case(w, f"T={T} Hq={Hq} Hkv={Hkv} D={D}")
