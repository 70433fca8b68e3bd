"""Chunked-prefill attention (paged_attention_prefill) against the oracle.

Query t of a T-token chunk sits at position L - T + t and sees keys
0 .. L - T + t, which is exactly the oracle's causal definition for any T.
Cases cover: a chunk with no cached prefix (L = T), prefixes ending on and
just past block and 32-key step boundaries, every GQA ratio, row groups that
fill only some waves of the workgroup, T = 1, sharp and overflowing scores,
poisoned unread slots, physical relabelling (bit-identical), repeatability,
and the 8B-shaped chunked-prefill batch (append then prefill) on sampled
sequences."""
import numpy as np
import pytest
import torch

import oracle
import workload
import paged_kv_cache_attention_amd as pkv
from gpu_util import (appended_oracle_pools, check_attention, check_attention_pbf16, check_lse, host, oracle_inputs,
                      upload)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def prefill(w, d, lse=True, piece_tokens=0):
    lse_t = torch.full((w.B, w.T, w.Hq), float("nan"), device="cuda") if lse else None
    out = torch.full_like(d["q"], float("nan"))
    pkv.paged_attention_prefill(d["q"], d["k"], d["v"], d["tables"], d["lens"], out=out, lse_out=lse_t,
                                scale=float(w.scale), piece_tokens=piece_tokens)
    torch.cuda.synchronize()
    return host(out), (host(lse_t) if lse else None)


def oracle_with_abs(q, kp, vp, tables, lens, scale, block_size):
    """The oracle's (out, lse) and its attention over |V| (the scale of the
    P-rounding bound of the prefill tile)."""
    ref, ref_lse = oracle.paged_attention(q, kp, vp, tables, lens, scale, block_size)
    abs_ref, _ = oracle.paged_attention(q, kp, np.abs(vp), tables, lens, scale, block_size)
    return ref, ref_lse, abs_ref


def check_vs_oracle(w, out, lse, where, seqs=None):
    ref, ref_lse, abs_ref = oracle_with_abs(*oracle_inputs(w, seqs), w.scale, w.block_size)
    sel = slice(None) if seqs is None else list(seqs)
    check_attention_pbf16(out[sel], ref, abs_ref, where)
    if lse is not None:
        check_lse(lse[sel], ref_lse, where)


SHAPES = [  # (D, Hq, Hkv, T, lens)
    (128, 32, 8, 64, [64, 65, 80, 96, 200, 333]),     # G=4, two row groups
    (64, 8, 8, 100, [100, 117, 260]),                 # G=1, last wave half full
    (128, 16, 8, 37, [37, 38, 500]),                  # G=2
    (64, 32, 4, 17, [17, 40, 1000]),                  # G=8, a second group of 8 rows
    (128, 32, 8, 1, [1, 30, 300]),                    # T=1 through the prefill path
    (128, 8, 8, 300, [300, 301, 700]),                # MHA, three row groups
    (64, 16, 4, 129, [129, 161, 192, 2000]),          # prefix ends on a 32-key step, long prefix
]


@pytest.mark.parametrize("D,Hq,Hkv,T,lens", SHAPES)
def test_prefill_shapes(D, Hq, Hkv, T, lens):
    w = workload.uniform_batch("prefill", seed=61 + T, B=len(lens), T=T, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16",
                               lens=lens)
    say("prefill", D, Hq, Hkv, T, lens)
    out, lse = prefill(w, upload(w))
    check_vs_oracle(w, out, lse, f"prefill D={D} Hq={Hq} Hkv={Hkv} T={T}")


@pytest.mark.parametrize("B,T,lmax", [(70, 40, 400), (520, 2, 60)])
def test_prefill_many_sequences(B, T, lmax):
    """Workgroups take their items longest first, the order searched over the
    lengths of all sequences: 70 sequences (more than one wave's worth, with
    repeated lengths, so ties in the order) and 520 (beyond the searched
    order, the plain order).  Every row and LSE is checked."""
    rng = np.random.default_rng(B)
    lens = rng.integers(T, lmax, size=B)
    lens[::7] = lens[0]
    w = workload.uniform_batch("many", seed=91 + B, B=B, T=T, Hq=4, Hkv=1, D=64, dtype="bf16", lens=lens.tolist())
    say("prefill many sequences", B, T)
    out, lse = prefill(w, upload(w))
    check_vs_oracle(w, out, lse, f"prefill B={B} T={T}")


@pytest.mark.parametrize("factor", [4.0, 64.0])
def test_prefill_sharp_and_overflowing_scores(factor):
    """q x4 sharpens the softmax; q x64 pushes scores far past the exp range."""
    w = workload.uniform_batch("sharp", seed=71, B=3, T=48, Hq=16, Hkv=4, D=128, dtype="bf16", lens=[48, 90, 400])
    w = workload.scaled_queries(w, factor)
    say("prefill sharp", factor)
    out, lse = prefill(w, upload(w))
    check_vs_oracle(w, out, lse, f"prefill q x{factor}")


def test_prefill_relabel_bit_identical_and_repeatable():
    w = workload.uniform_batch("relabel", seed=81, B=4, T=70, Hq=32, Hkv=8, D=128, dtype="bf16",
                               lens=[70, 100, 333, 1024])
    say("prefill relabel")
    d = upload(w)
    o1, l1 = prefill(w, d)
    o2, l2 = prefill(w, d)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    w2 = workload.relabel_physical(w, seed=5)
    o3, l3 = prefill(w2, upload(w2))
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


def test_prefill_rows_equal_decode_rows():
    """Row t of a chunk is the single-token decode of position L - T + t."""
    T = 20
    w = workload.uniform_batch("chain", seed=91, B=2, T=T, Hq=32, Hkv=8, D=128, dtype="bf16", lens=[60, 301])
    say("prefill vs decode rows")
    d = upload(w)
    out, _ = prefill(w, d, lse=False)
    for t in (0, 7, T - 1):
        lens_t = torch.from_numpy((w.context_lens - T + t + 1).astype(np.int32)).cuda()
        dec = pkv.paged_attention_decode(d["q"][:, t:t + 1].contiguous(), d["k"], d["v"], d["tables"], lens_t,
                                         scale=float(w.scale))
        torch.cuda.synchronize()
        ref, _, abs_ref = oracle_with_abs(w.values(w.q)[:, t:t + 1], w.values(w.k_pool), w.values(w.v_pool),
                                          w.block_tables, w.context_lens - T + t + 1, w.scale, w.block_size)
        check_attention_pbf16(out[:, t:t + 1], ref, abs_ref, f"prefill row {t}")
        check_attention(host(dec), ref, "bf16", f"decode row {t}")


def test_llama8b_chunked_prefill_full():
    """The 8B-shaped chunked-prefill batch as the benchmark runs it (append of
    the 512-token chunks, then prefill attention), sampled sequences against
    the oracle on the appended pools."""
    w = workload.llama8b_chunked_prefill()
    say("8B chunked prefill")
    d = upload(w)
    pkv.paged_kv_append(d["k_new"], d["v_new"], d["k"], d["v"], d["tables"], d["lens_pre"])
    out, lse = prefill(w, d)
    kp, vp = appended_oracle_pools(w)
    for b in (int(np.argmax(w.context_lens)), int(np.argmin(w.context_lens))):
        ref, ref_lse, abs_ref = oracle_with_abs(w.values(w.q)[b:b + 1], kp, vp, w.block_tables[b:b + 1],
                                                w.context_lens[b:b + 1], w.scale, w.block_size)
        check_attention_pbf16(out[b:b + 1], ref, abs_ref, f"8B prefill seq {b}")
        check_lse(lse[b:b + 1], ref_lse, f"8B prefill seq {b}")


def test_prefill_long_chunk_many_row_groups():
    """A 2048-token chunk after a 3000-token prefix and one with no prefix:
    64 row groups per KV head, key ranges up to 5048 (several LDS table
    windows of 512 blocks are not needed here, one window covers 8192 keys)."""
    w = workload.uniform_batch("long-chunk", seed=121, B=2, T=2048, Hq=8, Hkv=2, D=64, dtype="bf16",
                               lens=[2048 + 3000, 2048])
    say("prefill long chunk")
    out, lse = prefill(w, upload(w))
    check_vs_oracle(w, out, lse, "prefill T=2048")


def test_prefill_key_range_beyond_one_table_window():
    """Keys past 512 blocks (8192 tokens) make the tile reload its LDS table
    window mid-item."""
    w = workload.uniform_batch("window", seed=131, B=1, T=64, Hq=8, Hkv=8, D=64, dtype="bf16", lens=[8192 + 700])
    say("prefill table window")
    out, lse = prefill(w, upload(w))
    check_vs_oracle(w, out, lse, "prefill beyond a table window")


def test_prefill_maximum_chunk_sampled_rows():
    """The largest chunk the entry point takes (T = 8192) after an 8200-token
    prefix: 64 row groups of 128 rows per KV head, key ranges up to 16392
    (three LDS table windows).  Sampled rows, each checked as the
    one-token query at its own position (row t sees keys 0 .. L - T + t),
    with their LSE; every row must be finite."""
    T, pre = 8192, 8200
    w = workload.uniform_batch("max-chunk", seed=141, B=1, T=T, Hq=8, Hkv=8, D=64, dtype="bf16", lens=[pre + T])
    say("prefill maximum chunk")
    out, lse = prefill(w, upload(w))
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    rng = np.random.default_rng(7)
    rows = sorted({0, 1, 15, 16, 127, 128, 4095, 8191 - pre % 16, T - 2, T - 1, *rng.integers(0, T, size=6).tolist()})
    L = int(w.context_lens[0])
    for t in rows:
        ref, ref_lse, abs_ref = oracle_with_abs(w.values(w.q)[:, t:t + 1], w.values(w.k_pool), w.values(w.v_pool),
                                                w.block_tables, np.array([L - T + t + 1]), w.scale, w.block_size)
        check_attention_pbf16(out[:, t:t + 1], ref, abs_ref, f"max chunk row {t}")
        check_lse(lse[:, t:t + 1], ref_lse, f"max chunk row {t}")


PIECE_CASES = [  # (D, Hq, Hkv, T, lens, piece_tokens)
    (128, 32, 8, 64, [64, 65, 80, 96, 200, 333], 32),   # up to 11 pieces; rows with no key in later pieces
    (64, 16, 4, 129, [129, 161, 192, 2000], 96),        # pieces across 32-key steps and blocks
    (64, 8, 8, 100, [100, 117, 260], 64),
    (128, 16, 8, 37, [37, 38, 500], 160),               # some items in one piece, written directly
    (64, 32, 4, 17, [17, 40, 1000], 32),                # G = 8
    (128, 32, 8, 1, [1, 30, 300], 64),                  # T = 1: one row group, decode rows in pieces
    (128, 8, 8, 300, [300, 301, 700], 64),              # MHA: 300 rows, a full 256-row item and a partial one
    # grids of several waves of workgroups, pieces of mixed-length items ranked
    # ahead of the unsplit items: 40 and 70 sequences (the latter past 64, the
    # lengths in more than one register per lane)
    (128, 32, 8, 64, [64 + (i * 37) % 637 for i in range(40)], 64),
    (64, 16, 8, 8, [8 + (i * 53) % 300 for i in range(70)], 32),
]


@pytest.mark.parametrize("D,Hq,Hkv,T,lens,piece_tokens", PIECE_CASES)
def test_prefill_key_pieces(D, Hq, Hkv, T, lens, piece_tokens):
    """Items split into key pieces of piece_tokens tokens, one workgroup each,
    merged by log-sum-exp (at D = 128 the split launch runs 256-row items of
    8 waves): the oracle's result (and the unsplit call's, each within the
    P-rounding bound of the oracle), the unsplit call's LSE, and the same
    bits on a second call."""
    w = workload.uniform_batch("pieces", seed=151 + T, B=len(lens), T=T, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16",
                               lens=lens)
    say("prefill pieces", D, Hq, Hkv, T, lens, piece_tokens)
    d = upload(w)
    out, lse = prefill(w, d, piece_tokens=piece_tokens)
    check_vs_oracle(w, out, lse, f"prefill pieces of {piece_tokens} D={D} T={T}")
    out0, lse0 = prefill(w, d, piece_tokens=0)
    check_vs_oracle(w, out0, lse0, f"prefill unsplit D={D} T={T}")
    assert np.allclose(lse, lse0, atol=1e-4, rtol=0)
    out2, lse2 = prefill(w, d, piece_tokens=piece_tokens)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_prefill_key_pieces_overflowing_scores():
    """q x64: every piece has its own running max far from the others'."""
    w = workload.uniform_batch("sharp-pieces", seed=161, B=3, T=48, Hq=16, Hkv=4, D=128, dtype="bf16",
                               lens=[48, 90, 400])
    w = workload.scaled_queries(w, 64.0)
    say("prefill pieces q x64")
    out, lse = prefill(w, upload(w), piece_tokens=64)
    check_vs_oracle(w, out, lse, "prefill pieces q x64")


def test_prefill_one_sequence_long_prefix_suggested_pieces():
    """One 512-token chunk after an 8192-token prefix (the shape a serving
    loop prefills a long prompt in): 128 items, so the library suggests key
    pieces; sampled rows against the oracle, every row finite."""
    T, pre = 512, 8192
    w = workload.uniform_batch("one-long", seed=171, B=1, T=T, Hq=32, Hkv=8, D=128, dtype="bf16", lens=[pre + T])
    pt = pkv.pkv_prefill_piece_tokens(w.B, w.T, w.Hq, w.Hkv, w.D, w.block_size, w.max_blocks)
    say("prefill one long sequence, suggested pieces", pt)
    assert pt > 0
    out, lse = prefill(w, upload(w), piece_tokens=None)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    L = int(w.context_lens[0])
    rng = np.random.default_rng(3)
    for t in sorted({0, 1, 127, 128, 255, T - 1, *rng.integers(0, T, size=4).tolist()}):
        ref, ref_lse, abs_ref = oracle_with_abs(w.values(w.q)[:, t:t + 1], w.values(w.k_pool), w.values(w.v_pool),
                                                w.block_tables, np.array([L - T + t + 1]), w.scale, w.block_size)
        check_attention_pbf16(out[:, t:t + 1], ref, abs_ref, f"one long sequence row {t}")
        check_lse(lse[:, t:t + 1], ref_lse, f"one long sequence row {t}")
