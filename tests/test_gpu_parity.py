"""GPU parity: the HIP library (through its C ABI) against the fp64 CPU oracle.

Integer/byte work (append, gather) must be bit-exact; attention outputs must
meet the gates in gpu_util.  Every case is printed before it runs."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import workload
import paged_kv_cache_attention_amd as pkv
from gpu_util import (appended_oracle_pools, check_attention, check_lse, check_partials, dev, host, max_abs_finite,
                      mfma_floor, oracle_by_sequence, oracle_inputs, upload)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def c1():
    return workload.tiny_fp32()


@pytest.fixture(scope="module")
def c2():
    return workload.tinylm_mha_bf16()


@pytest.fixture(scope="module")
def c3():
    return workload.llama1b_gqa_append()


def run_decode(w, d, partition_size=None, with_lse=True):
    part = w.partition_size if partition_size is None else partition_size
    lse = torch.full((w.B, w.T, w.Hq), float("nan"), dtype=torch.float32, device="cuda") if with_lse else None
    out = pkv.paged_attention_decode(d["q"], d["k"], d["v"], d["tables"], d["lens"], lse_out=lse,
                                     scale=float(w.scale), partition_size=part)
    torch.cuda.synchronize()
    return out, lse


# ---------------------------------------------------------------- gather / append (bit-exact)

@pytest.mark.parametrize("name", ["tiny_fp32", "tinylm_mha_bf16", "llama1b_gqa_append"])
def test_gather_bit_exact(name):
    w = workload.WORKLOADS[name]()
    say("gather", name)
    d = upload(w)
    max_len = w.max_blocks * w.block_size
    k_out = torch.empty((w.B, max_len, w.Hkv, w.D), dtype=d["k"].dtype, device="cuda")
    v_out = torch.empty_like(k_out)
    pkv.paged_kv_gather(d["k"], d["v"], d["tables"], d["lens"], k_out, v_out)
    torch.cuda.synchronize()
    kh, vh = host(k_out), host(v_out)
    kp, vp = w.values(w.k_pool), w.values(w.v_pool)
    for b in range(w.B):
        L = int(w.context_lens[b])
        np.testing.assert_array_equal(kh[b, :L], oracle.gather_sequence(kp, w.block_tables[b], L, w.block_size))
        np.testing.assert_array_equal(vh[b, :L], oracle.gather_sequence(vp, w.block_tables[b], L, w.block_size))
        assert not kh[b, L:].any() and not vh[b, L:].any()


def test_append_bit_exact(c3):
    w = c3
    say("append", w.name)
    d = upload(w)
    pkv.paged_kv_append(d["k_new"], d["v_new"], d["k"], d["v"], d["tables"], d["lens_pre"])
    torch.cuda.synchronize()
    kp, vp = appended_oracle_pools(w)
    # compare storage bytes of the whole pool: appended slots and every canary byte elsewhere
    got_k = d["k"].view(torch.int16).cpu().numpy().view(np.uint16)
    got_v = d["v"].view(torch.int16).cpu().numpy().view(np.uint16)
    want_k = workload.f32_to_bf16_bits(kp.astype(np.float32))
    want_v = workload.f32_to_bf16_bits(vp.astype(np.float32))
    np.testing.assert_array_equal(got_k, want_k)
    np.testing.assert_array_equal(got_v, want_v)


def test_append_block_boundaries():
    """Pre-append lengths 15, 16, 31 and 0: the new row lands in a fresh or partly filled block."""
    w = workload.uniform_batch("append_edges", seed=31, B=4, T=1, Hq=8, Hkv=2, D=128, dtype="bf16",
                               lens=[16, 17, 32, 1], append=True)
    say("append edges", list(w.lens_pre))
    d = upload(w)
    pkv.paged_kv_append(d["k_new"], d["v_new"], d["k"], d["v"], d["tables"], d["lens_pre"])
    torch.cuda.synchronize()
    kp, vp = appended_oracle_pools(w)
    np.testing.assert_array_equal(host(d["k"]), kp)
    np.testing.assert_array_equal(host(d["v"]), vp)


# ---------------------------------------------------------------- attention parity

def test_tiny_fp32(c1):
    say("decode tiny_fp32")
    d = upload(c1)
    out, lse = run_decode(c1, d)
    ref, ref_lse = oracle.paged_attention(*oracle_inputs(c1), c1.scale, c1.block_size)
    check_attention(host(out), ref, "fp32", "tiny_fp32")
    check_lse(host(lse), ref_lse, "tiny_fp32")


@pytest.mark.parametrize("part", [0, 16, 64, 512])
def test_tinylm_mha_bf16(c2, part):
    say("decode tinylm_mha_bf16 partition", part)
    d = upload(c2)
    out, lse = run_decode(c2, d, partition_size=part)
    ref, ref_lse = oracle.paged_attention(*oracle_inputs(c2), c2.scale, c2.block_size)
    check_attention(host(out), ref, "bf16", f"tinylm part={part}")
    check_lse(host(lse), ref_lse, f"tinylm part={part}")


@pytest.mark.parametrize("part", [0, 512])
def test_llama1b_append_then_decode(c3, part):
    w = c3
    say("append+decode llama1b partition", part)
    d = upload(w)
    pkv.paged_kv_append(d["k_new"], d["v_new"], d["k"], d["v"], d["tables"], d["lens_pre"])
    out, lse = run_decode(w, d, partition_size=part)
    kp, vp = appended_oracle_pools(w)
    ref, ref_lse = oracle.paged_attention(w.values(w.q), kp, vp, w.block_tables, w.context_lens, w.scale,
                                          w.block_size)
    check_attention(host(out), ref, "bf16", f"llama1b part={part}")
    check_lse(host(lse), ref_lse, f"llama1b part={part}")


@pytest.fixture(scope="module")
def c4():
    """The 8B-shaped prefix-sharing batch (256 sequences), uploaded once, with
    the oracle's result for every sequence."""
    w = workload.llama8b_prefix_share()
    return w, upload(w), oracle_by_sequence(w)


@pytest.mark.parametrize("part", [0, 512])
def test_llama8b_prefix_share_full(c4, part):
    """The 8B-shaped prefix-sharing batch at full size, single pass (the
    launch configuration the benchmark times) and split into 512-token
    partitions: every one of the 256 sequences against the oracle."""
    w, d, (ref, ref_lse) = c4
    say("decode llama8b_prefix_share, all sequences, partition", part)
    out, lse = run_decode(w, d, partition_size=part)
    check_attention(host(out), ref, "bf16", f"llama8b part={part}", floor=mfma_floor(w))
    check_lse(host(lse), ref_lse, f"llama8b part={part}")


def test_llama8b_prefix_share_groups_not_adjacent(c4):
    """The same batch with its sequences reordered so that the members of a
    prefix group are 16 places apart: no sequence shares a block with its
    neighbours, so the tile streams V of the shared prefixes too (a cache
    hint only).  Every sequence against the oracle."""
    w, d, (ref, ref_lse) = c4
    perm = np.array([(i % 16) * 16 + i // 16 for i in range(w.B)])
    assert len(set(perm.tolist())) == w.B
    idx = torch.from_numpy(perm).cuda()
    dp = dict(q=d["q"].index_select(0, idx).contiguous(), k=d["k"], v=d["v"],
              tables=d["tables"].index_select(0, idx).contiguous(), lens=d["lens"].index_select(0, idx).contiguous())
    say("decode llama8b_prefix_share, groups spread over the batch")
    out, lse = run_decode(w, dp, partition_size=0)
    check_attention(host(out), ref[perm], "bf16", "llama8b groups not adjacent", floor=mfma_floor(w))
    check_lse(host(lse), ref_lse[perm], "llama8b groups not adjacent")


@pytest.fixture(scope="module")
def c5():
    """The long-context verify batch (16 sequences of 16K-64K tokens, T = 4),
    uploaded once, with the oracle's result for every sequence."""
    w = workload.longctx_verify()
    say("longctx lens", list(w.context_lens))
    ref = oracle_by_sequence(w)
    return w, upload(w), ref


def test_longctx_verify_full(c5):
    """Single pass (balanced split): all 16 sequences against the oracle."""
    w, d, (ref, ref_lse) = c5
    say("verify longctx, partition 0")
    out, lse = run_decode(w, d, partition_size=0)
    check_attention(host(out), ref, "bf16", "longctx part=0", floor=mfma_floor(w))
    check_lse(host(lse), ref_lse, "longctx part=0")


def test_longctx_verify_512_token_partitions(c5):
    """As configured: the KV split into 512-token partitions from position 0,
    each emitting a normalised partial and its log-sum-exp, merged by
    log-sum-exp.  Output and lse of all 16 sequences against the oracle, and
    the partials left in the workspace against the oracle's partitions for
    the two sequences with the most partitions (P_b > 64, so the merge runs
    its chunked loop over more than 64 partials)."""
    w, d, (ref, ref_lse) = c5
    part = 512
    ws_bytes = pkv.pkv_decode_workspace_bytes(w.B, w.T, w.Hq, w.D, w.max_blocks, w.block_size, part)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    lse = torch.full((w.B, w.T, w.Hq), float("nan"), dtype=torch.float32, device="cuda")
    say("verify longctx, partition 512")
    out = pkv.paged_attention_decode(d["q"], d["k"], d["v"], d["tables"], d["lens"], lse_out=lse,
                                     scale=float(w.scale), partition_size=part, workspace=ws)
    torch.cuda.synchronize()
    check_attention(host(out), ref, "bf16", "longctx part=512", floor=mfma_floor(w))
    check_lse(host(lse), ref_lse, "longctx part=512")
    P_max = -(-w.max_blocks * w.block_size // part)
    rows = w.B * w.T * w.Hq
    po = ws[: rows * P_max * w.D * 4].view(torch.float32).view(w.B, w.T, w.Hq, P_max, w.D)
    pl = ws[rows * P_max * w.D * 4: rows * P_max * (w.D + 1) * 4].view(torch.float32).view(w.B, w.T, w.Hq, P_max)
    Pb = -(-w.context_lens.astype(np.int64) // part)
    seqs = [int(b) for b in np.argsort(-Pb, kind="stable")[:2]]
    assert all(Pb[b] > 64 for b in seqs)
    ref_o, ref_l = oracle_by_sequence(w, seqs, partition_size=part)
    vmax = max_abs_finite(w, w.v_pool)
    for i, b in enumerate(seqs):
        n = int(Pb[b])
        say("  partials of sequence", b, "P_b", n)
        check_partials(host(po[b, :, :, :n]), host(pl[b, :, :, :n]), ref_o[i, :, :, :n], ref_l[i, :, :, :n], vmax,
                       f"longctx partials b={b}")
