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
from gpu_util import (appended_oracle_pools, check_attention, check_lse, dev, host, oracle_inputs, upload)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)



@pytest.fixture(autouse=True, params=["tile", "stream"])
def decode_kernel(request, monkeypatch):
    """Single-token decode through the MFMA tile and through the VALU stream
    kernel (PKV_DECODE_TILE, read by the library on each call)."""
    monkeypatch.setenv("PKV_DECODE_TILE", "1" if request.param == "tile" else "0")
    return request.param

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


def test_llama8b_prefix_share_full():
    w = workload.llama8b_prefix_share()
    say("decode llama8b_prefix_share partition", w.partition_size)
    d = upload(w)
    out, lse = run_decode(w, d)
    seqs = list(range(0, w.B, 5)) + [int(np.argmax(w.context_lens))]
    ref, ref_lse = oracle.paged_attention(*oracle_inputs(w, seqs), w.scale, w.block_size)
    check_attention(host(out)[seqs], ref, "bf16", "llama8b")
    check_lse(host(lse)[seqs], ref_lse, "llama8b")


def test_longctx_verify_full():
    w = workload.longctx_verify()
    say("verify longctx partition", w.partition_size, "lens", list(w.context_lens))
    d = upload(w)
    out, lse = run_decode(w, d)
    got, got_lse = host(out), host(lse)
    for b in [0, int(np.argmax(w.context_lens)), 7]:
        ref, ref_lse = oracle.paged_attention(*oracle_inputs(w, [b]), w.scale, w.block_size)
        check_attention(got[[b]], ref, "bf16", f"longctx b={b}")
        check_lse(got_lse[[b]], ref_lse, f"longctx b={b}")
        say("  sequence", b, "ok")
