"""The balanced split with its plan computed inside the decode launch (the
default while the unit list fits the workgroup's LDS: B*T + 1 <= 256 entries
per wave) against the same split planned by the separate planning kernel
(PKV_INLINE_PLAN=0, read by the library on each call).  Both plans are the
same numbers, so the outputs must agree bit for bit; each case is also checked
against the oracle.  Cases: unit lists just under and at the LDS capacity of
every workgroup width, ranges that span hundreds of one-block units (query
staging refilled many times), one long sequence among many short ones (a unit
cut by many range boundaries), multi-row units (T > 1 on the VALU path) and a
batch smaller than the number of ranges.  The multi-query verify tile plans
the same way (per-sequence block prefix sums, 512 LDS entries per wave)."""
import numpy as np
import pytest
import torch

import oracle
import workload
import paged_kv_cache_attention_amd as pkv
from gpu_util import check_attention, check_lse, host, oracle_inputs, upload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def run(w, d, monkeypatch, inline):
    monkeypatch.setenv("PKV_INLINE_PLAN", "1" if inline else "0")
    lse = torch.full((w.B, w.T, w.Hq), float("nan"), device="cuda")
    out = pkv.paged_attention_decode(d["q"], d["k"], d["v"], d["tables"], d["lens"], lse_out=lse,
                                     scale=float(w.scale), partition_size=0)
    torch.cuda.synchronize()
    return host(out), host(lse)


def both_plans_and_oracle(w, monkeypatch, where):
    d = upload(w)
    o_in, l_in = run(w, d, monkeypatch, True)
    o_pk, l_pk = run(w, d, monkeypatch, False)
    assert np.array_equal(o_in, o_pk), f"{where}: outputs differ between the two plans"
    assert np.array_equal(l_in, l_pk), f"{where}: lse differs between the two plans"
    ref, ref_lse = oracle.paged_attention(*oracle_inputs(w), w.scale, w.block_size)
    check_attention(o_in, ref, w.dtype, where)
    check_lse(l_in, ref_lse, where)


# (dtype, D, Hq, Hkv): workgroups of Hq/4 waves up to 8, LDS list of 256 entries per wave
WIDTHS = [("bf16", 128, 32, 8), ("bf16", 64, 16, 4), ("bf16", 64, 8, 8), ("fp32", 64, 4, 4)]


@pytest.mark.parametrize("dtype,D,Hq,Hkv", WIDTHS)
@pytest.mark.parametrize("edge", [-1, 0])
def test_unit_list_at_lds_capacity(monkeypatch, dtype, D, Hq, Hkv, edge):
    """B = capacity - 1 (planned inline) and B = capacity (too many units:
    the planning kernel runs even with the inline plan switched on)."""
    cap = 256 * min(Hq // 4, 8)
    B = cap + edge
    rng = np.random.Generator(np.random.PCG64(11 + B))
    lens = rng.integers(1, 49, size=B)
    w = workload.uniform_batch("cap", seed=12, B=B, T=1, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, lens=lens)
    say("cap", dtype, D, Hq, Hkv, "B", B)
    both_plans_and_oracle(w, monkeypatch, f"{dtype} Hq={Hq} B={B}")


def test_one_long_among_many_short(monkeypatch):
    """One 20000-token sequence between 600 one- and two-block sequences: the
    long unit is cut by many range boundaries, the short ones pack hundreds
    to a range."""
    rng = np.random.Generator(np.random.PCG64(21))
    lens = list(rng.integers(1, 33, size=300)) + [20000] + list(rng.integers(1, 33, size=300))
    w = workload.uniform_batch("long-short", seed=22, B=len(lens), T=1, Hq=32, Hkv=8, D=128, dtype="bf16",
                               lens=lens)
    say("long among short")
    both_plans_and_oracle(w, monkeypatch, "long among short")


@pytest.mark.parametrize("dtype,D,Hq,Hkv,T", [("bf16", 128, 32, 8, 5), ("fp32", 64, 16, 4, 3),
                                              ("bf16", 64, 8, 2, 16)])
def test_multi_row_units(monkeypatch, dtype, D, Hq, Hkv, T):
    """T > 1 outside the MFMA verify tile: each of the T rows of a sequence is
    its own unit, with its own causal limit."""
    rng = np.random.Generator(np.random.PCG64(31 + T))
    lens = np.maximum(T, rng.integers(1, 400, size=30))   # B*T + 1 within every LDS list
    w = workload.uniform_batch("rows", seed=32, B=len(lens), T=T, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, lens=lens)
    say("rows", dtype, D, Hq, Hkv, T)
    both_plans_and_oracle(w, monkeypatch, f"{dtype} T={T}")


def test_fewer_blocks_than_ranges(monkeypatch):
    """Three sequences, 11 blocks in all: one range of work, every other workgroup idle."""
    w = workload.uniform_batch("few", seed=41, B=3, T=1, Hq=32, Hkv=8, D=128, dtype="bf16", lens=[1, 40, 100])
    say("few")
    both_plans_and_oracle(w, monkeypatch, "few blocks")


def test_llama8b_shape_both_plans(monkeypatch):
    """The 8B-shaped prefix-sharing batch: both plans give the same bits; a
    sample of sequences against the oracle."""
    w = workload.llama8b_prefix_share()
    d = upload(w)
    say("8B both plans")
    o_in, l_in = run(w, d, monkeypatch, True)
    o_pk, l_pk = run(w, d, monkeypatch, False)
    assert np.array_equal(o_in, o_pk) and np.array_equal(l_in, l_pk)
    sel = list(range(3, 256, 23))
    ref, ref_lse = oracle.paged_attention(*oracle_inputs(w, sel), w.scale, w.block_size)
    check_attention(o_in[sel], ref, "bf16", "8B sample")
    check_lse(l_in[sel], ref_lse, "8B sample")


@pytest.mark.parametrize("Hq,Hkv,T,D,B", [(8, 2, 4, 128, 1023), (8, 2, 4, 128, 1024), (32, 8, 2, 64, 4095)])
def test_verify_prefix_at_lds_capacity(monkeypatch, Hq, Hkv, T, D, B):
    """Verify tile (T*G <= 16 rows per KV head), LDS list of 512 entries per
    wave: B + 1 at the capacity (planned inline) and one past it (planning
    kernel)."""
    rng = np.random.Generator(np.random.PCG64(51 + B))
    lens = rng.integers(T, 80, size=B)
    w = workload.uniform_batch("vcap", seed=52, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16", lens=lens)
    say("verify cap", Hq, Hkv, T, D, "B", B)
    both_plans_and_oracle(w, monkeypatch, f"verify Hq={Hq} Hkv={Hkv} T={T} B={B}")


def test_longctx_verify_both_plans(monkeypatch):
    """The long-context verify batch: both plans give the same bits; two
    sequences against the oracle."""
    w = workload.longctx_verify()
    d = upload(w)
    say("longctx both plans")
    o_in, l_in = run(w, d, monkeypatch, True)
    o_pk, l_pk = run(w, d, monkeypatch, False)
    assert np.array_equal(o_in, o_pk) and np.array_equal(l_in, l_pk)
    sel = [0, 9]
    ref, ref_lse = oracle.paged_attention(*oracle_inputs(w, sel), w.scale, w.block_size)
    check_attention(o_in[sel], ref, "bf16", "longctx sample")
    check_lse(l_in[sel], ref_lse, "longctx sample")
