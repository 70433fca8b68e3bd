"""The balanced split plans its ranges inside the decode launch while the
unit list fits the workgroup's LDS (B*T + 1 <= 256 entries per wave for the
VALU stream kernel, B + 1 <= 512 per wave for the MFMA tile) and with a
separate planning kernel beyond that.  Which one runs follows from the shape
alone, so the cases sit on both sides of each capacity and every output is
checked against the oracle.  Cases: unit lists just under and at the LDS
capacity of every workgroup width, ranges that span hundreds of one-block
units (query staging refilled many times), one long sequence among many short
ones (a unit cut by many range boundaries), multi-row units (T > 1 on the
VALU path) and a batch smaller than the number of ranges."""
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


def run(w, d):
    lse = torch.full((w.B, w.T, w.Hq), float("nan"), device="cuda")
    out = pkv.paged_attention_decode(d["q"], d["k"], d["v"], d["tables"], d["lens"], lse_out=lse,
                                     scale=float(w.scale), partition_size=0)
    torch.cuda.synchronize()
    return host(out), host(lse)


def check_with_oracle(w, where):
    d = upload(w)
    o, l = run(w, d)
    o2, l2 = run(w, d)
    assert np.array_equal(o, o2) and np.array_equal(l, l2), f"{where}: two runs differ"
    ref, ref_lse = oracle.paged_attention(*oracle_inputs(w), w.scale, w.block_size)
    check_attention(o, ref, w.dtype, where)
    check_lse(l, ref_lse, where)


# (dtype, D, Hq, Hkv) of single-token decode on the VALU stream kernel (fp32,
# or bf16 with more than 8 KV heads, not a multiple of 8, which the tile does
# not take): workgroups of Hq/4 waves up to 8, LDS list of 256 entries per wave
WIDTHS = [("bf16", 128, 12, 12), ("bf16", 64, 24, 12), ("fp32", 64, 32, 8), ("fp32", 64, 4, 4)]


@pytest.mark.parametrize("dtype,D,Hq,Hkv", WIDTHS)
@pytest.mark.parametrize("edge", [-1, 0])
def test_unit_list_at_lds_capacity(dtype, D, Hq, Hkv, edge):
    """B = capacity - 1 (planned inline) and B = capacity (too many units:
    the planning kernel runs first)."""
    cap = 256 * min(Hq // 4, 8)
    B = cap + edge
    rng = np.random.Generator(np.random.PCG64(11 + B))
    lens = rng.integers(1, 49, size=B)
    w = workload.uniform_batch("cap", seed=12, B=B, T=1, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, lens=lens)
    say("cap", dtype, D, Hq, Hkv, "B", B)
    check_with_oracle(w, f"{dtype} Hq={Hq} B={B}")


def test_one_long_among_many_short():
    """One 20000-token sequence between 600 one- and two-block sequences: the
    long unit is cut by many range boundaries, the short ones pack hundreds
    to a range."""
    rng = np.random.Generator(np.random.PCG64(21))
    lens = list(rng.integers(1, 33, size=300)) + [20000] + list(rng.integers(1, 33, size=300))
    w = workload.uniform_batch("long-short", seed=22, B=len(lens), T=1, Hq=32, Hkv=8, D=128, dtype="bf16",
                               lens=lens)
    say("long among short")
    check_with_oracle(w, "long among short")


@pytest.mark.parametrize("dtype,D,Hq,Hkv,T", [("bf16", 128, 32, 8, 5), ("fp32", 64, 16, 4, 3),
                                              ("bf16", 64, 8, 2, 16)])
def test_multi_row_units(dtype, D, Hq, Hkv, T):
    """T > 1 outside the MFMA verify tile: each of the T rows of a sequence is
    its own unit, with its own causal limit."""
    rng = np.random.Generator(np.random.PCG64(31 + T))
    lens = np.maximum(T, rng.integers(1, 400, size=30))   # B*T + 1 within every LDS list
    w = workload.uniform_batch("rows", seed=32, B=len(lens), T=T, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, lens=lens)
    say("rows", dtype, D, Hq, Hkv, T)
    check_with_oracle(w, f"{dtype} T={T}")


def test_fewer_blocks_than_ranges():
    """Three sequences, 11 blocks in all: one range of work, every other workgroup idle."""
    w = workload.uniform_batch("few", seed=41, B=3, T=1, Hq=32, Hkv=8, D=128, dtype="bf16", lens=[1, 40, 100])
    say("few")
    check_with_oracle(w, "few blocks")


@pytest.mark.parametrize("Hq,Hkv,T,D,B", [(8, 2, 4, 128, 1023), (8, 2, 4, 128, 1024), (32, 8, 2, 64, 4095)])
def test_verify_prefix_at_lds_capacity(Hq, Hkv, T, D, B):
    """Verify tile (T*G <= 16 rows per KV head), LDS list of 512 entries per
    wave: B + 1 at the capacity (planned inline) and one past it (planning
    kernel)."""
    rng = np.random.Generator(np.random.PCG64(51 + B))
    lens = rng.integers(T, 80, size=B)
    w = workload.uniform_batch("vcap", seed=52, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16", lens=lens)
    say("verify cap", Hq, Hkv, T, D, "B", B)
    check_with_oracle(w, f"verify Hq={Hq} Hkv={Hkv} T={T} B={B}")
