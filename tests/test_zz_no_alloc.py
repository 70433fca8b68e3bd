"""The allocation-free decode entry point (static device scratch) against
paged_attention_decode with a caller workspace: identical bits, two calls in a
row with the second batch smaller than the first (the scratch keeps the first
call's contents), each also checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workload
import paged_kv_cache_attention_amd as pkv
from gpu_util import check_attention, check_lse, host, mfma_floor, oracle_inputs, upload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def both(w, part):
    d = upload(w)
    lse_a = torch.full((w.B, w.T, w.Hq), float("nan"), device="cuda")
    out_a = pkv.paged_attention_decode(d["q"], d["k"], d["v"], d["tables"], d["lens"], lse_out=lse_a,
                                       scale=float(w.scale), partition_size=part)
    lse_b = torch.full_like(lse_a, float("nan"))
    out_b = torch.full_like(d["q"], float("nan"))
    pkv.paged_attention_decode_noalloc(d["q"], d["k"], d["v"], d["tables"], d["lens"], out_b, lse_out=lse_b,
                                       scale=float(w.scale), partition_size=part)
    torch.cuda.synchronize()
    return out_a, lse_a, out_b, lse_b


@pytest.mark.parametrize("part", [0, 512])
def test_noalloc_matches_workspace_entry_point(part):
    big = workload.uniform_batch("noalloc-big", seed=81, B=48, T=1, Hq=32, Hkv=8, D=128, dtype="bf16",
                                 lens=np.random.default_rng(81).integers(1, 3000, size=48))
    small = workload.uniform_batch("noalloc-small", seed=82, B=5, T=4, Hq=16, Hkv=4, D=64, dtype="bf16",
                                   lens=[4, 17, 300, 1030, 2049])
    for w in (big, small):
        say("noalloc", w.name, "partition", part)
        out_a, lse_a, out_b, lse_b = both(w, part)
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), f"{w.name}: outputs differ"
        assert torch.equal(lse_a, lse_b), f"{w.name}: lse differs"
        ref, ref_lse = oracle.paged_attention(*oracle_inputs(w), w.scale, w.block_size)
        check_attention(host(out_b), ref, "bf16", f"noalloc {w.name}", floor=mfma_floor(w))
        check_lse(host(lse_b), ref_lse, f"noalloc {w.name}")
