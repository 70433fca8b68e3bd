"""The binding on a stream other than torch's current one (a default-priority
side stream, as a serving loop uses): the library launches there, and the
workspace and outputs the binding allocates come from that stream's pool, so
work the current stream allocates meanwhile cannot take that memory while the
kernels still use it.  Every result is compared bit for bit with the same
call on the current stream, and the append with the oracle's pools."""
import numpy as np
import pytest
import torch

import oracle
import workload
import paged_kv_cache_attention_amd as pkv
from gpu_util import appended_oracle_pools, check_attention, check_lse, host, mfma_floor, oracle_inputs, upload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def churn():
    """Allocate, fill and free device memory on the current stream."""
    junk = [torch.full((4 << 20,), 7.0, dtype=torch.float32, device="cuda") for _ in range(4)]
    del junk


@pytest.mark.parametrize("part", [0, 512])
def test_decode_on_side_stream_bit_identical(part):
    w = workload.uniform_batch("side-stream", seed=91, B=24, T=1, Hq=32, Hkv=8, D=128, dtype="bf16",
                               lens=np.random.default_rng(91).integers(1, 3000, size=24))
    d = upload(w)
    say("decode on a side stream, partition", part)
    lse_ref = torch.full((w.B, w.T, w.Hq), float("nan"), device="cuda")
    ref = pkv.paged_attention_decode(d["q"], d["k"], d["v"], d["tables"], d["lens"], lse_out=lse_ref,
                                     scale=float(w.scale), partition_size=part)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()   # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lse = torch.full((w.B, w.T, w.Hq), float("nan"), device="cuda")
    out = pkv.paged_attention_decode(d["q"], d["k"], d["v"], d["tables"], d["lens"], lse_out=lse,
                                     scale=float(w.scale), partition_size=part, stream=side)
    churn()
    side.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "side-stream output differs"
    assert torch.equal(lse, lse_ref), "side-stream lse differs"
    r, rl = oracle.paged_attention(*oracle_inputs(w), w.scale, w.block_size)
    check_attention(host(out), r, "bf16", f"side stream part={part}", floor=mfma_floor(w))
    check_lse(host(lse), rl, f"side stream part={part}")


def test_append_then_prefill_on_side_stream():
    """Append a 96-token chunk per sequence, then attend it causally, both on
    the side stream; the pools and the output against the current stream's."""
    rng = np.random.default_rng(92)
    T = 96
    lens = rng.integers(T + 1, 1500, size=6)
    w = workload.uniform_batch("side-prefill", seed=92, B=6, T=T, Hq=32, Hkv=8, D=128, dtype="bf16", lens=lens,
                               append=True)
    say("append + prefill on a side stream")
    results = []
    for use_side in (False, True):
        d = upload(w)
        side = torch.cuda.Stream() if use_side else None
        if side is not None:
            side.wait_stream(torch.cuda.current_stream())
        pkv.paged_kv_append(d["k_new"], d["v_new"], d["k"], d["v"], d["tables"], d["lens_pre"], stream=side)
        out = pkv.paged_attention_prefill(d["q"], d["k"], d["v"], d["tables"], d["lens"], scale=float(w.scale),
                                          stream=side)
        if side is not None:
            churn()
            side.synchronize()
        else:
            torch.cuda.synchronize()
        bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
        results.append((bits(d["k"]), bits(d["v"]), bits(out)))
    for a, b, what in zip(results[0], results[1], ("k pool", "v pool", "prefill output")):
        assert np.array_equal(a, b), f"side stream: {what} differs"
    kp, vp = appended_oracle_pools(w)
    np.testing.assert_array_equal(results[1][0], workload.f32_to_bf16_bits(kp.astype(np.float32)))
    np.testing.assert_array_equal(results[1][1], workload.f32_to_bf16_bits(vp.astype(np.float32)))
