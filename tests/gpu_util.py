"""Helpers for the GPU parity tests: upload seeded workloads, read results back,
and the comparison gates."""
from __future__ import annotations

import numpy as np
import torch

import oracle

# Gates.  fp32: the stated max-abs 1e-5, plus the same bound on the relative
# Frobenius error.  bf16 (fp32 accumulate, bf16 output): the stated max-abs
# 1.5e-2; a relative Frobenius bound of 4e-3 (bf16 output rounding alone gives
# about 2^-9/sqrt(3) ~ 1.1e-3); and every element within one bf16 ulp of the
# correctly rounded reference unless it is within ULP_FLOOR of the exact value
# (near-zero outputs, where fp32 accumulation error of the summed terms is
# several ulps of the tiny result).
ULP_FLOOR = 1e-5
# MFMA tiles (verify, prefill) multiply P as bf16 hi + lo parts: |p - hi - lo|
# <= 2^-16 |p| (two roundings to 8-bit significands), so an output element
# sum_j p_j v_j / l is off by at most 2^-16 max_j |v_j| before accumulation
# error.  That bound, not ULP_FLOOR, is their floor for near-zero elements
# (cancelling sums of O(1) terms).
MFMA_P_REL = 2.0 ** -16
FP32_ATOL = 1e-5
BF16_ATOL = 1.5e-2
BF16_REL_FRO = 4e-3
LSE_ATOL = 2e-4


def dev(arr, dtype):
    a = np.ascontiguousarray(arr)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a.astype(np.float32, copy=False)).cuda()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def upload(w):
    d = dict(q=dev(w.q, w.dtype), k=dev(w.k_pool, w.dtype), v=dev(w.v_pool, w.dtype),
             tables=torch.from_numpy(w.block_tables.astype(np.int32)).cuda(),
             lens=torch.from_numpy(w.context_lens.astype(np.int32)).cuda())
    if w.lens_pre is not None:
        d["lens_pre"] = torch.from_numpy(w.lens_pre.astype(np.int32)).cuda()
        d["k_new"] = dev(w.k_new, w.dtype)
        d["v_new"] = dev(w.v_new, w.dtype)
    return d


def oracle_inputs(w, seqs=None):
    """(q, k_pool, v_pool, tables, lens) as float arrays, optionally for a subset of sequences."""
    sel = slice(None) if seqs is None else list(seqs)
    q = w.values(w.q)[sel]
    return q, w.values(w.k_pool), w.values(w.v_pool), w.block_tables[sel], w.context_lens[sel]


def appended_oracle_pools(w):
    kp, vp = oracle.kv_append(w.values(w.k_pool), w.values(w.v_pool), w.block_tables, w.lens_pre,
                              w.values(w.k_new), w.values(w.v_new), w.block_size)
    return kp, vp


def mfma_floor(w):
    """Near-zero floor of the MFMA tiles for workload w: 2^-16 max |V| (+ ULP_FLOOR)."""
    vmax = float(np.nanmax(np.abs(w.values(w.v_pool))))
    if w.v_new is not None:
        vmax = max(vmax, float(np.nanmax(np.abs(w.values(w.v_new)))))
    return MFMA_P_REL * vmax + ULP_FLOOR


def check_attention(got, ref, dtype, where="", floor=ULP_FLOOR):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    assert np.isfinite(got).all(), f"{where}: non-finite output"
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    if dtype == "fp32":
        assert err.max() <= FP32_ATOL, f"{where}: max abs {err.max():.3e}"
        assert rel <= FP32_ATOL, f"{where}: rel fro {rel:.3e}"
    else:
        atol = np.maximum(BF16_ATOL, 0.5 * oracle.bf16_ulp(ref) + 1e-5)
        assert (err <= atol).all(), f"{where}: max abs {err.max():.3e}"
        assert rel <= BF16_REL_FRO, f"{where}: rel fro {rel:.3e}"
        ulp_err = np.abs(got - oracle.round_to_bf16(ref)) / oracle.bf16_ulp(ref)
        bad = (ulp_err > 1.0) & (err > 0.5 * oracle.bf16_ulp(ref) + floor)
        if bad.any():
            i = np.unravel_index(np.argmax(np.where(bad, err, 0)), err.shape)
            raise AssertionError(f"{where}: {int(bad.sum())} elements more than 1 bf16 ulp off; worst at {i}: "
                                 f"got {got[i]!r} ref {ref[i]!r} ({ulp_err[i]:.2f} ulp)")
    return float(err.max()), float(rel)


def assert_within_bf16_ulp(got, base, where=""):
    """Two bf16 results agree to one ulp (or ULP_FLOOR for near-zero values)."""
    got = np.asarray(got, dtype=np.float64)
    base = np.asarray(base, dtype=np.float64)
    assert np.isfinite(got).all() and np.isfinite(base).all(), where
    d = np.abs(got - base)
    bad = (d > oracle.bf16_ulp(base)) & (d > ULP_FLOOR)
    assert not bad.any(), f"{where}: {int(bad.sum())} elements differ by more than 1 ulp; max diff {d.max():.3e}"


def check_lse(got, ref, where=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_inf = np.isneginf(got) & np.isneginf(ref)
    d = np.abs(np.where(both_inf, 0.0, got - ref))
    assert np.isfinite(d).all() and d.max() <= LSE_ATOL + 1e-6 * np.abs(np.where(both_inf, 0, ref)).max(), \
        f"{where}: lse max abs {d.max():.3e}"
