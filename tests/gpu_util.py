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


def max_abs_finite(w, arr):
    """Largest finite |value| of a storage array (NaN poison ignored)."""
    if w.dtype == "bf16":   # on the bit patterns: |x| orders like its low 15 bits
        mag = np.asarray(arr, dtype=np.uint16).ravel() & np.uint16(0x7FFF)
        mag = mag[mag < 0x7F80]
        return float(w.values(np.array([mag.max(initial=0)], dtype=np.uint16))[0])
    return float(np.nanmax(np.abs(np.asarray(arr, dtype=np.float32))))


def mfma_floor(w):
    """Near-zero floor of the MFMA tiles for workload w: 2^-16 max |V| (+ ULP_FLOOR)."""
    vmax = max_abs_finite(w, w.v_pool)
    if w.v_new is not None:
        vmax = max(vmax, max_abs_finite(w, w.v_new))
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


# The prefill tile rounds P once to bf16 for its P.V product (fp32
# accumulation, the denominator summed from the unrounded p).  bf16 keeps 8
# significant bits, so p~ = p (1 + e) with |e| <= 2^-8, and an output element
# moves by at most 2^-8 sum_j p_j |v_j| / l: attention over |V| ("abs_ref",
# the oracle's own definition applied to |V|) scaled by 2^-8.  The margin of
# 2^-11 on top covers fp32 accumulation and the exp2 approximation.
P_BF16_REL = 2.0 ** -8 + 2.0 ** -11


def check_attention_pbf16(got, ref, abs_ref, where=""):
    """bf16 attention with P rounded to bf16: per element
    |got - ref| <= b + 0.5 ulp(|ref| + b), b = P_BF16_REL * abs_ref + ULP_FLOOR
    (the computed value is within b of ref and then rounded to bf16); the
    stated max-abs 1.5e-2 wherever that bound is tighter (as in
    check_attention, bf16 rounding alone exceeds it beyond |out| = 2); and a
    relative Frobenius error within 4e-3."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    abs_ref = np.asarray(abs_ref, dtype=np.float64)
    assert got.shape == ref.shape == abs_ref.shape
    assert np.isfinite(got).all(), f"{where}: non-finite output"
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    b = P_BF16_REL * abs_ref + ULP_FLOOR
    tol = b + 0.5 * oracle.bf16_ulp(np.abs(ref) + b)
    assert (err <= np.maximum(BF16_ATOL, tol)).all(), f"{where}: max abs {err.max():.3e}"
    assert rel <= BF16_REL_FRO, f"{where}: rel fro {rel:.3e}"
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err / (b + 1e-30), 0)), err.shape)
        raise AssertionError(f"{where}: {int(bad.sum())} elements beyond the P-rounding bound; worst at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r} bound {b[i]:.3e}")
    return float(err.max()), float(rel)


def assert_within_bf16_ulp(got, base, where="", floor=ULP_FLOOR):
    """Two bf16 results agree to one ulp (or `floor` for near-zero values)."""
    got = np.asarray(got, dtype=np.float64)
    base = np.asarray(base, dtype=np.float64)
    assert np.isfinite(got).all() and np.isfinite(base).all(), where
    d = np.abs(got - base)
    bad = (d > oracle.bf16_ulp(base)) & (d > floor)
    assert not bad.any(), f"{where}: {int(bad.sum())} elements differ by more than 1 ulp; max diff {d.max():.3e}"


def check_lse(got, ref, where=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    both_inf = np.isneginf(got) & np.isneginf(ref)
    # empty rows must be -inf on both sides; they are taken out before subtracting
    g = np.where(both_inf, 0.0, got)
    r = np.where(both_inf, 0.0, ref)
    assert np.isfinite(g).all() and np.isfinite(r).all(), f"{where}: lse -inf/NaN where the other side is finite"
    d = np.abs(g - r)
    assert d.max(initial=0.0) <= LSE_ATOL + 1e-6 * np.abs(r).max(initial=0.0), f"{where}: lse max abs {d.max():.3e}"


def _compact(w, b, k_vals=None, v_vals=None):
    """Sequence b's own blocks as a small pool with table 0 .. nb-1 (a
    relabelling of physical ids, which leaves attention unchanged), widened
    from storage only for those blocks unless float pools are given."""
    nb = -(-int(w.context_lens[b]) // w.block_size)
    ids = np.asarray(w.block_tables[b, :nb], dtype=np.int64)
    kp = k_vals[ids] if k_vals is not None else w.values(w.k_pool[ids])
    vp = v_vals[ids] if v_vals is not None else w.values(w.v_pool[ids])
    return kp, vp, np.arange(nb, dtype=np.int64)[None, :]


def oracle_by_sequence(w, seqs=None, k_vals=None, v_vals=None, partition_size=0, threads=8):
    """The oracle on each listed sequence (all by default), one compact pool
    per sequence, in a thread pool.  Returns (out, lse) stacked over seqs, or
    with partition_size > 0 the oracle's partition partials (o, lse) with
    P_max = ceil(max_blocks * block_size / partition_size)."""
    from concurrent.futures import ThreadPoolExecutor
    seqs = list(range(w.B)) if seqs is None else list(seqs)
    qv = w.values(w.q)
    P_max = -(-w.max_blocks * w.block_size // partition_size) if partition_size else 0

    def one(b):
        kp, vp, tab = _compact(w, b, k_vals, v_vals)
        args = (qv[b:b + 1], kp, vp, tab, w.context_lens[b:b + 1], w.scale, w.block_size)
        if partition_size:
            return oracle.partition_attention(*args, partition_size, num_parts=P_max)
        return oracle.paged_attention(*args)

    with ThreadPoolExecutor(max(1, min(threads, len(seqs)))) as ex:
        res = list(ex.map(one, seqs))
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])


def check_partials(got_o, got_l, ref_o, ref_l, vmax, where):
    """fp32 split-KV partials (normalised o_p and lse_p) against the oracle's.
    Gate for o_p: 2^-16 max|V| (the MFMA tiles' hi + lo split of P) + 2e-6
    (fp32 accumulation); empty partitions must be exactly (0, -inf)."""
    got_o = np.asarray(got_o, dtype=np.float64)
    ref_o = np.asarray(ref_o, dtype=np.float64)
    check_lse(got_l, ref_l, where)
    empty = np.isneginf(np.asarray(ref_l))
    assert not got_o[empty].any(), f"{where}: empty partition with nonzero o"
    err = np.abs(got_o - ref_o)
    gate = MFMA_P_REL * vmax + 2e-6
    assert np.isfinite(got_o).all() and err.max(initial=0.0) <= gate, \
        f"{where}: partial max abs {err.max():.3e} > {gate:.3e}"
