"""Plain fp64 CPU oracle for paged decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg
use it.  It is deliberately slow and obvious: it rebuilds each sequence's
contiguous K/V from the block table and then evaluates softmax attention from
its definition in float64, with no blocking, fusion or online rescaling.

What the pages fix, and where:
  * The KV cache keeps each past key/value row so a decode step only computes
    the new token's query against all cached rows, and a cached decode must
    give the same result as recomputing the full prefix ("LLM Inference from
    Scratch", Architecture overview, M1 "prefill/decode equivalence"; "Efficient
    LLM Inference", learning route, "chunked computation equals a full-prefix
    forward pass").
  * The cache is paged: fixed-size physical blocks reached through a
    per-sequence block table ("Inference From Scratch", chapter table, ch. 10;
    "The Project", M13 mini-vLLM and M13b "paged greedy tokens equal the
    full-recompute reference").
  * Grouped-query attention: several query heads share one KV head ("The
    Project", milestone M2, MHA/GQA/MQA choice).
  * Online softmax / flash attention only reorganise this computation
    ("Inference From Scratch", chapter table, ch. 8); the oracle therefore does
    not use them.
  * A speculative verify step scores several drafted tokens with the big model
    in one pass ("LLM Inference from Scratch", M7): query token t of T sits at
    position L - T + t and sees keys 0 .. L - T + t.

Readings where the pages are silent (each also listed in the design notes):
  * query head h reads KV head h // (Hq / Hkv);
  * the context length L counts every cached token including the T query
    tokens; logical token j lives in slot j % block_size of physical block
    block_table[b][j // block_size];
  * a split-KV partition p covers logical tokens [p*P, (p+1)*P); each emits a
    normalised partial output and its natural-log log-sum-exp, and an empty
    partition emits (0, -inf); the partials combine by log-sum-exp weights.

Every input array may be float32 or float64; values are widened to float64.
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = float("-inf")


# --------------------------------------------------------------------------
# Small named helpers (kept separate so each reading is visible on its own).
# --------------------------------------------------------------------------

def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """GQA: query head h reads KV head h // (Hq/Hkv) (contiguous groups)."""
    return h // (Hq // Hkv)


def visible_tokens(L: int, T: int, t: int) -> int:
    """Number of keys query token t (of T) may attend to: positions 0 .. L-T+t."""
    return L - T + t + 1


def block_and_slot(j: int, block_size: int):
    """Logical token j -> (logical block index, slot inside the block)."""
    return j // block_size, j % block_size


# --------------------------------------------------------------------------
# Block-table gather and append (integer / byte work: exact).
# --------------------------------------------------------------------------

def gather_sequence(pool: np.ndarray, table_row: np.ndarray, length: int, block_size: int) -> np.ndarray:
    """Contiguous [length, Hkv, D] copy of one sequence's cached rows.

    Maps every logical token j through the block table, as the paged cache
    defines it; table entries past the last needed block are not read."""
    N, bs, Hkv, D = pool.shape
    assert bs == block_size
    j = np.arange(length)
    lb, slot = block_and_slot(j, block_size)
    phys = np.asarray(table_row)[lb].astype(np.int64)
    if length and (phys.min() < 0 or phys.max() >= N):
        raise IndexError(f"block table entry outside pool of {N} blocks")
    return pool[phys, slot]


def kv_append(k_pool, v_pool, block_tables, lens_pre, k_new, v_new, block_size):
    """Write T new rows per sequence at positions lens_pre[b] .. lens_pre[b]+T-1.

    Returns new pools; the inputs are not modified.  The target blocks must
    already be in the table (the caller's allocator places them)."""
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    B, T = k_new.shape[0], k_new.shape[1]
    N = k_pool.shape[0]
    for b in range(B):
        for t in range(T):
            pos = int(lens_pre[b]) + t
            lb, slot = block_and_slot(pos, block_size)
            phys = int(block_tables[b, lb])
            if not 0 <= phys < N:
                raise IndexError(f"block table entry {phys} outside pool of {N} blocks")
            k_out[phys, slot] = k_new[b, t]
            v_out[phys, slot] = v_new[b, t]
    return k_out, v_out


# --------------------------------------------------------------------------
# Attention from its definition.
# --------------------------------------------------------------------------

def softmax_attention_row(q_row: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """One query row against n key/value rows: (out[D], lse).

    out = sum_j softmax_j(scale * q.k_j) v_j; lse = log sum_j exp(scale * q.k_j).
    n == 0 gives (0, -inf)."""
    q64 = np.asarray(q_row, dtype=np.float64)
    K64 = np.asarray(K, dtype=np.float64)
    V64 = np.asarray(V, dtype=np.float64)
    D = q64.shape[0]
    if K64.shape[0] == 0:
        return np.zeros(D), NEG_INF
    s = float(scale) * (K64 @ q64)
    m = s.max()
    w = np.exp(s - m)
    z = w.sum()
    return (w @ V64) / z, m + math.log(z)


def paged_attention(q, k_pool, v_pool, block_tables, context_lens, scale, block_size):
    """Decode / verify attention over a paged cache.

    q: [B, T, Hq, D]; pools [N, block_size, Hkv, D]; block_tables [B, max_blocks];
    context_lens [B] (tokens cached, including the T query tokens).
    Returns (out [B, T, Hq, D] float64, lse [B, T, Hq] float64, natural log)."""
    B, T, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    out = np.zeros((B, T, Hq, D))
    lse = np.full((B, T, Hq), NEG_INF)
    for b in range(B):
        L = int(context_lens[b])
        if L < T:
            raise ValueError("context length must cover the query tokens")
        Kc = gather_sequence(k_pool, block_tables[b], L, block_size)
        Vc = gather_sequence(v_pool, block_tables[b], L, block_size)
        for t in range(T):
            n = visible_tokens(L, T, t)
            for h in range(Hq):
                kh = kv_head_of(h, Hq, Hkv)
                out[b, t, h], lse[b, t, h] = softmax_attention_row(q[b, t, h], Kc[:n, kh], Vc[:n, kh], scale)
    return out, lse


def num_partitions(L: int, partition_size: int) -> int:
    return -(-L // partition_size)


def partition_attention(q, k_pool, v_pool, block_tables, context_lens, scale, block_size, partition_size,
                        num_parts=None):
    """Split-KV partials: for each partition p, attention restricted to tokens
    [p*P, min((p+1)*P, visible)).  Returns (o [B,T,Hq,Pm,D], lse [B,T,Hq,Pm]);
    o is normalised within its partition, empty partitions are (0, -inf)."""
    B, T, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    if num_parts is None:
        num_parts = max(num_partitions(int(L), partition_size) for L in context_lens)
    o = np.zeros((B, T, Hq, num_parts, D))
    lse = np.full((B, T, Hq, num_parts), NEG_INF)
    for b in range(B):
        L = int(context_lens[b])
        Kc = gather_sequence(k_pool, block_tables[b], L, block_size)
        Vc = gather_sequence(v_pool, block_tables[b], L, block_size)
        for t in range(T):
            n = visible_tokens(L, T, t)
            for p in range(num_parts):
                lo, hi = p * partition_size, min((p + 1) * partition_size, n)
                if hi <= lo:
                    continue
                for h in range(Hq):
                    kh = kv_head_of(h, Hq, Hkv)
                    o[b, t, h, p], lse[b, t, h, p] = softmax_attention_row(
                        q[b, t, h], Kc[lo:hi, kh], Vc[lo:hi, kh], scale)
    return o, lse


def lse_combine(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge normalised partials by log-sum-exp weights over the last axis.

    o_parts [..., P, D], lse_parts [..., P].  With M = max_p lse_p and
    w_p = exp(lse_p - M): out = sum_p w_p o_p / sum_p w_p, lse = M + log sum_p w_p.
    Partitions with lse = -inf carry no weight and their o is never read; if
    every partition is empty the result is (0, -inf)."""
    o64 = np.asarray(o_parts, dtype=np.float64)
    l64 = np.asarray(lse_parts, dtype=np.float64)
    lead = l64.shape[:-1]
    D = o64.shape[-1]
    out = np.zeros(lead + (D,))
    lse = np.full(lead, NEG_INF)
    for idx in np.ndindex(*lead):
        ls = l64[idx]
        live = np.isfinite(ls)
        if not live.any():
            continue
        M = ls[live].max()
        w = np.exp(ls[live] - M)
        out[idx] = (w @ o64[idx][live]) / w.sum()
        lse[idx] = M + math.log(w.sum())
    return out, lse


# --------------------------------------------------------------------------
# Epilogue: fp32 accumulator -> storage dtype.
# --------------------------------------------------------------------------

def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value (8 significant bits), ties to even.

    Works on the float64 value directly: write |x| = m * 2^e with m in
    [0.5, 1), round m * 256 to an integer with ties to even, scale back.
    Zeros, infinities and NaN pass through."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.ldexp(np.round(m * 256.0), e - 8)
    return np.where(np.isfinite(x), r, x)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (for normal bf16 numbers)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.where(x > 0, x, 1.0))
    return np.ldexp(1.0, e - 8)
