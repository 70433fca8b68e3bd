"""Seeded synthetic inputs for paged decode attention.

This module only draws inputs: sequence lengths, physical block assignment
(block tables), and N(0,1) values for queries and the K/V block pools.  It
holds none of the attention arithmetic and is shared by the CPU oracle tests,
the GPU parity tests and the benchmark, so both sides see identical bytes.

Shapes follow the paged-KV layout used throughout: a pool of fixed-size
physical blocks ``[N_blocks, block_size, Hkv, D]`` addressed per sequence
through ``block_tables[B, max_blocks]`` (Inference From Scratch, chapter table,
"Paged attention, block tables"; The Project: Serve Your Own LLM, M13 "paged KV
cache").  The five workloads are shaped like the Llama-style decoders the pages
discuss (TinyLM's MHA decoder in "LLM Inference from Scratch", Architecture
overview; Llama-3.2-1B in "warpllama", Results) and extend them to an 8B-shaped
GQA batch with shared prefixes and a long-context speculative-verify batch.

Draw order for every workload (fixed so that a seed reproduces every byte):
lengths -> physical permutation -> q -> K pool -> V pool -> k_new -> v_new.
Values are float32 N(0,1); for bf16 workloads they are rounded to bf16 with
round-to-nearest-even on the float32 bit pattern.  ``poison=True`` writes NaN
into every pool slot that no sequence may read (unused blocks, the tail of a
sequence's last block, the slot an append is about to fill) and points table
padding at an all-NaN block, so any out-of-range read shows up as NaN.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BLOCK_SIZE = 16
BF16_NAN_BITS = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u + rounding) >> np.uint32(16)).astype(np.uint16)
    out[np.isnan(x)] = BF16_NAN_BITS
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Workload:
    """One batch of paged decode (or verify) attention inputs.

    ``context_lens[b]`` counts every token attention sees for sequence b,
    including the T query tokens and any token appended this step.
    ``lens_pre`` is set when the step starts with an append of T tokens: then
    ``context_lens == lens_pre + T`` and the appended slots are still empty
    (NaN when poisoned) until ``k_new``/``v_new`` are written there.
    Array members hold the storage form: float32 for ``dtype == "fp32"``,
    uint16 bf16 bit patterns for ``dtype == "bf16"``.
    """

    name: str
    B: int
    T: int
    Hq: int
    Hkv: int
    D: int
    block_size: int
    dtype: str
    partition_size: int
    context_lens: np.ndarray
    block_tables: np.ndarray
    N_blocks: int
    q: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    scale: np.float32
    poison_block: int
    lens_pre: Optional[np.ndarray] = None
    k_new: Optional[np.ndarray] = None
    v_new: Optional[np.ndarray] = None
    note: str = ""

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    def values(self, arr: Optional[np.ndarray]) -> Optional[np.ndarray]:
        """float32 values of a storage array (exact for bf16)."""
        if arr is None:
            return None
        if self.dtype == "bf16":
            return bf16_bits_to_f32(arr)
        return np.asarray(arr, dtype=np.float32)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


def _draw_values(rng: np.random.Generator, shape, dtype: str, chunk: int = 1 << 24) -> np.ndarray:
    """N(0,1) float32 draws, stored as float32 or bf16 bits; drawn in chunks."""
    n = int(np.prod(shape))
    if dtype == "fp32":
        return rng.standard_normal(n, dtype=np.float32).reshape(shape)
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = f32_to_bf16_bits(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


def _nan_value(dtype: str):
    return BF16_NAN_BITS if dtype == "bf16" else np.float32(np.nan)


def _layout_from_block_lists(per_seq_blocks, n_blocks_total, perm, max_blocks, handout=None):
    """Hand out physical ids ``perm[0], perm[1], ...`` to logical blocks.

    ``per_seq_blocks[b]`` is a list of logical block keys; equal keys denote a
    physically shared block.  Keys get ids in ``handout`` order when given,
    else in first-seen order.  Returns (tables, n_used, poison_block)."""
    B = len(per_seq_blocks)
    if handout is None:
        handout = list(dict.fromkeys(k for keys in per_seq_blocks for k in keys))
    key_to_phys = {k: int(perm[i]) for i, k in enumerate(handout)}
    tables = np.zeros((B, max_blocks), dtype=np.int32)
    for b, keys in enumerate(per_seq_blocks):
        for i, key in enumerate(keys):
            tables[b, i] = key_to_phys[key]
    n_used = len(handout)
    if n_used >= n_blocks_total:
        raise ValueError("pool has no spare block for table padding")
    poison_block = int(perm[n_used])
    for b, keys in enumerate(per_seq_blocks):
        tables[b, len(keys):] = poison_block
    return tables, n_used, poison_block


def _poison_pool(pool, tables, readable_lens, block_size, dtype):
    """NaN every slot that no sequence reads; ``readable_lens[b]`` tokens are live."""
    N = pool.shape[0]
    live = np.zeros((N, block_size), dtype=bool)
    for b in range(tables.shape[0]):
        L = int(readable_lens[b])
        nfull, rem = divmod(L, block_size)
        live[tables[b, :nfull], :] = True
        if rem:
            live[tables[b, nfull], :rem] = True
    pool[~live] = _nan_value(dtype)


def _finish(name, *, rng, B, T, Hq, Hkv, D, dtype, partition_size, context_lens, per_seq_blocks,
            n_blocks_total, perm, max_blocks, poison, append, handout=None, note="", structure_only=False):
    tables, n_used, poison_block = _layout_from_block_lists(per_seq_blocks, n_blocks_total, perm, max_blocks,
                                                            handout)
    if structure_only:
        return Workload(name=name, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, block_size=BLOCK_SIZE, dtype=dtype,
                        partition_size=partition_size, context_lens=context_lens.astype(np.int32),
                        block_tables=tables, N_blocks=n_blocks_total, q=None, k_pool=None, v_pool=None,
                        scale=np.float32(1.0 / math.sqrt(D)), poison_block=poison_block,
                        lens_pre=(context_lens - T).astype(np.int32) if append else None, note=note)
    q = _draw_values(rng, (B, T, Hq, D), dtype)
    k_pool = _draw_values(rng, (n_blocks_total, BLOCK_SIZE, Hkv, D), dtype)
    v_pool = _draw_values(rng, (n_blocks_total, BLOCK_SIZE, Hkv, D), dtype)
    lens_pre = k_new = v_new = None
    if append:
        lens_pre = (context_lens - T).astype(np.int32)
        k_new = _draw_values(rng, (B, T, Hkv, D), dtype)
        v_new = _draw_values(rng, (B, T, Hkv, D), dtype)
    if poison:
        readable = lens_pre if append else context_lens
        _poison_pool(k_pool, tables, readable, BLOCK_SIZE, dtype)
        _poison_pool(v_pool, tables, readable, BLOCK_SIZE, dtype)
    return Workload(name=name, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, block_size=BLOCK_SIZE, dtype=dtype,
                    partition_size=partition_size, context_lens=context_lens.astype(np.int32),
                    block_tables=tables, N_blocks=n_blocks_total, q=q, k_pool=k_pool, v_pool=v_pool,
                    scale=np.float32(1.0 / math.sqrt(D)), poison_block=poison_block,
                    lens_pre=lens_pre, k_new=k_new, v_new=v_new, note=note)


def _cdiv(a, b):
    return -(-a // b)


def uniform_batch(name, *, seed, B, T, Hq, Hkv, D, dtype, lens, pool_blocks=None, max_blocks=None,
                  partition_size=0, poison=True, append=False, note=""):
    """Generic batch: private blocks per sequence, ids from a seeded permutation.

    ``lens`` are the lengths attention sees (query/appended tokens included).
    ``pool_blocks`` defaults to ceil(1.1 * used blocks), with at least one spare."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = np.asarray(lens, dtype=np.int64)
    nblk = [_cdiv(int(L), BLOCK_SIZE) for L in lens]
    used = sum(nblk)
    if pool_blocks is None:
        pool_blocks = max(used + 1, _cdiv(11 * used, 10))
    if max_blocks is None:
        max_blocks = max(1, max(nblk) if nblk else 1)
    perm = rng.permutation(pool_blocks)
    per_seq = [[(b, i) for i in range(n)] for b, n in enumerate(nblk)]
    return _finish(name, rng=rng, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, partition_size=partition_size,
                   context_lens=lens, per_seq_blocks=per_seq, n_blocks_total=pool_blocks, perm=perm,
                   max_blocks=max_blocks, poison=poison, append=append, note=note)


def batch_from_block_lists(name, *, seed, T, Hq, Hkv, D, dtype, lens, per_seq_blocks, max_blocks=None,
                           pool_blocks=None, partition_size=0, poison=True, note=""):
    """Batch with an explicit block structure: ``per_seq_blocks[b]`` lists the
    logical block keys of sequence b (equal keys = one shared physical block).

    Physical ids come from a seeded permutation of the pool, handed out in
    first-seen key order; the pool defaults to ceil(1.1 * distinct keys)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = np.asarray(lens, dtype=np.int64)
    for b, L in enumerate(lens):
        if len(per_seq_blocks[b]) != _cdiv(int(L), BLOCK_SIZE):
            raise ValueError(f"sequence {b}: {len(per_seq_blocks[b])} blocks for {int(L)} tokens")
    used = len(dict.fromkeys(k for keys in per_seq_blocks for k in keys))
    if pool_blocks is None:
        pool_blocks = max(used + 1, _cdiv(11 * used, 10))
    if max_blocks is None:
        max_blocks = max(1, max(len(k) for k in per_seq_blocks))
    perm = rng.permutation(pool_blocks)
    return _finish(name, rng=rng, B=len(lens), T=T, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, partition_size=partition_size,
                   context_lens=lens, per_seq_blocks=per_seq_blocks, n_blocks_total=pool_blocks, perm=perm,
                   max_blocks=max_blocks, poison=poison, append=False, note=note)


# ---------------------------------------------------------------------------
# The five workloads.  Seeds equal the workload number.
# ---------------------------------------------------------------------------

def tiny_fp32(poison=True, structure_only=False):
    """B=2, MHA 4 heads, D=64, lengths {37, 100}, fp32, 16-block pool."""
    rng = np.random.Generator(np.random.PCG64(1))
    lens = np.array([37, 100], dtype=np.int64)
    perm = rng.permutation(16)
    per_seq = [[(0, i) for i in range(3)], [(1, i) for i in range(7)]]
    return _finish("tiny_fp32", rng=rng, B=2, T=1, Hq=4, Hkv=4, D=64, dtype="fp32", partition_size=0,
                   context_lens=lens, per_seq_blocks=per_seq, n_blocks_total=16, perm=perm, max_blocks=7,
                   poison=poison, append=False, structure_only=structure_only)


def tinylm_mha_bf16(poison=True, structure_only=False):
    """B=8, MHA 8 heads, D=64, lengths ~ U[1,512], bf16, 512-block pool."""
    rng = np.random.Generator(np.random.PCG64(2))
    lens = rng.integers(1, 512, size=8, endpoint=True)
    perm = rng.permutation(512)
    per_seq = [[(b, i) for i in range(_cdiv(int(L), BLOCK_SIZE))] for b, L in enumerate(lens)]
    return _finish("tinylm_mha_bf16", rng=rng, B=8, T=1, Hq=8, Hkv=8, D=64, dtype="bf16", partition_size=0,
                   context_lens=lens, per_seq_blocks=per_seq, n_blocks_total=512, perm=perm, max_blocks=32,
                   poison=poison, append=False, structure_only=structure_only)


def llama1b_gqa_append(poison=True, partition_size=0, structure_only=False):
    """B=64, GQA 32/8, D=64, pre-append lengths ~ U[128,4096], 1 token appended."""
    rng = np.random.Generator(np.random.PCG64(3))
    lens_pre = rng.integers(128, 4096, size=64, endpoint=True)
    lens = lens_pre + 1
    nblk = [_cdiv(int(L), BLOCK_SIZE) for L in lens]
    pool = _cdiv(11 * sum(nblk), 10)
    perm = rng.permutation(pool)
    per_seq = [[(b, i) for i in range(n)] for b, n in enumerate(nblk)]
    return _finish("llama1b_gqa_append", rng=rng, B=64, T=1, Hq=32, Hkv=8, D=64, dtype="bf16",
                   partition_size=partition_size, context_lens=lens, per_seq_blocks=per_seq,
                   n_blocks_total=pool, perm=perm, max_blocks=257, poison=poison, append=True, structure_only=structure_only)


PREFIX_TOKENS = 512
PREFIX_GROUP = 16


def llama8b_prefix_lens(rng):
    z = rng.standard_normal(256)
    return np.clip(np.rint(1024.0 * np.exp(0.8 * z)), 16, 8192).astype(np.int64)


def llama8b_prefix_share(poison=True, partition_size=0, structure_only=False):
    """B=256, GQA 32/8, D=128, lognormal lengths; groups of 16 share a 512-token prefix.

    A member with L < 512 points at the first ceil(L/16) blocks of its group's
    prefix; its own blocks start at logical block 32.  Ids are handed out group
    by group: the group's prefix blocks first, then each member's own blocks."""
    rng = np.random.Generator(np.random.PCG64(4))
    lens = llama8b_prefix_lens(rng)
    npref_max = PREFIX_TOKENS // BLOCK_SIZE
    per_seq = []
    for b, L in enumerate(lens):
        g = b // PREFIX_GROUP
        n = _cdiv(int(L), BLOCK_SIZE)
        per_seq.append([("prefix", g, i) if i < npref_max else (b, i) for i in range(n)])
    handout = []
    for g in range(len(lens) // PREFIX_GROUP):
        members = range(g * PREFIX_GROUP, (g + 1) * PREFIX_GROUP)
        npref = max(min(len(per_seq[b]), npref_max) for b in members)
        handout.extend(("prefix", g, i) for i in range(npref))
        for b in members:
            handout.extend(k for k in per_seq[b] if k[0] != "prefix")
    pool = _cdiv(11 * len(handout), 10)
    perm = rng.permutation(pool)
    return _finish("llama8b_prefix_share", rng=rng, B=256, T=1, Hq=32, Hkv=8, D=128, dtype="bf16",
                   partition_size=partition_size, context_lens=lens, per_seq_blocks=per_seq,
                   n_blocks_total=pool, perm=perm, max_blocks=512, poison=poison, append=False,
                   handout=handout, note=f"{len(handout)} unique blocks", structure_only=structure_only)


def longctx_verify(poison=True, partition_size=0, structure_only=False):
    """B=16, GQA 32/8, D=128, lengths ~ U[16384,65536], T=4 causal verify queries."""
    rng = np.random.Generator(np.random.PCG64(5))
    lens = rng.integers(16384, 65536, size=16, endpoint=True)
    nblk = [_cdiv(int(L), BLOCK_SIZE) for L in lens]
    pool = _cdiv(11 * sum(nblk), 10)
    perm = rng.permutation(pool)
    per_seq = [[(b, i) for i in range(n)] for b, n in enumerate(nblk)]
    return _finish("longctx_verify", rng=rng, B=16, T=4, Hq=32, Hkv=8, D=128, dtype="bf16",
                   partition_size=partition_size, context_lens=lens, per_seq_blocks=per_seq,
                   n_blocks_total=pool, perm=perm, max_blocks=4096, poison=poison, append=False, structure_only=structure_only)


def llama8b_chunked_prefill(poison=True, partition_size=0, structure_only=False):
    """B=8 sequences each prefilling a chunk of T=512 tokens (GQA 32/8, D=128,
    bf16) after a cached prefix ~ U[0, 3584] tokens: the chunk's K/V rows are
    appended at positions prefix .. prefix+511, then its 512 queries attend
    causally (L = prefix + 512 <= 4096)."""
    rng = np.random.Generator(np.random.PCG64(6))
    T = 512
    lens_pre = rng.integers(0, 3584, size=8, endpoint=True)
    lens = lens_pre + T
    nblk = [_cdiv(int(L), BLOCK_SIZE) for L in lens]
    pool = _cdiv(11 * sum(nblk), 10)
    perm = rng.permutation(pool)
    per_seq = [[(b, i) for i in range(n)] for b, n in enumerate(nblk)]
    return _finish("llama8b_chunked_prefill", rng=rng, B=8, T=T, Hq=32, Hkv=8, D=128, dtype="bf16",
                   partition_size=partition_size, context_lens=lens, per_seq_blocks=per_seq,
                   n_blocks_total=pool, perm=perm, max_blocks=256, poison=poison, append=True,
                   structure_only=structure_only)


def llama8b_long_prompt_chunk(poison=True, partition_size=0, structure_only=False):
    """One sequence prefilling a 512-token chunk of a long prompt (GQA 32/8,
    D=128, bf16) after 8192 cached tokens: the serving-loop shape of chunked
    prefill, where one request's chunk is attended at a time."""
    rng = np.random.Generator(np.random.PCG64(7))
    T, pre = 512, 8192
    lens = np.array([pre + T], dtype=np.int64)
    nblk = [_cdiv(int(L), BLOCK_SIZE) for L in lens]
    pool = _cdiv(11 * sum(nblk), 10)
    perm = rng.permutation(pool)
    per_seq = [[(0, i) for i in range(nblk[0])]]
    return _finish("llama8b_long_prompt_chunk", rng=rng, B=1, T=T, Hq=32, Hkv=8, D=128, dtype="bf16",
                   partition_size=partition_size, context_lens=lens, per_seq_blocks=per_seq,
                   n_blocks_total=pool, perm=perm, max_blocks=nblk[0], poison=poison, append=True,
                   structure_only=structure_only)


# Seed of each named workload (its PCG64 stream; also the workload number).
WORKLOAD_SEEDS = {"tiny_fp32": 1, "tinylm_mha_bf16": 2, "llama1b_gqa_append": 3, "llama8b_prefix_share": 4,
                  "longctx_verify": 5, "llama8b_chunked_prefill": 6, "llama8b_long_prompt_chunk": 7}

WORKLOADS = {
    "tiny_fp32": tiny_fp32,
    "tinylm_mha_bf16": tinylm_mha_bf16,
    "llama1b_gqa_append": llama1b_gqa_append,
    "llama8b_prefix_share": llama8b_prefix_share,
    "longctx_verify": longctx_verify,
    "llama8b_chunked_prefill": llama8b_chunked_prefill,
    "llama8b_long_prompt_chunk": llama8b_long_prompt_chunk,
}


def relabel_physical(w: Workload, seed: int) -> Workload:
    """Same logical data under a different physical block numbering.

    Block i of the pool moves to position perm[i] and every table entry is
    mapped through perm, so every sequence sees the same tokens."""
    rng = np.random.Generator(np.random.PCG64(seed))
    perm = rng.permutation(w.N_blocks)
    k_pool = np.empty_like(w.k_pool)
    v_pool = np.empty_like(w.v_pool)
    k_pool[perm] = w.k_pool
    v_pool[perm] = w.v_pool
    tables = perm[w.block_tables].astype(np.int32)
    return dataclasses.replace(w, k_pool=k_pool, v_pool=v_pool, block_tables=tables,
                               poison_block=int(perm[w.poison_block]))


def scaled_queries(w: Workload, factor: float) -> Workload:
    """Queries multiplied by a power of two (exact in bf16 and fp32): sharper softmax."""
    qv = w.values(w.q) * np.float32(factor)
    q = f32_to_bf16_bits(qv) if w.dtype == "bf16" else qv.astype(np.float32)
    return dataclasses.replace(w, q=q)
