"""Runs the engine's iteration plans on the device with the library's kernels.

Each iteration (the order of include/pkv_engine.h):
  1. copy-on-write block copies (paged_kv_copy_blocks);
  2. the K/V of every planned token, rotated at its position
     (paged_kv_append_rope; the queries are rotated in the same call);
  3. attention: one paged_attention_prefill per admitted request (its chunk of
     new tokens) and one paged_attention_decode for all decoding requests;
  4. one next token per planned request from the output of its last position.
The model around attention is not part of the library: the caller passes
``qkv(tokens) -> (q [n,Hq,D], k [n,Hkv,D], v [n,Hkv,D])`` (device tensors in the
pool dtype) and ``sample(plan, outputs) -> next tokens``.  This module only
moves arguments between the engine and the kernels.
"""
from __future__ import annotations

import numpy as np

from . import (Engine, PKV_ENGINE_DECODE, PKV_ENGINE_PREFILL, paged_attention_decode, paged_attention_prefill,
               paged_kv_append_rope, paged_kv_copy_blocks)


class PagedExecutor:
    def __init__(self, engine: Engine, k_pool, v_pool, Hq: int, rope_theta: float, qkv, sample, scale=None,
                 stream=None):
        self.engine, self.k_pool, self.v_pool = engine, k_pool, v_pool
        self.Hq, self.theta, self.qkv, self.sample = Hq, rope_theta, qkv, sample
        self.D = k_pool.shape[3]
        self.scale = scale if scale is not None else 1.0 / self.D ** 0.5
        self.stream = stream

    def _dev_i32(self, a):
        import torch
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(self.k_pool.device)

    def step(self):
        """Plan, execute and commit one iteration.  Returns (plan, outputs) with
        outputs[i] = [count_i, Hq, D] rows of planned request i, or None when idle."""
        plan = self.engine.schedule()
        if plan.n == 0:
            return None
        if len(plan.copy_src):
            paged_kv_copy_blocks(self.k_pool, self.v_pool, self._dev_i32(plan.copy_src), self._dev_i32(plan.copy_dst),
                                 stream=self.stream)
        outputs = [None] * plan.n
        dec = [i for i in range(plan.n) if plan.kind[i] == PKV_ENGINE_DECODE]
        for i in range(plan.n):
            if plan.kind[i] != PKV_ENGINE_PREFILL:
                continue
            tok = self._dev_i32(plan.tokens_of(i))
            q, k, v = self.qkv(tok)
            n = len(tok)
            tables = self._dev_i32(plan.block_tables[i:i + 1])
            q = q.reshape(1, n, self.Hq, self.D).contiguous()
            paged_kv_append_rope(k.reshape(1, n, *k.shape[1:]).contiguous(), v.reshape(1, n, *v.shape[1:]).contiguous(),
                                 self.k_pool, self.v_pool, tables, self._dev_i32(plan.start[i:i + 1]), self.theta, q=q,
                                 stream=self.stream)
            outputs[i] = paged_attention_prefill(q, self.k_pool, self.v_pool, tables,
                                                 self._dev_i32(plan.context_lens[i:i + 1]), scale=self.scale,
                                                 stream=self.stream)[0]
        if dec:
            idx = np.array(dec)
            tok = self._dev_i32(np.concatenate([plan.tokens_of(i) for i in dec]))
            q, k, v = self.qkv(tok)
            nd = len(dec)
            tables = self._dev_i32(plan.block_tables[idx])
            q = q.reshape(nd, 1, self.Hq, self.D).contiguous()
            paged_kv_append_rope(k.reshape(nd, 1, *k.shape[1:]).contiguous(), v.reshape(nd, 1, *v.shape[1:]).contiguous(),
                                 self.k_pool, self.v_pool, tables, self._dev_i32(plan.start[idx]), self.theta, q=q,
                                 stream=self.stream)
            out = paged_attention_decode(q, self.k_pool, self.v_pool, tables, self._dev_i32(plan.context_lens[idx]),
                                         scale=self.scale, stream=self.stream)
            for j, i in enumerate(dec):
                outputs[i] = out[j]
        self.engine.commit(self.sample(plan, outputs))
        return plan, outputs
