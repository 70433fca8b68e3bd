"""Rotary position embedding for the KV append -- oracle (test infrastructure only).

The decoder the pages build on is a Llama-style transformer with RoPE ("LLM
Inference from Scratch", Architecture overview), and the pages list a fused
RoPE kernel among the Llama milestones ("warpllama", Milestones).  The pages
fix no pairing or base, so this follows the plainest reading the rest
supports, Llama's: dimension i < D/2 of a head is paired with i + D/2, and the
pair at position p is rotated by the angle p * w_i, w_i = theta^(-2i/D):

    y[i]       = x[i] cos(p w_i) - x[i + D/2] sin(p w_i)
    y[i + D/2] = x[i + D/2] cos(p w_i) + x[i] sin(p w_i)

Everything is float64.  The fused append rotates each new key at the
position it is written to (lens_pre[b] + t) and copies the value unchanged.
"""
from __future__ import annotations

import numpy as np

from .attention import kv_append


def rope_angles(positions, D: int, theta: float) -> np.ndarray:
    """Angles p * w_i for i < D/2, shape positions.shape + (D/2,)."""
    if D % 2:
        raise ValueError("RoPE needs an even head dimension")
    i = np.arange(D // 2, dtype=np.float64)
    w = np.power(np.float64(theta), -2.0 * i / D)
    return np.asarray(positions, dtype=np.float64)[..., None] * w


def rope_rotate(x, positions, theta: float) -> np.ndarray:
    """Rotate x [..., H, D] whose leading dims match positions [...] (one
    position per token, shared by its heads)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    ang = rope_angles(positions, D, theta)[..., None, :]   # [..., 1, D/2]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def token_positions(lens_pre, T: int) -> np.ndarray:
    """Position of new token t of sequence b: lens_pre[b] + t, shape [B, T]."""
    return np.asarray(lens_pre, dtype=np.int64)[:, None] + np.arange(T)[None, :]


def kv_append_rope(k_pool, v_pool, block_tables, lens_pre, k_new, v_new, block_size, theta):
    """The KV append of k_new rotated at its positions, v_new as given."""
    T = k_new.shape[1]
    k_rot = rope_rotate(k_new, token_positions(lens_pre, T), theta)
    return kv_append(k_pool, v_pool, block_tables, lens_pre, k_rot, v_new, block_size)
