"""Python binding of libpkv: paged KV-cache decode attention for MI355X (gfx950).

Argument marshalling only: each function takes torch tensors that already
live on the GPU, checks their shapes, and passes raw device pointers, sizes
and the current HIP stream to the C ABI declared in include/pkv.h, where every
step runs in hand-written HIP kernels.  torch supplies device memory and
streams, nothing else.  There is no CPU fallback: if libpkv.so is missing or
a call fails, a RuntimeError is raised.
"""
from __future__ import annotations

import ctypes
import pathlib

LIB_PATH = pathlib.Path(__file__).resolve().with_name("libpkv.so")

PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EWORKSPACE, PKV_EHIP = range(5)
PKV_FP32, PKV_BF16 = 0, 1
STATUS_NAMES = {0: "PKV_OK", 1: "PKV_EINVAL", 2: "PKV_EUNSUPPORTED", 3: "PKV_EWORKSPACE", 4: "PKV_EHIP"}
EXPORTS = ("paged_kv_append", "paged_kv_append_rope", "paged_kv_gather", "pkv_decode_workspace_bytes", "paged_attention_decode",
           "paged_attention_prefill", "lse_reduce", "pkv_last_error")

_lib = None


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def load_library(path: pathlib.Path = LIB_PATH) -> ctypes.CDLL:
    """Load libpkv.so and declare the C signatures.  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not path.exists():
        raise RuntimeError(f"{path} is not built; run `python -m paged_kv_cache_attention_amd.build`")
    lib = ctypes.CDLL(str(path))
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.paged_kv_append.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, I, P]
    lib.paged_kv_append.restype = I
    lib.paged_kv_append_rope.argtypes = [P, I, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P]
    lib.paged_kv_append_rope.restype = I
    lib.paged_kv_gather.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, I, P]
    lib.paged_kv_gather.restype = I
    lib.pkv_decode_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.pkv_decode_workspace_bytes.restype = S
    lib.paged_attention_decode.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, P, S, I, P]
    lib.paged_attention_decode.restype = I
    lib.paged_attention_prefill.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, P]
    lib.paged_attention_prefill.restype = I
    lib.lse_reduce.argtypes = [P, P, P, P, I, I, I, I, I, I, P]
    lib.lse_reduce.restype = I
    lib.pkv_last_error.argtypes = []
    lib.pkv_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != PKV_OK:
        raise PkvError(status, load_library().pkv_last_error().decode())


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return PKV_FP32
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _i32(t, name):
    torch = _torch()
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    return _ptr(t)


def _stream(stream, device):
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def pkv_decode_workspace_bytes(B, T, Hq, D, max_blocks, block_size, partition_size) -> int:
    return int(load_library().pkv_decode_workspace_bytes(B, T, Hq, D, max_blocks, block_size, partition_size))


def paged_kv_append(k_new, v_new, k_pool, v_pool, block_tables, context_lens_pre, stream=None):
    """Write k_new/v_new [B,T,Hkv,D] at positions context_lens_pre[b]+t of each sequence."""
    lib = load_library()
    B, T, Hkv, D = k_new.shape
    N, bs = k_pool.shape[0], k_pool.shape[1]
    _check(lib.paged_kv_append(_ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool),
                               _i32(block_tables, "block_tables"), _i32(context_lens_pre, "context_lens_pre"),
                               B, T, Hkv, D, bs, block_tables.shape[1], N, _dtype_code(k_pool),
                               _stream(stream, k_pool.device)))


def paged_kv_append_rope(k_new, v_new, k_pool, v_pool, block_tables, context_lens_pre, rope_theta, q=None,
                         stream=None):
    """paged_kv_append with k_new rotated by RoPE at its positions; q [B,T,Hq,D],
    when given, is rotated in place at the same positions."""
    lib = load_library()
    B, T, Hkv, D = k_new.shape
    N, bs = k_pool.shape[0], k_pool.shape[1]
    Hq = q.shape[2] if q is not None else 0
    _check(lib.paged_kv_append_rope(_ptr(q), Hq, _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool),
                                    _i32(block_tables, "block_tables"), _i32(context_lens_pre, "context_lens_pre"),
                                    B, T, Hkv, D, bs, block_tables.shape[1], N, float(rope_theta),
                                    _dtype_code(k_pool), _stream(stream, k_pool.device)))


def paged_kv_gather(k_pool, v_pool, block_tables, context_lens, k_out, v_out, stream=None):
    """Contiguous copy of each sequence's cached rows into k_out/v_out [B,max_len,Hkv,D]."""
    lib = load_library()
    B, max_len, Hkv, D = k_out.shape
    N, bs = k_pool.shape[0], k_pool.shape[1]
    _check(lib.paged_kv_gather(_ptr(k_pool), _ptr(v_pool), _i32(block_tables, "block_tables"),
                               _i32(context_lens, "context_lens"), _ptr(k_out), _ptr(v_out), B, max_len, Hkv, D, bs,
                               block_tables.shape[1], N, _dtype_code(k_pool), _stream(stream, k_pool.device)))


def paged_attention_decode(q, k_pool, v_pool, block_tables, context_lens, out=None, lse_out=None, scale=None,
                           partition_size=0, workspace=None, stream=None):
    """Attention of q [B,T,Hq,D] over the paged cache; returns out [B,T,Hq,D].

    When the library needs workspace (pkv_decode_workspace_bytes > 0) and none
    is given, one is allocated with torch (device memory only; all computation
    is in the library)."""
    torch = _torch()
    lib = load_library()
    B, T, Hq, D = q.shape
    N, bs, Hkv = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    max_blocks = block_tables.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if scale is None:
        scale = 1.0 / D ** 0.5
    need = pkv_decode_workspace_bytes(B, T, Hq, D, max_blocks, bs, partition_size)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.paged_attention_decode(_ptr(q), _ptr(k_pool), _ptr(v_pool), _i32(block_tables, "block_tables"),
                                      _i32(context_lens, "context_lens"), _ptr(out), _ptr(lse_out), B, T, Hq, Hkv, D,
                                      bs, max_blocks, N, float(scale), int(partition_size), _ptr(workspace), ws_bytes,
                                      _dtype_code(q), _stream(stream, q.device)))
    return out


def paged_attention_prefill(q, k_pool, v_pool, block_tables, context_lens, out=None, lse_out=None, scale=None,
                            stream=None):
    """Chunked-prefill attention of q [B,T,Hq,D] (bf16) over the paged cache;
    query t of sequence b sees keys 0 .. context_lens[b] - T + t.  Returns out."""
    torch = _torch()
    lib = load_library()
    B, T, Hq, D = q.shape
    N, bs, Hkv = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    max_blocks = block_tables.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if scale is None:
        scale = 1.0 / D ** 0.5
    _check(lib.paged_attention_prefill(_ptr(q), _ptr(k_pool), _ptr(v_pool), _i32(block_tables, "block_tables"),
                                       _i32(context_lens, "context_lens"), _ptr(out), _ptr(lse_out), B, T, Hq, Hkv, D,
                                       bs, max_blocks, N, float(scale), _dtype_code(q), _stream(stream, q.device)))
    return out


def lse_reduce(part_out, part_lse, out, lse_out=None, stream=None):
    """Merge float32 partials part_out [B,T,Hq,P,D] / part_lse [B,T,Hq,P] into out [B,T,Hq,D]."""
    lib = load_library()
    B, T, Hq, P, D = part_out.shape
    _check(lib.lse_reduce(_ptr(part_out), _ptr(part_lse), _ptr(out), _ptr(lse_out), B, T, Hq, D, P,
                          _dtype_code(out), _stream(stream, out.device)))
    return out
