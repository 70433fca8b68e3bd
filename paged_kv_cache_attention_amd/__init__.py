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
EXPORTS = ("paged_kv_append", "paged_kv_append_rope", "paged_kv_copy_blocks", "paged_kv_gather",
           "pkv_decode_workspace_bytes", "paged_attention_decode", "paged_attention_decode_noalloc",
           "paged_attention_prefill",
           "pkv_prefill_workspace_bytes", "pkv_prefill_piece_tokens", "lse_reduce",
           "pkv_last_error",
           "pkv_engine_create", "pkv_engine_destroy", "pkv_engine_last_error", "pkv_engine_add_request",
           "pkv_engine_schedule", "pkv_engine_commit", "pkv_engine_get_stats", "pkv_engine_request_tokens",
           "pkv_engine_block_ref")

_lib = None


class EngineConfig(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int), ("block_size", ctypes.c_int), ("max_blocks_per_seq", ctypes.c_int),
                ("max_running", ctypes.c_int), ("max_prefill_tokens", ctypes.c_int),
                ("enable_prefix_cache", ctypes.c_int), ("pad_block", ctypes.c_int)]


_I32P = ctypes.POINTER(ctypes.c_int32)
_I64P = ctypes.POINTER(ctypes.c_int64)


class EnginePlan(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int), ("request_id", _I64P), ("kind", _I32P), ("start", _I32P), ("count", _I32P),
                ("token_offset", _I32P), ("tokens", _I32P), ("block_tables", _I32P), ("context_lens", _I32P),
                ("max_blocks_per_seq", ctypes.c_int), ("n_copies", ctypes.c_int), ("copy_src", _I32P),
                ("copy_dst", _I32P), ("n_preempted", ctypes.c_int), ("preempted", _I64P)]


class EngineStats(ctypes.Structure):
    _fields_ = [(k, ctypes.c_int64) for k in ("iterations", "preemptions", "cow_copies", "prefix_hit_tokens",
                                              "computed_tokens", "finished")] + \
               [(k, ctypes.c_int) for k in ("waiting", "running", "free_blocks", "cached_blocks", "cache_entries")]


PKV_ENGINE_PREFILL, PKV_ENGINE_DECODE = 0, 1


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
    lib.paged_attention_decode_noalloc.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, I, P]
    lib.paged_attention_decode_noalloc.restype = I
    lib.paged_attention_prefill.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, P, S, I, P]
    lib.paged_attention_prefill.restype = I
    lib.pkv_prefill_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I]
    lib.pkv_prefill_workspace_bytes.restype = S
    lib.pkv_prefill_piece_tokens.argtypes = [I, I, I, I, I, I, I]
    lib.pkv_prefill_piece_tokens.restype = I
    lib.lse_reduce.argtypes = [P, P, P, P, I, I, I, I, I, I, P]
    lib.lse_reduce.restype = I
    lib.paged_kv_copy_blocks.argtypes = [P, P, P, P, I, I, I, I, I, I, P]
    lib.paged_kv_copy_blocks.restype = I
    E = ctypes.c_void_p
    lib.pkv_engine_create.argtypes = [ctypes.POINTER(EngineConfig)]
    lib.pkv_engine_create.restype = E
    lib.pkv_engine_destroy.argtypes = [E]
    lib.pkv_engine_destroy.restype = None
    lib.pkv_engine_last_error.argtypes = [E]
    lib.pkv_engine_last_error.restype = ctypes.c_char_p
    lib.pkv_engine_add_request.argtypes = [E, ctypes.c_int64, P, I, I]
    lib.pkv_engine_add_request.restype = I
    lib.pkv_engine_schedule.argtypes = [E, ctypes.POINTER(EnginePlan)]
    lib.pkv_engine_schedule.restype = I
    lib.pkv_engine_commit.argtypes = [E, P]
    lib.pkv_engine_commit.restype = I
    lib.pkv_engine_get_stats.argtypes = [E, ctypes.POINTER(EngineStats)]
    lib.pkv_engine_get_stats.restype = I
    lib.pkv_engine_request_tokens.argtypes = [E, ctypes.c_int64, P, I]
    lib.pkv_engine_request_tokens.restype = I
    lib.pkv_engine_block_ref.argtypes = [E, I]
    lib.pkv_engine_block_ref.restype = I
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


def _alloc(shape, dtype, device, stream):
    """Device memory for the library (a workspace, or an output it was not
    given), owned by torch's caching allocator.

    It is allocated on `stream` (torch's current stream when None), the stream
    the library launches on, so the allocator does not hand it to other work
    while those kernels may still use it after this call returns."""
    torch = _torch()
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def check_attention_args(q, k_pool, v_pool, block_tables, context_lens, out=None, lse_out=None):
    """Shape, dtype and device agreement of the attention arguments.

    The C ABI takes raw pointers and sizes, so a pool of another dtype or head
    size than q, or an out or lse_out of the wrong size, would make the
    kernels read or write past the end of a buffer: the binding checks here,
    from the tensors' metadata only (it runs on any tensor, without a GPU).
    Raises ValueError or TypeError."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError(f"q must be [B, T, Hq, D], got shape {tuple(q.shape)}")
    B, T, Hq, D = q.shape
    if k_pool.dim() != 4 or tuple(k_pool.shape) != tuple(v_pool.shape):
        raise ValueError(f"k_pool and v_pool must both be [N_blocks, block_size, Hkv, D], got "
                         f"{tuple(k_pool.shape)} and {tuple(v_pool.shape)}")
    if k_pool.shape[3] != D:
        raise ValueError(f"pool head size {k_pool.shape[3]} differs from q's {D}")
    if Hq % k_pool.shape[2]:
        raise ValueError(f"Hq = {Hq} is not a multiple of the pool's Hkv = {k_pool.shape[2]}")
    for name, t in (("k_pool", k_pool), ("v_pool", v_pool), ("out", out)):
        if t is not None and t.dtype != q.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, q has {q.dtype}")
    if out is not None and tuple(out.shape) != tuple(q.shape):
        raise ValueError(f"out must have q's shape {tuple(q.shape)}, got {tuple(out.shape)}")
    if lse_out is not None:
        if lse_out.dtype != torch.float32 or tuple(lse_out.shape) != (B, T, Hq):
            raise ValueError(f"lse_out must be float32 [B, T, Hq] = {(B, T, Hq)}, got {lse_out.dtype} "
                             f"{tuple(lse_out.shape)}")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError(f"block_tables must be [B = {B}, max_blocks], got {tuple(block_tables.shape)}")
    if context_lens.dim() != 1 or context_lens.shape[0] != B:
        raise ValueError(f"context_lens must be [B = {B}], got {tuple(context_lens.shape)}")
    for name, t in (("block_tables", block_tables), ("context_lens", context_lens)):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32, got {t.dtype}")
    devs = {t.device for t in (q, k_pool, v_pool, block_tables, context_lens, out, lse_out) if t is not None}
    if len(devs) != 1:
        raise ValueError(f"all tensors must be on one device, got {sorted(map(str, devs))}")


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
    lib = load_library()
    check_attention_args(q, k_pool, v_pool, block_tables, context_lens, out, lse_out)
    B, T, Hq, D = q.shape
    N, bs, Hkv = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    max_blocks = block_tables.shape[1]
    if out is None:
        out = _alloc(q.shape, q.dtype, q.device, stream)
    if scale is None:
        scale = 1.0 / D ** 0.5
    need = pkv_decode_workspace_bytes(B, T, Hq, D, max_blocks, bs, partition_size)
    if need and workspace is None:
        workspace = _alloc(need, _torch().uint8, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.paged_attention_decode(_ptr(q), _ptr(k_pool), _ptr(v_pool), _i32(block_tables, "block_tables"),
                                      _i32(context_lens, "context_lens"), _ptr(out), _ptr(lse_out), B, T, Hq, Hkv, D,
                                      bs, max_blocks, N, float(scale), int(partition_size), _ptr(workspace), ws_bytes,
                                      _dtype_code(q), _stream(stream, q.device)))
    return out


PKV_NOALLOC_SCRATCH_BYTES = 64 << 20


def paged_attention_decode_noalloc(q, k_pool, v_pool, block_tables, context_lens, out, lse_out=None, scale=None,
                                   partition_size=0, stream=None):
    """paged_attention_decode without a workspace: the library works in its
    static device scratch (PKV_NOALLOC_SCRATCH_BYTES per GPU) and neither it
    nor this binding allocates.  `out` must be given.  Calls in flight at once
    on one GPU share that scratch and race."""
    lib = load_library()
    check_attention_args(q, k_pool, v_pool, block_tables, context_lens, out, lse_out)
    B, T, Hq, D = q.shape
    N, bs, Hkv = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    if scale is None:
        scale = 1.0 / D ** 0.5
    _check(lib.paged_attention_decode_noalloc(_ptr(q), _ptr(k_pool), _ptr(v_pool), _i32(block_tables, "block_tables"),
                                              _i32(context_lens, "context_lens"), _ptr(out), _ptr(lse_out), B, T, Hq,
                                              Hkv, D, bs, block_tables.shape[1], N, float(scale), int(partition_size),
                                              _dtype_code(q), _stream(stream, q.device)))
    return out


def pkv_prefill_workspace_bytes(B, T, Hq, Hkv, D, block_size, max_blocks, piece_tokens):
    return int(load_library().pkv_prefill_workspace_bytes(B, T, Hq, Hkv, D, block_size, max_blocks, piece_tokens))


def pkv_prefill_piece_tokens(B, T, Hq, Hkv, D, block_size, max_blocks):
    return int(load_library().pkv_prefill_piece_tokens(B, T, Hq, Hkv, D, block_size, max_blocks))


def paged_attention_prefill(q, k_pool, v_pool, block_tables, context_lens, out=None, lse_out=None, scale=None,
                            piece_tokens=None, workspace=None, stream=None):
    """Chunked-prefill attention of q [B,T,Hq,D] (bf16) over the paged cache;
    query t of sequence b sees keys 0 .. context_lens[b] - T + t.  Returns out.

    piece_tokens None takes the library's suggestion for this shape on the
    current device (pkv_prefill_piece_tokens); 0 never splits keys.  When
    pieces need workspace and none is given, one is allocated."""
    lib = load_library()
    check_attention_args(q, k_pool, v_pool, block_tables, context_lens, out, lse_out)
    B, T, Hq, D = q.shape
    N, bs, Hkv = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    max_blocks = block_tables.shape[1]
    if out is None:
        out = _alloc(q.shape, q.dtype, q.device, stream)
    if scale is None:
        scale = 1.0 / D ** 0.5
    if piece_tokens is None:
        piece_tokens = pkv_prefill_piece_tokens(B, T, Hq, Hkv, D, bs, max_blocks)
    need = pkv_prefill_workspace_bytes(B, T, Hq, Hkv, D, bs, max_blocks, piece_tokens)
    if need and workspace is None:
        workspace = _alloc(need, _torch().uint8, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.paged_attention_prefill(_ptr(q), _ptr(k_pool), _ptr(v_pool), _i32(block_tables, "block_tables"),
                                       _i32(context_lens, "context_lens"), _ptr(out), _ptr(lse_out), B, T, Hq, Hkv, D,
                                       bs, max_blocks, N, float(scale), int(piece_tokens), _ptr(workspace), ws_bytes,
                                       _dtype_code(q), _stream(stream, q.device)))
    return out


def paged_kv_copy_blocks(k_pool, v_pool, src, dst, stream=None):
    """Copy block src[i] to dst[i] in both pools (src, dst: int32 device tensors)."""
    lib = load_library()
    N, bs, Hkv, D = k_pool.shape
    n = int(src.numel())
    _check(lib.paged_kv_copy_blocks(_ptr(k_pool), _ptr(v_pool), _i32(src, "src"), _i32(dst, "dst"), n, Hkv, D, bs, N,
                                    _dtype_code(k_pool), _stream(stream, k_pool.device)))


class Plan:
    """One iteration planned by the engine, copied out of the library's arrays."""

    def __init__(self, p: "EnginePlan"):
        import numpy as np
        n, mb = p.n, p.max_blocks_per_seq

        def arr(ptr, count, dtype):
            return np.ctypeslib.as_array(ptr, shape=(count,)).astype(dtype, copy=True) if count else np.zeros(0, dtype)
        self.n = n
        self.request_id = arr(p.request_id, n, np.int64)
        self.kind = arr(p.kind, n, np.int32)
        self.start = arr(p.start, n, np.int32)
        self.count = arr(p.count, n, np.int32)
        self.token_offset = arr(p.token_offset, n + 1, np.int32) if n else np.zeros(1, np.int32)
        self.tokens = arr(p.tokens, int(self.token_offset[-1]), np.int32)
        self.block_tables = arr(p.block_tables, n * mb, np.int32).reshape(n, mb)
        self.context_lens = arr(p.context_lens, n, np.int32)
        self.copy_src = arr(p.copy_src, p.n_copies, np.int32)
        self.copy_dst = arr(p.copy_dst, p.n_copies, np.int32)
        self.preempted = arr(p.preempted, p.n_preempted, np.int64)

    def tokens_of(self, i):
        return self.tokens[self.token_offset[i]:self.token_offset[i + 1]]


class Engine:
    """Block manager + continuous-batching scheduler of the library (host only)."""

    def __init__(self, num_blocks, block_size, max_blocks_per_seq, max_running, max_prefill_tokens,
                 prefix_cache=True, pad_block=0):
        self._lib = load_library()
        cfg = EngineConfig(num_blocks, block_size, max_blocks_per_seq, max_running, max_prefill_tokens,
                           int(bool(prefix_cache)), pad_block)
        self._h = self._lib.pkv_engine_create(ctypes.byref(cfg))
        if not self._h:
            raise PkvError(PKV_EINVAL, "invalid engine configuration")

    def _ok(self, status):
        if status != PKV_OK:
            raise PkvError(status, self._lib.pkv_engine_last_error(self._h).decode())

    def add_request(self, request_id, prompt, max_new_tokens):
        import numpy as np
        a = np.ascontiguousarray(prompt, dtype=np.int32)
        self._ok(self._lib.pkv_engine_add_request(self._h, int(request_id),
                                                  a.ctypes.data_as(ctypes.c_void_p), len(a), int(max_new_tokens)))

    def schedule(self) -> Plan:
        p = EnginePlan()
        self._ok(self._lib.pkv_engine_schedule(self._h, ctypes.byref(p)))
        return Plan(p)

    def commit(self, next_tokens):
        import numpy as np
        a = np.ascontiguousarray(next_tokens, dtype=np.int32)
        self._ok(self._lib.pkv_engine_commit(self._h, a.ctypes.data_as(ctypes.c_void_p)))

    def stats(self) -> dict:
        st = EngineStats()
        self._ok(self._lib.pkv_engine_get_stats(self._h, ctypes.byref(st)))
        return {k: getattr(st, k) for k, _ in EngineStats._fields_}

    def request_tokens(self, request_id):
        import numpy as np
        n = self._lib.pkv_engine_request_tokens(self._h, int(request_id), None, 0)
        if n < 0:
            raise KeyError(request_id)
        out = np.zeros(n, dtype=np.int32)
        self._lib.pkv_engine_request_tokens(self._h, int(request_id), out.ctypes.data_as(ctypes.c_void_p), n)
        return out

    def block_ref(self, block):
        return self._lib.pkv_engine_block_ref(self._h, int(block))

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pkv_engine_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()


def lse_reduce(part_out, part_lse, out, lse_out=None, stream=None):
    """Merge float32 partials part_out [B,T,Hq,P,D] / part_lse [B,T,Hq,P] into out [B,T,Hq,D]."""
    lib = load_library()
    B, T, Hq, P, D = part_out.shape
    _check(lib.lse_reduce(_ptr(part_out), _ptr(part_lse), _ptr(out), _ptr(lse_out), B, T, Hq, D, P,
                          _dtype_code(out), _stream(stream, out.device)))
    return out
