"""The C ABI library loads and exports what include/pkv.h declares; host-side
argument checks return the documented status without launching anything.
CPU only: no call here reaches a kernel launch."""
import ctypes
import pathlib
import re

import pytest

import paged_kv_cache_attention_amd as pkv

INCLUDE = pathlib.Path(__file__).resolve().parent.parent / "include"
P = ctypes.c_void_p(256)      # non-null dummy pointers, never dereferenced on these paths
Q, K, V, TAB, LENS, OUT = (ctypes.c_void_p(4096 * (i + 1)) for i in range(6))


def declared_functions():
    names = []
    for h in sorted(INCLUDE.glob("*.h")):
        names += re.findall(r"^(?:pkv_status|size_t|const char\*|pkv_engine\*|void|int)\s+(\w+)\s*\(", h.read_text(),
                            flags=re.M)
    return names


def test_library_exports_every_declared_symbol():
    lib = pkv.load_library()
    names = declared_functions()
    assert set(names) == set(pkv.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def test_workspace_sizing():
    f = pkv.pkv_decode_workspace_bytes
    assert f(4, 1, 32, 128, 64, 16, 0) > 0          # balanced split needs its own workspace

    def partitioned(B, T, Hq, D, P):
        """The documented partials (offset 0), rounded up to 256 bytes, then
        the tile's plan (a header, B + 1 prefix sums, 2048 range starts,
        B + 1 descriptors, each area rounded to 256 bytes), one piece slot of
        T * Hq rows per (range, sequence) -- at most 2048 * min(16, T * Hq)
        + B * T * Hq rows -- and two slots of min(16, T * Hq) rows per range
        for the 2048 ranges of Hkv = 1."""
        r = lambda n: -(-n // 256) * 256
        partials = r(B * T * Hq * P * (D + 1) * 4)
        plan = 256 + r((B + 1) * 4) + r(2048 * 4) + r((B + 1) * 16)
        pieces = (2048 * min(16, T * Hq) + B * T * Hq) * (D + 1) * 4
        return partials + plan + pieces + 2 * 2048 * min(16, T * Hq) * (D + 1) * 4
    # P_max = ceil(64*16/256) = 4 partitions
    assert f(4, 1, 32, 128, 64, 16, 256) == partitioned(4, 1, 32, 128, 4)
    assert f(16, 4, 32, 128, 4096, 16, 512) == partitioned(16, 4, 32, 128, 128)
    assert f(1, 1, 1, 64, 3, 16, 32) == partitioned(1, 1, 1, 64, 2)
    assert f(16, 4, 32, 128, 4096, 16, 512) >= 16 * 4 * 32 * 128 * 129 * 4


def _decode(**kw):
    args = dict(q=Q, k=K, v=V, tab=TAB, lens=LENS, out=OUT, lse=None, B=2, T=1, Hq=8, Hkv=2, D=128, bs=16, mb=4, N=8,
                scale=0.088, part=0, ws=None, wsb=0, dt=pkv.PKV_BF16)
    args.update(kw)
    lib = pkv.load_library()
    st = lib.paged_attention_decode(args["q"], args["k"], args["v"], args["tab"], args["lens"], args["out"],
                                    args["lse"], args["B"], args["T"], args["Hq"], args["Hkv"], args["D"], args["bs"],
                                    args["mb"], args["N"], args["scale"], args["part"], args["ws"], args["wsb"],
                                    args["dt"], None)
    return st, lib.pkv_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), pkv.PKV_EINVAL),
    (dict(out=None), pkv.PKV_EINVAL),
    (dict(Hq=6, Hkv=4), pkv.PKV_EINVAL),
    (dict(T=0), pkv.PKV_EINVAL),
    (dict(Hkv=0), pkv.PKV_EINVAL),
    (dict(part=24), pkv.PKV_EINVAL),
    (dict(part=-16), pkv.PKV_EINVAL),
    (dict(scale=float("nan")), pkv.PKV_EINVAL),
    (dict(dt=7), pkv.PKV_EINVAL),
    (dict(out=Q), pkv.PKV_EINVAL),            # out aliases q
    (dict(D=96), pkv.PKV_EUNSUPPORTED),
    (dict(bs=32), pkv.PKV_EUNSUPPORTED),
    (dict(T=17), pkv.PKV_EUNSUPPORTED),
    (dict(Hq=24, Hkv=2), pkv.PKV_EUNSUPPORTED),     # Hq/Hkv = 12
    (dict(Hq=6, Hkv=6), pkv.PKV_EUNSUPPORTED),      # Hq not a multiple of 4
    (dict(Hq=8, Hkv=8, D=128, dt=pkv.PKV_FP32), pkv.PKV_EUNSUPPORTED),
    (dict(part=16), pkv.PKV_EWORKSPACE),
    (dict(part=0), pkv.PKV_EWORKSPACE),
    (dict(part=16, ws=P, wsb=100), pkv.PKV_EWORKSPACE),
])
def test_decode_argument_errors(kw, status):
    st, msg = _decode(**kw)
    assert st == status, msg
    assert msg


def test_decode_empty_batch_is_a_noop():
    st, _ = _decode(B=0, q=None, out=None)
    assert st == pkv.PKV_OK


def _prefill(**kw):
    args = dict(q=Q, k=K, v=V, tab=TAB, lens=LENS, out=OUT, lse=None, B=2, T=64, Hq=8, Hkv=2, D=128, bs=16, mb=8,
                N=16, scale=0.088, pt=0, ws=None, wsb=0, dt=pkv.PKV_BF16)
    args.update(kw)
    lib = pkv.load_library()
    st = lib.paged_attention_prefill(args["q"], args["k"], args["v"], args["tab"], args["lens"], args["out"],
                                     args["lse"], args["B"], args["T"], args["Hq"], args["Hkv"], args["D"], args["bs"],
                                     args["mb"], args["N"], args["scale"], args["pt"], args["ws"], args["wsb"],
                                     args["dt"], None)
    return st, lib.pkv_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), pkv.PKV_EINVAL),
    (dict(out=None), pkv.PKV_EINVAL),
    (dict(out=K), pkv.PKV_EINVAL),                  # out aliases k_pool
    (dict(Hq=6, Hkv=4), pkv.PKV_EINVAL),
    (dict(T=0), pkv.PKV_EINVAL),
    (dict(scale=float("inf")), pkv.PKV_EINVAL),
    (dict(dt=3), pkv.PKV_EINVAL),
    (dict(dt=pkv.PKV_FP32), pkv.PKV_EUNSUPPORTED),
    (dict(D=80), pkv.PKV_EUNSUPPORTED),
    (dict(bs=8), pkv.PKV_EUNSUPPORTED),
    (dict(T=8193), pkv.PKV_EUNSUPPORTED),
    (dict(Hq=32, Hkv=2), pkv.PKV_EUNSUPPORTED),     # Hq/Hkv = 16
    (dict(pt=-32), pkv.PKV_EINVAL),
    (dict(pt=48), pkv.PKV_EINVAL),                   # not a multiple of 32
    (dict(pt=32), pkv.PKV_EWORKSPACE),               # 128 keys in 4 pieces: partials need a workspace
    (dict(pt=32, ws=ctypes.c_void_p(1 << 20), wsb=64), pkv.PKV_EWORKSPACE),   # too small
    (dict(pt=32, ws=ctypes.c_void_p((1 << 20) + 4), wsb=1 << 30), pkv.PKV_EINVAL),   # misaligned
])
def test_prefill_argument_errors(kw, status):
    st, msg = _prefill(**kw)
    assert st == status, msg
    assert msg


def test_prefill_empty_batch_is_a_noop():
    st, _ = _prefill(B=0, q=None, out=None)
    assert st == pkv.PKV_OK


def test_prefill_workspace_and_piece_policy():
    """Workspace: one 128-row slot of D + 1 floats per (sequence, row group,
    KV head, piece) when any item can have more than one piece, else none.
    The suggested piece length leaves grids that fill the device unsplit and
    cuts the key bound of a one-sequence chunk into multiples of 32 tokens
    (without a GPU the library assumes 256 CUs)."""
    lib = pkv.load_library()
    wsb = lib.pkv_prefill_workspace_bytes
    # B=2, T=64, G=4: 256 rows, 2 row groups; 8 blocks = 128 keys in pieces of 32: 4 pieces
    assert wsb(2, 64, 8, 2, 128, 16, 8, 32) == 2 * 2 * 2 * 4 * 128 * 129 * 4
    assert wsb(2, 64, 8, 2, 128, 16, 8, 0) == 0
    assert wsb(2, 64, 8, 2, 128, 16, 8, 128) == 0    # one piece covers every key
    assert wsb(2, 64, 8, 2, 128, 16, 8, -32) == 0 and wsb(2, 64, 8, 2, 128, 8, 8, 32) == 0
    pt = lib.pkv_prefill_piece_tokens
    assert pt(8, 512, 32, 8, 128, 16, 256) == 0       # 1024 items for 512 slots: no split
    assert pt(1, 512, 32, 8, 128, 16, 544) == 2176   # 128 items: 4 pieces of the 8704-token bound
    assert pt(1, 512, 32, 8, 64, 16, 544) == 1088    # D = 64: 1024 slots, 8 pieces
    assert pt(1, 512, 32, 8, 128, 16, 8) == 0        # 128 keys: never below 512 tokens
    assert pt(1, 512, 32, 8, 80, 16, 544) == 0       # unsupported head dim


def test_append_rope_argument_errors():
    lib = pkv.load_library()
    f = lib.paged_kv_append_rope
    ok = (P, 8, P, P, P, P, P, P, 2, 1, 2, 64, 16, 4, 8)
    assert f(*ok, 0.0, pkv.PKV_BF16, None) == pkv.PKV_EINVAL            # theta must be > 0
    assert f(*ok, float("nan"), pkv.PKV_BF16, None) == pkv.PKV_EINVAL
    assert f(P, 5, *ok[2:], 10000.0, pkv.PKV_BF16, None) == pkv.PKV_EINVAL      # Hq not a multiple of Hkv
    assert f(P, 8, P, None, *ok[4:], 10000.0, pkv.PKV_BF16, None) == pkv.PKV_EINVAL   # v_new missing
    assert f(P, 8, P, P, P, P, P, P, 2, 1, 2, 96, 16, 4, 8, 10000.0, pkv.PKV_BF16, None) == pkv.PKV_EUNSUPPORTED
    assert f(P, 8, P, P, P, P, P, P, 0, 1, 2, 64, 16, 4, 8, 10000.0, pkv.PKV_BF16, None) == pkv.PKV_OK   # B = 0
    assert f(P, 8, P, P, P, P, P, P, 2, 1, 2, 64, 16, 4, 8, 10000.0, 5, None) == pkv.PKV_EINVAL        # dtype


def test_append_gather_reduce_argument_errors():
    lib = pkv.load_library()
    assert lib.paged_kv_append(P, P, P, P, P, None, 2, 1, 8, 64, 16, 4, 8, pkv.PKV_BF16, None) == pkv.PKV_EINVAL
    assert lib.paged_kv_append(P, P, P, P, P, P, 2, 1, 8, 64, 8, 4, 8, pkv.PKV_BF16, None) == pkv.PKV_EUNSUPPORTED
    assert lib.paged_kv_append(P, P, P, P, P, P, 0, 1, 8, 64, 16, 4, 8, pkv.PKV_BF16, None) == pkv.PKV_OK
    assert lib.paged_kv_gather(P, P, P, P, None, P, 2, 64, 8, 64, 16, 4, 8, pkv.PKV_BF16, None) == pkv.PKV_EINVAL
    assert lib.paged_kv_gather(P, P, P, P, P, P, 2, 64, 8, 80, 16, 4, 8, pkv.PKV_BF16, None) == pkv.PKV_EUNSUPPORTED
    assert lib.lse_reduce(P, None, P, None, 2, 1, 8, 128, 4, pkv.PKV_BF16, None) == pkv.PKV_EINVAL
    assert lib.lse_reduce(P, P, P, None, 2, 1, 8, 100, 4, pkv.PKV_BF16, None) == pkv.PKV_EUNSUPPORTED
    assert lib.lse_reduce(P, P, P, None, 2, 1, 8, 128, 0, pkv.PKV_BF16, None) == pkv.PKV_EINVAL


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(pkv, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        pkv.load_library(tmp_path / "missing.so")


def test_misaligned_tensors_rejected():
    """Rows move with 16-byte vector accesses: a tensor argument that is not
    16-byte aligned is an argument error, reported before any launch."""
    lib = pkv.load_library()
    odd = ctypes.c_void_p(4096 * 9 + 8)
    st, msg = _decode(q=odd)
    assert st == pkv.PKV_EINVAL and "16-byte" in msg
    st, msg = _decode(out=odd)
    assert st == pkv.PKV_EINVAL and "16-byte" in msg
    st, msg = _prefill(k=odd)
    assert st == pkv.PKV_EINVAL and "16-byte" in msg
    assert lib.paged_kv_append(odd, P, P, P, P, P, 2, 1, 8, 64, 16, 4, 8, pkv.PKV_BF16, None) == pkv.PKV_EINVAL
    assert lib.paged_kv_copy_blocks(P, odd, P, P, 1, 8, 64, 16, 8, pkv.PKV_BF16, None) == pkv.PKV_EINVAL
    assert lib.paged_kv_gather(P, P, P, P, odd, P, 2, 64, 8, 64, 16, 4, 8, pkv.PKV_BF16, None) == pkv.PKV_EINVAL
    assert "16-byte" in lib.pkv_last_error().decode()


def test_binding_checks_attention_arguments():
    """The binding rejects tensors whose dtype, shape or device disagree before
    any pointer reaches the library (metadata only, CPU tensors)."""
    import torch
    B, T, Hq, Hkv, D, N = 3, 2, 8, 2, 64, 10
    bf = torch.bfloat16
    q = torch.zeros(B, T, Hq, D, dtype=bf)
    kp = torch.zeros(N, 16, Hkv, D, dtype=bf)
    tab = torch.zeros(B, 4, dtype=torch.int32)
    lens = torch.ones(B, dtype=torch.int32)
    ok = dict(q=q, k_pool=kp, v_pool=kp.clone(), block_tables=tab, context_lens=lens,
              out=torch.zeros_like(q), lse_out=torch.zeros(B, T, Hq))
    pkv.check_attention_args(**ok)
    bad = [
        (dict(q=q.float()), TypeError),                                       # fp32 q, bf16 pools
        (dict(out=torch.zeros(B, T, Hq, D)), TypeError),                       # fp32 out, bf16 q
        (dict(v_pool=torch.zeros(N, 16, Hkv, 2 * D, dtype=bf)), ValueError),   # pools differ
        (dict(k_pool=torch.zeros(N, 16, Hkv, 2 * D, dtype=bf),
              v_pool=torch.zeros(N, 16, Hkv, 2 * D, dtype=bf)), ValueError),   # head size differs from q
        (dict(k_pool=torch.zeros(N, 16, 3, D, dtype=bf), v_pool=torch.zeros(N, 16, 3, D, dtype=bf)), ValueError),
        (dict(out=torch.zeros(B, T, Hq, D // 2, dtype=bf)), ValueError),
        (dict(lse_out=torch.zeros(B, T, Hq, dtype=torch.float64)), ValueError),
        (dict(lse_out=torch.zeros(B, Hq)), ValueError),
        (dict(block_tables=torch.zeros(B * 4, dtype=torch.int32)), ValueError),
        (dict(block_tables=torch.zeros(B + 1, 4, dtype=torch.int32)), ValueError),
        (dict(block_tables=tab.long()), TypeError),
        (dict(context_lens=torch.ones(B + 1, dtype=torch.int32)), ValueError),
        (dict(context_lens=lens.long()), TypeError),
        (dict(q=q[0]), ValueError),
        (dict(lse_out=torch.zeros(B, T, Hq, device="meta")), ValueError),    # two devices
    ]
    for change, exc in bad:
        with pytest.raises(exc):
            pkv.check_attention_args(**dict(ok, **change))


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """The allocation-free decode refuses, before touching a device, a call
    whose workspace would not fit its static scratch (here: the long-context
    verify shape split into 512-token partitions, about 169 MB)."""
    lib = pkv.load_library()
    need = pkv.pkv_decode_workspace_bytes(16, 4, 32, 128, 4096, 16, 512)
    assert need > pkv.PKV_NOALLOC_SCRATCH_BYTES
    st = lib.paged_attention_decode_noalloc(Q, K, V, TAB, LENS, OUT, None, 16, 4, 32, 8, 128, 16, 4096, 50000,
                                            0.088, 512, pkv.PKV_BF16, None)
    assert st == pkv.PKV_EWORKSPACE
    msg = lib.pkv_last_error().decode()
    assert str(need) in msg and str(pkv.PKV_NOALLOC_SCRATCH_BYTES) in msg
    # argument errors come first, as for paged_attention_decode
    assert lib.paged_attention_decode_noalloc(None, K, V, TAB, LENS, OUT, None, 2, 1, 8, 2, 128, 16, 4, 8, 0.088, 0,
                                              pkv.PKV_BF16, None) == pkv.PKV_EINVAL
    # the 8B-shaped single-token batch fits
    assert pkv.pkv_decode_workspace_bytes(256, 1, 32, 128, 512, 16, 0) <= pkv.PKV_NOALLOC_SCRATCH_BYTES
