"""Benchmark: paged decode attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--partition P]

A step is one pass of the hot path over one batch: the KV append when the
workload has one, then paged_attention_decode (split-KV partitions plus the
log-sum-exp merge when the workload is split).  Inputs are seeded synthetic
tensors already resident in HBM.  Prints ONE JSON line with seq-steps/s, the
roofline of the decode call (algorithmic bytes / event-timed duration against
the 8 TB/s HBM peak) and the CPU oracle timed on a bounded sample.

The roofline figure is warm: consecutive calls on the same batch, as in a
decode loop.  roofline.cold_cache repeats the call after reading a 1 GiB
buffer (evicting the caches, outside the timed events) and reports its
percentiles beside it.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workload  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix peak of MI355X
METRIC = "seq-steps/s and achieved HBM GB/s (% of peak) for paged decode attention"
DEFAULT_WORKLOAD = "llama8b_prefix_share"


def live_slots(w):
    """Number of distinct (physical block, slot) pairs attention reads."""
    live = np.zeros((w.N_blocks, w.block_size), dtype=bool)
    for b in range(w.B):
        L = int(w.context_lens[b])
        nfull, rem = divmod(L, w.block_size)
        live[w.block_tables[b, :nfull], :] = True
        if rem:
            live[w.block_tables[b, nfull], :rem] = True
    return int(live.sum())


def algorithmic_bytes(w, part=0):
    """Bytes the decode call must move (unique), and the logical KV bytes
    (each sequence in full).  With split-KV partitions of `part` tokens the
    call also writes each partition's normalised partial and lse (fp32, D + 1
    values per row) for every sequence of more than one partition; the
    reduce folds them on chip, so they are not read back."""
    e = w.elem_bytes
    row = w.Hkv * w.D * e                      # one token, all KV heads, K or V
    kv_unique = 2 * row * live_slots(w)
    kv_logical = 2 * row * int(w.context_lens.sum())
    qo = 2 * w.B * w.T * w.Hq * w.D * e        # q read + out written
    tables = 4 * int(np.sum(-(-w.context_lens // w.block_size))) + 4 * w.B
    append = 2 * 2 * w.B * w.T * row if w.lens_pre is not None else 0   # k_new+v_new read and written
    partials = 0
    if part:
        pb = -(-w.context_lens.astype(np.int64) // part)
        partials = int(np.sum(np.where(pb > 1, pb, 0))) * w.T * w.Hq * (w.D + 1) * 4
    return dict(decode=kv_unique + qo + tables + partials, logical=kv_logical + qo + tables + partials,
                append=append, kv_unique=kv_unique, kv_logical=kv_logical, partials=partials)


# Decode-kernel sources whose hash guards the committed traffic figures (both
# single-pass kernels: a change to either retires every figure).
TRAFFIC_SOURCES = ("pkv_stream.hip", "pkv_verify.hip", "pkv_tile.h", "pkv_device.h", "pkv_internal.h")


def decode_uses_tile(w):
    """Which single-pass kernel paged_attention_decode runs for w (the
    library's choice, restated: the MFMA tile for bf16, D in {64, 128},
    T * G <= 16 query rows per KV head and Hkv <= 8 or a multiple of 8)."""
    G = w.Hq // w.Hkv
    return (w.dtype == "bf16" and w.D in (64, 128) and w.T * G <= 16 and (w.Hkv <= 8 or w.Hkv % 8 == 0)
            and w.B <= 8192)


def measured_traffic(workload_name, part=0):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary (FETCH_SIZE + WRITE_SIZE, calibrated), or None when there
    is none for this workload and partition size or the kernel sources
    changed since."""
    import hashlib
    import re
    suffix = f"_partitions_{part}" if part else ""
    prof = os.path.join(ROOT, "profiles", f"paged_decode_{workload_name}{suffix}.md")
    if not os.path.exists(prof):
        return None
    m = re.search(r"traffic-bytes: fetch=(\d+) write=(\d+) source-sha256=([0-9a-f]+)", open(prof).read())
    if not m:
        return None
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != m.group(3):
        return None
    return int(m.group(1)) + int(m.group(2))


def attention_flops(w):
    """Useful flops of the attention: 4*D per (query row, visible key) pair
    (2*D for q.k, 2*D for p*v); masked pairs are not counted."""
    t = np.arange(w.T)
    vis = np.clip(w.context_lens[:, None].astype(np.int64) - w.T + t[None, :] + 1, 0, None)
    return int(vis.sum()) * w.Hq * 4 * w.D


def host_cores():
    """Cores this process may run on, capped at the 16-core share of one GPU."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, budget_s, repeats=3):
    """The fp64 oracle, untuned, on a bounded sample of the same batch, on the
    host's cores.

    The oracle evaluates one sequence per call (the whole batch of its query
    rows); the sample is the first n sequences in batch order, n chosen from a
    one-sequence calibration so that one pass takes about budget_s / repeats
    seconds on `cores` threads, each thread taking whole sequences with one
    BLAS thread of its own.  The pass is timed `repeats` times (median
    reported, all listed); a one-thread pass over a smaller sample is reported
    beside it."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits

    q_all, kp, vp = w.values(w.q), w.values(w.k_pool), w.values(w.v_pool)
    cores = host_cores()

    def one(b):
        oracle.paged_attention(q_all[b:b + 1], kp, vp, w.block_tables[b:b + 1], w.context_lens[b:b + 1],
                               w.scale, w.block_size)

    def timed_pass(seqs, threads):
        t0 = time.perf_counter()
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, seqs))
        return time.perf_counter() - t0

    with threadpool_limits(limits=1):
        t_one = timed_pass([0], 1)   # calibration, untimed in the result
        per_tok = t_one / max(1, int(w.context_lens[0]))
        order = [b % w.B for b in range(64 * w.B)]
        cum = np.cumsum([int(w.context_lens[b]) for b in order]) * per_tok

        def sample(seconds):
            return order[:max(1, int(np.searchsorted(cum, seconds)) + 1)]
        seqs = sample(budget_s / repeats * cores * 0.8)
        times = [timed_pass(seqs, cores) for _ in range(repeats)]
        seqs1 = sample(budget_s / (2 * repeats))
        t1 = timed_pass(seqs1, 1)
    med = float(np.median(times))
    return {"value": round(len(seqs) / med, 2), "unit": "seq-steps/s", "cores": cores, "kind": "oracle",
            "repeats_s": [round(t, 3) for t in times],
            "one_thread": {"value": round(len(seqs1) / t1, 2), "sequences": len(seqs1), "s": round(t1, 3)},
            "cpu_model": cpu_model(),
            "sample": f"{len(seqs)} sequence-steps of {w.name} in batch order ({min(len(seqs), w.B)} distinct "
                      f"sequences), fp64 NumPy oracle, {cores} threads over sequences with 1 BLAS thread each, "
                      f"median of {repeats} passes"}


def provenance(torch, w):
    """What produced the numbers: device, ROCm and hipcc versions, commit, seed, host CPU."""
    from paged_kv_cache_attention_amd import build as pkv_build
    props = torch.cuda.get_device_properties(0)
    info = {"gpu": torch.cuda.get_device_name(0), "gpu_arch": getattr(props, "gcnArchName", None),
            "gpu_cus": props.multi_processor_count, "torch": torch.__version__, "torch_hip": torch.version.hip,
            "hipcc": None, "seed": workload.WORKLOAD_SEEDS.get(w.name), "host_cpu": cpu_model(),
            "host_cores": host_cores()}
    try:
        info["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        info["rocm"] = None
    info["sources_sha256"] = pkv_build.sources_sha256()
    info["commit"] = None
    try:   # the commit and hipcc the library was built with, recorded by the build while the sources still match
        bi = json.loads(pkv_build.BUILD_INFO.read_text())
        if bi.get("sources_sha256") == info["sources_sha256"]:
            info["commit"] = bi.get("commit")
            info["hipcc"] = bi.get("hipcc")
    except (OSError, ValueError):
        pass
    return info


def read_ceiling(torch, dev, nbytes=2 << 30, reps=10):
    """Read bandwidth of the diagnostic probe: random 32 KB blocks of a 2 GiB pool, read as
    4 KB head slices (the KV-pool pattern), no compute; 8 and 16 waves per CU."""
    import ctypes
    from paged_kv_cache_attention_amd import build as pkv_build
    lib = ctypes.CDLL(str(pkv_build.PROBE_LIB))
    nblocks = nbytes // 32768
    pool = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    g = torch.Generator().manual_seed(0)
    order = torch.randperm(nblocks, generator=g).to(torch.int32).to(dev)
    res = {}
    for grid in (512, 1024):
        sink = torch.empty(grid * 256, dtype=torch.int32, device=dev)
        call = lambda: lib.pkv_probe_slice_read(ctypes.c_void_p(pool.data_ptr()), ctypes.c_void_p(order.data_ptr()),
                                                nblocks, grid, ctypes.c_void_p(sink.data_ptr()), None)
        for _ in range(2):
            assert call() == 0
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            call()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        res[f"GBps_{grid * 4 // 256}_waves_per_cu"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    return res


def copy_ceiling(torch, dev, nbytes=1 << 30, reps=20):
    """Read+write bandwidth of a plain device copy of nbytes (torch's copy kernel)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    return {"bytes_read": nbytes, "bytes_written": nbytes, "ms": round(ms, 4),
            "GBps_read_plus_write": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}


def serve_bench(torch, dev, iters=200):
    """The host runtime: (1) schedule + commit cost per iteration of the native
    engine with 256 running requests (CPU only); (2) a 16-request serving run
    on the device through PagedExecutor (continuous batching with preemption,
    prefix cache, RoPE append, prefill and decode kernels), wall clock."""
    import paged_kv_cache_attention_amd as pkv
    from paged_kv_cache_attention_amd.serve import PagedExecutor
    rng = np.random.default_rng(9)
    eng = pkv.Engine(num_blocks=40000, block_size=16, max_blocks_per_seq=512, max_running=256,
                     max_prefill_tokens=1 << 22, prefix_cache=True)
    for r in range(256):
        eng.add_request(r, rng.integers(0, 32000, size=int(rng.integers(16, 2048))), 2000)
    plan = eng.schedule()
    eng.commit(np.zeros(plan.n, np.int32))
    toks = np.arange(256, dtype=np.int32)
    t0 = time.perf_counter()
    for _ in range(iters):
        plan = eng.schedule()
        eng.commit(toks[:plan.n])
    host_us = (time.perf_counter() - t0) * 1e6 / iters
    eng.close()

    V, HQ, HKV, D = 997, 8, 2, 64
    g = torch.Generator().manual_seed(1234)
    emb = [torch.randn(V, h, D, generator=g).to(torch.bfloat16).to(dev) for h in (HQ, HKV, HKV)]
    common = rng.integers(0, V, size=37)   # one shared prompt ending inside a block
    reqs = []
    for r in range(16):
        p = rng.integers(0, V, size=int(rng.integers(5, 150)))
        if r in (0, 5, 9, 13):
            p = common.copy()
        if r in (2, 7):
            p = np.concatenate([common, p[: len(p) // 3]])
        reqs.append((r, p, 40 if r == 0 else int(rng.integers(3, 30))))
    worst = sum(-(-(len(p) + m) // 16) for _, p, m in reqs)
    kp = torch.zeros(worst // 3, 16, HKV, D, dtype=torch.bfloat16, device=dev)
    vp = torch.zeros_like(kp)

    def serve_once():
        eng = pkv.Engine(worst // 3, 16, max_blocks_per_seq=16, max_running=8, max_prefill_tokens=256,
                         prefix_cache=True)
        for rid, p, m in reqs:
            eng.add_request(rid, p, m)
        ex = PagedExecutor(eng, kp, vp, HQ, 10000.0, lambda t: tuple(e[t.long()] for e in emb),
                           lambda plan, outs: ((plan.request_id * 7 + plan.context_lens) % V).astype(np.int32))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while ex.step() is not None:
            pass
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        st = eng.stats()
        eng.close()
        return wall, st

    serve_once()   # first launches of every kernel and torch op, untimed
    wall, st = serve_once()
    gen = sum(m for _, _, m in reqs)
    return {"engine_host_us_per_iteration_256_running": round(host_us, 2),
            "serve16": {"iterations": st["iterations"], "preemptions": st["preemptions"],
                        "prefix_hit_tokens": st["prefix_hit_tokens"], "cow_copies": st["cow_copies"],
                        "generated_tokens": gen, "wall_s": round(wall, 4),
                        "generated_tokens_per_s": round(gen / wall, 1),
                        "ms_per_iteration": round(wall * 1e3 / st["iterations"], 3)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(workload.WORKLOADS))
    ap.add_argument("--partition", type=int, default=None, help="split-KV partition size (tokens); 0 = single pass")
    ap.add_argument("--cpu-seconds", type=float, default=24.0,
                    help="oracle time budget of the cpu_baseline leg (its passes together)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rope-theta", type=float, default=None,
                    help="append workloads: fused RoPE append (paged_kv_append_rope, queries rotated too)")
    ap.add_argument("--serve", action="store_true",
                    help="measure the host runtime (engine) and a 16-request serving run instead of one batch")
    ap.add_argument("--piece-tokens", type=int, default=None,
                    help="prefill workloads: piece_tokens for the call (0: no key pieces; default: the library's "
                         "suggestion for the shape)")
    ap.add_argument("--cold-reps", type=int, default=20,
                    help="extra untimed-region reps, each after a 1 GiB cache flush, for the cold-cache figure")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_attention_amd as pkv

    if args.serve:
        res = {"mode": "serve", "n_gpus": 1, "data": "synthetic"}
        res.update(serve_bench(torch, torch.device("cuda:0")))
        print(json.dumps(res), flush=True)
        return

    t_gen = time.time()
    w = workload.WORKLOADS[args.workload](poison=False)
    part = w.partition_size if args.partition is None else args.partition
    print(f"# generated {w.name} in {time.time() - t_gen:.1f}s; partition {part}", file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")

    def up(a):
        a = np.ascontiguousarray(a)
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    q, kp, vp = up(w.q), up(w.k_pool), up(w.v_pool)
    tables = torch.from_numpy(w.block_tables).to(dev)
    lens = torch.from_numpy(w.context_lens).to(dev)
    has_append = w.lens_pre is not None
    if has_append:
        k_new, v_new = up(w.k_new), up(w.v_new)
        lens_pre = torch.from_numpy(w.lens_pre).to(dev)
    out = torch.empty_like(q)
    need = pkv.pkv_decode_workspace_bytes(w.B, w.T, w.Hq, w.D, w.max_blocks, w.block_size, part)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    scale = float(w.scale)

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    prefill = w.T > 16   # a chunked-prefill workload: paged_attention_prefill
    if prefill:   # the library's key-piece choice for this shape, workspace allocated up front
        pieces = (pkv.pkv_prefill_piece_tokens(w.B, w.T, w.Hq, w.Hkv, w.D, w.block_size, w.max_blocks)
                  if args.piece_tokens is None else args.piece_tokens)
        pneed = pkv.pkv_prefill_workspace_bytes(w.B, w.T, w.Hq, w.Hkv, w.D, w.block_size, w.max_blocks, pieces)
        pws = torch.empty(max(pneed, 16), dtype=torch.uint8, device=dev)

    def attention():
        if prefill:
            pkv.paged_attention_prefill(q, kp, vp, tables, lens, out=out, scale=scale, piece_tokens=pieces,
                                        workspace=pws, stream=stream)
        else:
            pkv.paged_attention_decode(q, kp, vp, tables, lens, out=out, scale=scale, partition_size=part,
                                       workspace=ws, stream=stream)

    aev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]

    def step(i=None):
        if has_append:
            if i is not None:
                aev[i][0].record(stream)
            if args.rope_theta is not None:
                pkv.paged_kv_append_rope(k_new, v_new, kp, vp, tables, lens_pre, args.rope_theta, q=q, stream=stream)
            else:
                pkv.paged_kv_append(k_new, v_new, kp, vp, tables, lens_pre, stream=stream)
            if i is not None:
                aev[i][1].record(stream)
        if i is not None:
            ev[i][0].record(stream)
        attention()
        if i is not None:
            ev[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    decode_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))

    warm = np.array([a.elapsed_time(b) for a, b in ev])

    # Cold cache: before each rep a 1 GiB buffer is read (more than the 256 MB
    # last-level cache plus the L2s), outside the timed events.  Reading only
    # leaves no dirty lines whose write-back would land in the timed call.
    cold = np.array([])
    if args.cold_reps > 0:
        flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        sink = torch.empty((), dtype=torch.float32, device=dev)
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.cold_reps)]
        for a, b in cev:
            torch.amax(flush, dim=0, out=sink)
            a.record(stream)
            attention()
            b.record(stream)
        torch.cuda.synchronize()
        cold = np.array([a.elapsed_time(b) for a, b in cev])
        del flush

    nb = algorithmic_bytes(w, part)
    achieved = nb["decode"] / (decode_ms * 1e-3) / 1e9
    seq_steps = w.B / (ms_step * 1e-3)
    result = {
        "metric": METRIC, "value": round(seq_steps, 1), "unit": "seq-steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
                   "block_size": w.block_size, "partition_size": part, "total_tokens": int(w.context_lens.sum()),
                   "append": has_append},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(w.name, part),
                     "kernel": (("paged_attention_decode call (balanced MFMA tile with split-KV partitions"
                                 " + piece merge)" if decode_uses_tile(w) else
                                 "paged_attention_decode call (fixed partitions + lse merge)") if part
                                else "paged_attention_decode call (balanced MFMA tile + piece merge)" if decode_uses_tile(w)
                                else "paged_attention_decode call (plan + balanced decode + boundary merge)"),
                     "bytes_per_launch": nb["decode"], "partial_bytes": nb["partials"],
                     "launch_ms": round(decode_ms, 5),
                     "launch_ms_p10_p50_p90": [round(float(np.percentile(warm, p)), 5) for p in (10, 50, 90)],
                     "logical_GBps": round(nb["logical"] / (decode_ms * 1e-3) / 1e9, 1)},
    }
    if prefill:
        # compute-bound: useful flops against the dense bf16 matrix peak
        fl = attention_flops(w)
        tf = fl / (decode_ms * 1e-3) / 1e12
        result["roofline"] = {
            "bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
            "kernel": ("paged_attention_prefill (MFMA tiles, LDS-staged K/V)" if not pieces else
                       f"paged_attention_prefill (MFMA tiles, LDS-staged K/V; {pieces}-token key pieces + merge)"),
            "piece_tokens": pieces, "flops_per_launch": fl,
            "launch_ms": round(decode_ms, 5),
            "launch_ms_p10_p50_p90": [round(float(np.percentile(warm, p)), 5) for p in (10, 50, 90)],
            "bytes_per_launch": nb["decode"], "hbm_GBps": round(achieved, 1)}
        result["tokens_per_s"] = round(w.B * w.T / (ms_step * 1e-3), 1)
    if has_append:
        app_ms = float(np.mean([a.elapsed_time(b) for a, b in aev]))
        rope = args.rope_theta is not None
        app_bytes = nb["append"] + (2 * w.B * w.T * w.Hq * w.D * w.elem_bytes if rope else 0)   # + q read and written
        result["append"] = {"kernel": "paged_kv_append_rope" if rope else "paged_kv_append",
                            "rope_theta": args.rope_theta, "launch_ms": round(app_ms, 5), "bytes_per_launch": app_bytes,
                            "GBps": round(app_bytes / (app_ms * 1e-3) / 1e9, 1)}
    if cold.size:
        cold_med = float(np.median(cold))
        cc = {"reps": int(cold.size),
              "launch_ms_p10_p50_p90": [round(float(np.percentile(cold, p)), 5) for p in (10, 50, 90)]}
        if prefill:
            cc["TFLOPs_at_median"] = round(attention_flops(w) / (cold_med * 1e-3) / 1e12, 1)
        else:
            cc["GBps_at_median"] = round(nb["decode"] / (cold_med * 1e-3) / 1e9, 1)
            cc["frac_at_median"] = round(nb["decode"] / (cold_med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        result["roofline"]["cold_cache"] = cc
    # the practical ceilings, measured in the same run: the read probe (the
    # decode kernels' access pattern, no arithmetic) and a plain device copy
    result["read_ceiling"] = read_ceiling(torch, dev)
    result["copy_ceiling"] = copy_ceiling(torch, dev)
    result["provenance"] = provenance(torch, w)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
