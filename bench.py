"""Benchmark: block-sparse attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload winglobal128k]

A step is one bsa_forward over the whole workload (every q-block of every
head; one kernel launch) with inputs already resident in HBM.  Prints ONE JSON
line: ms per forward and effective TFLOP/s on the active tiles
(4 * block^2 * head_dim FLOPs per planned tile), the roofline of the kernel
(HIP-event time of the launch on its stream), the oracle's CPU rate on a
bounded sample of the same workload, and context timings (the 256K GQA
window+global workload and the same shape with a dense causal mask, run by
the same kernel).
"""
from __future__ import annotations

import argparse
import json
import math
import multiprocessing as mp
import os
import sys
import time

import numpy as np
import torch

from block_sparse_flash_bsa_amd import bsattn
from block_sparse_flash_bsa_amd import workloads as wl

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA (published)
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def time_forward(p, q, k, v, out, lse, steps, warmup):
    """Warm up, then time `steps` forwards: wall clock around the loop and a
    HIP event pair per launch on the stream the kernel is launched on."""
    for _ in range(warmup):
        bsattn.forward(q, k, v, p, out, lse)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        bsattn.forward(q, k, v, p, out, lse)
        b.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ev_ms = [a.elapsed_time(b) for a, b in evs]
    return wall_ms, ev_ms


def plan_for(w, lay, **kw):
    return bsattn.plan(w.batch, w.heads, w.kv_heads, w.seq_len, w.head_dim, w.block, w.dtype, lay, **kw)


# ------------------------------------------------------------- CPU baseline
_CPU = {}


def _cpu_init(path, lay, bs):
    """Worker start-up (spawned process): memory-map one head's Q/K/V."""
    os.environ["OMP_NUM_THREADS"] = "1"
    import oracle  # test infrastructure: only this baseline leg of the benchmark uses it
    _CPU.update(oracle=oracle, lay=lay, bs=bs, h0=0,
                q=np.load(path + "_q.npy", mmap_mode="r"), k=np.load(path + "_k.npy", mmap_mode="r"),
                v=np.load(path + "_v.npy", mmap_mode="r"))


def _cpu_worker(args):
    """Run the oracle on random runs of 128 consecutive query rows (one
    q-block) for `seconds`; return (rows, elapsed)."""
    seed, seconds = args
    d = _CPU
    N = d["q"].shape[2]
    rng = np.random.default_rng(seed)
    done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        q0 = int(rng.integers(0, N // 128)) * 128
        q1 = min(N, q0 + 128)
        d["oracle"].forward_query_range(d["q"][0, 0, q0:q1], d["k"][0, 0], d["v"][0, 0], d["lay"], d["bs"],
                                        d["h0"], q0)
        done += q1 - q0
    return done, time.perf_counter() - t0


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (empty if unavailable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def cpu_baseline(w, lay, q, k, v, flops, seconds=15.0):
    """The oracle, as it is, on a bounded sample of the workload's rows.

    One head's Q/K/V (exact float32 copies of the bf16 inputs) is written to
    /tmp and memory-mapped by spawned worker processes (one thread each); each
    worker evaluates random q-blocks (128 consecutive query rows, the oracle's
    query-range form of the definition) for `seconds`.  The full-job time is
    extrapolated from the measured rows per second."""
    import tempfile
    B, H, N = w.batch, w.heads, w.seq_len
    group = w.heads // w.kv_heads
    h0 = H // 2
    tmp = tempfile.mkdtemp(prefix="bsa_cpu_")
    path = os.path.join(tmp, "head")
    np.save(path + "_q.npy", q[0:1, h0:h0 + 1].float().cpu().numpy())
    np.save(path + "_k.npy", k[0:1, h0 // group:h0 // group + 1].float().cpu().numpy())
    np.save(path + "_v.npy", v[0:1, h0 // group:h0 // group + 1].float().cpu().numpy())
    lay1 = dict(lay)
    if lay.get("bitmap") is not None:
        lay1["bitmap"] = np.asarray(lay["bitmap"][h0:h0 + 1])
    host_cpus = os.cpu_count() or 1
    cores = max(1, min(16, host_cpus))
    ctx = mp.get_context("spawn")
    # One BLAS thread per worker: the spawned processes read these at import.
    saved = {n: os.environ.get(n) for n in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS")}
    os.environ.update(OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1")
    try:
        with ctx.Pool(cores, initializer=_cpu_init, initargs=(path, lay1, w.block)) as pool:
            pool.map(_cpu_worker, [(s, 0.5) for s in range(cores)])       # warm-up
            t0 = time.perf_counter()
            res = []
            for r in pool.imap_unordered(_cpu_worker, [(100 + s, seconds) for s in range(cores)]):
                res.append(r)
                log(f"[bench] cpu worker done: {r[0]} rows in {r[1]:.1f} s")
            wall = time.perf_counter() - t0
    finally:
        for n, val in saved.items():
            if val is None:
                os.environ.pop(n, None)
            else:
                os.environ[n] = val
        for suffix in ("_q.npy", "_k.npy", "_v.npy"):
            if os.path.exists(path + suffix):
                os.remove(path + suffix)
        os.rmdir(tmp)
    rows = sum(r[0] for r in res)
    full_s = wall * (B * H * N) / rows
    return {"value": flops / full_s / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "host_cpu_count": host_cpus, "host_cpu_model": cpu_model(),
            "sample": f"{rows} query rows (random q-blocks of 128 consecutive rows) of head {h0} of "
                      f"{w.name}, evaluated by the float64 oracle's query-range form in {cores} "
                      f"single-threaded processes over {wall:.1f} s (host: {host_cpus} CPUs); "
                      f"full-job time extrapolated to {B * H * N} rows = {full_s:.0f} s",
            "extrapolated_full_s": round(full_s, 1)}


# Sources a kernel's code is compiled from: its own file and the headers it
# includes.  A counter summary records their combined SHA-256.
KERNEL_SOURCES = {
    "forward": ("forward.hip", "queue.h", "internal.h"),
    "backward": ("backward.hip", "queue.h", "internal.h"),
}


def sources_sha256(kind):
    """SHA-256 over the concatenated sources of one kernel family (None when one is missing)."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        path = os.path.join(here, "block_sparse_flash_bsa_amd", "csrc", name)
        if not os.path.exists(path):
            return None
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by its plain-copy calibration).
    None when there is no summary for this kernel and workload, or when the
    kernel's sources changed since the counters were taken."""
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", f"{kernel}_{workload}_hbm.txt")
    sha = sources_sha256("forward")
    if not os.path.exists(path) or sha is None:
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if not line.startswith("#") and ":" in line:
                key, val = line.split(":", 1)
                rec[key.strip()] = val.strip()
    if rec.get("forward_sources_sha256") != sha or "traffic_bytes_per_launch" not in rec:
        return None
    return int(rec["traffic_bytes_per_launch"])


def calibrate_copy(mib):
    """A plain device copy of known size, for scaling HBM byte counters."""
    x = torch.ones(mib * 2 ** 18, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": x.numel() * 4, "copy_bytes_written": y.numel() * 4,
                      "launches": 3}), flush=True)


def dynamic_plan_context():
    """Device-side CSR from a device bitmap (bsa_plan_set_bitmap) against the host planner
    on the same bitmap: the 32K random layout's per-head Bernoulli(0.10) bitmap, and a
    256K causal per-head bitmap of the density of the 256K windowed layout (2%)."""
    res = {}
    w = wl.WORKLOADS["random32k"]
    cases = {"random32k": (w, wl.layout_of(w)["bitmap"], False)}
    g = torch.Generator(device="cuda").manual_seed(5)
    nb = 262144 // 128
    bm = (torch.rand((32, nb, nb), generator=g, device="cuda") < 0.02).to(torch.uint8)
    bm[:, torch.arange(nb), torch.arange(nb)] = 1
    rw = wl.Workload("router256k", 1, 32, 8, 262144, 128, 128, torch.bfloat16, 5, {})
    cases["router256k"] = (rw, bm.cpu().numpy(), True)
    del bm
    for name, (cw, bitmap, causal) in cases.items():
        lay = dict(causal=causal, unit="blocks", window_left=-1, window_right=-1, global_keys=0,
                   global_queries=0, bitmap=bitmap)
        t = time.perf_counter()
        hp = plan_for(cw, lay)
        host_ms = (time.perf_counter() - t) * 1e3
        dp = bsattn.plan_dynamic(cw.batch, cw.heads, cw.kv_heads, cw.seq_len, cw.head_dim, cw.block,
                                 cw.dtype, causal, bitmap.shape[0])
        dbm = torch.from_numpy(np.ascontiguousarray(bitmap, dtype=np.uint8)).cuda()
        nnz = torch.zeros(1, dtype=torch.int64, device="cuda")
        for _ in range(3):
            dp.set_bitmap(dbm, nnz)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            dp.set_bitmap(dbm, nnz)
        e1.record()
        torch.cuda.synchronize()
        res[name] = {"bitmap": list(bitmap.shape), "causal": causal, "nnz": int(nnz.item()),
                     "host_plan_ms": round(host_ms, 2),
                     "device_plan_us": round(e0.elapsed_time(e1) * 1e3 / 20, 1),
                     "nnz_matches_host": int(nnz.item()) == hp.info["nnz"]}
        # The forward through each plan (same bitmap, same inputs), alternating.
        q, k, v = wl.make_qkv(cw, "cuda")
        out, lse = bsattn.forward(q, k, v, hp)
        ms = {"static": [], "dynamic": []}
        for _ in range(3):
            for kind, pl in (("static", hp), ("dynamic", dp)):
                bsattn.forward(q, k, v, pl, out, lse)
                torch.cuda.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(5):
                    bsattn.forward(q, k, v, pl, out, lse)
                b.record()
                torch.cuda.synchronize()
                ms[kind].append(a.elapsed_time(b) / 5)
        res[name]["forward_static_ms"] = round(float(np.median(ms["static"])), 4)
        res[name]["forward_dynamic_ms"] = round(float(np.median(ms["dynamic"])), 4)
        log(f"[bench] dynamic plan {name}: {res[name]}")
        del dbm, dp, hp, q, k, v, out, lse
    res["backward_long_columns"] = dynamic_backward_context()
    return res


def dynamic_backward_context(steps=5):
    """The backward through a dynamic plan against the static plan of the same
    bitmap, where key-block columns are dense (global key blocks read by every
    q-block): B=1, H=32, Hkv=8, N=64K, causal, per-head Bernoulli(0.05) bitmap
    with the diagonal and key blocks 0 and 1 on.  bsa_plan_set_bitmap cuts
    the long dK/dV walks on the device, as the host planner does."""
    w = wl.Workload("globalcols64k", 1, 32, 8, 65536, 128, 128, torch.bfloat16, 6, {})
    nb = w.seq_len // w.block
    g = torch.Generator(device="cuda").manual_seed(6)
    bm = (torch.rand((w.heads, nb, nb), generator=g, device="cuda") < 0.05).to(torch.uint8)
    bm[:, torch.arange(nb), torch.arange(nb)] = 1
    bm[:, :, :2] = 1
    lay = dict(causal=True, unit="blocks", window_left=-1, window_right=-1, global_keys=0, global_queries=0,
               bitmap=bm.cpu().numpy())
    sp = plan_for(w, lay)
    dp = bsattn.plan_dynamic(w.batch, w.heads, w.kv_heads, w.seq_len, w.head_dim, w.block, w.dtype, True, w.heads)
    dp.set_bitmap(bm)
    q, k, v = wl.make_qkv(w, "cuda")
    do = wl.make_dout(w, "cuda")
    res = {"bitmap": [w.heads, nb, nb], "active_tiles": sp.info["active_blocks"]}
    for name, p in (("static", sp), ("dynamic", dp)):
        out, lse = bsattn.forward(q, k, v, p)
        res[f"{name}_ms"] = round(float(np.mean(time_backward(p, q, k, v, out, lse, do, steps, 1))), 3)
        res[f"{name}_split_columns"] = p.read_work_kv()[1]
    res["dynamic_over_static"] = round(res["dynamic_ms"] / res["static_ms"], 3)
    log(f"[bench] dynamic-plan backward with dense key-block columns: {res}")
    del q, k, v, do, sp, dp, bm
    torch.cuda.empty_cache()
    return res


def merge_context(steps=20):
    """bsa_lse_merge of two partial results of the 128K workload's output shape
    (bf16 O [32, 131072, 128] and fp32 LSE per part): an HBM-bound kernel that
    reads each part once and writes the result once; GB/s against 8 TB/s."""
    P, rows, D = 2, 32 * 131072, 128
    g = torch.Generator(device="cuda").manual_seed(9)
    O = torch.randn((P, rows, D), generator=g, device="cuda").to(torch.bfloat16)
    L = torch.randn((P, rows), generator=g, device="cuda")
    out = torch.empty((rows, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    for _ in range(3):
        bsattn.lse_merge(O, L, out, lse)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        bsattn.lse_merge(O, L, out, lse)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    nbytes = (P + 1) * rows * (D * 2 + 4)
    res = {"parts": P, "rows": rows, "head_dim": D, "ms": round(ms, 4), "bytes": nbytes,
           "gb_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
           "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / (PEAK_HBM_GBS * 1e9), 4)}
    log(f"[bench] lse_merge: {res}")
    del O, L, out, lse
    torch.cuda.empty_cache()
    return res


def time_backward(p, q, k, v, out, lse, do, steps, warmup):
    """Warm up, then time `steps` backwards (three launches each) with a HIP
    event pair around each on the launch stream; returns the per-step ms."""
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    for _ in range(warmup):
        bsattn.backward(q, k, v, out, lse, do, p, dq, dk, dv, delta)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        bsattn.backward(q, k, v, out, lse, do, p, dq, dk, dv, delta)
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def backward_context(names, steps=5):
    """bsa_backward on the workloads: ms per backward (Delta, dQ and dK/dV
    kernels), TFLOP/s counting the five GEMMs of an attention backward per
    active tile (S recomputed, dP, dV, dK, dQ: 10 * block^2 * head_dim, the
    usual 2.5x of the forward) against the dtype's peak, and the seven the
    kernels execute (S and dP are formed in both the dQ and the dK/dV
    kernel)."""
    res = {}
    for name in names:
        w = wl.WORKLOADS[name]
        p = plan_for(w, wl.layout_of(w))
        q, k, v = wl.make_qkv(w, "cuda")
        do = wl.make_dout(w, "cuda")
        out, lse = bsattn.forward(q, k, v, p)
        ms = float(np.mean(time_backward(p, q, k, v, out, lse, do, steps, 1)))
        tiles = p.info["active_blocks"]
        unit = w.block * w.block * w.head_dim
        alg = 10.0 * unit * tiles / (ms * 1e-3) / 1e12
        peak = PEAK_BF16_TFLOPS if w.dtype == torch.bfloat16 else PEAK_F32_TFLOPS
        res[name] = {"ms_per_backward": round(ms, 3), "tflops_algorithmic": round(alg, 1),
                     "pct_of_peak": round(100 * alg / peak, 2),
                     "tflops_mfma_executed": round(1.4 * alg, 1), "active_tiles": tiles}
        log(f"[bench] backward {name}: {res[name]}")
        del q, k, v, do, out, lse, p
        torch.cuda.empty_cache()
    return res


def lengths_context(steps=5):
    """Sequence lengths the block does not divide, and variable-length batches,
    on the 128K window+global rule at B=4, H=32, N=32K: the whole-block kernels,
    the ragged-tail kernels at N - 64, and the variable-length forward and
    backward at full and at mixed lengths; TFLOP/s counts the active tiles of
    each entry's own length."""
    base = wl.WORKLOADS["winglobal128k"]
    lay = wl.layout_of(base)
    res = {}

    def rate(flops, ms):
        return round(flops / (ms * 1e-3) / 1e12, 1)

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]))

    N = 32768
    for name, n in (("whole_blocks", N), ("ragged_tail", N - 64)):
        w = base.with_shape(name=name, batch=4, seq_len=n)
        p = plan_for(w, lay)
        q, k, v = wl.make_qkv(w, "cuda")
        do = wl.make_dout(w, "cuda")
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        ms = timed(lambda: bsattn.forward(q, k, v, p, out, lse))
        bms = timed(lambda: bsattn.backward(q, k, v, out, lse, do, p, dq, dk, dv, delta))
        # the backward's algorithmic work is 2.5x the forward's (5 GEMMs per tile against 2)
        res[name] = {"seq_len": n, "ms_per_forward": round(ms, 4), "tflops": rate(p.flops(), ms),
                     "ms_per_backward": round(bms, 4), "backward_tflops": rate(2.5 * p.flops(), bms)}
        if name == "whole_blocks":
            for lname, lens in (("varlen_full", [N] * 4), ("varlen_mixed", [N, 24000, 16000, 7000])):
                sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
                ms = timed(lambda: bsattn.forward_varlen(q, k, v, p, sl, out, lse))
                bms = timed(lambda: bsattn.backward_varlen(q, k, v, out, lse, do, p, sl, dq, dk, dv, delta))
                useful = sum(plan_for(base.with_shape(batch=1, seq_len=L), lay, host_only=True).flops()
                             for L in lens)
                res[lname] = {"seq_lens": lens, "ms_per_forward": round(ms, 4), "tflops": rate(useful, ms),
                              "ms_per_backward": round(bms, 4), "backward_tflops": rate(2.5 * useful, bms)}
        del q, k, v, do, out, lse, dq, dk, dv, delta, p
        torch.cuda.empty_cache()
    log(f"[bench] lengths: {res}")
    return res


def mfma_probe(workgroups=512, iters=200000):
    """Sustained bf16 MFMA rate of this GPU (libbsattn_probe: independent
    v_mfma_f32_32x32x16_bf16 chains on register operands, 2 waves per SIMD on
    every CU): the measured peak the attention kernel is also reported
    against, since the chip clocks down under sustained matrix load."""
    import ctypes
    from block_sparse_flash_bsa_amd import build as bld
    L = ctypes.CDLL(bld.PROBE_LIB)
    L.bsa_probe_mfma.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    L.bsa_probe_mfma.restype = ctypes.c_int32
    L.bsa_probe_mfma_flops.argtypes = [ctypes.c_int64, ctypes.c_int32]
    L.bsa_probe_mfma_flops.restype = ctypes.c_double
    out = torch.empty(workgroups * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    run = lambda n: L.bsa_probe_mfma(n, workgroups, ctypes.c_void_p(out.data_ptr()),
                                     ctypes.c_void_p(stream.cuda_stream))
    if run(iters // 10) != 0:
        raise RuntimeError("MFMA probe launch failed")
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    run(iters)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    tf = L.bsa_probe_mfma_flops(iters, workgroups) / (ms * 1e-3) / 1e12
    log(f"[bench] MFMA probe: {ms:.1f} ms, {tf:.1f} TFLOP/s")
    return {"tflops": round(tf, 1), "ms": round(ms, 2), "workgroups": workgroups, "iters": iters,
            "instruction": "v_mfma_f32_32x32x16_bf16"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="winglobal128k", choices=sorted(wl.WORKLOADS))
    ap.add_argument("--schedule", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--backward-only", action="store_true",
                    help="only time bsa_backward on --workload (for profiling) and print its JSON")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MiB",
                    help="only run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE={world}): "
              "this forward has no multi-GPU path; shard heads or batch entries across GPUs with "
              "independent processes instead.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    bsattn.lib()
    if args.backward_only:
        print(json.dumps({"backward": backward_context([args.workload], args.steps)}), flush=True)
        return

    w = wl.WORKLOADS[args.workload]
    lay = wl.layout_of(w)
    # The plan (host CSR, work orders, upload) is built and timed apart from
    # the forward: median of 5 builds; the last one is used.
    plan_times = []
    for _ in range(5):
        t = time.perf_counter()
        p = plan_for(w, lay, schedule=args.schedule)
        plan_times.append((time.perf_counter() - t) * 1e3)
    plan_ms = float(np.median(plan_times))
    flops = p.flops()
    log(f"[bench] {w.name}: plan {plan_ms:.1f} ms, {p.info['active_blocks']} active tiles, "
        f"{flops / 1e12:.2f} TFLOP per forward")
    q, k, v = wl.make_qkv(w, "cuda")
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    wall_ms, ev_ms = time_forward(p, q, k, v, out, lse, args.steps, args.warmup)
    kern_ms = float(np.mean(ev_ms))
    peak = PEAK_BF16_TFLOPS if w.dtype == torch.bfloat16 else PEAK_F32_TFLOPS
    value = flops / (wall_ms * 1e-3) / 1e12
    achieved = flops / (kern_ms * 1e-3) / 1e12
    log(f"[bench] {args.steps} steps: {wall_ms:.3f} ms/forward wall, kernel {kern_ms:.3f} ms "
        f"(min {min(ev_ms):.3f}, max {max(ev_ms):.3f}) -> {achieved:.1f} TFLOP/s")
    kernel = "fwd_bf16_d128" if w.dtype == torch.bfloat16 else "fwd_f32"
    elem = 2 if w.dtype == torch.bfloat16 else 4
    min_bytes = (q.numel() + k.numel() + v.numel() + out.numel()) * elem + lse.numel() * 4
    result = {
        "metric": "block-sparse attn fwd: ms/fwd + effective TFLOP/s on active blocks (% MFMA peak)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic: seeded iid N(0,1) Q/K/V drawn on the GPU",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "kv_heads": w.kv_heads,
                   "seq_len": w.seq_len, "head_dim": w.head_dim, "block": w.block,
                   "layout": {k_: v_ for k_, v_ in w.layout.items() if k_ != "bitmap"},
                   "active_tiles": p.info["active_blocks"], "schedule": args.schedule},
        "pct_of_mfma_peak": round(100 * value / peak, 2),
        # Kernel-event percentiles over the timed launches, and the rate that
        # counts only allowed (q, k) pairs (4 * head_dim FLOPs each) instead
        # of whole tiles.
        "kernel_ms_p10_p50_p90": [round(float(x), 4) for x in np.percentile(ev_ms, [10, 50, 90])],
        "token_exact_tflops": round(4.0 * w.head_dim * p.info["allowed_pairs"] / (kern_ms * 1e-3) / 1e12, 2),
        "plan_ms_median_of_5": round(plan_ms, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": recorded_traffic(kernel, w.name), "traffic_unit": "HBM bytes per launch",
                     "kernel": kernel,
                     "kernel_ms": round(kern_ms, 4),
                     "algorithmic_flops": flops, "min_hbm_bytes": min_bytes},
    }
    if w.dtype == torch.bfloat16:
        probe = mfma_probe()
        result["roofline"]["measured_peak"] = probe["tflops"]
        result["roofline"]["frac_of_measured_peak"] = round(achieved / probe["tflops"], 4)
        result["mfma_probe"] = probe
    if not args.no_context:
        # The other workloads, timed the same way (kernel HIP events), and the
        # dense causal comparator of the 256K shape on the same kernel.
        ctx = {}
        for name in ("tiny_f32", "window16k", "random32k", "gqa256k", "dense256k"):
            if name == w.name:
                continue
            cw = wl.WORKLOADS[name]
            clay = wl.layout_of(cw)
            cp = plan_for(cw, clay)
            del q, k, v, out, lse
            torch.cuda.empty_cache()
            q, k, v = wl.make_qkv(cw, "cuda")
            out = torch.empty_like(q)
            lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
            steps = {"dense256k": 2, "gqa256k": 5}.get(name, 20)
            cw_ms, cev = time_forward(cp, q, k, v, out, lse, steps, 2)
            cpeak = PEAK_BF16_TFLOPS if cw.dtype == torch.bfloat16 else PEAK_F32_TFLOPS
            tf = cp.flops() / (np.mean(cev) * 1e-3) / 1e12
            ctx[name] = {"ms_per_forward": round(float(np.mean(cev)), 4),
                         "tflops": round(float(tf), 1), "pct_of_peak": round(100 * tf / cpeak, 2),
                         "active_tiles": cp.info["active_blocks"]}
            if name in ("tiny_f32", "window16k"):
                # Microsecond-scale launches: 100 back to back between one event pair.
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(100):
                    bsattn.forward(q, k, v, cp, out, lse)
                b.record()
                torch.cuda.synchronize()
                ctx[name]["ms_per_forward_100_back_to_back"] = round(a.elapsed_time(b) / 100, 4)
            log(f"[bench] context {name}: {ctx[name]}")
        ctx["dense_over_sparse_time"] = round(ctx["dense256k"]["ms_per_forward"] /
                                              ctx["gqa256k"]["ms_per_forward"], 2)
        del q, k, v, out, lse
        torch.cuda.empty_cache()
        ctx["dynamic_plan"] = dynamic_plan_context()
        ctx["lse_merge"] = merge_context()
        ctx["lengths"] = lengths_context()
        ctx["backward"] = backward_context(["tiny_f32", "window16k", "random32k", "winglobal128k", "gqa256k"])
        result["context"] = ctx
    if not args.no_cpu_baseline:
        if not args.no_context:      # the context runs replaced the inputs
            q, k, v = wl.make_qkv(w, "cuda")
        log("[bench] timing the CPU oracle on a sample ...")
        result["cpu_baseline"] = cpu_baseline(w, lay, q, k, v, flops, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
