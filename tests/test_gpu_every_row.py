"""Every-row parity of bsa_forward at full size against the float64 oracle.

Each bf16 workload runs once on the GPU in the benchmark's launch
configuration (default plan and work order); then every output row of the
selected heads is compared with the oracle's definition (masked softmax
attention over the row's allowed keys, in float64), evaluated by a pool of
spawned CPU processes over runs of 128 consecutive query rows.  Tolerances
(max abs error over all rows): 2e-2 on O, 1e-3 on LSE; a row's LSE must be
finite exactly when the oracle's is.

Heads: every head of every workload by default.  BSA_EVERY_ROW_HEADS=n
limits each workload to n heads spread over the head range (first and last
included), for quicker local runs.
"""
import multiprocessing as mp
import os
import shutil
import sys
import tempfile
import time

import numpy as np
import pytest
import torch

from block_sparse_flash_bsa_amd import bsattn
from block_sparse_flash_bsa_amd import workloads as wl
from tests import every_row_worker

pytestmark = pytest.mark.gpu

TOL_O, TOL_L = 2e-2, 1e-3
ROWS_PER_TASK = 2048


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsattn.lib()
    torch.cuda.set_device(0)


def heads_to_check(w):
    n = os.environ.get("BSA_EVERY_ROW_HEADS", "all")
    pairs = [(b, h) for b in range(w.batch) for h in range(w.heads)]
    if n == "all" or int(n) >= len(pairs):
        return pairs
    idx = np.unique(np.linspace(0, len(pairs) - 1, int(n)).round().astype(int))
    return [pairs[i] for i in idx]


def scratch_dir():
    base = "/dev/shm" if os.access("/dev/shm", os.W_OK) else None
    return tempfile.mkdtemp(prefix="bsa_rows_", dir=base)


def dump(path, name, t):
    a = t.cpu()
    if a.dtype == torch.bfloat16:
        a = a.view(torch.int16)
    arr = a.numpy()
    if arr.dtype == np.int16:
        arr = arr.view(np.uint16)
    np.save(os.path.join(path, name + ".npy"), arr)


@pytest.mark.parametrize("name", ["window16k", "winglobal128k", "random32k", "gqa256k"])
def test_every_row_full_size(name):
    w = wl.WORKLOADS[name]
    lay = wl.layout_of(w)
    say(f"[every-row] {w.name} B={w.batch} H={w.heads}/{w.kv_heads} N={w.seq_len}")
    q, k, v = wl.make_qkv(w, "cuda")
    p = bsattn.plan(w.batch, w.heads, w.kv_heads, w.seq_len, w.head_dim, w.block, w.dtype, lay)
    out, lse = bsattn.forward(q, k, v, p)
    torch.cuda.synchronize()
    pairs = heads_to_check(w)
    path = scratch_dir()
    saved = {}
    t0 = time.perf_counter()
    try:
        for nm, t in (("q", q), ("k", k), ("v", v), ("o", out), ("lse", lse)):
            dump(path, nm, t)
        del q, k, v, out, lse
        torch.cuda.empty_cache()
        lay_np = dict(lay)
        if lay_np.get("bitmap") is not None:
            lay_np["bitmap"] = lay_np["bitmap"].numpy().astype(np.uint8)
        tasks = [(b, h, q0, min(w.seq_len, q0 + ROWS_PER_TASK))
                 for b, h in pairs for q0 in range(0, w.seq_len, ROWS_PER_TASK)]
        workers = max(1, min(16, os.cpu_count() or 1))
        say(f"[every-row] {w.name}: {len(pairs)} heads, {len(tasks)} tasks, {workers} workers "
            f"(dump {time.perf_counter() - t0:.1f} s)")
        ctx = mp.get_context("spawn")
        # One BLAS thread per worker process (read by each worker at import).
        for n in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS"):
            saved[n] = os.environ.get(n)
            os.environ[n] = "1"
        rows = bad = 0
        eo = el = 0.0
        wo = wl_ = None
        done = 0
        with ctx.Pool(workers, initializer=every_row_worker.init,
                      initargs=(path, lay_np, w.block, "bf16")) as pool:
            for r in pool.imap_unordered(every_row_worker.check, tasks, chunksize=4):
                n, o_err, o_at, l_err, l_at, b_ = r
                rows += n
                bad += b_
                if o_err > eo:
                    eo, wo = o_err, o_at
                if l_err > el:
                    el, wl_ = l_err, l_at
                done += 1
                if done % max(1, len(tasks) // 8) == 0:
                    say(f"[every-row] {w.name}: {done}/{len(tasks)} tasks, max|dO| {eo:.3e}, "
                        f"max|dLSE| {el:.3e} ({time.perf_counter() - t0:.0f} s)")
    finally:
        for n, val in saved.items():
            if val is None:
                os.environ.pop(n, None)
            else:
                os.environ[n] = val
        shutil.rmtree(path, ignore_errors=True)
    say(f"[every-row] {w.name}: {rows} rows, max|dO| {eo:.3e} at {wo}, max|dLSE| {el:.3e} at {wl_}, "
        f"finiteness mismatches {bad}, {time.perf_counter() - t0:.1f} s")
    assert rows == len(pairs) * w.seq_len
    assert bad == 0
    assert eo <= TOL_O, (eo, wo)
    assert el <= TOL_L, (el, wl_)
