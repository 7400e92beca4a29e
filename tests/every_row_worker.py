"""Worker side of the every-row parity check (spawned processes, CPU only).

The parent writes the full-size inputs and the GPU's outputs as raw arrays
(bfloat16 as their 16-bit patterns) into a scratch directory; each worker
memory-maps them, evaluates runs of 128 consecutive query rows with the
oracle's query-range form, and returns the largest differences it saw.
Imports numpy and the oracle only.
"""
import os

import numpy as np

_S = {}


def bf16_to_f32(u16):
    """Exact float32 values of bfloat16 bit patterns."""
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def init(path, layout, block, dtype):
    os.environ["OMP_NUM_THREADS"] = "1"
    import oracle  # test infrastructure
    _S.update(oracle=oracle, layout=layout, block=block, dtype=dtype, cache={},
              **{n: np.load(os.path.join(path, n + ".npy"), mmap_mode="r")
                 for n in ("q", "k", "v", "o", "lse")})


def _rows(a):
    return bf16_to_f32(a) if _S["dtype"] == "bf16" else np.asarray(a, dtype=np.float32)


def _kv(b, hk):
    key = (b, hk)
    c = _S["cache"]
    if key not in c:
        c.clear()
        c[key] = (_rows(_S["k"][b, hk]), _rows(_S["v"][b, hk]))
    return c[key]


def check(task):
    """task = (b, h, q0, q1): every row in [q0, q1) of head h of batch entry b.

    Returns (rows, max|dO|, (b, h, q) of it, max|dLSE|, (b, h, q) of it,
    rows whose LSE finiteness differs)."""
    b, h, q0, q1 = task
    o_ = _S["oracle"]
    H, Hk = _S["q"].shape[1], _S["k"].shape[1]
    Kh, Vh = _kv(b, o_.kv_head(h, H // Hk))
    bs = _S["block"]
    eo, where_o, el, where_l, bad = 0.0, None, 0.0, None, 0
    for r0 in range(q0, q1, 128):
        r1 = min(q1, r0 + 128)
        O, L = o_.forward_query_range(_rows(_S["q"][b, h, r0:r1]), Kh, Vh, _S["layout"], bs, h, r0)
        Og = _rows(_S["o"][b, h, r0:r1]).astype(np.float64)
        Lg = np.asarray(_S["lse"][b, h, r0:r1], dtype=np.float64)
        d = np.abs(Og - O).max(axis=1)
        i = int(d.argmax())
        if d[i] > eo:
            eo, where_o = float(d[i]), (b, h, r0 + i)
        fin = np.isfinite(L)
        bad += int((np.isfinite(Lg) != fin).sum())
        if fin.any():
            dl = np.where(fin, np.abs(Lg - np.where(fin, L, 0.0)), 0.0)
            i = int(dl.argmax())
            if dl[i] > el:
                el, where_l = float(dl[i]), (b, h, r0 + i)
    return q1 - q0, eo, where_o, el, where_l, bad
