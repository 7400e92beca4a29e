"""GPU parity of bsa_backward against the CPU oracle, through the C ABI.

* every element of dQ, dK and dV for each workload's rule at a size the
  oracle finishes in seconds (several tiles, partial tiles, GQA groups,
  per-head bitmaps, rows with no allowed key);
* full-size workloads in the benchmark's launch configuration: sampled dQ
  rows and sampled dK/dV keys against the oracle's per-row / per-key forms;
* determinism, and UNSUPPORTED for plans without a backward kernel.

Tolerance, for each of dQ, dK, dV: max abs error <= 1e-2 * max |reference|.
Derivation: the kernels round P and dS to bf16 before their products
(relative 2^-9 per term, independent between terms, so a sum's error stays
below 2^-9 of the sum of |terms|, which for these workloads is within a
small factor of the largest gradient), Delta uses the bf16 output O
(relative 2^-9), and the result is rounded to bf16 once more (2^-9 of the
value); 1e-2 is about five times their sum.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from block_sparse_flash_bsa_amd import bsattn
from block_sparse_flash_bsa_amd import workloads as wl

pytestmark = pytest.mark.gpu

RTOL_OF_MAX = 1e-2

SMALL = {
    "window16k": wl.small_variant(wl.WORKLOADS["window16k"], 2048, heads=2, kv_heads=2),
    "winglobal128k": wl.small_variant(wl.WORKLOADS["winglobal128k"], 2048, heads=2, kv_heads=2),
    "random32k": wl.small_variant(wl.WORKLOADS["random32k"], 2048, heads=2, kv_heads=2, batch=2),
    "gqa256k": wl.small_variant(wl.WORKLOADS["gqa256k"], 5120, heads=4, kv_heads=1),
    "dense256k": wl.small_variant(wl.WORKLOADS["dense256k"], 1024, heads=4, kv_heads=2),
}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsattn.lib()      # raises if the library is missing: no fallback
    torch.cuda.set_device(0)


def gpu_plan(w, layout, **kw):
    return bsattn.plan(w.batch, w.heads, w.kv_heads, w.seq_len, w.head_dim, w.block, w.dtype,
                       layout, **kw)


def fwd_bwd(p, q, k, v, do):
    out, lse = bsattn.forward(q, k, v, p)
    dq, dk, dv = bsattn.backward(q, k, v, out, lse, do, p)
    torch.cuda.synchronize()
    return dq, dk, dv


def check(name, got, ref):
    got = np.asarray(got, dtype=np.float64)
    assert not np.isnan(got).any(), f"{name}: NaN"
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    say(f"  {name}: max|err| = {err:.3e}, max|ref| = {scale:.3e}, ratio {err / max(scale, 1e-30):.2e}")
    assert err <= RTOL_OF_MAX * scale, f"{name}: error {err} > {RTOL_OF_MAX} * {scale}"


# ----------------------------------------------------- every element, small sizes
@pytest.mark.parametrize("name", list(SMALL))
def test_backward_all_elements_small(name):
    w = SMALL[name]
    say(f"[bwd-small] {w.name} B={w.batch} H={w.heads}/{w.kv_heads} N={w.seq_len}")
    lay = wl.layout_of(w)
    q, k, v = wl.make_qkv(w, "cpu")
    do = wl.make_dout(w, "cpu")
    p = gpu_plan(w, lay)
    dq, dk, dv = fwd_bwd(p, q.cuda(), k.cuda(), v.cuda(), do.cuda())
    rq, rk, rv = oracle.backward(q, k, v, do, lay, w.block)
    check("dQ", dq.float().cpu().numpy(), rq)
    check("dK", dk.float().cpu().numpy(), rk)
    check("dV", dv.float().cpu().numpy(), rv)


def test_backward_per_head_bitmap_with_empty_rows():
    """Per-head causal bitmaps; q-block 3 of head 0 has no active block at all,
    and under causality the first rows of blocks whose only block is above
    the diagonal have no allowed key either."""
    w = wl.WORKLOADS["random32k"].with_shape(name="bitmap-empty", batch=1, heads=2, kv_heads=1,
                                             seq_len=1024)
    nb = w.num_blocks
    rng = np.random.default_rng(5)
    bm = rng.random((2, nb, nb)) < 0.3
    bm[0, 3, :] = False
    bm[1, 5, :] = False
    bm[1, 5, 6] = True                     # above the diagonal: cut away entirely by causality
    lay = dict(causal=True, unit="blocks", window_left=-1, window_right=-1, global_keys=0,
               global_queries=0, bitmap=torch.from_numpy(bm))
    q, k, v = wl.make_qkv(w, "cpu")
    do = wl.make_dout(w, "cpu")
    p = gpu_plan(w, lay)
    dq, dk, dv = fwd_bwd(p, q.cuda(), k.cuda(), v.cuda(), do.cuda())
    rq, rk, rv = oracle.backward(q, k, v, do, lay, w.block)
    assert torch.all(dq[0, 0, 3 * 128:4 * 128] == 0)
    check("dQ", dq.float().cpu().numpy(), rq)
    check("dK", dk.float().cpu().numpy(), rk)
    check("dV", dv.float().cpu().numpy(), rv)


def test_backward_token_rule_both_sides_gqa():
    """Token window on both sides plus global keys and global query rows, GQA 4:1."""
    w = wl.WORKLOADS["gqa256k"].with_shape(name="two-sided", heads=4, kv_heads=1, seq_len=1536)
    lay = dict(causal=False, unit="tokens", window_left=200, window_right=77, global_keys=5,
               global_queries=3, bitmap=None)
    q, k, v = wl.make_qkv(w, "cpu")
    do = wl.make_dout(w, "cpu")
    p = gpu_plan(w, lay)
    dq, dk, dv = fwd_bwd(p, q.cuda(), k.cuda(), v.cuda(), do.cuda())
    rq, rk, rv = oracle.backward(q, k, v, do, lay, w.block)
    check("dQ", dq.float().cpu().numpy(), rq)
    check("dK", dk.float().cpu().numpy(), rk)
    check("dV", dv.float().cpu().numpy(), rv)


def test_backward_split_columns():
    """Walks longer than twice the mean are cut into chunks whose float32
    partials a reduction kernel adds: the 8 global keys' k-block (read by
    every q-block of all 4 heads) and, with per-head bitmaps, dense columns."""
    w = wl.WORKLOADS["gqa256k"].with_shape(name="split-global", heads=4, kv_heads=1, seq_len=4096)
    lay = dict(causal=True, unit="tokens", window_left=255, window_right=0, global_keys=8,
               global_queries=0, bitmap=None)
    nb = w.num_blocks
    rng = np.random.default_rng(6)
    bm = rng.random((4, nb, nb)) < 0.05
    bm[:, :, 3] = True                      # k-block 3 read by every q-block of every head
    bm[1, :, 17] = True
    bm[:, np.arange(nb), np.arange(nb)] = True
    lay_bm = dict(causal=False, unit="blocks", window_left=-1, window_right=-1, global_keys=0,
                  global_queries=0, bitmap=torch.from_numpy(bm))
    for name, ly in (("global keys", lay), ("dense bitmap columns", lay_bm)):
        say(f"[bwd-split] {name}")
        p = gpu_plan(w, ly)
        work = p.work_kv()
        assert len(work[work >= 0]) > len(np.unique(work[work >= 0])), "expected split columns"
        q, k, v = wl.make_qkv(w, "cpu")
        do = wl.make_dout(w, "cpu")
        dq, dk, dv = fwd_bwd(p, q.cuda(), k.cuda(), v.cuda(), do.cuda())
        rq, rk, rv = oracle.backward(q, k, v, do, ly, w.block)
        check("dQ", dq.float().cpu().numpy(), rq)
        check("dK", dk.float().cpu().numpy(), rk)
        check("dV", dv.float().cpu().numpy(), rv)


def test_backward_ragged_split_last_column():
    """A split walk on the short last block of a ragged sequence: the
    reduction writes only the rows below N of that block."""
    N = 4000                                      # 32 blocks, the last with 32 rows
    w = wl.WORKLOADS["gqa256k"].with_shape(name="ragged-split", heads=4, kv_heads=1, seq_len=N)
    nb = -(-N // 128)
    rng = np.random.default_rng(7)
    bm = rng.random((4, nb, nb)) < 0.05
    bm[:, :, nb - 1] = True                       # every q-block reads the short last block
    bm[:, np.arange(nb), np.arange(nb)] = True
    lay = dict(causal=False, unit="blocks", window_left=-1, window_right=-1, global_keys=0,
               global_queries=0, bitmap=torch.from_numpy(bm))
    p = gpu_plan(w, lay)
    work = p.work_kv()
    assert np.sum(work == nb - 1) > 1, "expected the last column's walk to be split"
    q, k, v = wl.make_qkv(w, "cpu")
    do = wl.make_dout(w, "cpu")
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    out, lse = bsattn.forward(qc, kc, vc, p)
    n = int(np.prod(k.shape))
    bufk = torch.full((n + 4096,), float("nan"), dtype=torch.bfloat16, device="cuda")
    bufv = torch.full((n + 4096,), float("nan"), dtype=torch.bfloat16, device="cuda")
    dk, dv = bufk[:n].view(k.shape), bufv[:n].view(v.shape)
    dq, _, _ = bsattn.backward(qc, kc, vc, out, lse, doc, p, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.isnan(bufk[n:]).all() and torch.isnan(bufv[n:]).all(), "write beyond the last row"
    rq, rk, rv = oracle.backward(q, k, v, do, lay, w.block)
    check("dQ", dq.float().cpu().numpy(), rq)
    check("dK", dk.float().cpu().numpy(), rk)
    check("dV", dv.float().cpu().numpy(), rv)


@pytest.mark.parametrize("N,causal", [(1000, True), (700, False)])
def test_backward_ragged_length(N, causal):
    """The block does not divide N: rows beyond N exist nowhere, gradients of
    the last rows are exact, and nothing is written beyond the last row."""
    w = wl.WORKLOADS["gqa256k"].with_shape(name=f"ragged{N}", heads=4, kv_heads=1, seq_len=N)
    lay = dict(causal=causal, unit="tokens", window_left=200, window_right=0 if causal else 90,
               global_keys=5, global_queries=0 if causal else 2, bitmap=None)
    q, k, v = wl.make_qkv(w, "cpu")
    do = wl.make_dout(w, "cpu")
    p = gpu_plan(w, lay)
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    out, lse = bsattn.forward(qc, kc, vc, p)

    def guarded(shape):
        n = int(np.prod(shape))
        buf = torch.full((n + 4096,), float("nan"), dtype=torch.bfloat16, device="cuda")
        return buf[:n].view(shape), buf[n:]
    dq, gq = guarded(tuple(q.shape))
    dk, gk = guarded(tuple(k.shape))
    dv, gv = guarded(tuple(v.shape))
    bsattn.backward(qc, kc, vc, out, lse, doc, p, dq, dk, dv)
    torch.cuda.synchronize()
    for g in (gq, gk, gv):
        assert torch.isnan(g).all(), "write beyond the last row"
    rq, rk, rv = oracle.backward(q, k, v, do, lay, w.block)
    check("dQ", dq.float().cpu().numpy(), rq)
    check("dK", dk.float().cpu().numpy(), rk)
    check("dV", dv.float().cpu().numpy(), rv)


# ---------------------------------------------------------- full size, sampled
FULL_KEYS = {
    # keys away from global blocks (a global key is read by every query of the
    # sequence, which the per-key oracle would take minutes to sum)
    "window16k": [(0, 0, 0), (0, 31, 8191), (0, 17, 16383), (0, 5, 700)],
    "winglobal128k": [(0, 3, 65541), (0, 31, 131071), (0, 0, 131072 - 900)],
    "random32k": [(1, 15, 32767), (0, 2, 20000), (1, 7, 128)],
    "gqa256k": [(0, 7, 262143), (0, 0, 100000), (0, 3, 262144 - 1500)],
}


def sample_rows(w, n_random=32, seed=0):
    rng = np.random.default_rng(seed)
    N, H, B = w.seq_len, w.heads, w.batch
    qs = [0, 1, 127, 128, 511, 512, 4095, 4096, 4104, N // 2, N - 129, N - 1]
    rows = [(int(rng.integers(0, B)), int(rng.integers(0, H)), qq) for qq in qs if qq < N]
    rows += [(int(rng.integers(0, B)), int(rng.integers(0, H)), int(rng.integers(0, N)))
             for _ in range(n_random)]
    return rows


@pytest.mark.parametrize("name", list(FULL_KEYS))
def test_backward_full_size_sampled(name):
    w = wl.WORKLOADS[name]
    say(f"[bwd-full] {w.name} B={w.batch} H={w.heads}/{w.kv_heads} N={w.seq_len}")
    lay = wl.layout_of(w)
    q, k, v = wl.make_qkv(w, "cuda")
    do = wl.make_dout(w, "cuda")
    p = gpu_plan(w, lay)
    dq, dk, dv = fwd_bwd(p, q, k, v, do)
    group = w.heads // w.kv_heads
    rows = sample_rows(w)
    keys = FULL_KEYS[name]
    heads = sorted({(b, h) for b, h, _ in rows} | {(b, hk * group + g) for b, hk, _ in keys for g in range(group)})
    kvh = sorted({(b, h // group) for b, h in heads})
    # Host copies of only the heads the samples touch, indexed like the full
    # tensors: Q and dO stay bf16 (read one row at a time), K and V are
    # upcast once to float64 (gathered thousands of rows at a time).
    parts = {"q": {bh: q[bh].cpu() for bh in heads}, "do": {bh: do[bh].cpu() for bh in heads},
             "k": {bk: k[bk].double().cpu().numpy() for bk in kvh},
             "v": {bk: v[bk].double().cpu().numpy() for bk in kvh}}

    class View:
        """Minimal [b, h] / [b, h, q] indexing over the host copies for the oracle."""
        def __init__(self, part, shape):
            self.part, self.shape = part, shape

        def __getitem__(self, idx):
            if len(idx) == 2:
                return self.part[idx]
            return self.part[idx[:2]][idx[2]]

    qs_, ks_ = (w.batch, w.heads, w.seq_len, w.head_dim), (w.batch, w.kv_heads, w.seq_len, w.head_dim)
    Qv, dOv = View(parts["q"], qs_), View(parts["do"], qs_)
    Kv, Vv = View(parts["k"], ks_), View(parts["v"], ks_)
    say(f"  host copies ready: {len(heads)} query heads, {len(kvh)} KV heads")
    rq = oracle.backward_dq_rows(Qv, Kv, Vv, dOv, lay, w.block, rows)
    idx = tuple(torch.tensor(x) for x in zip(*rows))
    check("dQ rows", dq[idx].float().cpu().numpy(), rq)
    say("  dQ rows checked; summing the sampled keys' columns")
    rk, rv = oracle.backward_dkv_keys(Qv, Kv, Vv, dOv, lay, w.block, keys)
    kidx = tuple(torch.tensor(x) for x in zip(*keys))
    check("dK keys", dk[kidx].float().cpu().numpy(), rk)
    check("dV keys", dv[kidx].float().cpu().numpy(), rv)


# ------------------------------------------------------------------ behaviour
def test_backward_deterministic_and_overwrites():
    w = SMALL["gqa256k"]
    lay = wl.layout_of(w)
    q, k, v = (x.cuda() for x in wl.make_qkv(w, "cpu"))
    do = wl.make_dout(w, "cuda")
    p = gpu_plan(w, lay)
    out, lse = bsattn.forward(q, k, v, p)
    a = bsattn.backward(q, k, v, out, lse, do, p)
    poisoned = [torch.full_like(x, float("nan")) for x in a]
    delta = torch.full((w.batch, w.heads, w.seq_len), float("nan"), device="cuda")
    b = bsattn.backward(q, k, v, out, lse, do, p, *poisoned, delta=delta)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert not torch.isnan(delta).any()


@pytest.mark.parametrize("kind", ["plain", "ragged", "varlen", "varlen_f32"])
def test_delta_workspace_is_row_dot_of_dout_and_out(kind):
    """The dQ kernel forms Delta_q = <dO_q, O_q> for its own rows and writes it
    to the caller's workspace before the dK/dV kernel reads it: every row of
    a NaN-poisoned workspace comes back as the float64 dot of the bf16 O and
    dO rows, to float32 rounding of 128 products, and rows at or beyond a
    batch entry's length (whose padding holds NaN) as 0."""
    if kind == "plain":
        w = SMALL["gqa256k"]
        lay, lens = wl.layout_of(w), None
    elif kind == "ragged":
        w = wl.WORKLOADS["gqa256k"].with_shape(name="delta-ragged", batch=1, heads=4, kv_heads=2, seq_len=1000)
        lay, lens = wl.layout_of(w), None
    else:
        w, lay, lens = _varlen_case("window")
        if kind == "varlen_f32":
            w = w.with_shape(name="varlen-f32", dtype=torch.float32, head_dim=64, block=64)
    say(f"[delta] {kind} B={w.batch} H={w.heads}/{w.kv_heads} N={w.seq_len} lens={lens}")
    q, k, v = wl.make_qkv(w, "cpu")
    do = wl.make_dout(w, "cpu")
    if lens is not None:
        for b, L in enumerate(lens):
            for t in (q, k, v, do):
                t[b, :, L:] = float("nan")
    p = gpu_plan(w, lay)
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    delta = torch.full((w.batch, w.heads, w.seq_len), float("nan"), device="cuda")
    if lens is None:
        out, lse = bsattn.forward(qc, kc, vc, p)
        bsattn.backward(qc, kc, vc, out, lse, doc, p, delta=delta)
    else:
        sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
        out, lse = bsattn.forward_varlen(qc, kc, vc, p, sl)
        bsattn.backward_varlen(qc, kc, vc, out, lse, doc, p, sl, delta=delta)
    torch.cuda.synchronize()
    got = delta.cpu().double().numpy()
    o64 = out.cpu().double().numpy()
    d64 = do.double().numpy()
    valid = np.ones(got.shape, dtype=bool)
    if lens is not None:
        for b, L in enumerate(lens):
            valid[b, :, L:] = False
            d64[b, :, L:] = 0.0
    ref = np.einsum("bhnd,bhnd->bhn", o64, d64)
    mag = np.einsum("bhnd,bhnd->bhn", np.abs(o64), np.abs(d64))
    assert not np.isnan(got).any(), "unwritten or NaN rows of Delta"
    assert np.all(got[~valid] == 0.0), "rows beyond an entry's length are not 0"
    err = np.abs(got - ref)[valid]
    bound = (1e-5 * mag + 1e-30)[valid]
    say(f"  max|err| = {err.max():.3e}, worst err/bound = {(err / bound).max():.3f}")
    assert np.all(err <= bound)


def test_backward_launch_queues_over_many_calls():
    """The dQ and dK/dV launch queues (the last eighth of each XCD's rows
    drained by workgroups of any XCD, counters taken per launch in turn from
    the plan's 64 sets): 45 forward + backward calls of one plan (135 queued
    launches, twice round the sets) on two alternating streams, each into
    NaN-poisoned gradients, give bit for bit the gradients of the LPT order,
    whose launches have no queue."""
    w = wl.small_variant(wl.WORKLOADS["winglobal128k"], 16384, heads=8, kv_heads=8)
    lay = wl.layout_of(w)
    q, k, v = (x.cuda() for x in wl.make_qkv(w, "cpu"))
    do = wl.make_dout(w, "cuda")
    p = gpu_plan(w, lay)
    assert len(p.work()) // 8 >= 16 and len(p.work_kv()) // 8 >= 16
    ref = fwd_bwd(gpu_plan(w, lay, schedule=2), q, k, v, do)
    grads = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    streams = [torch.cuda.current_stream(), torch.cuda.Stream()]
    for call in range(45):
        st = streams[call % 2]
        st.wait_stream(streams[(call + 1) % 2])
        with torch.cuda.stream(st):
            for g in grads:
                g.fill_(float("nan"))
            out, lse = bsattn.forward(q, k, v, p)
            bsattn.backward(q, k, v, out, lse, do, p, *grads)
        st.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), grads, ref):
            assert torch.equal(a, b), f"call {call}: {name} differs"


def test_backward_custom_scale_stream_and_empty_problems():
    """A non-default scale (enters P and the scale of dQ, dK), a non-default
    stream, and problems with no work items (returns at once)."""
    w = wl.WORKLOADS["window16k"].with_shape(name="scale", heads=2, kv_heads=2, seq_len=1024)
    lay = wl.layout_of(w)
    q, k, v = wl.make_qkv(w, "cpu")
    do = wl.make_dout(w, "cpu")
    p = gpu_plan(w, lay, scale=0.05)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
        out, lse = bsattn.forward(qc, kc, vc, p)
        dq, dk, dv = bsattn.backward(qc, kc, vc, out, lse, doc, p)
    stream.synchronize()
    rq, rk, rv = oracle.backward(q, k, v, do, lay, w.block, scale=0.05)
    check("dQ", dq.float().cpu().numpy(), rq)
    check("dK", dk.float().cpu().numpy(), rk)
    check("dV", dv.float().cpu().numpy(), rv)
    for B, N in ((0, 1024), (1, 0)):
        pe = bsattn.plan(B, 2, 2, N, 128, 128, torch.bfloat16, lay)
        z = torch.empty((B, 2, N, 128), dtype=torch.bfloat16, device="cuda")
        l0 = torch.empty((B, 2, N), dtype=torch.float32, device="cuda")
        bsattn.backward(z, z, z, z, l0, z, pe)


F32_TOL = 1e-5


@pytest.mark.parametrize("D,BS,N,causal", [(64, 64, 1024, False), (128, 128, 1024, True), (64, 128, 700, True),
                                           (128, 64, 1000, False)])
def test_backward_f32_all_elements(D, BS, N, causal):
    """The exact-precision path: float32 inputs, fp32 FMAs throughout.
    Tolerance: max abs error <= 1e-5 * max(1, max |reference|); the fp32
    accumulations over at most N terms of magnitude ~1 stay far below it."""
    base = wl.WORKLOADS["tiny_f32"]
    w = base.with_shape(name=f"f32-{D}-{BS}-{N}", heads=4, kv_heads=2, seq_len=N, head_dim=D, block=BS)
    lay = (wl.layout_of(base) if (D, BS, N) == (64, 64, 1024) else
           dict(causal=causal, unit="tokens", window_left=150, window_right=-1 if not causal else 0,
                global_keys=3, global_queries=2, bitmap=None))
    say(f"[bwd-f32] D={D} block={BS} N={N} {lay}")
    q, k, v = wl.make_qkv(w, "cpu")
    do = wl.make_dout(w, "cpu")
    p = gpu_plan(w, lay)
    dq, dk, dv = fwd_bwd(p, q.cuda(), k.cuda(), v.cuda(), do.cuda())
    rq, rk, rv = oracle.backward(q, k, v, do, lay, w.block)
    for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        err = float(np.abs(g.double().cpu().numpy() - r).max())
        tol = F32_TOL * max(1.0, float(np.abs(r).max()))
        say(f"  {name}: max|err| = {err:.3e} (tol {tol:.1e})")
        assert err <= tol, f"{name}: {err} > {tol}"


@pytest.mark.parametrize("causal", [False, True])
def test_backward_through_dynamic_plan(causal):
    """A dynamic plan builds the transposed lists on the device; its backward
    equals the static plan's of the same bitmap bit for bit (no walk is split
    at this density) and the oracle within tolerance."""
    w = SMALL["random32k"]
    lay = wl.layout_of(w)
    lay["causal"] = causal
    bm = lay["bitmap"].to(torch.uint8)
    q, k, v = wl.make_qkv(w, "cpu")
    do = wl.make_dout(w, "cpu")
    ps = gpu_plan(w, lay)
    work = ps.work_kv()
    assert len(work[work >= 0]) == len(np.unique(work[work >= 0]))
    pd = bsattn.plan_dynamic(w.batch, w.heads, w.kv_heads, w.seq_len, w.head_dim, w.block, w.dtype,
                             causal=causal, bitmap_heads=w.heads)
    pd.set_bitmap(bm.cuda().contiguous())
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    gs = fwd_bwd(ps, qc, kc, vc, doc)
    gd = fwd_bwd(pd, qc, kc, vc, doc)
    for a, b_ in zip(gs, gd):
        assert torch.equal(a, b_)
    rq, rk, rv = oracle.backward(q, k, v, do, lay, w.block)
    check("dQ", gd[0].float().cpu().numpy(), rq)
    check("dK", gd[1].float().cpu().numpy(), rk)
    check("dV", gd[2].float().cpu().numpy(), rv)


def test_beyond_2g_elements_forward_backward():
    """The 256K GQA rule with batch 2: Q, O, dO and dQ hold 2^31 elements
    each, so the last rows sit beyond every 32-bit element index.  Sampled
    output rows, dQ rows and dK/dV keys at the ends of the buffers."""
    w = wl.WORKLOADS["gqa256k"].with_shape(name="gqa256k-b2", batch=2)
    assert w.batch * w.heads * w.seq_len * w.head_dim >= 2 ** 31
    say(f"[max-size] {w.name} B={w.batch} H={w.heads}/{w.kv_heads} N={w.seq_len}")
    lay = wl.layout_of(w)
    q, k, v = wl.make_qkv(w, "cuda")
    do = wl.make_dout(w, "cuda")
    p = gpu_plan(w, lay)
    out, lse = bsattn.forward(q, k, v, p)
    dq, dk, dv = bsattn.backward(q, k, v, out, lse, do, p)
    torch.cuda.synchronize()
    N = w.seq_len
    rows = [(1, 31, N - 1), (1, 31, N - 129), (1, 30, N // 2), (0, 0, 0), (1, 0, 4096), (1, 17, 200000)]
    keys = [(1, 7, N - 1), (1, 7, N - 700)]
    heads = sorted({(b, h) for b, h, _ in rows} | {(b, hk * 4 + g) for b, hk, _ in keys for g in range(4)})
    kvh = sorted({(b, h // 4) for b, h in heads})
    parts = {"q": {bh: q[bh].cpu() for bh in heads}, "do": {bh: do[bh].cpu() for bh in heads},
             "k": {bk: k[bk].double().cpu().numpy() for bk in kvh},
             "v": {bk: v[bk].double().cpu().numpy() for bk in kvh}}

    class View:
        def __init__(self, part, shape):
            self.part, self.shape = part, shape

        def __getitem__(self, idx):
            return self.part[idx] if len(idx) == 2 else self.part[idx[:2]][idx[2]]

    qs_, ks_ = tuple(q.shape), tuple(k.shape)
    Qv, dOv, Kv, Vv = View(parts["q"], qs_), View(parts["do"], qs_), View(parts["k"], ks_), View(parts["v"], ks_)
    O_ref, L_ref = oracle.forward(Qv, Kv, Vv, lay, w.block, rows=rows)
    idx = tuple(torch.tensor(x) for x in zip(*rows))
    eo = float(np.abs(out[idx].float().cpu().numpy() - O_ref).max())
    el = float(np.abs(lse[idx].cpu().numpy() - L_ref).max())
    say(f"  O: max|err| {eo:.3e}, LSE: max|err| {el:.3e}")
    assert eo <= 2e-2 and el <= 1e-3
    check("dQ rows", dq[idx].float().cpu().numpy(), oracle.backward_dq_rows(Qv, Kv, Vv, dOv, lay, w.block, rows))
    rk, rv = oracle.backward_dkv_keys(Qv, Kv, Vv, dOv, lay, w.block, keys)
    kidx = tuple(torch.tensor(x) for x in zip(*keys))
    check("dK keys", dk[kidx].float().cpu().numpy(), rk)
    check("dV keys", dv[kidx].float().cpu().numpy(), rv)


# ------------------------------------------------------ variable-length batches
def _varlen_case(kind):
    """(workload, layout, lengths) of a padded variable-length batch."""
    if kind == "split":
        # GQA group of 4 over one KV head; k-blocks 3 and the last are read by
        # every q-block, so their dK/dV walks are split into chunks, and the
        # shorter entries end inside those walks.
        N, lens = 4000, [4000, 2500, 1000]
        w = wl.WORKLOADS["gqa256k"].with_shape(name="varlen-split", batch=3, heads=4, kv_heads=1, seq_len=N)
        nb = -(-N // 128)
        bm = np.random.default_rng(11).random((4, nb, nb)) < 0.05
        bm[:, :, 3] = True
        bm[:, :, nb - 1] = True
        bm[:, np.arange(nb), np.arange(nb)] = True
        lay = dict(causal=False, unit="blocks", window_left=-1, window_right=-1, global_keys=0,
                   global_queries=0, bitmap=torch.from_numpy(bm))
        return w, lay, lens
    N, lens = 1500, [1500, 640, 333, 0]
    w = wl.WORKLOADS["gqa256k"].with_shape(name=f"varlen-{kind}", batch=4, heads=4, kv_heads=2, seq_len=N)
    if kind == "window":
        lay = dict(causal=True, unit="tokens", window_left=300, window_right=0, global_keys=5,
                   global_queries=0, bitmap=None)
    else:
        nb = -(-N // 128)
        bm = np.random.default_rng(9).random((4, nb, nb)) < 0.3
        bm[:, np.arange(nb), np.arange(nb)] = True
        lay = dict(causal=False, unit="blocks", window_left=-1, window_right=-1, global_keys=0,
                   global_queries=0, bitmap=torch.from_numpy(bm))
    return w, lay, lens


@pytest.mark.parametrize("kind", ["window", "bitmap", "split"])
def test_backward_varlen_parity(kind):
    """Batch entry b uses its first lens[b] positions: its gradients match the
    oracle's on the trimmed sequence, rows beyond the length are zero, and
    the NaN padding of Q, K, V and dO is never read."""
    w, lay, lens = _varlen_case(kind)
    say(f"[bwd-varlen] {kind} B={w.batch} H={w.heads}/{w.kv_heads} Nmax={w.seq_len} lens={lens}")
    q, k, v = wl.make_qkv(w, "cpu")
    do = wl.make_dout(w, "cpu")
    for b, L in enumerate(lens):
        for t in (q, k, v, do):
            t[b, :, L:] = float("nan")
    p = gpu_plan(w, lay)
    if kind == "split":
        work = p.work_kv()
        assert len(work[work >= 0]) > len(np.unique(work[work >= 0])), "expected split columns"
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    out, lse = bsattn.forward_varlen(qc, kc, vc, p, sl)
    dq, dk, dv = bsattn.backward_varlen(qc, kc, vc, out, lse, doc, p, sl)
    torch.cuda.synchronize()
    dq, dk, dv = (x.float().cpu().numpy() for x in (dq, dk, dv))
    for b, L in enumerate(lens):
        for name, g in (("dQ", dq), ("dK", dk), ("dV", dv)):
            assert np.all(g[b, :, L:] == 0), f"entry {b}: {name} rows beyond {L} not zero"
        if L == 0:
            continue
        ly = dict(lay)
        if ly["bitmap"] is not None:
            nbl = -(-L // 128)
            ly["bitmap"] = ly["bitmap"][:, :nbl, :nbl]
        sl_b = (slice(b, b + 1), slice(None), slice(0, L))
        rq, rk, rv = oracle.backward(q[sl_b], k[sl_b], v[sl_b], do[sl_b], ly, w.block)
        check(f"entry {b} (L={L}) dQ", dq[sl_b], rq)
        check(f"entry {b} (L={L}) dK", dk[sl_b], rk)
        check(f"entry {b} (L={L}) dV", dv[sl_b], rv)


@pytest.mark.parametrize("N", [1500, 1024])
def test_backward_varlen_full_lengths_equal_plain_backward(N):
    """With every length at the maximum, the variable-length backward gives
    bit for bit what bsa_backward gives."""
    w = wl.WORKLOADS["gqa256k"].with_shape(name="varlen-full", batch=2, heads=4, kv_heads=2, seq_len=N)
    lay = wl.layout_of(w)
    q, k, v = (x.cuda() for x in wl.make_qkv(w, "cpu"))
    do = wl.make_dout(w, "cuda")
    p = gpu_plan(w, lay)
    out, lse = bsattn.forward(q, k, v, p)
    g1 = bsattn.backward(q, k, v, out, lse, do, p)
    g2 = bsattn.backward_varlen(q, k, v, out, lse, do, p, torch.full((2,), N, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("D,BS,kind", [(64, 64, "window"), (128, 128, "bitmap"), (64, 128, "bitmap"),
                                       (128, 64, "window")])
def test_backward_varlen_parity_f32(D, BS, kind):
    """The float32 kernels' variable-length backward: each entry's gradients
    match the oracle's on the trimmed sequence (max abs error <= 1e-5 *
    max(1, max|reference|)), rows beyond the length are zero, and the NaN
    padding of Q, K, V and dO is never read."""
    N, lens = 1000, [1000, 640, 2 * BS, 0]
    w = wl.WORKLOADS["tiny_f32"].with_shape(name=f"bwd-varlen-f32-{kind}", batch=4, heads=4, kv_heads=2,
                                            seq_len=N, head_dim=D, block=BS)
    nb = -(-N // BS)
    if kind == "window":
        lay = dict(causal=True, unit="tokens", window_left=200, window_right=0, global_keys=3,
                   global_queries=0, bitmap=None)
    else:
        bm = np.random.default_rng(BS + D).random((4, nb, nb)) < 0.4
        bm[:, np.arange(nb), np.arange(nb)] = True
        lay = dict(causal=False, unit="blocks", window_left=-1, window_right=-1, global_keys=0,
                   global_queries=0, bitmap=torch.from_numpy(bm))
    say(f"[bwd-varlen-f32] D={D} block={BS} {kind} N={N} lens={lens}")
    q, k, v = wl.make_qkv(w, "cpu")
    do = wl.make_dout(w, "cpu")
    for b, L in enumerate(lens):
        for t in (q, k, v, do):
            t[b, :, L:] = float("nan")
    p = gpu_plan(w, lay)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    out, lse = bsattn.forward_varlen(qc, kc, vc, p, sl)
    dq, dk, dv = bsattn.backward_varlen(qc, kc, vc, out, lse, doc, p, sl)
    torch.cuda.synchronize()
    dq, dk, dv = (x.double().cpu().numpy() for x in (dq, dk, dv))
    for b, L in enumerate(lens):
        for name, g in (("dQ", dq), ("dK", dk), ("dV", dv)):
            assert np.all(g[b, :, L:] == 0), f"entry {b}: {name} rows beyond {L} not zero"
        if L == 0:
            continue
        ly = dict(lay)
        if ly["bitmap"] is not None:
            nbl = -(-L // BS)
            ly["bitmap"] = ly["bitmap"][:, :nbl, :nbl]
        sl_b = (slice(b, b + 1), slice(None), slice(0, L))
        rq, rk, rv = oracle.backward(q[sl_b], k[sl_b], v[sl_b], do[sl_b], ly, BS)
        for name, g, r in (("dQ", dq[sl_b], rq), ("dK", dk[sl_b], rk), ("dV", dv[sl_b], rv)):
            err = float(np.abs(g - r).max())
            tol = F32_TOL * max(1.0, float(np.abs(r).max()))
            say(f"  entry {b} (L={L}) {name}: max|err| = {err:.3e} (tol {tol:.1e})")
            assert err <= tol, f"entry {b} {name}: {err} > {tol}"


def test_backward_varlen_rejects_bad_arguments():
    wb = wl.small_variant(wl.WORKLOADS["window16k"], 1024, heads=2, kv_heads=2)
    pb = gpu_plan(wb, wl.layout_of(wb))
    y = wl.make_qkv(wb, "cpu")[0].cuda()
    host_lens = torch.full((1,), 512, dtype=torch.int32)
    ptr = y.data_ptr()
    st = bsattn.lib().bsa_backward_varlen(ptr, ptr, ptr, ptr, ptr, ptr, pb.handle, host_lens.data_ptr(), ptr, ptr,
                                          ptr, ptr, None)
    assert st == bsattn.ERR_INVALID_ARGUMENT                # host memory for seq_lens


def test_varlen_lengths_are_clamped():
    """Lengths below 0 or above seq_len act as 0 and seq_len (forward and
    backward give bit for bit the results of the clamped lengths)."""
    N = 1000
    w = wl.WORKLOADS["gqa256k"].with_shape(name="varlen-clamp", batch=3, heads=4, kv_heads=2, seq_len=N)
    lay = wl.layout_of(w)
    q, k, v = (x.cuda() for x in wl.make_qkv(w, "cpu"))
    do = wl.make_dout(w, "cuda")
    p = gpu_plan(w, lay)
    res = []
    for lens in ([-7, N + 333, 2 ** 31 - 1], [0, N, N]):
        sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
        o, l = bsattn.forward_varlen(q, k, v, p, sl)
        res.append((o, l) + bsattn.backward_varlen(q, k, v, o, l, do, p, sl))
    torch.cuda.synchronize()
    for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), *res):
        assert torch.equal(a, b), f"{name} differs"
    assert torch.all(res[0][0][0] == 0) and torch.all(res[0][1][0] == -float("inf"))
