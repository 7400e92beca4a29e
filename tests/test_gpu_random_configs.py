"""A seeded sweep of random problems through the C ABI against the oracle.

Each case draws its shape (batch, query and KV heads, a sequence length the
block may not divide), its dtype and kernel shape (bf16 128/128 on MFMA or
float32 with head_dim and block 64 or 128) and its layout (token or block
windows on either side with global keys and queries, causal or not, or a
per-head or shared bitmap of random density) from one generator, then
compares every output row of the forward, and for every third case every
element of dQ, dK and dV, with the oracle.  Tolerances as elsewhere: fp32
1e-5 on O and LSE, bf16 2e-2 on O and 1e-3 on LSE; gradients within 1% of
the largest reference element (bf16), or 1e-5 of it (at least 1e-5; fp32).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from block_sparse_flash_bsa_amd import bsattn
from block_sparse_flash_bsa_amd import workloads as wl

pytestmark = pytest.mark.gpu

CASES = 192


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsattn.lib()      # raises if the library is missing: no fallback
    torch.cuda.set_device(0)


def draw(case):
    """(workload, layout) of random case `case` (same draw on every run)."""
    rng = np.random.default_rng(7000 + case)
    bf16 = rng.random() < 0.65
    D, bs = (128, 128) if bf16 else (int(rng.choice([64, 128])), int(rng.choice([64, 128])))
    Hkv = int(rng.integers(1, 3))
    H = Hkv * int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 3))
    N = int(rng.integers(bs // 2, 6 * bs + 1))
    nb = -(-N // bs)
    kind = rng.choice(["tokens", "blocks", "bitmap"])
    causal = bool(rng.random() < 0.5)
    if kind == "bitmap":
        lh = int(rng.choice([1, H]))
        bm = (rng.random((lh, nb, nb)) < rng.uniform(0.05, 0.6)).astype(np.uint8)
        if rng.random() < 0.7:
            bm[:, np.arange(nb), np.arange(nb)] = 1      # else some rows may stay empty
        lay = dict(causal=causal, unit="blocks", window_left=-1, window_right=-1, global_keys=0,
                   global_queries=0, bitmap=bm)
    else:
        span = N if kind == "tokens" else nb
        wlft = int(rng.integers(-1, span + 1))
        wrgt = int(rng.integers(-1, span + 1)) if not causal else int(rng.integers(-1, 2))
        gk = int(rng.integers(0, max(2, span // 4))) if rng.random() < 0.5 else 0
        gq = int(rng.integers(0, max(2, span // 4))) if rng.random() < 0.3 else 0
        lay = wl.spec(causal, kind, wlft, wrgt, gk, gq)
    w = wl.Workload(f"random-{case}", B, H, Hkv, N, D, bs, torch.bfloat16 if bf16 else torch.float32,
                    100 + case, {})
    return w, lay


def describe(w, lay):
    if lay.get("bitmap") is not None:
        bm = lay["bitmap"]
        form = f"bitmap {bm.shape[0]}x{bm.shape[1]}x{bm.shape[2]} density {bm.mean():.2f}"
    else:
        form = (f"{lay['unit']} window ({lay['window_left']}, {lay['window_right']}) "
                f"globals ({lay['global_keys']}, {lay['global_queries']})")
    return (f"{str(w.dtype).split('.')[-1]} D={w.head_dim} block={w.block} B={w.batch} H={w.heads}/{w.kv_heads} "
            f"N={w.seq_len} causal={lay['causal']} {form}")


@pytest.mark.parametrize("case", range(CASES))
def test_random_problem_against_oracle(case):
    w, lay = draw(case)
    say(f"[random {case}] {describe(w, lay)}")
    q, k, v = wl.make_qkv(w, "cpu")
    p = bsattn.plan(w.batch, w.heads, w.kv_heads, w.seq_len, w.head_dim, w.block, w.dtype, lay)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    out = torch.full((w.batch, w.heads, w.seq_len, w.head_dim), float("nan"), dtype=w.dtype, device="cuda")
    lse = torch.full((w.batch, w.heads, w.seq_len), float("nan"), dtype=torch.float32, device="cuda")
    bsattn.forward(qc, kc, vc, p, out, lse)
    torch.cuda.synchronize()
    O = out.float().cpu().numpy().astype(np.float64)
    L = lse.cpu().numpy().astype(np.float64)
    O_ref, L_ref = oracle.forward(q, k, v, lay, w.block)
    to, tl = (2e-2, 1e-3) if w.dtype == torch.bfloat16 else (1e-5, 1e-5)
    assert not np.isnan(O).any() and not np.isnan(L).any(), "unwritten or NaN outputs"
    fin = np.isfinite(L_ref)
    assert np.array_equal(np.isfinite(L), fin), "empty-row pattern differs"
    eo = float(np.abs(O - O_ref).max())
    el = float(np.abs(L[fin] - L_ref[fin]).max()) if fin.any() else 0.0
    say(f"  forward: max|dO| {eo:.2e} (tol {to}), max|dLSE| {el:.2e} (tol {tl}), empty rows {int((~fin).sum())}")
    assert eo <= to and el <= tl
    assert np.all(O[~fin] == 0)
    if case % 3:
        return
    do = wl.make_dout(w, "cpu")
    dq, dk, dv = bsattn.backward(qc, kc, vc, out, lse, do.cuda(), p)
    torch.cuda.synchronize()
    ref = oracle.backward(q, k, v, do, lay, w.block)
    rel = 1e-2 if w.dtype == torch.bfloat16 else 1e-5
    for name, got, r in (("dQ", dq, ref[0]), ("dK", dk, ref[1]), ("dV", dv, ref[2])):
        g = got.float().cpu().numpy().astype(np.float64)
        assert not np.isnan(g).any(), f"{name}: NaN"
        amax = float(np.abs(r).max())
        scale = max(amax, 1e-30) if w.dtype == torch.bfloat16 else max(amax, 1.0)
        err = float(np.abs(g - r).max())
        say(f"  {name}: max|err| {err:.2e}, {err / scale:.2e} of max|ref|")
        assert err <= rel * scale, f"{name}: {err} > {rel} * {scale}"


VARLEN_CASES = 64


@pytest.mark.parametrize("case", range(VARLEN_CASES))
def test_random_variable_length_batch_against_oracle(case):
    """The same draws as a padded batch of 2 to 4 entries with random lengths
    (0 to N): each entry's rows match the oracle on its trimmed sequence,
    rows beyond its length are empty (O = 0, LSE = -inf) and their gradients
    zero, and NaN padding of the inputs is never read."""
    w, lay = draw(1000 + case)
    rng = np.random.default_rng(9000 + case)
    w = w.with_shape(batch=int(rng.integers(2, 5)))
    lens = [int(x) for x in rng.integers(0, w.seq_len + 1, size=w.batch)]
    lens[int(rng.integers(0, w.batch))] = w.seq_len          # one entry at full length
    say(f"[random varlen {case}] {describe(w, lay)} lens={lens}")
    q, k, v = wl.make_qkv(w, "cpu")
    do = wl.make_dout(w, "cpu")
    for b, L in enumerate(lens):
        for t in (q, k, v, do):
            t[b, :, L:] = float("nan")
    p = bsattn.plan(w.batch, w.heads, w.kv_heads, w.seq_len, w.head_dim, w.block, w.dtype, lay)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    out, lse = bsattn.forward_varlen(qc, kc, vc, p, sl)
    backward = case % 2 == 0
    if backward:
        dq, dk, dv = bsattn.backward_varlen(qc, kc, vc, out, lse, doc, p, sl)
    torch.cuda.synchronize()
    O = out.float().cpu().numpy().astype(np.float64)
    L_ = lse.cpu().numpy().astype(np.float64)
    to, tl = (2e-2, 1e-3) if w.dtype == torch.bfloat16 else (1e-5, 1e-5)
    rel = 1e-2 if w.dtype == torch.bfloat16 else 1e-5
    grads = tuple(x.float().cpu().numpy().astype(np.float64) for x in (dq, dk, dv)) if backward else ()
    for b, L in enumerate(lens):
        assert np.all(O[b, :, L:] == 0) and np.all(L_[b, :, L:] == -np.inf), f"entry {b}: rows beyond {L}"
        for g in grads:
            assert np.all(g[b, :, L:] == 0), f"entry {b}: gradient rows beyond {L}"
        if L == 0:
            continue
        ly = dict(lay)
        if ly.get("bitmap") is not None:
            nbl = -(-L // w.block)
            ly["bitmap"] = ly["bitmap"][:, :nbl, :nbl]
        sb = (slice(b, b + 1), slice(None), slice(0, L))
        O_ref, L_ref = oracle.forward(q[sb], k[sb], v[sb], ly, w.block)
        fin = np.isfinite(L_ref)
        Ob, Lb = O[sb], L_[sb]
        assert np.array_equal(np.isfinite(Lb), fin), f"entry {b}: empty-row pattern differs"
        eo = float(np.abs(Ob - O_ref).max())
        el = float(np.abs(Lb[fin] - L_ref[fin]).max()) if fin.any() else 0.0
        say(f"  entry {b} (L={L}): max|dO| {eo:.2e}, max|dLSE| {el:.2e}")
        assert eo <= to and el <= tl
        if backward:
            ref = oracle.backward(q[sb], k[sb], v[sb], do[sb], ly, w.block)
            for name, g, r in zip(("dQ", "dK", "dV"), grads, ref):
                amax = float(np.abs(r).max())
                scale = max(amax, 1e-30) if w.dtype == torch.bfloat16 else max(amax, 1.0)
                err = float(np.abs(g[sb] - r).max())
                assert err <= rel * scale, f"entry {b} {name}: {err} > {rel} * {scale}"


DYNAMIC_CASES = 48


@pytest.mark.parametrize("case", range(DYNAMIC_CASES))
def test_random_dynamic_plan_equals_static(case):
    """Random bitmaps through a dynamic plan (CSR, transposed lists, split
    walks and launch order built on the device) give, bit for bit, the
    forward and backward of the static plan of the same bitmap."""
    rng = np.random.default_rng(11000 + case)
    bf16 = rng.random() < 0.7
    D, bs = (128, 128) if bf16 else (int(rng.choice([64, 128])), int(rng.choice([64, 128])))
    Hkv = int(rng.integers(1, 3))
    H = Hkv * int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 3))
    N = int(rng.integers(bs, 8 * bs + 1))
    nb = -(-N // bs)
    causal = bool(rng.random() < 0.5)
    lh = int(rng.choice([1, H]))
    bm = (rng.random((lh, nb, nb)) < rng.uniform(0.05, 0.5)).astype(np.uint8)
    if rng.random() < 0.5:
        bm[:, :, int(rng.integers(0, nb))] = 1            # a dense key-block column
    w = wl.Workload(f"dyn-{case}", B, H, Hkv, N, D, bs, torch.bfloat16 if bf16 else torch.float32, 300 + case, {})
    lay = dict(causal=causal, unit="blocks", window_left=-1, window_right=-1, global_keys=0, global_queries=0,
               bitmap=bm)
    say(f"[random dynamic {case}] {describe(w, lay)}")
    q, k, v = (x.cuda() for x in wl.make_qkv(w, "cpu"))
    do = wl.make_dout(w, "cuda")
    sp = bsattn.plan(B, H, Hkv, N, D, bs, w.dtype, lay)
    dp = bsattn.plan_dynamic(B, H, Hkv, N, D, bs, w.dtype, causal, lh)
    dp.set_bitmap(torch.from_numpy(bm).cuda())
    o1, l1 = bsattn.forward(q, k, v, sp)
    o2, l2 = bsattn.forward(q, k, v, dp)
    g1 = bsattn.backward(q, k, v, o1, l1, do, sp)
    g2 = bsattn.backward(q, k, v, o2, l2, do, dp)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "forward differs"
    for name, a, b in zip(("dQ", "dK", "dV"), g1, g2):
        assert torch.equal(a, b), f"{name} differs"
