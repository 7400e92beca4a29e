"""Pins for the oracle's sampled-row and query-range forms, and full-size
brute-force plan counts.

* `oracle.forward(..., rows=...)` (the checker of the smoke run and of the
  sampled full-size GPU tests) against the full per-query form evaluated on
  KV heads expanded to one per query head, which involves no head mapping at
  all, on token, block and bitmap rules with GQA and random Q/K/V;
* `oracle.forward_query_range` (the checker of the every-row full-size GPU
  tests) against the per-query form, library attention (SDPA) and
  brute-force masked attention;
* the allowed key sets against the layout predicate written out over every
  key, at full sequence length on sampled queries;
* plan counts by brute-force enumeration of A(q) for every query at full N of
  the two token-unit workloads, against the interval path and the C++ planner;
* planted mistakes in the head mapping, which the pins must catch.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import bsa_oracle
from block_sparse_flash_bsa_amd import workloads as wl


def spec(causal, unit, w_left=-1, w_right=-1, gk=0, gq=0, bitmap=None):
    return dict(causal=causal, unit=unit, window_left=w_left, window_right=w_right,
                global_keys=gk, global_queries=gq, bitmap=bitmap)


def rand_qkv(B, H, Hk, N, D, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(B, H, N, D, generator=g, dtype=torch.float64),
            torch.randn(B, Hk, N, D, generator=g, dtype=torch.float64),
            torch.randn(B, Hk, N, D, generator=g, dtype=torch.float64))


def bitmap_layout(causal, H, nb, seed, p=0.35):
    rng = np.random.default_rng(seed)
    bm = (rng.random((H, nb, nb)) < p).astype(np.uint8)
    bm[1 % H, 2, :] = 0                      # an empty block row: its queries have no key
    return spec(causal, "blocks", bitmap=bm)


RULES = {
    "tokens_window_globals": (spec(True, "tokens", 37, 0, 5, 3), 32),
    "tokens_two_sided": (spec(False, "tokens", 20, 11, 2, 0), 32),
    "blocks_window_globals": (spec(True, "blocks", 2, 0, 1, 1), 32),
    "blocks_symmetric": (spec(False, "blocks", 1, 1, 0, 0), 32),
    "bitmap_causal": (bitmap_layout(True, 4, 6, 5), 32),
    "bitmap": (bitmap_layout(False, 4, 6, 6), 32),
}


def rows_of(B, H, N, seed, n=60):
    rng = np.random.default_rng(seed)
    edge = [0, 1, 31, 32, 33, 63, 64, 95, N - 1]
    rows = {(b, h, q) for b in range(B) for h in range(H) for q in edge if q < N}
    rows |= {(int(rng.integers(0, B)), int(rng.integers(0, H)), int(rng.integers(0, N))) for _ in range(n)}
    return sorted(rows)


# ------------------------------------------------------- sampled-row form
def check_rows_form(name, N=190, seed=0):
    """Max differences of rows= against the full form on expanded KV heads."""
    lay, bs = RULES[name]
    Q, K, V = rand_qkv(2, 4, 2, N, 16, seed)
    Ke, Ve = K.repeat_interleave(2, 1), V.repeat_interleave(2, 1)   # one KV head per query head
    Of, Lf = oracle.forward(Q, Ke, Ve, lay, bs)
    rows = rows_of(2, 4, N, seed)
    Or, Lr = oracle.forward(Q, K, V, lay, bs, rows=rows)
    idx = tuple(np.array(x) for x in zip(*rows))
    lf = Lf[idx]
    fin = np.isfinite(lf)
    assert np.array_equal(fin, np.isfinite(Lr))
    return float(np.abs(Or - Of[idx]).max()), float(np.abs(Lr[fin] - lf[fin]).max(initial=0.0))


@pytest.mark.parametrize("name", sorted(RULES))
def test_rows_form_equals_full_form_gqa(name):
    eo, el = check_rows_form(name)
    assert eo <= 1e-13 and el <= 1e-13, (eo, el)


def test_rows_form_covers_empty_rows():
    lay, bs = RULES["bitmap_causal"]
    Q, K, V = rand_qkv(1, 4, 2, 190, 16, 3)
    rows = [(0, 1, q) for q in range(64, 96)]          # block row 2 of head 1 is empty
    O, L = oracle.forward(Q, K, V, lay, bs, rows=rows)
    assert np.all(O == 0) and np.all(L == -np.inf)


@pytest.mark.parametrize("plant", ["own_head", "interleaved"])
def test_pins_catch_planted_kv_head(monkeypatch, plant):
    """Reading K[b, h] (or an interleaved head map) for K[b, h // group]."""
    wrong = {"own_head": lambda h, group: min(h, 1), "interleaved": lambda h, group: h % 2}[plant]
    monkeypatch.setattr(bsa_oracle, "kv_head", wrong)
    caught = 0
    for name in ("tokens_window_globals", "blocks_window_globals", "bitmap"):
        eo, el = check_rows_form(name)
        caught += not (eo <= 1e-13 and el <= 1e-13)
    assert caught == 3


# ------------------------------------------------------- query-range form
def range_vs_rows(lay, bs, N, H, Hk, ranges, seed, D=16):
    Q, K, V = rand_qkv(1, H, Hk, N, D, seed)
    g = H // Hk
    worst = 0.0
    for h in range(H):
        for q0, q1 in ranges:
            O, L = oracle.forward_query_range(Q[0, h, q0:q1].numpy(), K[0, h // g].numpy(),
                                              V[0, h // g].numpy(), lay, bs, h, q0)
            Or, Lr = oracle.forward(Q, K, V, lay, bs, rows=[(0, h, q) for q in range(q0, q1)])
            fin = np.isfinite(Lr)
            assert np.array_equal(fin, np.isfinite(L))
            assert np.all(O[~fin] == 0)
            worst = max(worst, float(np.abs(O - Or).max()), float(np.abs(L[fin] - Lr[fin]).max(initial=0.0)))
    return worst


@pytest.mark.parametrize("name", sorted(RULES))
def test_query_range_equals_per_query(name):
    lay, bs = RULES[name]
    N = 190                                   # a ragged last block of 30 rows
    ranges = [(0, 32), (5, 70), (64, 96), (150, 190), (37, 38)]
    assert range_vs_rows(lay, bs, N, 4, 2, ranges, 7) <= 1e-12


def test_query_range_dense_equals_sdpa():
    Q, K, V = rand_qkv(1, 2, 2, 256, 32, 8)
    for causal in (False, True):
        lay = spec(causal, "tokens")
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=causal)[0]
        S = (Q @ K.transpose(-1, -2))[0] / math.sqrt(32)
        if causal:
            S = S.masked_fill(torch.ones(256, 256, dtype=torch.bool).triu(1), -math.inf)
        lse = torch.logsumexp(S, -1)
        for h in range(2):
            O, L = oracle.forward_query_range(Q[0, h].numpy(), K[0, h].numpy(), V[0, h].numpy(),
                                              lay, 64, h, 0)
            np.testing.assert_allclose(O, ref[h].numpy(), atol=1e-12)
            np.testing.assert_allclose(L, lse[h].numpy(), atol=1e-12)


def test_query_range_bruteforce_masked():
    """Against attention with an N x N mask built here from the rule's definition."""
    N, bs, W, G = 300, 64, 45, 3
    Q, K, V = rand_qkv(1, 1, 1, N, 8, 9)
    q = np.arange(N)[:, None]
    k = np.arange(N)[None, :]
    mask = (k <= q) & ((q - k <= W) | (k < G))
    S = np.where(mask, (Q[0, 0].numpy() @ K[0, 0].numpy().T) / math.sqrt(8), -np.inf)
    m = S.max(1)
    P = np.exp(S - m[:, None])
    ref_o = P @ V[0, 0].numpy() / P.sum(1)[:, None]
    ref_l = m + np.log(P.sum(1))
    O, L = oracle.forward_query_range(Q[0, 0].numpy(), K[0, 0].numpy(), V[0, 0].numpy(),
                                      spec(True, "tokens", W, 0, G), bs, 0, 0)
    np.testing.assert_allclose(O, ref_o, atol=1e-12)
    np.testing.assert_allclose(L, ref_l, atol=1e-12)


# --------------------------------------------- allowed sets vs the predicate
def predicate_all_keys(lay, N, bs, h, q):
    """The layout predicate evaluated for one query over every key."""
    k = np.arange(N)
    if lay.get("bitmap") is not None:
        bm = np.asarray(lay["bitmap"])
        ok = bm[0 if bm.shape[0] == 1 else h, q // bs, k // bs].astype(bool)
    else:
        qu, ku = (q, k) if lay["unit"] == "tokens" else (q // bs, k // bs)
        ok = np.ones(N, dtype=bool)
        if lay["window_left"] >= 0:
            ok &= qu - ku <= lay["window_left"]
        if lay["window_right"] >= 0:
            ok &= ku - qu <= lay["window_right"]
        ok |= (ku < lay["global_keys"]) | (qu < lay["global_queries"])
    if lay["causal"]:
        ok &= k <= q
    return np.flatnonzero(ok)


@pytest.mark.parametrize("name", ["window16k", "winglobal128k", "gqa256k", "dense256k", "random32k",
                                  "tiny_f32"])
def test_allowed_keys_equal_predicate_full_size(name):
    w = wl.WORKLOADS[name]
    lay = wl.layout_of(w)
    if lay.get("bitmap") is not None:
        lay = dict(lay, bitmap=np.asarray(lay["bitmap"]))
    N = w.seq_len
    rng = np.random.default_rng(31)
    qs = {0, 1, 127, 128, 511, 512, 4095, 4096, 4103, 4104, N - 1} | set(rng.integers(0, N, 40).tolist())
    for q in sorted(x for x in qs if x < N):
        for h in (0, w.heads - 1):
            np.testing.assert_array_equal(oracle.allowed_keys(lay, N, w.block, h, q),
                                          predicate_all_keys(lay, N, w.block, h, q), err_msg=f"q={q}")


# ------------------------------------------------ full-size brute-force plan
@pytest.mark.slow
@pytest.mark.parametrize("name", ["window16k", "gqa256k"])
def test_plan_bruteforce_full_size(name):
    """Brute force: A(q) enumerated for every one of the N queries, counted
    per tile; equals the interval counts and the C++ host planner."""
    from block_sparse_flash_bsa_amd import bsattn
    w = wl.WORKLOADS[name]
    lay = wl.layout_of(w)
    brute = oracle.plan(lay, w.seq_len, w.block, brute=True)
    fast = oracle.plan(lay, w.seq_len, w.block, brute=False)
    p = bsattn.plan(w.batch, w.heads, w.kv_heads, w.seq_len, w.head_dim, w.block, w.dtype, lay,
                    host_only=True)
    got = p.csr(0)
    for key in ("row_ptr", "col_idx", "flags"):
        np.testing.assert_array_equal(brute[0][key], fast[0][key], err_msg=key)
        np.testing.assert_array_equal(brute[0][key], got[key], err_msg=key)
