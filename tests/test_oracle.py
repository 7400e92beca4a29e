"""Pins for the CPU oracle: checks against things other than the oracle itself.

* a library routine: torch's scaled_dot_product_attention and logsumexp in
  float64 for dense layouts;
* brute-force dense masked attention whose N x N masks are built here with
  triu/tril/kron (the naive masked formulation of the pages), not from the
  oracle's interval code;
* invariants: weights sum to one (V = 1 gives O = 1), a window >= N is dense,
  a single allowed key returns that key's V row;
* closed forms for |A(q)| and for the plan's entry counts, derived by hand
  from each workload's rule;
* a value the pages print (tests/golden/window_flop_ratio.json);
* planted mistakes in the oracle that these pins must catch.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import bsa_oracle
from block_sparse_flash_bsa_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def spec(causal, unit, w_left=-1, w_right=-1, gk=0, gq=0, bitmap=None):
    return dict(causal=causal, unit=unit, window_left=w_left, window_right=w_right,
                global_keys=gk, global_queries=gq, bitmap=bitmap)


def rand_qkv(B, H, Hk, N, D, seed=0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(B, H, N, D, generator=g, dtype=torch.float64),
            torch.randn(B, Hk, N, D, generator=g, dtype=torch.float64),
            torch.randn(B, Hk, N, D, generator=g, dtype=torch.float64))


def dense_masked(Q, K, V, mask, scale=None):
    """Materialised masked softmax attention (float64, tiny shapes only)."""
    Q, K, V = (x.numpy() for x in (Q, K, V))
    B, H, N, D = Q.shape
    g = H // K.shape[1]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    O = np.zeros((B, H, N, D))
    L = np.full((B, H, N), -np.inf)
    for b in range(B):
        for h in range(H):
            mk = mask if mask.ndim == 2 else mask[h]
            S = np.where(mk, scale * Q[b, h] @ K[b, h // g].T, -np.inf)
            m = S.max(axis=1)
            ok = np.isfinite(m)
            W = np.where(mk, np.exp(S - np.where(ok, m, 0)[:, None]), 0.0)
            l = W.sum(axis=1)
            O[b, h, ok] = W[ok] @ V[b, h // g] / l[ok, None]
            L[b, h, ok] = m[ok] + np.log(l[ok])
    return O, L


def assert_close(O, L, O2, L2, tol=1e-12):
    np.testing.assert_allclose(O, O2, atol=tol, rtol=0)
    fin = np.isfinite(L2)
    assert np.array_equal(np.isfinite(L), fin)
    np.testing.assert_allclose(L[fin], L2[fin], atol=tol, rtol=0)


# ---------------------------------------------------------------- library pins
def test_full_bitmap_equals_sdpa():
    B, H, Hk, N, D, bs = 2, 4, 2, 256, 32, 32
    Q, K, V = rand_qkv(B, H, Hk, N, D, 1)
    nb = N // bs
    lay = spec(False, "blocks", bitmap=np.ones((1, nb, nb), np.uint8))
    O, L = oracle.forward(Q, K, V, lay, bs)
    Ke, Ve = K.repeat_interleave(H // Hk, 1), V.repeat_interleave(H // Hk, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, Ke, Ve)
    lse = torch.logsumexp(Q @ Ke.transpose(-1, -2) / math.sqrt(D), dim=-1)
    assert_close(O, L, ref.numpy(), lse.numpy())


def test_causal_dense_equals_sdpa_causal():
    B, H, Hk, N, D, bs = 1, 2, 1, 192, 16, 64
    Q, K, V = rand_qkv(B, H, Hk, N, D, 2)
    O, L = oracle.forward(Q, K, V, spec(True, "tokens", -1, 0), bs)
    Ke, Ve = K.repeat_interleave(H // Hk, 1), V.repeat_interleave(H // Hk, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, Ke, Ve, is_causal=True)
    S = Q @ Ke.transpose(-1, -2) / math.sqrt(D)
    S = S.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), -math.inf)
    assert_close(O, L, ref.numpy(), torch.logsumexp(S, -1).numpy())


def test_custom_scale_matches_sdpa():
    Q, K, V = rand_qkv(1, 1, 1, 64, 8, 3)
    O, L = oracle.forward(Q, K, V, spec(False, "tokens"), 32, scale=0.3)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=0.3)
    assert_close(O, L, ref.numpy(), torch.logsumexp(0.3 * Q @ K.transpose(-1, -2), -1).numpy())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("unit,w", [("tokens", 256), ("tokens", 10_000), ("blocks", 4), ("blocks", 99)])
def test_window_at_least_n_is_dense(causal, unit, w):
    N, bs = 256, 64
    Q, K, V = rand_qkv(1, 2, 2, N, 16, 4)
    O, L = oracle.forward(Q, K, V, spec(causal, unit, w, w), bs)
    O2, L2 = oracle.forward(Q, K, V, spec(causal, "tokens", -1, -1), bs)
    assert_close(O, L, O2, L2)
    mask = np.tril(np.ones((N, N), bool)) if causal else np.ones((N, N), bool)
    assert_close(O, L, *dense_masked(Q, K, V, mask))


# ---------------------------------------------------- brute force, tiny shapes
def band(N, lo, hi):
    """Boolean mask of pairs with -lo <= k - q <= hi, via triu/tril."""
    one = np.ones((N, N), bool)
    return np.triu(one, -lo) & np.tril(one, hi)


@pytest.mark.parametrize("W", [0, 1, 7, 33])
def test_symmetric_window_bruteforce(W):
    N = 160
    Q, K, V = rand_qkv(1, 2, 1, N, 8, 5)
    mask = ~(np.triu(np.ones((N, N), bool), W + 1) | np.tril(np.ones((N, N), bool), -W - 1))
    assert_close(*oracle.forward(Q, K, V, spec(False, "tokens", W, W), 32),
                 *dense_masked(Q, K, V, mask))


@pytest.mark.parametrize("W,G,GQ", [(15, 0, 0), (15, 3, 0), (40, 5, 2), (0, 1, 0)])
def test_causal_window_globals_bruteforce(W, G, GQ):
    N = 192
    Q, K, V = rand_qkv(1, 2, 2, N, 8, 6)
    mask = band(N, W, 0)
    mask[:, :G] = True
    mask[:GQ, :] = True
    mask &= np.tril(np.ones((N, N), bool))
    assert_close(*oracle.forward(Q, K, V, spec(True, "tokens", W, 0, G, GQ), 64),
                 *dense_masked(Q, K, V, mask))


@pytest.mark.parametrize("causal", [False, True])
def test_bitmap_per_head_bruteforce(causal):
    N, bs, H = 256, 32, 3
    nb = N // bs
    rng = np.random.default_rng(7)
    bm = (rng.random((H, nb, nb)) < 0.3).astype(np.uint8)
    bm[:, 2, :] = 0                                   # an empty q-block row
    Q, K, V = rand_qkv(2, H, H, N, 8, 8)
    mask = np.stack([np.kron(bm[h], np.ones((bs, bs), np.uint8)).astype(bool) for h in range(H)])
    if causal:
        mask &= np.tril(np.ones((N, N), bool))[None]
    O, L = oracle.forward(Q, K, V, spec(causal, "blocks", bitmap=bm), bs)
    O2, L2 = dense_masked(Q, K, V, mask)
    assert_close(O, L, O2, L2)
    assert np.all(L[:, :, 2 * bs:3 * bs] == -np.inf) and np.all(O[:, :, 2 * bs:3 * bs] == 0)


def test_tiny_workload_rule_bruteforce():
    """Block (i, j) active iff |i-j| <= 2 or i == 0 or j == 0, via kron of the block grid."""
    N, bs = 512, 64
    nb = N // bs
    i, j = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    grid = (np.abs(i - j) <= 2) | (i == 0) | (j == 0)
    mask = np.kron(grid, np.ones((bs, bs))).astype(bool)
    Q, K, V = rand_qkv(1, 2, 2, N, 16, 9)
    assert_close(*oracle.forward(Q, K, V, spec(False, "blocks", 2, 2, 1, 1), bs),
                 *dense_masked(Q, K, V, mask))


# ------------------------------------------------------------------ invariants
def test_weights_sum_to_one():
    N = 256
    Q, K, _ = rand_qkv(1, 2, 2, N, 16, 10)
    V = torch.ones(1, 2, N, 16, dtype=torch.float64)
    O, L = oracle.forward(Q, K, V, spec(True, "tokens", 50, 0, 3), 64)
    np.testing.assert_allclose(O, 1.0, atol=1e-14)
    assert np.all(np.isfinite(L))


def test_single_allowed_key_returns_its_value_row():
    N, D = 128, 16
    Q, K, V = rand_qkv(1, 2, 2, N, D, 11)
    O, L = oracle.forward(Q, K, V, spec(True, "tokens", 0, 0), 64)
    np.testing.assert_array_equal(O, V.numpy())
    s = (Q * K).sum(-1).numpy() / math.sqrt(D)
    np.testing.assert_allclose(L, s, atol=1e-14)


def test_gqa_head_mapping():
    """Query head h reads KV head h // group: permuting KV heads permutes outputs."""
    Q, K, V = rand_qkv(1, 4, 2, 64, 8, 12)
    O, _ = oracle.forward(Q, K, V, spec(False, "tokens", 5, 5), 32)
    Ke, Ve = K.repeat_interleave(2, 1), V.repeat_interleave(2, 1)
    O2, _ = oracle.forward(Q, Ke, Ve, spec(False, "tokens", 5, 5), 32)
    np.testing.assert_array_equal(O, O2)


# -------------------------------------------------------------- closed forms
def closed_form_count(name, q, N):
    """|A(q)| for each workload's rule, derived by hand from the rule."""
    if name == "window16k":
        return min(q + 1, 512)
    if name == "gqa256k":
        return min(q + 1, 4096) + min(8, max(0, q - 4095))
    if name == "dense256k":
        return q + 1
    if name == "winglobal128k":
        i = q // 128
        row = min(i + 1, 64) + min(4, max(0, i - 63))
        return 128 * (row - 1) + q % 128 + 1
    if name == "tiny_f32":
        i, nb = q // 64, N // 64
        blocks = nb if i == 0 else len({j for j in range(nb) if abs(i - j) <= 2 or j == 0})
        return 64 * blocks
    raise KeyError(name)


def count_mismatches(orc, name, N, qs):
    lay = wl.WORKLOADS[name].layout
    bs = wl.WORKLOADS[name].block
    return [q for q in qs if orc.allowed_count(lay, N, bs, 0, q) != closed_form_count(name, q, N)]


def sample_queries(N, n=300, seed=0):
    rng = np.random.default_rng(seed)
    edges = [0, 1, 7, 8, 9, 127, 128, 129, 511, 512, 513, 4094, 4095, 4096, 4097, 4103, 4104,
             8191, 8192, 8193, N - 1]
    return sorted({q for q in edges if q < N} | set(rng.integers(0, N, n).tolist()))


@pytest.mark.parametrize("name", ["window16k", "winglobal128k", "gqa256k", "dense256k", "tiny_f32"])
def test_allowed_count_closed_form(name):
    N = wl.WORKLOADS[name].seq_len
    assert count_mismatches(oracle, name, N, sample_queries(N)) == []


@pytest.mark.parametrize("name", ["window16k", "gqa256k", "tiny_f32"])
def test_zero_q_lse_is_log_count(name):
    """Q = 0 makes every score 0, so LSE = ln |A(q)| exactly."""
    w = wl.WORKLOADS[name]
    N = 1024 if name != "gqa256k" else 8192 + 256
    Q = torch.zeros(1, 1, N, 16, dtype=torch.float64)
    K = torch.randn(1, 1, N, 16, dtype=torch.float64)
    V = torch.randn(1, 1, N, 16, dtype=torch.float64)
    qs = sample_queries(N, 40)
    _, L = oracle.forward(Q, K, V, w.layout, w.block, rows=[(0, 0, q) for q in qs])
    np.testing.assert_allclose(L, [math.log(closed_form_count(name, q, N)) for q in qs], atol=1e-12)


def plan_counts(p):
    return sum(len(x["col_idx"]) for x in p), sum(int((x["flags"] == 0).sum()) for x in p)


def closed_form_plan(name):
    """(nnz, FULL) per workload, summed over q-blocks from the hand-derived rows."""
    if name == "window16k":            # 4 window blocks: rows i<4 have i FULL + diag
        rows = [(i + 1, i) if i < 4 else (5, 3) for i in range(128)]
    elif name == "gqa256k":            # 32 window blocks + global block 0 from row 33 on
        rows = [(i + 1, i) if i < 32 else (33, 31) if i == 32 else (34, 31) for i in range(2048)]
    elif name == "winglobal128k":      # every j < i FULL, diagonal PARTIAL
        rows = [(min(i + 1, 64) + min(4, max(0, i - 63)),) * 2 for i in range(1024)]
        rows = [(n, n - 1) for n, _ in rows]
    elif name == "dense256k":
        rows = [(i + 1, i) for i in range(2048)]
    elif name == "tiny_f32":
        rows = []
        for i in range(16):
            n = 16 if i == 0 else len({j for j in range(16) if abs(i - j) <= 2 or j == 0})
            rows.append((n, n))
    return sum(r[0] for r in rows), sum(r[1] for r in rows)


@pytest.mark.parametrize("name,expect", [
    ("tiny_f32", (100, 100)), ("window16k", (630, 378)), ("winglobal128k", (67354, 66330)),
    ("gqa256k", (69071, 62992)), ("dense256k", (2098176, 2096128))])
def test_plan_closed_form_counts(name, expect):
    w = wl.WORKLOADS[name]
    assert closed_form_plan(name) == expect
    assert plan_counts(oracle.plan(w.layout, w.seq_len, w.block)) == expect


def test_random_bitmap_plan_counts():
    w = wl.WORKLOADS["random32k"]
    lay = wl.layout_of(w)
    p = oracle.plan(lay, w.seq_len, w.block)
    assert len(p) == 16
    assert plan_counts(p) == (108398, 108398)
    lens = np.concatenate([np.diff(x["row_ptr"]) for x in p])
    assert lens.min() == 9 and lens.max() == 44
    for h in range(16):   # CSR == nonzero pattern of the bitmap, row by row
        bm = lay["bitmap"][h].numpy()
        for i in (0, 17, 255):
            cols = p[h]["col_idx"][p[h]["row_ptr"][i]:p[h]["row_ptr"][i + 1]]
            np.testing.assert_array_equal(cols, np.flatnonzero(bm[i]))


# ------------------------------------------------ plan: intervals vs brute force
def random_specs(n, seed):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        bs = int(rng.choice([8, 16, 32]))
        N = bs * int(rng.integers(1, 9))
        unit = str(rng.choice(["tokens", "blocks"]))
        lim = N if unit == "tokens" else N // bs
        yield N, bs, spec(bool(rng.integers(0, 2)), unit,
                          int(rng.integers(-1, lim + 2)), int(rng.integers(-1, lim + 2)),
                          int(rng.integers(0, lim + 1)), int(rng.integers(0, lim + 1)))


def test_plan_intervals_match_bruteforce():
    for N, bs, lay in random_specs(150, 13):
        fast = oracle.plan(lay, N, bs, brute=False)
        slow = oracle.plan(lay, N, bs, brute=True)
        for a, b in zip(fast, slow):
            for key in ("row_ptr", "col_idx", "flags"):
                np.testing.assert_array_equal(a[key], b[key], err_msg=f"{lay} N={N} bs={bs}")


def test_plan_blocks_spec_equals_bitmap_of_same_rule():
    N, bs = 2048, 64
    nb = N // bs
    i, j = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    grid = ((i - j <= 5) & (j - i <= 1)) | (j < 2) | (i < 1)
    for causal in (False, True):
        a = oracle.plan(spec(causal, "blocks", 5, 1, 2, 1), N, bs)[0]
        b = oracle.plan(spec(causal, "blocks", bitmap=grid[None].astype(np.uint8)), N, bs)[0]
        for key in ("row_ptr", "col_idx", "flags"):
            np.testing.assert_array_equal(a[key], b[key])


# ----------------------------------------------------------- printed value
def test_golden_window_flop_ratio():
    """The pages print that a 4096 window at n = 128K cuts attention work 32x."""
    with open(os.path.join(GOLDEN, "window_flop_ratio.json")) as f:
        g = json.load(f)
    N, W = g["n"], g["window"]
    lay = spec(True, "tokens", W - 1, 0)
    qs = np.arange(0, N, 97)
    mean = np.mean([oracle.allowed_count(lay, N, 128, 0, int(q)) for q in qs])
    ratio = N / mean                      # full attention has N keys per query
    assert abs(ratio - g["printed_ratio"]) < g["abs_tolerance"], ratio
    sym = spec(False, "tokens", W, W)     # the symmetric |i-j| <= W reading gives ~16x
    mean_sym = np.mean([oracle.allowed_count(sym, N, 128, 0, int(q)) for q in qs[::10]])
    assert abs(N / mean_sym - g["printed_ratio"]) > 10


# ----------------------------------------------------------- planted mistakes
def test_pins_catch_planted_window_off_by_one(monkeypatch):
    orig = bsa_oracle._token_pieces

    def wider(layout, N, q):
        pieces = orig(layout, N, q)
        return [(max(0, lo - 1), hi) for lo, hi in pieces]   # one extra key on the left
    monkeypatch.setattr(bsa_oracle, "_token_pieces", wider)
    assert count_mismatches(bsa_oracle, "window16k", 16384, sample_queries(16384)) != []


def test_pins_catch_planted_dropped_global(monkeypatch):
    orig = bsa_oracle._token_pieces
    monkeypatch.setattr(bsa_oracle, "_token_pieces", lambda lay, N, q: orig(lay, N, q)[:1])
    assert count_mismatches(bsa_oracle, "gqa256k", 262144, sample_queries(262144)) != []


def test_pins_catch_planted_transposed_operand(monkeypatch):
    """Swapping K and V roles in the row kernel must break the SDPA pin."""
    orig = bsa_oracle.attend_row
    monkeypatch.setattr(bsa_oracle, "attend_row", lambda q, Kr, Vr, s: orig(q, Vr, Kr, s))
    Q, K, V = rand_qkv(1, 1, 1, 64, 8, 14)
    O, _ = bsa_oracle.forward(Q, K, V, spec(False, "tokens"), 32)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V).numpy()
    assert np.abs(O - ref).max() > 1e-3


def test_pins_catch_planted_missing_scale(monkeypatch):
    orig = bsa_oracle.attend_row
    monkeypatch.setattr(bsa_oracle, "attend_row", lambda q, Kr, Vr, s: orig(q, Kr, Vr, 1.0))
    Q, K, V = rand_qkv(1, 1, 1, 64, 8, 15)
    _, L = bsa_oracle.forward(Q, K, V, spec(False, "tokens"), 32)
    lse = torch.logsumexp(Q @ K.transpose(-1, -2) / math.sqrt(8), -1).numpy()
    assert np.abs(L - lse).max() > 1e-3


# ------------------------------------------- ragged lengths (bs does not divide N)
# The last block holds N mod bs rows; keys and queries at or beyond N do not
# exist.  The masks below are built for exactly N positions (triu/tril/kron
# trimmed to N), independently of the oracle's block and interval code.
@pytest.mark.parametrize("N,W,G,GQ", [(200, 37, 3, 0), (130, 0, 0, 0), (333, 100, 8, 5)])
def test_ragged_token_rule_bruteforce(N, W, G, GQ):
    Q, K, V = rand_qkv(1, 2, 1, N, 8, 20)
    mask = band(N, W, 0)
    mask[:, :G] = True
    mask[:GQ, :] = True
    mask &= np.tril(np.ones((N, N), bool))
    assert_close(*oracle.forward(Q, K, V, spec(True, "tokens", W, 0, G, GQ), 64),
                 *dense_masked(Q, K, V, mask))


@pytest.mark.parametrize("causal", [False, True])
def test_ragged_block_rule_and_bitmap_bruteforce(causal):
    N, bs = 300, 64                                  # 5 blocks, the last with 44 rows
    nb = -(-N // bs)
    i, j = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    grid = (np.abs(i - j) <= 1) | (j < 1)
    mask = np.kron(grid, np.ones((bs, bs))).astype(bool)[:N, :N]
    if causal:
        mask &= np.tril(np.ones((N, N), bool))
    Q, K, V = rand_qkv(1, 2, 2, N, 8, 21)
    assert_close(*oracle.forward(Q, K, V, spec(causal, "blocks", 1, 1, 1, 0), bs), *dense_masked(Q, K, V, mask))
    bm = grid[None].astype(np.uint8)
    assert_close(*oracle.forward(Q, K, V, spec(causal, "blocks", bitmap=bm), bs), *dense_masked(Q, K, V, mask))


def test_ragged_dense_equals_sdpa():
    N = 190
    Q, K, V = rand_qkv(1, 2, 2, N, 16, 22)
    O, L = oracle.forward(Q, K, V, spec(True, "tokens"), 64)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True)
    assert_close(O, L, ref.numpy(), torch.logsumexp(
        (Q @ K.transpose(-1, -2) / 4.0).masked_fill(~torch.ones(N, N, dtype=torch.bool).tril(), -math.inf),
        -1).numpy())


def test_ragged_plan_counts_bruteforce_and_flags():
    rng = np.random.default_rng(23)
    for _ in range(60):
        bs = int(rng.choice([8, 16, 32]))
        N = bs * int(rng.integers(1, 7)) + int(rng.integers(1, bs))
        unit = str(rng.choice(["tokens", "blocks"]))
        lim = N if unit == "tokens" else -(-N // bs)
        lay = spec(bool(rng.integers(0, 2)), unit, int(rng.integers(-1, lim + 2)), int(rng.integers(-1, lim + 2)),
                   int(rng.integers(0, lim + 1)), int(rng.integers(0, lim + 1)))
        fast = oracle.plan(lay, N, bs, brute=False)[0]
        slow = oracle.plan(lay, N, bs, brute=True)[0]
        for key in ("row_ptr", "col_idx", "flags"):
            np.testing.assert_array_equal(fast[key], slow[key], err_msg=f"{lay} N={N} bs={bs}")
        nb = -(-N // bs)
        last = slow["col_idx"] == nb - 1     # tiles touching the short block are never FULL
        assert np.all(slow["flags"][last] == oracle.PARTIAL)
        rows_last = slice(slow["row_ptr"][nb - 1], slow["row_ptr"][nb])
        assert np.all(slow["flags"][rows_last] == oracle.PARTIAL)
