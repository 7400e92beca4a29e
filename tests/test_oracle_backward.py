"""Pins for the oracle's backward (dQ, dK, dV), checked against things other
than the oracle's own gradient code:

* a library routine: torch autograd through scaled_dot_product_attention in
  float64 for dense layouts (causal and not, GQA by repeated KV heads);
* brute force: torch autograd through materialised masked softmax attention
  whose N x N masks are built here with triu/tril/kron;
* finite differences of the oracle's (separately pinned) forward: the
  directional derivative of sum(dO * O) along a random direction;
* invariants of the softmax Jacobian: sum_k dK_k = 0, sum_k dV_k = sum of dO
  over non-empty rows, constant V rows give dQ = dK = 0, a single allowed key
  gives dQ = dK = 0 and dV_k = dO_k;
* the transposed enumeration allowed_queries against allowed_keys by brute
  force, and the sampled-row/-key functions against the full backward;
* planted mistakes in the gradient code that these pins must catch.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import bsa_oracle


def spec(causal, unit, w_left=-1, w_right=-1, gk=0, gq=0, bitmap=None):
    return dict(causal=causal, unit=unit, window_left=w_left, window_right=w_right,
                global_keys=gk, global_queries=gq, bitmap=bitmap)


def rand4(B, H, Hk, N, D, seed=0):
    g = torch.Generator().manual_seed(seed)
    Q = torch.randn(B, H, N, D, generator=g, dtype=torch.float64)
    K = torch.randn(B, Hk, N, D, generator=g, dtype=torch.float64)
    V = torch.randn(B, Hk, N, D, generator=g, dtype=torch.float64)
    dO = torch.randn(B, H, N, D, generator=g, dtype=torch.float64)
    return Q, K, V, dO


def autograd_masked(Q, K, V, dO, mask):
    """Gradients of sum(dO * O) for materialised masked attention (float64).

    mask: bool [N, N] or [H, N, N]; every row must have an allowed key.
    """
    Q, K, V = (x.clone().requires_grad_(True) for x in (Q, K, V))
    g = Q.shape[1] // K.shape[1]
    Ke, Ve = K.repeat_interleave(g, 1), V.repeat_interleave(g, 1)
    S = Q @ Ke.transpose(-1, -2) / math.sqrt(Q.shape[-1])
    m = torch.as_tensor(mask)
    S = S.masked_fill(~m, -math.inf)
    O = torch.softmax(S, dim=-1) @ Ve
    (O * dO).sum().backward()
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


def close3(a, b, tol=1e-11):
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, atol=tol, rtol=0)


def band(N, lo, hi):
    one = np.ones((N, N), bool)
    return np.triu(one, -lo) & np.tril(one, hi)


# ---------------------------------------------------------------- library pins
@pytest.mark.parametrize("causal", [False, True])
def test_dense_equals_sdpa_autograd(causal):
    B, H, Hk, N, D, bs = 1, 4, 2, 128, 16, 32
    Q, K, V, dO = rand4(B, H, Hk, N, D, 1)
    lay = spec(causal, "tokens")
    got = oracle.backward(Q, K, V, dO, lay, bs)
    Qr, Kr, Vr = (x.clone().requires_grad_(True) for x in (Q, K, V))
    O = torch.nn.functional.scaled_dot_product_attention(
        Qr, Kr.repeat_interleave(2, 1), Vr.repeat_interleave(2, 1), is_causal=causal)
    (O * dO).sum().backward()
    close3(got, (Qr.grad.numpy(), Kr.grad.numpy(), Vr.grad.numpy()))


# ---------------------------------------------------- brute force, tiny shapes
@pytest.mark.parametrize("W,G,GQ", [(15, 0, 0), (15, 3, 0), (40, 5, 2), (0, 1, 0)])
def test_causal_window_globals_bruteforce(W, G, GQ):
    N = 160
    Q, K, V, dO = rand4(1, 2, 1, N, 8, 2)
    mask = band(N, W, 0)
    mask[:, :G] = True
    mask[:GQ, :] = True
    mask &= np.tril(np.ones((N, N), bool))
    close3(oracle.backward(Q, K, V, dO, spec(True, "tokens", W, 0, G, GQ), 32),
           autograd_masked(Q, K, V, dO, mask))


@pytest.mark.parametrize("W", [0, 3, 20])
def test_symmetric_window_bruteforce(W):
    N = 128
    Q, K, V, dO = rand4(1, 2, 2, N, 8, 3)
    close3(oracle.backward(Q, K, V, dO, spec(False, "tokens", W, W), 32),
           autograd_masked(Q, K, V, dO, band(N, W, W)))


@pytest.mark.parametrize("causal", [False, True])
def test_bitmap_per_head_bruteforce(causal):
    N, bs, H = 192, 32, 3
    nb = N // bs
    rng = np.random.default_rng(4)
    bm = (rng.random((H, nb, nb)) < 0.35).astype(np.uint8)
    bm[:, np.arange(nb), np.arange(nb)] = 1           # every row keeps its diagonal block
    Q, K, V, dO = rand4(1, H, H, N, 8, 5)
    mask = np.stack([np.kron(bm[h], np.ones((bs, bs), np.uint8)).astype(bool) for h in range(H)])
    if causal:
        mask &= np.tril(np.ones((N, N), bool))[None]
    close3(oracle.backward(Q, K, V, dO, spec(causal, "blocks", bitmap=bm), bs),
           autograd_masked(Q, K, V, dO, mask))


def test_block_units_window_globals_bruteforce():
    """Causal, block window 2 plus one global key block and one global query block."""
    N, bs = 256, 32
    nb = N // bs
    i, j = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    grid = ((i - j) <= 2) | (j < 1) | (i < 1)
    mask = np.kron(grid, np.ones((bs, bs))).astype(bool) & np.tril(np.ones((N, N), bool))
    Q, K, V, dO = rand4(1, 4, 2, N, 8, 6)
    close3(oracle.backward(Q, K, V, dO, spec(True, "blocks", 2, 0, 1, 1), bs),
           autograd_masked(Q, K, V, dO, mask))


# ------------------------------------------------- finite differences of forward
def test_directional_derivative_matches_forward_differences():
    """<dX, U> equals d/dt sum(dO * O(X + tU)) at t = 0 (central differences)."""
    N, bs = 96, 32
    lay = spec(True, "tokens", 20, 0, 2)
    Q, K, V, dO = rand4(1, 2, 1, N, 8, 7)
    grads = oracle.backward(Q, K, V, dO, lay, bs)
    rng = np.random.default_rng(8)
    eps = 1e-5
    for which, grad in zip(range(3), grads):
        U = rng.standard_normal(grad.shape)

        def loss(t):
            X = [Q.numpy().copy(), K.numpy().copy(), V.numpy().copy()]
            X[which] = X[which] + t * U
            O, _ = oracle.forward(*X, lay, bs)
            return float((O * dO.numpy()).sum())
        fd = (loss(eps) - loss(-eps)) / (2 * eps)
        assert abs(fd - float((grad * U).sum())) < 1e-7 * max(1.0, abs(fd)), which


# ------------------------------------------------------------------ invariants
def test_softmax_jacobian_invariants():
    N, bs = 192, 64
    lay = spec(True, "tokens", 30, 0, 3)
    Q, K, V, dO = rand4(2, 4, 2, N, 8, 9)
    dQ, dK, dV = oracle.backward(Q, K, V, dO, lay, bs)
    # each row's score gradients sum to zero, so sum_k dK_k = scale * sum_q Q_q * 0
    np.testing.assert_allclose(dK.sum(axis=2), 0.0, atol=1e-12)
    # each row's weights sum to one: sum_k dV_k = sum over the group's rows of dO
    np.testing.assert_allclose(dV.sum(axis=2),
                               dO.numpy().reshape(2, 2, 2, N, 8).sum(axis=(2, 3)), atol=1e-12)


def test_constant_value_rows_give_zero_score_gradients():
    N, bs = 128, 32
    Q, K, _, dO = rand4(1, 2, 2, N, 8, 10)
    V = torch.randn(1, 2, 1, 8, dtype=torch.float64).expand(1, 2, N, 8).contiguous()
    dQ, dK, _ = oracle.backward(Q, K, V, dO, spec(False, "tokens", 9, 4, 1), bs)
    assert np.abs(dQ).max() < 1e-13 and np.abs(dK).max() < 1e-13


def test_single_allowed_key():
    N, bs = 128, 32
    Q, K, V, dO = rand4(1, 2, 2, N, 8, 11)
    dQ, dK, dV = oracle.backward(Q, K, V, dO, spec(True, "tokens", 0, 0), bs)
    assert np.abs(dQ).max() == 0 and np.abs(dK).max() == 0
    np.testing.assert_array_equal(dV, dO.numpy())


def test_empty_rows_contribute_nothing():
    N, bs = 128, 32
    nb = N // bs
    bm = np.ones((1, nb, nb), np.uint8)
    bm[0, 1, :] = 0                                    # q-block 1 sees nothing
    Q, K, V, dO = rand4(1, 1, 1, N, 8, 12)
    dQ, dK, dV = oracle.backward(Q, K, V, dO, spec(False, "blocks", bitmap=bm), bs)
    assert np.all(dQ[:, :, bs:2 * bs] == 0)
    dO2 = dO.clone()
    dO2[:, :, bs:2 * bs] = 1e3                          # their upstream gradient is irrelevant
    dQ2, dK2, dV2 = oracle.backward(Q, K, V, dO2, spec(False, "blocks", bitmap=bm), bs)
    np.testing.assert_array_equal(dK, dK2)
    np.testing.assert_array_equal(dV, dV2)


# ------------------------------------------- transposed enumeration and samples
@pytest.mark.parametrize("lay", [
    spec(True, "tokens", 20, 0, 3, 2), spec(False, "tokens", 5, 9, 0, 1),
    spec(True, "blocks", 1, 0, 1, 1), spec(False, "blocks", 1, 2, 0, 0)])
def test_allowed_queries_is_transpose_of_allowed_keys(lay):
    N, bs = 160, 32
    M = np.zeros((N, N), bool)
    for q in range(N):
        M[q, oracle.allowed_keys(lay, N, bs, 0, q)] = True
    for k in range(N):
        np.testing.assert_array_equal(oracle.allowed_queries(lay, N, bs, 0, k), np.flatnonzero(M[:, k]))


def test_allowed_queries_bitmap_transpose():
    N, bs, H = 128, 32, 2
    nb = N // bs
    bm = (np.random.default_rng(13).random((H, nb, nb)) < 0.4).astype(np.uint8)
    lay = spec(True, "blocks", bitmap=bm)
    for h in range(H):
        M = np.zeros((N, N), bool)
        for q in range(N):
            M[q, oracle.allowed_keys(lay, N, bs, h, q)] = True
        for k in range(0, N, 7):
            np.testing.assert_array_equal(oracle.allowed_queries(lay, N, bs, h, k), np.flatnonzero(M[:, k]))


def test_sampled_rows_and_keys_match_full_backward():
    N, bs = 160, 32
    lay = spec(True, "tokens", 40, 0, 3)
    Q, K, V, dO = rand4(1, 4, 2, N, 8, 14)
    dQ, dK, dV = oracle.backward(Q, K, V, dO, lay, bs)
    rows = [(0, h, q) for h in range(4) for q in (0, 1, 39, 40, 41, 159)]
    got = oracle.backward_dq_rows(Q, K, V, dO, lay, bs, rows)
    np.testing.assert_allclose(got, np.stack([dQ[r] for r in rows]), atol=1e-13, rtol=0)
    keys = [(0, hk, k) for hk in range(2) for k in (0, 2, 3, 100, 120, 159)]
    gk, gv = oracle.backward_dkv_keys(Q, K, V, dO, lay, bs, keys)
    np.testing.assert_allclose(gk, np.stack([dK[r] for r in keys]), atol=1e-13, rtol=0)
    np.testing.assert_allclose(gv, np.stack([dV[r] for r in keys]), atol=1e-13, rtol=0)


# ----------------------------------------------------------- planted mistakes
def _dense_case():
    N = 64
    Q, K, V, dO = rand4(1, 1, 1, N, 8, 15)
    return Q, K, V, dO, autograd_masked(Q, K, V, dO, np.ones((N, N), bool))


def test_pins_catch_planted_dropped_softmax_term(monkeypatch):
    """ds = p * dp (the -sum p dp term dropped) must break the autograd pin."""
    orig = bsa_oracle.grad_row

    def wrong(q, do, Kr, Vr, scale):
        p, _ = orig(q, do, Kr, Vr, scale)
        return p, p * (Vr @ do)
    monkeypatch.setattr(bsa_oracle, "grad_row", wrong)
    Q, K, V, dO, ref = _dense_case()
    got = bsa_oracle.backward(Q, K, V, dO, spec(False, "tokens"), 32)
    assert np.abs(got[0] - ref[0]).max() > 1e-3 and np.abs(got[1] - ref[1]).max() > 1e-3


def test_pins_catch_planted_unscaled_scores(monkeypatch):
    orig = bsa_oracle.grad_row
    monkeypatch.setattr(bsa_oracle, "grad_row", lambda q, do, Kr, Vr, s: orig(q, do, Kr, Vr, 1.0))
    Q, K, V, dO, ref = _dense_case()
    got = bsa_oracle.backward(Q, K, V, dO, spec(False, "tokens"), 32)
    assert max(np.abs(g - r).max() for g, r in zip(got, ref)) > 1e-3


def test_pins_catch_planted_swapped_key_value_roles(monkeypatch):
    """dp formed from K instead of V must break the autograd pin."""
    orig = bsa_oracle.grad_row
    monkeypatch.setattr(bsa_oracle, "grad_row", lambda q, do, Kr, Vr, s: orig(q, do, Kr, Kr, s))
    Q, K, V, dO, ref = _dense_case()
    got = bsa_oracle.backward(Q, K, V, dO, spec(False, "tokens"), 32)
    assert np.abs(got[0] - ref[0]).max() > 1e-3


@pytest.mark.parametrize("N,causal", [(200, True), (150, False)])
def test_ragged_length_bruteforce(N, causal):
    """A last, shorter block (bs = 64 does not divide N): autograd through the
    masked attention of exactly N positions."""
    Q, K, V, dO = rand4(1, 2, 1, N, 8, 16)
    mask = band(N, 30, 0 if causal else 30)
    mask[:, :2] = True
    if causal:
        mask &= np.tril(np.ones((N, N), bool))
    close3(oracle.backward(Q, K, V, dO, spec(causal, "tokens", 30, 0 if causal else 30, 2), 64),
           autograd_masked(Q, K, V, dO, mask))
