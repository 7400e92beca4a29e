"""CPU pins of the oracle's LSE merge (partial attention results over disjoint
key sets of the same queries combined into the result over their union).

* Library attention: torch scaled_dot_product_attention in float64 over two
  (or three) disjoint key ranges, each part's LSE from torch.logsumexp of its
  scaled scores, merged, against SDPA over all keys.
* The oracle's own forward over a per-head bitmap split into disjoint block
  subsets, merged, against its forward over the whole bitmap (rows empty in
  one part, in every part, GQA).
* Algebra: a part with no key changes nothing, the order of parts does not
  matter, large LSEs (where forgetting the max would overflow) merge exactly,
  and planted mistakes (weights e^{L} without the max, a plain average, a
  dropped part) fail.
"""
import numpy as np
import pytest
import torch

import oracle


def sdpa_part(q, k, v):
    """Partial attention of q over keys k (float64): (O, LSE)."""
    s = (q @ k.transpose(-1, -2)) / np.sqrt(q.shape[-1])
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v)
    return o.numpy(), torch.logsumexp(s, dim=-1).numpy()


@pytest.mark.parametrize("cuts", [[0, 300, 700], [0, 1, 700], [0, 200, 450, 700]])
def test_merge_of_key_ranges_is_sdpa_over_all_keys(cuts):
    g = torch.Generator().manual_seed(len(cuts))
    q = torch.randn(2, 3, 50, 32, generator=g, dtype=torch.float64)
    k = torch.randn(2, 3, 700, 32, generator=g, dtype=torch.float64)
    v = torch.randn(2, 3, 700, 32, generator=g, dtype=torch.float64)
    parts = [sdpa_part(q, k[:, :, a:b], v[:, :, a:b]) for a, b in zip(cuts[:-1], cuts[1:])]
    O, L = oracle.lse_merge([p[0] for p in parts], [p[1] for p in parts])
    ref_o, ref_l = sdpa_part(q, k, v)
    assert np.abs(O - ref_o).max() < 1e-12
    assert np.abs(L - ref_l).max() < 1e-12


def split_bitmap(layout_bm, parts, seed):
    rng = np.random.default_rng(seed)
    owner = rng.integers(0, parts, size=layout_bm.shape)
    return [(layout_bm.astype(bool) & (owner == p)).astype(np.uint8) for p in range(parts)]


@pytest.mark.parametrize("parts,causal", [(2, False), (2, True), (3, False)])
def test_merge_of_split_bitmaps_is_the_union(parts, causal):
    N, bs, H, Hkv, D = 320, 32, 4, 2, 16
    nb = N // bs
    rng = np.random.default_rng(parts + causal)
    bm = (rng.random((H, nb, nb)) < 0.5).astype(np.uint8)
    bm[0, 3, :] = 0                                   # a row empty everywhere
    g = torch.Generator().manual_seed(7)
    Q = torch.randn(1, H, N, D, generator=g, dtype=torch.float64)
    K = torch.randn(1, Hkv, N, D, generator=g, dtype=torch.float64)
    V = torch.randn(1, Hkv, N, D, generator=g, dtype=torch.float64)

    def lay(b):
        return dict(causal=causal, unit="blocks", window_left=-1, window_right=-1, global_keys=0,
                    global_queries=0, bitmap=b)
    outs = [oracle.forward(Q, K, V, lay(b), bs) for b in split_bitmap(bm, parts, seed=3)]
    O, L = oracle.lse_merge([o for o, _ in outs], [l for _, l in outs])
    ref_o, ref_l = oracle.forward(Q, K, V, lay(bm), bs)
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(L), fin)
    assert not fin.all() and fin.any()
    assert np.abs(O - ref_o).max() < 1e-12
    assert np.abs(L[fin] - ref_l[fin]).max() < 1e-12
    assert np.all(O[~fin] == 0)


def test_merge_algebra():
    rng = np.random.default_rng(0)
    O = rng.standard_normal((3, 5, 8))
    L = rng.standard_normal((3, 5)) * 3
    # an empty part changes nothing
    O2 = np.concatenate([O, rng.standard_normal((1, 5, 8))])
    L2 = np.concatenate([L, np.full((1, 5), -np.inf)])
    a, b = oracle.lse_merge(O, L), oracle.lse_merge(O2, L2)
    assert np.allclose(a[0], b[0], atol=1e-15) and np.allclose(a[1], b[1], atol=1e-15)
    # order of parts
    c = oracle.lse_merge(O[::-1], L[::-1])
    assert np.allclose(a[0], c[0], atol=1e-14) and np.allclose(a[1], c[1], atol=1e-14)
    # one part: itself
    d = oracle.lse_merge(O[:1], L[:1])
    assert np.array_equal(d[0], O[0]) and np.allclose(d[1], L[0], atol=1e-15)
    # equal LSEs: the mean of the parts, LSE + ln P
    e = oracle.lse_merge(O, np.zeros((3, 5)))
    assert np.allclose(e[0], O.mean(axis=0), atol=1e-15) and np.allclose(e[1], np.log(3), atol=1e-15)
    # large LSEs merge exactly (e^{L} alone would overflow)
    f = oracle.lse_merge(O[:2], np.stack([np.full(5, 1000.0), np.full(5, 1000.0 + np.log(3))]))
    assert np.allclose(f[0], 0.25 * O[0] + 0.75 * O[1], atol=1e-14)
    assert np.allclose(f[1], 1000.0 + np.log(4), atol=1e-12)
    # rows empty in every part
    g = oracle.lse_merge(O, np.full((3, 5), -np.inf))
    assert np.all(g[0] == 0) and np.all(np.isneginf(g[1]))


def test_planted_merge_mistakes_fail():
    """Plausible mistakes in a merge fail the split-union pin's arithmetic."""
    rng = np.random.default_rng(1)
    O = rng.standard_normal((2, 6, 4))
    L = rng.standard_normal((2, 6)) * 2
    good, lgood = oracle.lse_merge(O, L)
    w = np.exp(L) / np.exp(L).sum(axis=0)
    assert np.allclose(good, (w[..., None] * O).sum(axis=0), atol=1e-13)   # the law itself
    mean = O.mean(axis=0)                                                   # plain average
    assert np.abs(mean - good).max() > 1e-3
    dropped = O[0]                                                          # a dropped part
    assert np.abs(dropped - good).max() > 1e-3
    wrong_lse = L.max(axis=0)                                               # max instead of logaddexp
    assert np.abs(wrong_lse - lgood).max() > 1e-3
