"""GPU tests of bsa_lse_merge (partial attention results over disjoint key
sets combined into the result over their union), through the C ABI.

* The kernel against the oracle's merge on the same inputs: bf16 and float32,
  2 and 5 parts, parts without keys, rows empty in every part, LSEs near
  1000; one part is returned unchanged.
* End to end: forwards over a bitmap split into disjoint block subsets,
  merged on the GPU, against the oracle's forward over the whole bitmap on
  every row (R12 tolerances: bf16 2e-2 on O and 1e-3 on LSE, float32 1e-5).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from block_sparse_flash_bsa_amd import bsattn

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsattn.lib()
    torch.cuda.set_device(0)


@pytest.mark.parametrize("dtype,P", [(torch.bfloat16, 2), (torch.bfloat16, 5), (torch.float32, 2),
                                     (torch.float32, 5)])
def test_merge_kernel_against_oracle(dtype, P):
    g = torch.Generator().manual_seed(P)
    rows, D = 3000, 128
    O = torch.randn(P, rows, D, generator=g).to(dtype)
    L = torch.randn(P, rows, generator=g) * 4
    L[0, ::7] = float("-inf")                          # part 0 has no key in some rows
    L[:, 5] = float("-inf")                            # a row empty in every part
    L[:, 6] = 1000.0 + torch.arange(P, dtype=torch.float32)   # large LSEs
    out, lse = bsattn.lse_merge(O.cuda(), L.cuda())
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.lse_merge(O.double().numpy(), L.double().numpy())
    o = out.double().cpu().numpy()
    l = lse.double().cpu().numpy()
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(l), fin) and not fin[5]
    assert np.all(o[5] == 0)
    eo = float(np.abs(o - ref_o).max())
    el = float(np.abs(l[fin] - ref_l[fin]).max())
    tol_o = 2.0 ** -8 * float(np.abs(ref_o).max()) if dtype == torch.bfloat16 else 1e-5
    say(f"  {dtype} P={P}: max|dO| {eo:.2e} (tol {tol_o:.1e}), max|dLSE| {el:.2e}")
    assert eo <= tol_o and el <= 1e-4


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_merge_of_one_part_is_the_part(dtype):
    g = torch.Generator().manual_seed(3)
    O = torch.randn(1, 2, 4, 256, 128, generator=g).to(dtype).cuda()
    L = torch.randn(1, 2, 4, 256, generator=g).cuda()
    out, lse = bsattn.lse_merge(O, L)
    torch.cuda.synchronize()
    assert torch.equal(out, O[0])
    assert float((lse - L[0]).abs().max()) <= 1e-5


def split(bm, parts, seed):
    owner = np.random.default_rng(seed).integers(0, parts, size=bm.shape)
    return [(bm.astype(bool) & (owner == p)).astype(np.uint8) for p in range(parts)]


@pytest.mark.parametrize("dtype,parts,causal", [(torch.bfloat16, 2, False), (torch.bfloat16, 3, True),
                                                (torch.float32, 2, True)])
def test_split_forwards_merged_equal_the_union(dtype, parts, causal):
    """Forwards over a bitmap split into disjoint block subsets, merged,
    against the oracle over the whole bitmap on every row."""
    if dtype == torch.bfloat16:
        B, H, Hkv, N, D, bs = 1, 4, 2, 2048, 128, 128
    else:
        B, H, Hkv, N, D, bs = 1, 4, 2, 1024, 64, 64
    nb = N // bs
    rng = np.random.default_rng(parts)
    bm = (rng.random((H, nb, nb)) < 0.4).astype(np.uint8)
    bm[:, np.arange(nb), np.arange(nb)] = 1
    bm[1, 2, :] = 0                                    # a row empty in every part
    g = torch.Generator().manual_seed(11)
    q = torch.randn(B, H, N, D, generator=g).to(dtype)
    k = torch.randn(B, Hkv, N, D, generator=g).to(dtype)
    v = torch.randn(B, Hkv, N, D, generator=g).to(dtype)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()

    def lay(b):
        return dict(causal=causal, unit="blocks", window_left=-1, window_right=-1, global_keys=0,
                    global_queries=0, bitmap=b)
    outs, lses = [], []
    for part in split(bm, parts, seed=5):
        p = bsattn.plan(B, H, Hkv, N, D, bs, dtype, lay(part))
        o, l = bsattn.forward(qc, kc, vc, p)
        outs.append(o)
        lses.append(l)
    out, lse = bsattn.lse_merge(torch.stack(outs), torch.stack(lses))
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.forward(q, k, v, lay(bm), bs)
    o = out.double().cpu().numpy()
    l = lse.double().cpu().numpy()
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(l), fin) and not fin.all()
    eo = float(np.abs(o - ref_o).max())
    el = float(np.abs(l[fin] - ref_l[fin]).max())
    to, tl = (2e-2, 1e-3) if dtype == torch.bfloat16 else (1e-5, 1e-5)
    say(f"  {dtype} parts={parts} causal={causal}: max|dO| {eo:.2e} max|dLSE| {el:.2e}")
    assert eo <= to and el <= tl
    assert np.all(o[~fin] == 0)
