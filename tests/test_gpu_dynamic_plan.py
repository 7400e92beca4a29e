"""GPU tests of dynamic plans: the CSR that bsa_plan_set_bitmap derives on the
device from a device bitmap must equal, bit for bit, the host planner's CSR
for the same bitmap and the oracle's plan (entries exist iff the tile has an
allowed pair; PARTIAL iff fewer than block^2), and a forward through a
dynamic plan must equal a forward through the host-built plan bit for bit
(same entries, same kernel; only the launch order differs) and match the
oracle within the library tolerances."""
import sys

import numpy as np
import pytest
import torch

import oracle
from block_sparse_flash_bsa_amd import bsattn
from block_sparse_flash_bsa_amd import workloads as wl

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsattn.lib()
    torch.cuda.set_device(0)


def bitmap_layout(bm, causal):
    return dict(causal=causal, unit="blocks", window_left=-1, window_right=-1, global_keys=0,
                global_queries=0, bitmap=bm)


def random_bitmap(lh, nb, density, seed):
    rng = np.random.default_rng(seed)
    bm = (rng.random((lh, nb, nb)) < density).astype(np.uint8)
    bm[:, np.arange(nb), np.arange(nb)] = 1
    return bm


def assert_same_csr(a, b, what):
    for key in ("row_ptr", "col_idx", "flags"):
        assert np.array_equal(np.asarray(a[key]), np.asarray(b[key])), f"{what}: {key} differs"


@pytest.mark.parametrize("lh,H,nb,bs,density,causal,cut", [
    (1, 2, 37, 64, 0.3, False, 0),
    (1, 2, 37, 64, 0.3, True, 0),
    (4, 4, 64, 64, 0.15, True, 0),
    (16, 16, 256, 128, 0.10, False, 0),
    (2, 2, 130, 64, 0.2, True, 0),
    # seq_len = nb * bs - cut: a shorter last block, whose tiles are PARTIAL
    (1, 2, 37, 64, 0.3, False, 63),
    (2, 2, 37, 64, 0.3, True, 1),
    (4, 4, 20, 128, 0.25, True, 100),
    (16, 16, 256, 128, 0.10, False, 27),
])
def test_device_csr_matches_host_plan_and_oracle(lh, H, nb, bs, density, causal, cut):
    bm = random_bitmap(lh, nb, density, seed=nb + lh)
    bm[0, 3, :] = 0                                  # an empty row (the diagonal too)
    bm[-1, nb - 2, :] = 1                            # a full row
    bm[-1, :, nb - 1] = 1                            # a full last column (the short block when cut > 0)
    N = nb * bs - cut
    lay = bitmap_layout(bm, causal)
    dtype = torch.float32 if bs == 64 else torch.bfloat16
    D = 64 if bs == 64 else 128
    hp = bsattn.plan(1, H, H, N, D, bs, dtype, lay, host_only=True)
    ref = oracle.plan(lay, N, bs)
    dp = bsattn.plan_dynamic(1, H, H, N, D, bs, dtype, causal, lh)
    nnz = torch.zeros(1, dtype=torch.int64, device="cuda")
    dp.set_bitmap(torch.from_numpy(bm).cuda(), nnz)
    torch.cuda.synchronize()
    total = 0
    for h in range(lh):
        got = dp.read_csr(h)
        assert_same_csr(got, hp.csr(h), f"head {h} vs host plan")
        assert_same_csr(got, ref[h], f"head {h} vs oracle")
        total += len(got["col_idx"])
        # The transposed lists built on the device: per column j, the rows i
        # whose oracle list holds j, ascending, with the same flags.
        gt = dp.read_csr_transposed(h)
        rp, ci, fl = (np.asarray(ref[h][key]) for key in ("row_ptr", "col_idx", "flags"))
        cols = [[] for _ in range(nb)]
        for i in range(nb):
            for e in range(rp[i], rp[i + 1]):
                cols[ci[e]].append((i, fl[e]))
        want_ptr = np.concatenate([[0], np.cumsum([len(c) for c in cols])])
        assert np.array_equal(gt["col_ptr"], want_ptr), f"head {h}: col_ptr"
        assert np.array_equal(gt["row_idx"], [i for c in cols for i, _ in c]), f"head {h}: row_idx"
        assert np.array_equal(gt["flags"], [f for c in cols for _, f in c]), f"head {h}: flags"
        ht = hp.csr_transposed(h)
        assert all(np.array_equal(gt[key], ht[key]) for key in ("col_ptr", "row_idx", "flags"))
    assert int(nnz.item()) == total == hp.info["nnz"]
    if cut:
        flags = np.concatenate([np.asarray(dp.read_csr(h)["flags"]) for h in range(lh)])
        assert flags.sum() > 0
    say(f"  lh={lh} nb={nb} N={N} causal={causal}: {total} entries identical, transposed lists too")


@pytest.mark.parametrize("lh,nb,causal", [(8, 1100, False), (8, 1100, True), (64, 1024, False), (64, 1024, True),
                                           (6, 2100, False), (32, 2052, True)])
def test_device_csr_many_rows_matches_host_plan(lh, nb, causal):
    """More rows than the one-workgroup scan takes (8 x 1100 and 64 x 1024
    rows): the blocked three-kernel scan gives the host planner's CSR and
    transposed lists bit for bit; 64 x 1024 also takes the column kernels'
    4-byte loads (256 strips of 256 columns).  With nb above 2048 a wave's
    chunk of rows exceeds what the column fill keeps in registers, so it
    reads its strip again: one byte per lane (6 x 2100) and four (32 x 2052,
    288 strips)."""
    bs = 64
    bm = random_bitmap(lh, nb, 0.01, seed=17)
    bm[2, 700, :] = 1                                # a full row
    bm[5, :, 9] = 1                                  # a full column
    lay = bitmap_layout(bm, causal)
    hp = bsattn.plan(1, lh, lh, nb * bs, 64, bs, torch.float32, lay, host_only=True)
    dp = bsattn.plan_dynamic(1, lh, lh, nb * bs, 64, bs, torch.float32, causal, lh)
    nnz = torch.zeros(1, dtype=torch.int64, device="cuda")
    dp.set_bitmap(torch.from_numpy(bm).cuda(), nnz)
    torch.cuda.synchronize()
    assert int(nnz.item()) == hp.info["nnz"]
    for h in range(lh):
        assert_same_csr(dp.read_csr(h), hp.csr(h), f"head {h}")
        gt, ht = dp.read_csr_transposed(h), hp.csr_transposed(h)
        for key in ("col_ptr", "row_idx", "flags"):
            assert np.array_equal(gt[key], ht[key]), f"head {h}: transposed {key}"
    say(f"  causal={causal}: {hp.info['nnz']} entries identical")


def test_forward_through_dynamic_plan_is_bitwise_the_static_one():
    w = wl.small_variant(wl.WORKLOADS["random32k"], 4096, heads=4, kv_heads=2, batch=2)
    bm = random_bitmap(4, 32, 0.2, seed=3)
    for causal in (False, True):
        lay = bitmap_layout(bm, causal)
        q, k, v = wl.make_qkv(w, "cpu")
        sp = bsattn.plan(w.batch, w.heads, w.kv_heads, w.seq_len, w.head_dim, w.block, w.dtype, lay)
        dp = bsattn.plan_dynamic(w.batch, w.heads, w.kv_heads, w.seq_len, w.head_dim, w.block, w.dtype,
                                 causal, 4)
        dp.set_bitmap(torch.from_numpy(bm).cuda())
        o1, l1 = bsattn.forward(q.cuda(), k.cuda(), v.cuda(), sp)
        o2, l2 = bsattn.forward(q.cuda(), k.cuda(), v.cuda(), dp)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"causal={causal}"
        rows = [(b, h, qq) for b in range(2) for h in range(4) for qq in (0, 1, 127, 128, 2049, 4095)]
        O_ref, L_ref = oracle.forward(q, k, v, lay, w.block, rows=rows)
        idx = tuple(torch.tensor(x) for x in zip(*rows))
        eo = float(np.abs(o2[idx].float().cpu().numpy() - O_ref).max())
        fin = np.isfinite(L_ref)
        el = float(np.abs(l2[idx].cpu().numpy()[fin] - L_ref[fin]).max()) if fin.any() else 0.0
        say(f"  causal={causal}: max|dO| {eo:.2e} max|dLSE| {el:.2e}")
        assert eo <= 2e-2 and el <= 1e-3
        assert np.array_equal(np.isfinite(l2[idx].cpu().numpy()), fin)


@pytest.mark.parametrize("lh", [1, 4])
def test_dynamic_order_is_longest_row_first(lh):
    """bsa_plan_set_bitmap re-sorts the launch order of a dynamic plan without
    the causal cut: every slot keeps its (b, h) (so its XCD run), the q-blocks
    of each (b, h) appear once each, and along each (KV head, batch entry) run
    of the order at creation the row lengths of the group's first head come
    non-increasing; a causal plan keeps its order; the forward through the
    re-sorted plan into NaN-poisoned outputs equals the static plan's bit for
    bit."""
    B, H, Hkv, nb, bs = 2, 4, 2, 64, 128
    group = H // Hkv
    rng = np.random.default_rng(21 + lh)
    dens = rng.random((lh, nb, 1)) * 0.5          # rows of very different lengths
    bm = (rng.random((lh, nb, nb)) < dens).astype(np.uint8)
    bm[:, np.arange(nb), np.arange(nb)] = 1
    w = wl.WORKLOADS["random32k"].with_shape(name="order", batch=B, heads=H, kv_heads=Hkv, seq_len=nb * bs)
    for causal in (False, True):
        dp = bsattn.plan_dynamic(B, H, Hkv, nb * bs, 128, bs, torch.bfloat16, causal, lh)
        base = dp.work()
        dp.set_bitmap(torch.from_numpy(bm).cuda())
        got = dp.read_work()
        assert got.shape == base.shape
        assert np.array_equal(got < 0, base < 0)
        live = base >= 0
        if causal:
            assert np.array_equal(got, base), "a causal dynamic plan keeps its order"
            continue
        assert np.array_equal(got[live] // nb, base[live] // nb), "a slot changed its (b, h)"
        for bh in range(B * H):
            qs = np.sort(got[live][got[live] // nb == bh] % nb)
            assert np.array_equal(qs, np.arange(nb)), f"(b, h) {bh}: q-blocks not a permutation"
        # Position of each slot in the order at creation: (KV head, batch entry,
        # q-block, group member), outer to inner.
        it = base[live]
        i0, bh0 = it % nb, it // nb
        h0, b0 = bh0 % H, bh0 // H
        pos = ((h0 // group * B + b0) * nb + i0) * group + h0 % group
        srt = np.argsort(pos)
        new_i = (got[live] % nb)[srt]
        hk_s = (h0 // group)[srt]
        b_s = b0[srt]
        lens = bm.sum(axis=2).astype(np.int64)       # [lh, nb] row lengths (no causal cut)
        for hk in range(Hkv):
            head = hk * group if lh > 1 else 0
            for b in range(B):
                seq = np.minimum(lens[head][new_i[(hk_s == hk) & (b_s == b)]], 1023)
                assert np.all(np.diff(seq) <= 0), f"run (hk {hk}, b {b}) not longest first"
        q, k, v = (x.cuda() for x in wl.make_qkv(w, "cpu"))
        sp = bsattn.plan(B, H, Hkv, nb * bs, 128, bs, torch.bfloat16, bitmap_layout(bm, False))
        o1, l1 = bsattn.forward(q, k, v, sp)
        o2 = torch.full_like(o1, float("nan"))
        l2 = torch.full_like(l1, float("nan"))
        bsattn.forward(q, k, v, dp, o2, l2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_new_bitmap_replaces_the_old_one():
    nb, bs, H = 48, 64, 2
    dp = bsattn.plan_dynamic(1, H, H, nb * bs, 64, bs, torch.float32, False, 1)
    first = np.ones((1, nb, nb), np.uint8)
    second = random_bitmap(1, nb, 0.05, seed=11)
    q = torch.randn(1, H, nb * bs, 64, generator=torch.Generator().manual_seed(1))
    k = torch.randn(1, H, nb * bs, 64, generator=torch.Generator().manual_seed(2))
    v = torch.randn(1, H, nb * bs, 64, generator=torch.Generator().manual_seed(3))
    for bm in (first, second):
        dp.set_bitmap(torch.from_numpy(bm).cuda())
        lay = bitmap_layout(bm, False)
        assert_same_csr(dp.read_csr(0), oracle.plan(lay, nb * bs, bs)[0], "after update")
        out, lse = bsattn.forward(q.cuda(), k.cuda(), v.cuda(), dp)
        torch.cuda.synchronize()
        rows = [(0, h, qq) for h in range(H) for qq in (0, 700, 3071)]
        O_ref, L_ref = oracle.forward(q, k, v, lay, bs, rows=rows)
        idx = tuple(torch.tensor(x) for x in zip(*rows))
        assert float(np.abs(out[idx].cpu().numpy() - O_ref).max()) <= 1e-5
        assert float(np.abs(lse[idx].cpu().numpy() - L_ref).max()) <= 1e-5


def test_fresh_and_empty_dynamic_plans_give_empty_rows():
    nb, bs, H = 16, 128, 2
    dp = bsattn.plan_dynamic(1, H, H, nb * bs, 128, bs, torch.bfloat16, True, H)
    q = torch.randn(1, H, nb * bs, 128, device="cuda").to(torch.bfloat16)
    for step in ("fresh", "zeros"):
        if step == "zeros":
            dp.set_bitmap(torch.zeros((H, nb, nb), dtype=torch.uint8, device="cuda"))
        out, lse = bsattn.forward(q, q, q, dp)
        torch.cuda.synchronize()
        assert torch.all(out == 0) and torch.all(torch.isneginf(lse)), step


def test_set_bitmap_rejects_host_memory_and_static_plans():
    nb, bs = 8, 64
    dp = bsattn.plan_dynamic(1, 1, 1, nb * bs, 64, bs, torch.float32, False, 1)
    host = np.ones((1, nb, nb), np.uint8)
    st = bsattn.lib().bsa_plan_set_bitmap(dp.handle, host.ctypes.data, None, None)
    assert st == bsattn.ERR_INVALID_ARGUMENT
    sp = bsattn.plan(1, 1, 1, nb * bs, 64, bs, torch.float32, bitmap_layout(host, False))
    dev = torch.from_numpy(host).cuda()
    st = bsattn.lib().bsa_plan_set_bitmap(sp.handle, dev.data_ptr(), None, None)
    assert st == bsattn.ERR_INVALID_ARGUMENT


def test_varlen_through_dynamic_plan_is_bitwise_the_static_one():
    """Variable-length forward and backward through a dynamic plan equal, bit
    for bit, the same calls through the host-built plan (lengths that end
    inside a block, on a block edge, and zero)."""
    w = wl.small_variant(wl.WORKLOADS["random32k"], 2048, heads=4, kv_heads=2, batch=4)
    bm = random_bitmap(4, 16, 0.25, seed=5)
    lens = torch.tensor([2048, 1000, 512, 0], dtype=torch.int32, device="cuda")
    for causal in (False, True):
        lay = bitmap_layout(bm, causal)
        q, k, v = (x.cuda() for x in wl.make_qkv(w, "cpu"))
        do = wl.make_dout(w, "cuda")
        sp = bsattn.plan(w.batch, w.heads, w.kv_heads, w.seq_len, w.head_dim, w.block, w.dtype, lay)
        dp = bsattn.plan_dynamic(w.batch, w.heads, w.kv_heads, w.seq_len, w.head_dim, w.block, w.dtype,
                                 causal, 4)
        dp.set_bitmap(torch.from_numpy(bm).cuda())
        res = []
        for p in (sp, dp):
            o, l = bsattn.forward_varlen(q, k, v, p, lens)
            res.append((o, l) + bsattn.backward_varlen(q, k, v, o, l, do, p, lens))
        torch.cuda.synchronize()
        for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), *res):
            assert torch.equal(a, b), f"causal={causal}: {name} differs"
        say(f"  causal={causal}: forward and backward bitwise equal")


@pytest.mark.parametrize("dtype,seq_len,block,D", [(torch.bfloat16, 4000, 128, 128), (torch.float32, 1000, 64, 64)])
def test_ragged_seq_len_through_dynamic_plan(dtype, seq_len, block, D):
    """A seq_len the block does not divide: forward and backward through a
    dynamic plan equal, bit for bit, the same calls through the host-built plan
    of the same bitmap (the short last block's tiles PARTIAL in both), and the
    oracle within the library tolerances on sampled rows, including the last
    row and every row of the short block's first and last tokens."""
    nb = -(-seq_len // block)
    H, Hkv, B = 4, 2, 2
    bm = random_bitmap(H, nb, 0.25, seed=seq_len)
    bm[1, :, nb - 1] = 1                             # every q-block sees the short block
    bm[2, nb - 1, :] = 1                             # the short block sees every key block
    tol_o, tol_l = (2e-2, 1e-3) if dtype == torch.bfloat16 else (1e-5, 1e-5)
    for causal in (False, True):
        lay = bitmap_layout(bm, causal)
        g = torch.Generator().manual_seed(seq_len + causal)
        q, k, v, do = (torch.randn(B, h, seq_len, D, generator=g).to(dtype) for h in (H, Hkv, Hkv, H))
        qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
        sp = bsattn.plan(B, H, Hkv, seq_len, D, block, dtype, lay)
        dp = bsattn.plan_dynamic(B, H, Hkv, seq_len, D, block, dtype, causal, H)
        assert dp.info["num_blocks"] == nb
        dp.set_bitmap(torch.from_numpy(bm).cuda())
        for h in range(H):
            assert_same_csr(dp.read_csr(h), sp.csr(h), f"head {h}")
        res = []
        for p in (sp, dp):
            o, l = bsattn.forward(qc, kc, vc, p)
            res.append((o, l) + bsattn.backward(qc, kc, vc, o, l, doc, p))
        torch.cuda.synchronize()
        for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), *res):
            assert torch.equal(a, b), f"causal={causal}: {name} differs"
        o, l = res[1][0], res[1][1]
        tail = (nb - 1) * block
        rows = [(b, h, qq) for b in range(B) for h in range(H)
                for qq in (0, 1, block - 1, tail - 1, tail, seq_len - 2, seq_len - 1)]
        O_ref, L_ref = oracle.forward(q, k, v, lay, block, rows=rows)
        idx = tuple(torch.tensor(x) for x in zip(*rows))
        eo = float(np.abs(o[idx].float().cpu().numpy() - O_ref).max())
        fin = np.isfinite(L_ref)
        el = float(np.abs(l[idx].cpu().numpy()[fin] - L_ref[fin]).max()) if fin.any() else 0.0
        assert np.array_equal(np.isfinite(l[idx].cpu().numpy()), fin)
        say(f"  {dtype} N={seq_len} causal={causal}: bitwise equal to the static plan; "
            f"max|dO| {eo:.2e} max|dLSE| {el:.2e}")
        assert eo <= tol_o and el <= tol_l


def chunks_of(desc):
    """The launch descriptors as a sorted list of (item, begin, end, split?),
    independent of slot positions and partial-tile numbering."""
    return sorted((int(a), int(b), int(c), int(p >= 0)) for a, b, c, p in desc if a >= 0)


def grads(p, q, k, v, do):
    o, l = bsattn.forward(q, k, v, p)
    g = bsattn.backward(q, k, v, o, l, do, p)
    torch.cuda.synchronize()
    return (o, l) + g


@pytest.mark.parametrize("causal", [False, True])
def test_dynamic_plan_splits_long_walks_like_the_static_plan(causal):
    """Full bitmap columns (a global key block read by every q-block): the
    device cuts their dK/dV walks by the host planner's rule, so the
    descriptors hold the same chunks, the backward equals the static plan's
    bit for bit and matches the oracle on every element; a second bitmap with
    no long column leaves no chunk behind."""
    B, H, Hkv, N, bs = 1, 8, 1, 4096, 128
    nb = N // bs
    bm = random_bitmap(H, nb, 0.05, seed=21)
    bm[:, :, 0] = 1
    bm[:, :, 5] = 1
    bm[0, :, 20] = 1
    g = torch.Generator().manual_seed(5 + causal)
    q, do = (torch.randn(B, H, N, 128, generator=g).to(torch.bfloat16) for _ in range(2))
    k, v = (torch.randn(B, Hkv, N, 128, generator=g).to(torch.bfloat16) for _ in range(2))
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    dp = bsattn.plan_dynamic(B, H, Hkv, N, 128, bs, torch.bfloat16, causal, H)
    for step, bmap in (("long columns", bm), ("no long column", random_bitmap(H, nb, 0.05, seed=22))):
        lay = bitmap_layout(bmap, causal)
        sp = bsattn.plan(B, H, Hkv, N, 128, bs, torch.bfloat16, lay)
        dp.set_bitmap(torch.from_numpy(bmap).cuda())
        ds, nd = dp.read_work_kv()
        ss, ns = sp.read_work_kv()
        assert chunks_of(ds) == chunks_of(ss) and nd == ns, step
        if step == "long columns":
            assert ns > 0, "expected the full columns' walks to be split"
        else:
            assert ns == 0 and all(d[3] < 0 for d in ds if d[0] >= 0)
        a, b = grads(sp, qc, kc, vc, doc), grads(dp, qc, kc, vc, doc)
        for name, x, y in zip(("O", "LSE", "dQ", "dK", "dV"), a, b):
            assert torch.equal(x, y), f"{step}: {name} differs from the static plan"
        say(f"  causal={causal} {step}: {ns} split columns, bitwise equal to the static plan")
    # Oracle, every element, for the bitmap with the long columns.
    lay = bitmap_layout(bm, causal)
    dp.set_bitmap(torch.from_numpy(bm).cuda())
    _, _, dq, dk, dv = grads(dp, qc, kc, vc, doc)
    rq, rk, rv = oracle.backward(q, k, v, do, lay, bs)
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        got = got.double().cpu().numpy()
        err, scale = float(np.abs(got - ref).max()), float(np.abs(ref).max())
        say(f"  {name}: max|err| {err:.3e} (max|ref| {scale:.3e})")
        assert err <= 1e-2 * scale


def test_dynamic_split_budget_doubles_the_chunk():
    """More chunks than the plan's partial-tile budget (1024 tiles; 18 batch
    entries x 30 long columns x 2 chunks = 1080): the device doubles the chunk
    length, here until no walk is split, while the static plan splits all 540
    columns; the gradients still match the oracle on sampled keys of long and
    short columns and the static plan's within bf16 rounding."""
    B, H, Hkv, nb, bs = 18, 4, 1, 72, 128
    N = nb * bs
    bm = np.zeros((1, nb, nb), np.uint8)
    for j in range(30):                              # 30 columns of 36 q-blocks each
        bm[0, (j + np.arange(36)) % nb, j] = 1
    bm[0, np.arange(nb), np.arange(nb)] = 1          # the diagonal: no empty row
    lay = bitmap_layout(bm, False)
    sp = bsattn.plan(B, H, Hkv, N, 128, bs, torch.bfloat16, lay)
    dp = bsattn.plan_dynamic(B, H, Hkv, N, 128, bs, torch.bfloat16, False, 1)
    dp.set_bitmap(torch.from_numpy(bm).cuda())
    ds, nd = dp.read_work_kv()
    ss, ns = sp.read_work_kv()
    say(f"  static plan: {ns} split columns; dynamic plan: {nd}")
    assert ns == 30 * B and nd == 0
    assert all(p < 0 for a, _, _, p in ds if a >= 0)
    g = torch.Generator().manual_seed(9)
    q, do = (torch.randn(B, H, N, 128, generator=g).to(torch.bfloat16) for _ in range(2))
    k, v = (torch.randn(B, Hkv, N, 128, generator=g).to(torch.bfloat16) for _ in range(2))
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    a, b = grads(sp, qc, kc, vc, doc), grads(dp, qc, kc, vc, doc)
    for name, x, y in zip(("O", "LSE", "dQ"), a[:3], b[:3]):
        assert torch.equal(x, y), name
    for name, x, y in zip(("dK", "dV"), a[3:], b[3:]):
        err, scale = float((x.float() - y.float()).abs().max()), float(y.float().abs().max())
        say(f"  {name}: max|dynamic - static| {err:.3e} (max {scale:.3e})")
        assert err <= 2 ** -7 * scale
    # Host float64 copies of the batch entries the sampled keys sit in.
    keys = [(17, 0, 29 * bs + 77), (7, 0, 50 * bs + 3)]   # a long and a short column
    sel = sorted({kb for kb, _, _ in keys})
    f64 = {name: {kb: t[kb].double().numpy() for kb in sel} for name, t in (("q", q), ("k", k), ("v", v), ("do", do))}

    class View:
        """[b, h] / [b, h, q] indexing over the per-batch-entry host copies."""
        def __init__(self, part, shape):
            self.part, self.shape = part, shape

        def __getitem__(self, idx):
            return self.part[idx[0]][idx[1:]]

    views = [View(f64[name], t.shape) for name, t in (("q", q), ("k", k), ("v", v), ("do", do))]
    for key in keys:
        rk, rv = oracle.backward_dkv_keys(*views, lay, bs, [key])
        for name, got, ref in (("dK", b[3][key], rk[0]), ("dV", b[4][key], rv[0])):
            got = got.double().cpu().numpy()
            err, scale = float(np.abs(got - ref).max()), float(np.abs(ref).max())
            say(f"  {name} at key {key}: max|err| {err:.3e} (max|ref| {scale:.3e})")
            assert err <= 1e-2 * scale
