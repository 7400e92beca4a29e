"""CPU tests of the C-ABI library: symbol exports, the host planner against
the oracle's plan (bit-exact), the work order, and every error path that can
be reached without a GPU (bsa_plan_host makes no HIP call)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import oracle
from block_sparse_flash_bsa_amd import bsattn
from block_sparse_flash_bsa_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsattn.h")


def spec(causal, unit, w_left=-1, w_right=-1, gk=0, gq=0, bitmap=None):
    return dict(causal=causal, unit=unit, window_left=w_left, window_right=w_right,
                global_keys=gk, global_queries=gq, bitmap=bitmap)


def host_plan(w, layout=None, **kw):
    return bsattn.plan(w.batch, w.heads, w.kv_heads, w.seq_len, w.head_dim, w.block, w.dtype,
                       layout if layout is not None else wl.layout_of(w), host_only=True, **kw)


# ------------------------------------------------------------------ exports
def test_library_exports_every_declared_symbol():
    text = open(HEADER).read()
    declared = set(re.findall(r"\b(bsa_\w+)\s*\(", text))
    assert declared == set(bsattn.EXPORTS)
    L = ctypes.CDLL(bsattn.LIB_PATH)
    for name in declared:
        assert hasattr(L, name), name
    assert bsattn.lib().bsa_abi_version() == int(re.search(r"BSA_ABI_VERSION (\d+)", text).group(1))


def test_status_strings():
    L = bsattn.lib()
    assert L.bsa_status_string(0) == b"BSA_OK"
    assert L.bsa_status_string(2) == b"BSA_ERR_UNSUPPORTED"
    assert L.bsa_status_string(99) == b"BSA_ERR_UNKNOWN"


def test_struct_layouts_match_header():
    assert ctypes.sizeof(bsattn.Problem) == 40
    assert ctypes.sizeof(bsattn.Layout) == 56
    assert bsattn.Layout.bitmap.offset == 40


# --------------------------------------------------------- plan bit-exactness
def assert_same_plan(p, ref):
    assert len(ref) == p.info["layout_heads"]
    for lh, r in enumerate(ref):
        got = p.csr(lh)
        for key in ("row_ptr", "col_idx", "flags"):
            np.testing.assert_array_equal(got[key], r[key], err_msg=f"{key} head {lh}")


@pytest.mark.parametrize("name", ["tiny_f32", "window16k", "winglobal128k", "random32k", "gqa256k",
                                  "dense256k"])
def test_plan_matches_oracle_full_size(name):
    w = wl.WORKLOADS[name]
    lay = wl.layout_of(w)
    p = host_plan(w, lay)
    assert_same_plan(p, oracle.plan(lay, w.seq_len, w.block))


def test_plan_matches_oracle_bruteforce_random_specs():
    rng = np.random.default_rng(21)
    for _ in range(120):
        bs = 64 if rng.random() < 0.5 else 128
        nb = int(rng.integers(1, 9))
        N = bs * nb
        unit = "tokens" if rng.random() < 0.6 else "blocks"
        lim = N if unit == "tokens" else nb
        lay = spec(bool(rng.integers(0, 2)), unit, int(rng.integers(-1, lim + 2)),
                   int(rng.integers(-1, lim + 2)), int(rng.integers(0, lim + 1)),
                   int(rng.integers(0, lim + 1)))
        p = bsattn.plan(1, 2, 1, N, 64, bs, torch.float32, lay, host_only=True)
        assert_same_plan(p, oracle.plan(lay, N, bs, brute=True))


def test_plan_bitmap_per_head_and_causal_cut():
    rng = np.random.default_rng(22)
    nb, bs = 12, 64
    bm = (rng.random((3, nb, nb)) < 0.4).astype(np.uint8)
    bm[1, 5, :] = 0
    for causal in (False, True):
        lay = spec(causal, "blocks", bitmap=bm)
        p = bsattn.plan(2, 3, 3, nb * bs, 64, bs, torch.float32, lay, host_only=True)
        assert_same_plan(p, oracle.plan(lay, nb * bs, bs, brute=True))
        assert p.info["active_blocks"] == 2 * sum(len(x["col_idx"]) for x in oracle.plan(lay, nb * bs, bs))


def test_plan_info_counts():
    w = wl.WORKLOADS["gqa256k"]
    p = host_plan(w)
    i = p.info
    assert (i["nnz"], i["nnz_partial"], i["active_blocks"], i["max_row_entries"]) == (69071, 6079, 2210272, 34)
    q = np.arange(w.seq_len)
    from tests.closed_forms import count
    assert i["allowed_pairs"] == 32 * int(count("gqa256k", q, w.seq_len).sum())
    assert p.flops() == 4.0 * 128 * 128 * 128 * 2210272


# ---------------------------------------------------------------- work order
@pytest.mark.parametrize("schedule", [0, 1, 2, 3])
@pytest.mark.parametrize("name", ["winglobal128k", "random32k", "gqa256k"])
def test_work_order_is_a_permutation(name, schedule):
    w = wl.WORKLOADS[name]
    p = host_plan(w, schedule=schedule)
    work = p.work()
    items = work[work >= 0]
    n = w.batch * w.heads * w.num_blocks
    assert p.info["work_items"] == n and p.info["launch_slots"] == len(work)
    np.testing.assert_array_equal(np.sort(items), np.arange(n))


def test_xcd_schedule_runs_are_local_and_balanced():
    w = wl.WORKLOADS["gqa256k"]
    p = host_plan(w, schedule=bsattn.SCHEDULE_XCD)
    work = p.work()
    nb, H, group = w.num_blocks, w.heads, w.heads // w.kv_heads
    lens = np.diff(p.csr(0)["row_ptr"])
    costs = []
    for x in range(8):
        run = work[x::8]
        run = run[run >= 0]
        i, h, b = run % nb, (run // nb) % H, run // (nb * H)
        # within a run: KV head major, then batch entry, q-block, the heads of the group
        key = (((h // group) * w.batch + b) * nb + i) * group + h % group
        assert np.all(np.diff(key) > 0)
        costs.append(int((lens[i] + 1).sum()))
    assert max(costs) - min(costs) <= lens.max() + 1


def test_xcd_schedule_takes_bitmap_rows_longest_first():
    """For a bitmap layout each head's q-blocks run longest row first (ties in
    q-block order), so the workgroups running together sweep the key blocks
    at the same pace; heads stay contiguous per XCD run."""
    w = wl.WORKLOADS["random32k"]
    p = host_plan(w, schedule=bsattn.SCHEDULE_XCD)
    work = p.work()
    nb, H = w.num_blocks, w.heads
    lens = [np.diff(p.csr(h)["row_ptr"]) for h in range(H)]
    for x in range(8):
        run = work[x::8]
        run = run[run >= 0]
        i, h, b = run % nb, (run // nb) % H, run // (nb * H)
        grp = h * w.batch + b                  # head outer, batch entry next
        assert np.all(np.diff(grp) >= 0)
        for g in np.unique(grp):
            ii = i[grp == g]
            c = lens[g // w.batch][ii]
            assert np.all(np.diff(c) <= 0)
            ties = np.diff(c) == 0
            assert np.all(np.diff(ii)[ties] > 0)


def test_xcd_schedule_of_bitmaps_cuts_runs_by_item_count():
    """A bitmap plan's XCD runs hold equal item counts, so whole (head, batch
    entry) runs sit on one XCD when they divide evenly (the random 32K layout:
    32 runs over 8 XCDs, 4 each)."""
    w = wl.WORKLOADS["random32k"]
    p = host_plan(w, schedule=bsattn.SCHEDULE_XCD)
    work = p.work()
    nb, H = w.num_blocks, w.heads
    counts, owners = [], {}
    for x in range(8):
        run = work[x::8]
        run = run[run >= 0]
        counts.append(len(run))
        for g in np.unique((run // (nb * H)) + w.batch * ((run // nb) % H)):
            owners.setdefault(int(g), set()).add(x)
    assert max(counts) - min(counts) <= 1
    assert all(len(v) == 1 for v in owners.values()), "a (head, batch entry) run spans two XCDs"


def test_xcd_schedule_keeps_causal_bitmap_rows_ascending():
    """Under the causal cut a bitmap plan keeps each head's q-blocks in
    ascending order (a row's length grows with its q-block anyway)."""
    nb, H, B = 64, 4, 2
    rng = np.random.default_rng(4)
    bm = (rng.random((H, nb, nb)) < 0.3).astype(np.uint8)
    bm[:, np.arange(nb), np.arange(nb)] = 1
    lay = dict(causal=True, unit="blocks", window_left=-1, window_right=-1, global_keys=0, global_queries=0,
               bitmap=bm)
    p = bsattn.plan(B, H, H, nb * 128, 128, 128, torch.bfloat16, lay, host_only=True)
    work = p.work()
    for x in range(8):
        run = work[x::8]
        run = run[run >= 0]
        i, grp = run % nb, run // nb
        for g in np.unique(grp):
            assert np.all(np.diff(i[grp == g]) > 0)


def test_lpt_schedule_is_longest_first():
    w = wl.WORKLOADS["random32k"]
    p = host_plan(w, schedule=bsattn.SCHEDULE_LPT)
    work = p.work()
    nb, H = w.num_blocks, w.heads
    lens = [np.diff(p.csr(h)["row_ptr"]) for h in range(H)]
    c = np.array([lens[(it // nb) % H][it % nb] for it in work])
    assert np.all(np.diff(c) <= 0)


# ------------------------------------------------------------------- errors
def expect_error(status, **over):
    args = dict(batch=1, num_heads=4, num_kv_heads=2, seq_len=1024, head_dim=128, block_size=128,
                dtype=torch.bfloat16, layout=spec(True, "tokens", 100, 0))
    args.update(over)
    with pytest.raises(bsattn.BsaError) as ei:
        bsattn.plan(host_only=True, **args)
    assert ei.value.status == status, ei.value
    assert ei.value.detail  # bsa_last_error() explains it


def test_invalid_arguments():
    E = bsattn.ERR_INVALID_ARGUMENT
    expect_error(E, seq_len=-128)
    expect_error(E, num_heads=3, num_kv_heads=2)
    expect_error(E, num_kv_heads=0)
    expect_error(E, batch=-1)
    expect_error(E, scale=float("nan"))
    expect_error(E, scale=-1.0)
    expect_error(E, schedule=9)
    expect_error(E, layout=spec(True, "tokens", -2, 0))
    expect_error(E, layout=spec(True, "tokens", 4, 0, gk=-1))
    expect_error(E, layout=spec(True, "blocks", bitmap=np.ones((3, 8, 8), np.uint8)))
    with pytest.raises(bsattn.BsaError) as ei:
        pr = bsattn.make_problem(1, 4, 2, 1024, 128, 128, torch.bfloat16)
        lay, _ = bsattn.make_layout(spec(True, "tokens"))
        lay.causal = 2
        h = ctypes.c_void_p()
        bsattn._check(bsattn.lib().bsa_plan_host(ctypes.byref(pr), ctypes.byref(lay), ctypes.byref(h)))
    assert ei.value.status == E


def test_null_arguments():
    L = bsattn.lib()
    h = ctypes.c_void_p()
    assert L.bsa_plan_host(None, None, ctypes.byref(h)) == bsattn.ERR_INVALID_ARGUMENT
    pr = bsattn.make_problem(1, 1, 1, 128, 128, 128, torch.bfloat16)
    lay, _ = bsattn.make_layout(spec(False, "tokens"))
    assert L.bsa_plan_host(ctypes.byref(pr), ctypes.byref(lay), None) == bsattn.ERR_INVALID_ARGUMENT
    assert L.bsa_plan_get_info(None, None) == bsattn.ERR_INVALID_ARGUMENT
    assert L.bsa_plan_active_blocks(None) == -1
    L.bsa_plan_destroy(None)


def test_unsupported_shapes():
    U = bsattn.ERR_UNSUPPORTED
    expect_error(U, head_dim=96, seq_len=1152)
    expect_error(U, head_dim=64)                          # bf16 kernel is head_dim 128
    expect_error(U, block_size=64, seq_len=1024)          # bf16 kernel is block 128
    expect_error(U, dtype=torch.float32, head_dim=256)


def test_host_plan_cannot_run_forward():
    p = bsattn.plan(1, 1, 1, 128, 128, 128, torch.bfloat16, spec(False, "tokens"), host_only=True)
    st = bsattn.lib().bsa_forward(None, None, None, p.handle, None, None, None)
    assert st == bsattn.ERR_INVALID_ARGUMENT
    assert b"bsa_plan_host" in bsattn.lib().bsa_last_error()


def test_csr_head_out_of_range():
    p = bsattn.plan(1, 2, 2, 256, 128, 128, torch.bfloat16, spec(False, "tokens"), host_only=True)
    with pytest.raises(bsattn.BsaError):
        p.csr(1)


def test_empty_problems():
    p = bsattn.plan(0, 2, 2, 256, 128, 128, torch.bfloat16, spec(True, "tokens"), host_only=True)
    assert p.info["work_items"] == 0 and p.info["active_blocks"] == 0
    p = bsattn.plan(1, 2, 2, 0, 128, 128, torch.bfloat16, spec(True, "tokens"), host_only=True)
    assert p.info["num_blocks"] == 0 and p.info["nnz"] == 0 and p.work().size == 0


def test_empty_rows_have_no_entries():
    bm = np.zeros((1, 4, 4), np.uint8)
    bm[0, 1, 2] = 1
    p = bsattn.plan(1, 1, 1, 512, 128, 128, torch.bfloat16, spec(False, "blocks", bitmap=bm),
                    host_only=True)
    np.testing.assert_array_equal(p.csr(0)["row_ptr"], [0, 0, 1, 1, 1])
    # causal removes the only block above the diagonal
    p = bsattn.plan(1, 1, 1, 512, 128, 128, torch.bfloat16, spec(True, "blocks", bitmap=bm),
                    host_only=True)
    assert p.info["nnz"] == 0


BF16_TILE_KERNELS = [
    ("forward.hip", "_ZN3bsa12_GLOBAL__N_113fwd_bf16_d128ILb0EEEvNS0_9FwdParamsEPKi"),
    ("forward.hip", "_ZN3bsa12_GLOBAL__N_113fwd_bf16_d128ILb1EEEvNS0_9FwdParamsEPKi"),
    ("backward.hip", "_ZN3bsa12_GLOBAL__N_118bwd_dkdv_bf16_d128ILb0EEEvNS0_9BwdParamsE"),
    ("backward.hip", "_ZN3bsa12_GLOBAL__N_118bwd_dkdv_bf16_d128ILb1EEEvNS0_9BwdParamsE"),
    ("backward.hip", "_ZN3bsa12_GLOBAL__N_116bwd_dq_bf16_d128ILb0EEEvNS0_9BwdParamsE"),
    ("backward.hip", "_ZN3bsa12_GLOBAL__N_116bwd_dq_bf16_d128ILb1EEEvNS0_9BwdParamsE")]

_ASM = {}


def _device_asm(source):
    """gfx950 assembly of one HIP source, compiled once per test session
    (hipcc cross-compiles without a GPU)."""
    if source not in _ASM:
        import subprocess
        import tempfile
        from block_sparse_flash_bsa_amd import build as bld
        src = os.path.join(ROOT, "block_sparse_flash_bsa_amd", "csrc", source)
        out = os.path.join(tempfile.mkdtemp(prefix="bsa_asm_"), source + ".s")
        cmd = [bld.hipcc(), "-x", "hip", *bld.HIP_FLAGS, "-O3", "-std=c++17", "--cuda-device-only", "-S",
               "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "block_sparse_flash_bsa_amd", "csrc"),
               src, "-o", out]
        subprocess.run(cmd, check=True, capture_output=True)
        with open(out) as f:
            _ASM[source] = f.read()
    return _ASM[source]


@pytest.mark.parametrize("source,symbol", BF16_TILE_KERNELS)
def test_bf16_kernel_m0_only_set_for_lds_loads(source, symbol):
    """The bf16 forward and dK/dV kernels write M0 in inline assembly right
    before each HBM->LDS load; the compiler treats M0 as reserved and does not
    honour it as a clobber, so its own code must never rely on M0 across those
    loads.  Check on the kernel's gfx950 assembly that every M0 access in it
    is one of those load sequences."""
    asm = _device_asm(source)
    start = asm.index(symbol + ":")
    body = [l.strip() for l in asm[start:asm.index(".Lfunc_end", start)].splitlines()]
    body = [l for l in body if l and not l.startswith(";")]
    uses = [k for k, l in enumerate(body) if re.search(r"\bm0\b", l)]
    assert uses, "expected the HBM->LDS load sequences"
    for k in uses:
        assert body[k].startswith("s_mov_b32 m0, s"), body[k]
        assert body[k + 1].startswith("s_nop") and body[k + 2].startswith("global_load_lds_dwordx4"), body[k:k + 3]


@pytest.mark.parametrize("source,symbol", BF16_TILE_KERNELS)
def test_bf16_kernel_fits_two_workgroups_per_cu(source, symbol):
    """Every bf16 tile kernel runs two 4-wave workgroups per CU, so that each
    SIMD interleaves two independent waves: at most half of the CU's 160 KB
    of LDS per workgroup and at most 256 registers (arithmetic plus
    accumulation) per wave, from the kernel metadata of its gfx950 build.
    The forward kernels and the whole-block backward kernels (the benchmark
    paths) spill no vector registers and use no scratch memory (a few scalar
    registers may be parked in vector-register lanes)."""
    import yaml
    asm = _device_asm(source)
    meta = asm[asm.index(".amdgpu_metadata") + len(".amdgpu_metadata"):asm.index(".end_amdgpu_metadata")]
    meta = meta[meta.index("---"):meta.rindex("...") + 3]        # the YAML document
    kernels = {k[".name"]: k for k in yaml.safe_load(meta)["amdhsa.kernels"]}
    k = kernels[symbol]
    assert k[".max_flat_workgroup_size"] == 256
    assert k[".group_segment_fixed_size"] <= 160 * 1024 // 2, k[".group_segment_fixed_size"]
    assert k[".vgpr_count"] + k.get(".agpr_count", 0) <= 256, (k[".vgpr_count"], k.get(".agpr_count"))
    if source == "forward.hip" or "ILb0E" in symbol:
        assert k[".vgpr_spill_count"] == 0 and k[".private_segment_fixed_size"] == 0


# ------------------------------------------------------------ dynamic plans
def test_dynamic_plan_argument_errors():
    L = bsattn.lib()
    pr = bsattn.make_problem(1, 2, 2, 1024, 64, 64, torch.float32)
    h = ctypes.c_void_p()

    def lay(**kw):
        x = bsattn.Layout()
        x.causal, x.unit = kw.get("causal", 0), bsattn.UNIT_BLOCKS
        x.window_left, x.window_right = kw.get("wl", -1), -1
        x.global_keys, x.global_queries = kw.get("gk", 0), 0
        x.bitmap_heads = kw.get("heads", 1)
        bm = kw.get("bitmap")
        x.bitmap = bm.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)) if bm is not None else None
        return x

    bm = np.ones((1, 16, 16), np.uint8)
    for bad in (lay(bitmap=bm), lay(wl=3), lay(gk=1), lay(heads=3), lay(causal=2)):
        assert L.bsa_plan_dynamic(ctypes.byref(pr), ctypes.byref(bad), ctypes.byref(h)) == \
            bsattn.ERR_INVALID_ARGUMENT
        assert bsattn.lib().bsa_last_error()
    assert L.bsa_plan_dynamic(ctypes.byref(pr), ctypes.byref(lay()), None) == bsattn.ERR_INVALID_ARGUMENT
    # A sequence length the block does not divide passes the argument checks
    # (a shorter last block, as for static plans): with no GPU the call gets as
    # far as the device query.
    ragged = bsattn.make_problem(1, 2, 2, 1000, 64, 64, torch.float32)
    st = L.bsa_plan_dynamic(ctypes.byref(ragged), ctypes.byref(lay()), ctypes.byref(h))
    if st == bsattn.OK:
        L.bsa_plan_destroy(h)
    else:
        assert st == bsattn.ERR_DEVICE, bsattn.lib().bsa_last_error()
    # Up to 2^31 - 1 possible entries (one int32 offset space).
    big = bsattn.make_problem(1, 32, 32, 16384 * 64, 64, 64, torch.float32)
    assert L.bsa_plan_dynamic(ctypes.byref(big), ctypes.byref(lay(heads=32)), ctypes.byref(h)) == \
        bsattn.ERR_INVALID_ARGUMENT
    # A static (host) plan is neither updatable nor readable as a dynamic one.
    hp = bsattn.plan(1, 2, 2, 1024, 64, 64, torch.float32, spec(False, "blocks", 1, 1), host_only=True)
    assert L.bsa_plan_set_bitmap(hp.handle, bm.ctypes.data, None, None) == bsattn.ERR_INVALID_ARGUMENT
    rp = np.zeros(17, np.int32)
    n = ctypes.c_int64()
    assert L.bsa_plan_read_csr(hp.handle, 0, rp.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), None, None,
                               0, ctypes.byref(n)) == bsattn.ERR_INVALID_ARGUMENT
    assert L.bsa_plan_set_bitmap(None, bm.ctypes.data, None, None) == bsattn.ERR_INVALID_ARGUMENT


# ------------------------------------------------ transposed CSR (backward)
def transpose_of(ref, nb):
    """Per k-block lists of (q-block, flag) from the oracle's per-q-block lists."""
    cols = [[] for _ in range(nb)]
    for i in range(nb):
        for e in range(ref["row_ptr"][i], ref["row_ptr"][i + 1]):
            cols[ref["col_idx"][e]].append((i, ref["flags"][e]))
    col_ptr = np.cumsum([0] + [len(c) for c in cols]).astype(np.int32)
    row_idx = np.array([i for c in cols for i, _ in c], np.int32)
    flags = np.array([f for c in cols for _, f in c], np.uint8)
    return col_ptr, row_idx, flags


@pytest.mark.parametrize("name", ["tiny_f32", "window16k", "winglobal128k", "random32k", "gqa256k"])
def test_transposed_csr_matches_oracle_plan(name):
    w = wl.WORKLOADS[name]
    lay = wl.layout_of(w)
    p = host_plan(w, lay)
    ref = oracle.plan(lay, w.seq_len, w.block)
    for lh, r in enumerate(ref):
        got = p.csr_transposed(lh)
        cp, ri, fl = transpose_of(r, w.num_blocks)
        np.testing.assert_array_equal(got["col_ptr"], cp)
        np.testing.assert_array_equal(got["row_idx"], ri)
        np.testing.assert_array_equal(got["flags"], fl)


@pytest.mark.parametrize("name", ["winglobal128k", "random32k", "gqa256k"])
def test_kv_work_order_is_a_permutation(name):
    w = wl.WORKLOADS[name]
    p = host_plan(w)
    work = p.work_kv()
    items = work[work >= 0]
    # every item is covered; only long walks (global-key columns) take several slots
    np.testing.assert_array_equal(np.unique(items), np.arange(w.batch * w.kv_heads * w.num_blocks))
    assert len(items) - len(np.unique(items)) < 0.05 * len(items)
    # slot s runs on XCD s % 8: each XCD's items form one contiguous, ordered
    # run of the locality order (KV head, batch entry, k-block)
    # (for a bitmap, each (KV head, batch entry)'s k-blocks go longest walk first)
    nb, B, Hkv, group = w.num_blocks, w.batch, w.kv_heads, w.heads // w.kv_heads
    lay = wl.layout_of(w)
    if lay.get("bitmap") is not None:
        col = p.csr_transposed
        walk = np.zeros((B * Hkv * nb,), dtype=np.int64)
        for it in range(len(walk)):
            j, hk = it % nb, (it // nb) % Hkv
            walk[it] = sum(int(np.diff(col(h)["col_ptr"])[j]) for h in range(hk * group, (hk + 1) * group))
    seen = []
    for x in range(8):
        run = work[x::8]
        run = run[run >= 0]
        j, hk, b = run % nb, (run // nb) % Hkv, run // (nb * Hkv)
        grp = hk * B + b
        assert np.all(np.diff(grp) >= 0)
        if lay.get("bitmap") is None:
            key = grp * nb + j
            assert np.all(np.diff(key) >= 0) and np.all(np.diff(key) <= 1)
        else:
            for g in np.unique(grp):
                wk = walk[run[grp == g]]
                assert np.all(np.diff(wk) <= 0), "k-blocks of a group must go longest walk first"
        seen.append(run)


def test_transposed_csr_errors():
    p = bsattn.plan(1, 2, 2, 256, 128, 128, torch.bfloat16, spec(False, "tokens"), host_only=True)
    with pytest.raises(bsattn.BsaError):
        p.csr_transposed(2)


def test_backward_rejects_host_only_plan():
    p = bsattn.plan(1, 1, 1, 128, 128, 128, torch.bfloat16, spec(False, "tokens"), host_only=True)
    st = bsattn.lib().bsa_backward(1, 1, 1, 1, 1, 1, p.handle, 1, 1, 1, 1, None)
    assert st == bsattn.ERR_INVALID_ARGUMENT
    assert b"bsa_plan_host" in bsattn.lib().bsa_last_error()


def test_backward_operand_offset_identities():
    """The backward kernels address LDS operands as one per-lane base XOR-ed
    with a per-operand constant.  The identities behind that, written out for
    every lane: the tile layout (chunk c of row r at c ^ (4 (r & 3) +
    ((r >> 2) & 3))), the row layout (c ^ (r & 15)) and the transposing reads
    (lane 4 r4 + c4 of 16-lane group g reads row 4 hf + r4 + 8 s, columns
    32 dt + 16 (g & 1) + 4 c4 .. +3, in the tile layout)."""
    def tile_swz(r):
        return 4 * (r & 3) + ((r >> 2) & 3)

    def tile_off(r, c):
        return r * 256 + 16 * (c ^ tile_swz(r))

    def rows_off(r, c):
        return r * 256 + 16 * (c ^ (r & 15))

    def col_read(lane, dt, s):
        hf, r4, c4, gp = lane >> 5, (lane & 15) >> 2, lane & 3, (lane >> 4) & 1
        row = 4 * hf + r4 + 8 * s
        return tile_off(row, 4 * dt + 2 * gp + (c4 >> 1)) + 8 * (c4 & 1)

    for w in range(4):
        for lane in range(64):
            r32, hf = lane & 31, lane >> 5
            r4, c4, gp = (lane & 15) >> 2, lane & 3, (lane >> 4) & 1
            f = tile_swz(r32)
            tile_rows_base = r32 * 256 + 16 * (hf ^ (f & 1)) + 16 * (f & 14)
            rows_rows_base = (32 * w + r32) * 256 + 16 * (hf ^ (r32 & 1)) + 16 * (r32 & 14)
            for cc in range(8):
                assert tile_rows_base ^ (32 * cc) == tile_off(r32, 2 * cc + hf)
                assert rows_rows_base ^ (32 * cc) == rows_off(32 * w + r32, 2 * cc + hf)
            for s in (0, 1):
                cols_base = ((4 * hf + r4 + 8 * s) * 256 + 16 * ((2 * gp + (c4 >> 1)) ^ (hf + 2 * s))
                             + 8 * (c4 & 1) + 64 * r4)
                for dt in range(4):
                    assert cols_base ^ (64 * dt) == col_read(lane, dt, s)
                for kc in range(8):         # 16 kc more rows keep the row's swizzle
                    assert tile_swz(4 * hf + r4 + 8 * s + 16 * kc) == tile_swz(4 * hf + r4 + 8 * s)


# -------------------------------------------------- ragged lengths (host plans)
RAGGED_LAYOUTS = [
    dict(causal=True, unit="tokens", window_left=300, window_right=0, global_keys=5, global_queries=0, bitmap=None),
    dict(causal=False, unit="tokens", window_left=77, window_right=200, global_keys=0, global_queries=3, bitmap=None),
    dict(causal=True, unit="blocks", window_left=2, window_right=0, global_keys=1, global_queries=1, bitmap=None),
    dict(causal=False, unit="blocks", window_left=1, window_right=1, global_keys=0, global_queries=0, bitmap=None),
]


@pytest.mark.parametrize("N", [1, 127, 129, 1000, 4097])
@pytest.mark.parametrize("li", range(len(RAGGED_LAYOUTS)))
def test_ragged_plan_matches_oracle(N, li):
    lay = RAGGED_LAYOUTS[li]
    for dtype, D, bs in ((torch.bfloat16, 128, 128), (torch.float32, 64, 64)):
        p = bsattn.plan(1, 2, 1, N, D, bs, dtype, lay, host_only=True)
        assert p.info["num_blocks"] == -(-N // bs)
        assert_same_plan(p, oracle.plan(lay, N, bs, brute=N <= 1024))
        if N <= 1000:
            assert p.info["allowed_pairs"] == 2 * sum(oracle.allowed_count(lay, N, bs, 0, q) for q in range(N))


def test_ragged_bitmap_plan_matches_oracle():
    N, bs = 1000, 128
    nb = -(-N // bs)
    bm = (np.random.default_rng(31).random((2, nb, nb)) < 0.4).astype(np.uint8)
    for causal in (False, True):
        lay = spec(causal, "blocks", bitmap=bm)
        p = bsattn.plan(1, 2, 2, N, 128, bs, torch.bfloat16, lay, host_only=True)
        assert_same_plan(p, oracle.plan(lay, N, bs, brute=True))
        total = sum(oracle.allowed_count(lay, N, bs, h, q) for h in range(2) for q in range(N))
        assert p.info["allowed_pairs"] == total


def test_probe_library_exports_its_header():
    """The benchmark's MFMA-rate probe (include/bsattn_probe.h) is built into a
    library of its own and exports exactly what its header declares."""
    from block_sparse_flash_bsa_amd import build as bld
    text = open(os.path.join(ROOT, "include", "bsattn_probe.h")).read()
    declared = set(re.findall(r"\b(bsa_\w+)\s*\(", text))
    assert declared == {"bsa_probe_mfma", "bsa_probe_mfma_flops"}
    L = ctypes.CDLL(bld.PROBE_LIB)
    for name in declared:
        assert hasattr(L, name), name
    L.bsa_probe_mfma_flops.argtypes = [ctypes.c_int64, ctypes.c_int32]
    L.bsa_probe_mfma_flops.restype = ctypes.c_double
    assert L.bsa_probe_mfma_flops(10, 3) == 3 * 4 * 4 * 10 * 32768
    L.bsa_probe_mfma.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    assert L.bsa_probe_mfma(0, 1, None, None) == 1          # argument errors return before any HIP call


def test_lse_merge_argument_errors():
    """Errors bsa_lse_merge reports before touching the device; zero rows is
    a no-op."""
    L = bsattn.lib()
    one = ctypes.c_void_p(1)
    for args, what in (((0, 10, 128, bsattn.BF16), b"parts"), ((2, -1, 128, bsattn.BF16), b"rows"),
                       ((2, 10, 128, 7), b"dtype"), ((2, 10, 4, bsattn.BF16), b"head_dim"),
                       ((2, 10, 2, bsattn.F32), b"head_dim")):
        assert L.bsa_lse_merge(*args, one, one, one, one, None) == bsattn.ERR_INVALID_ARGUMENT
        assert what in L.bsa_last_error()
    assert L.bsa_lse_merge(2, 10, 128, bsattn.BF16, None, one, one, one, None) == bsattn.ERR_INVALID_ARGUMENT
    assert L.bsa_lse_merge(2, 0, 128, bsattn.BF16, None, None, None, None, None) == bsattn.OK
    # host memory is refused (or, with no GPU, the device query fails first)
    host = np.zeros(4096, np.float32)
    st = L.bsa_lse_merge(1, 4, 128, bsattn.F32, host.ctypes.data, host.ctypes.data, host.ctypes.data,
                         host.ctypes.data, None)
    assert st in (bsattn.ERR_INVALID_ARGUMENT, bsattn.ERR_DEVICE)


def test_varlen_and_transposed_read_argument_errors():
    """Errors the variable-length entry points and the transposed-list read
    report before touching the device."""
    L = bsattn.lib()
    one = ctypes.c_void_p(1)
    assert L.bsa_forward_varlen(one, one, one, None, one, one, one, None) == bsattn.ERR_INVALID_ARGUMENT
    assert L.bsa_backward_varlen(one, one, one, one, one, one, None, one, one, one, one, one, None) == \
        bsattn.ERR_INVALID_ARGUMENT
    # Both dtypes have variable-length kernels; a NULL seq_lens is refused first.
    f32 = bsattn.plan(1, 2, 2, 1024, 64, 64, torch.float32, spec(False, "blocks", 1, 1), host_only=True)
    bf = bsattn.plan(2, 2, 2, 1024, 128, 128, torch.bfloat16, spec(True, "tokens", 300), host_only=True)
    for pl in (f32, bf):
        assert L.bsa_forward_varlen(one, one, one, pl.handle, None, one, one, None) == bsattn.ERR_INVALID_ARGUMENT
        assert b"seq_lens" in L.bsa_last_error()
        assert L.bsa_backward_varlen(one, one, one, one, one, one, pl.handle, None, one, one, one, one, None) == \
            bsattn.ERR_INVALID_ARGUMENT
        assert b"seq_lens" in L.bsa_last_error()
    # The transposed lists of a static plan are read with bsa_plan_csr_transposed, not from the device.
    cp = np.zeros(9, np.int32)
    n = ctypes.c_int64()
    i32 = ctypes.POINTER(ctypes.c_int32)
    assert L.bsa_plan_read_csr_transposed(bf.handle, 0, cp.ctypes.data_as(i32), None, None, 0,
                                          ctypes.byref(n)) == bsattn.ERR_INVALID_ARGUMENT
    assert L.bsa_plan_read_csr_transposed(None, 0, cp.ctypes.data_as(i32), None, None, 0,
                                          ctypes.byref(n)) == bsattn.ERR_INVALID_ARGUMENT


def test_xcd_runs_hold_every_batch_entry():
    """The XCD-local orders put KV heads outermost and batch entries next, so
    each XCD's run holds all batch entries (variable-length batches stay
    balanced across XCDs)."""
    w = wl.WORKLOADS["gqa256k"].with_shape(name="b4", batch=4, heads=16, kv_heads=8, seq_len=8192)
    p = host_plan(w, schedule=bsattn.SCHEDULE_XCD)
    nb = w.num_blocks
    for work, per_b in ((p.work(), nb * w.heads), (p.work_kv(), nb * w.kv_heads)):
        for x in range(8):
            run = work[x::8]
            run = run[run >= 0]
            assert set((run // per_b).tolist()) == set(range(w.batch)), f"XCD {x}"


# ------------------------------------------------ binding argument checks
class _CudaStandIn:
    """Duck-typed stand-in for a CUDA tensor (no GPU here): it only answers
    the attributes the binding inspects before calling into the library."""

    def __init__(self, shape, dtype, contiguous=True):
        self.shape, self.dtype, self._c = tuple(shape), dtype, contiguous
        self.is_cuda = True
        self.device = torch.device("cuda", 0)

    def is_contiguous(self):
        return self._c

    def data_ptr(self):
        raise AssertionError("the binding reached the library call")


def test_binding_rejects_bad_out_and_lse_before_any_launch():
    w = wl.small_variant(wl.WORKLOADS["window16k"], 1024, heads=2, kv_heads=2)
    p = host_plan(w)
    B, H, N, D = w.batch, w.heads, w.seq_len, w.head_dim
    bf = torch.bfloat16
    q = _CudaStandIn((B, H, N, D), bf)
    k = _CudaStandIn((B, H, N, D), bf)
    v = _CudaStandIn((B, H, N, D), bf)
    lens = _CudaStandIn((B,), torch.int32)
    good_out = _CudaStandIn((B, H, N, D), bf)
    good_lse = _CudaStandIn((B, H, N), torch.float32)
    bad = {
        "cpu out": (torch.empty((B, H, N, D), dtype=bf), good_lse),
        "cpu lse": (good_out, torch.empty((B, H, N), dtype=torch.float32)),
        "strided out": (_CudaStandIn((B, H, N, D), bf, contiguous=False), good_lse),
        "strided lse": (good_out, _CudaStandIn((B, H, N), torch.float32, contiguous=False)),
        "fp32 out": (_CudaStandIn((B, H, N, D), torch.float32), good_lse),
    }
    for what, (o, l) in bad.items():
        with pytest.raises(ValueError):
            bsattn.forward_varlen(q, k, v, p, lens, o, l)
        with pytest.raises(ValueError):
            bsattn.forward(q, k, v, p, o, l)
    with pytest.raises(ValueError):       # lengths in host memory
        bsattn.forward_varlen(q, k, v, p, torch.zeros(B, dtype=torch.int32), good_out, good_lse)
    with pytest.raises(ValueError):       # q in host memory
        bsattn.forward(torch.empty((B, H, N, D), dtype=bf), k, v, p, good_out, good_lse)


def test_read_work_argument_errors():
    """bsa_plan_read_work refuses NULL arguments and host-only plans before any
    device call."""
    L = bsattn.lib()
    hp = bsattn.plan(1, 2, 2, 1024, 128, 128, torch.bfloat16, spec(True, "tokens", 300), host_only=True)
    w = np.zeros(64, np.int32)
    n = ctypes.c_int64()
    assert L.bsa_plan_read_work(None, w.ctypes.data, 64, ctypes.byref(n)) == bsattn.ERR_INVALID_ARGUMENT
    assert L.bsa_plan_read_work(hp.handle, w.ctypes.data, 64, None) == bsattn.ERR_INVALID_ARGUMENT
    assert L.bsa_plan_read_work(hp.handle, None, 64, ctypes.byref(n)) == bsattn.ERR_INVALID_ARGUMENT
    assert L.bsa_plan_read_work(hp.handle, w.ctypes.data, 64, ctypes.byref(n)) == bsattn.ERR_INVALID_ARGUMENT
    assert b"bsa_plan_host" in L.bsa_last_error()
