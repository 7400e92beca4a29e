"""bsa_backward_noalloc against bsa_backward, through the C ABI.

The allocation-free entry point keeps Delta in the library's static per-GPU
workspace instead of a caller buffer and runs the same kernels, so its
gradients must equal bsa_backward's bit for bit.  Two calls in a row, the
second on a smaller problem (the workspace keeps the first call's contents),
plus the size limit, which is refused before anything is launched.
"""
import ctypes

import pytest
import torch

from block_sparse_flash_bsa_amd import bsattn
from block_sparse_flash_bsa_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsattn.lib()
    torch.cuda.set_device(0)


def noalloc(q, k, v, out, lse, do, p, dq, dk, dv):
    stream = torch.cuda.current_stream().cuda_stream
    return bsattn.lib().bsa_backward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                            lse.data_ptr(), do.data_ptr(), p.handle, dq.data_ptr(),
                                            dk.data_ptr(), dv.data_ptr(), ctypes.c_void_p(stream))


def case(w, lay):
    p = bsattn.plan(w.batch, w.heads, w.kv_heads, w.seq_len, w.head_dim, w.block, w.dtype, lay)
    q, k, v = (t.cuda() for t in wl.make_qkv(w, "cpu"))
    do = wl.make_dout(w, "cpu").cuda()
    out, lse = bsattn.forward(q, k, v, p)
    ref = bsattn.backward(q, k, v, out, lse, do, p)
    got = tuple(torch.full_like(t, float("nan")) for t in ref)
    st = noalloc(q, k, v, out, lse, do, p, *got)
    torch.cuda.synchronize()
    assert st == bsattn.OK, bsattn.lib().bsa_last_error().decode()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), f"{w.name}: {name} differs from bsa_backward"
    return p


def test_noalloc_equals_backward_two_calls():
    # First: a GQA problem whose dK/dV walks of the global keys are split.
    big = wl.WORKLOADS["gqa256k"].with_shape(name="noalloc-big", heads=4, kv_heads=1, seq_len=4096)
    lay = dict(causal=True, unit="tokens", window_left=255, window_right=0, global_keys=8,
               global_queries=0, bitmap=None)
    p = case(big, lay)
    work = p.work_kv()
    assert len(work[work >= 0]) > len(set(work[work >= 0].tolist())), "expected split columns"
    # Second, right after: a smaller problem (fewer rows than the workspace holds from the first).
    small = wl.small_variant(wl.WORKLOADS["window16k"], 1000, heads=2, kv_heads=2)
    case(small, wl.layout_of(small))
    # And the tiny fp32 workload through the same workspace.
    tiny = wl.WORKLOADS["tiny_f32"]
    case(tiny, wl.layout_of(tiny))


def test_noalloc_rejects_problems_beyond_the_workspace():
    # 1 x 65 x 262144 = 17,039,360 query rows > 16,777,216: refused on the host.
    lay = dict(causal=True, unit="tokens", window_left=127, window_right=0, global_keys=0,
               global_queries=0, bitmap=None)
    p = bsattn.plan(1, 65, 65, 262144, 128, 128, torch.bfloat16, lay)
    one = ctypes.c_void_p(1)           # never dereferenced: the size check comes first
    st = bsattn.lib().bsa_backward_noalloc(one, one, one, one, one, one, p.handle, one, one, one, None)
    assert st == bsattn.ERR_INVALID_ARGUMENT
    assert b"static workspace" in bsattn.lib().bsa_last_error()
