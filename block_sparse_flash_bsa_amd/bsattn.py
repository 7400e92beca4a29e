"""ctypes binding over libbsattn (include/bsattn.h).

Argument marshalling only: every step of the forward and backward runs in
the library's HIP kernels; PyTorch provides device memory and the current
stream.

    p = plan(batch=1, num_heads=32, num_kv_heads=32, seq_len=16384, head_dim=128,
             block_size=128, dtype=torch.bfloat16,
             layout=dict(causal=True, unit="tokens", window_left=511, window_right=0,
                         global_keys=0, global_queries=0, bitmap=None))
    out, lse = forward(q, k, v, p)
    dq, dk, dv = backward(q, k, v, out, lse, dout, p)

The library is loaded on first use; if it has not been built the call raises
(there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_uint8, c_void_p
from typing import Dict, Optional

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbsattn.so")

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_OUT_OF_MEMORY, ERR_DEVICE = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
UNIT_TOKENS, UNIT_BLOCKS = 0, 1
SCHEDULE_DEFAULT, SCHEDULE_XCD, SCHEDULE_LPT, SCHEDULE_ROWMAJOR = 0, 1, 2, 3

# Every entry point include/bsattn.h declares.
EXPORTS = ("bsa_plan", "bsa_plan_host", "bsa_plan_destroy", "bsa_plan_csr", "bsa_plan_get_info",
           "bsa_plan_work", "bsa_plan_active_blocks", "bsa_plan_dynamic", "bsa_plan_set_bitmap",
           "bsa_plan_read_csr", "bsa_plan_read_csr_transposed", "bsa_forward",
           "bsa_plan_csr_transposed", "bsa_plan_work_kv", "bsa_plan_read_work", "bsa_plan_read_work_kv",
           "bsa_backward", "bsa_backward_noalloc", "bsa_forward_varlen", "bsa_backward_varlen", "bsa_lse_merge",
           "bsa_status_string", "bsa_last_error",
           "bsa_abi_version")


class Problem(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("num_heads", c_int32), ("num_kv_heads", c_int32),
                ("head_dim", c_int32), ("seq_len", c_int64), ("block_size", c_int32),
                ("dtype", c_int32), ("scale", c_float), ("schedule", c_int32)]


class Layout(ctypes.Structure):
    _fields_ = [("causal", c_int32), ("unit", c_int32), ("window_left", c_int64),
                ("window_right", c_int64), ("global_keys", c_int64), ("global_queries", c_int64),
                ("bitmap", POINTER(c_uint8)), ("bitmap_heads", c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("layout_heads", c_int32), ("num_blocks", c_int32), ("nnz", c_int64),
                ("nnz_partial", c_int64), ("active_blocks", c_int64), ("allowed_pairs", c_int64),
                ("work_items", c_int64), ("launch_slots", c_int64), ("max_row_entries", c_int32),
                ("on_device", c_int32)]


class BsaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.detail = detail
        super().__init__(f"{_status_name(status)}: {detail}")


_lib = None


def lib():
    """Load libbsattn.so once; raise if it is missing (no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libbsattn.so is not built ({LIB_PATH}); run "
                           "`python -m block_sparse_flash_bsa_amd.build` or __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    P = c_void_p
    L.bsa_plan.argtypes = [POINTER(Problem), POINTER(Layout), POINTER(P)]
    L.bsa_plan_host.argtypes = [POINTER(Problem), POINTER(Layout), POINTER(P)]
    L.bsa_plan_destroy.argtypes = [P]
    L.bsa_plan_destroy.restype = None
    L.bsa_plan_csr.argtypes = [P, c_int32, POINTER(POINTER(c_int32)), POINTER(POINTER(c_int32)),
                               POINTER(POINTER(c_uint8)), POINTER(c_int64)]
    L.bsa_plan_get_info.argtypes = [P, POINTER(PlanInfo)]
    L.bsa_plan_work.argtypes = [P, POINTER(POINTER(c_int32)), POINTER(c_int64)]
    L.bsa_plan_active_blocks.argtypes = [P]
    L.bsa_plan_active_blocks.restype = c_int64
    L.bsa_plan_dynamic.argtypes = [POINTER(Problem), POINTER(Layout), POINTER(P)]
    L.bsa_plan_set_bitmap.argtypes = [P, c_void_p, c_void_p, c_void_p]
    L.bsa_plan_read_csr.argtypes = [P, c_int32, POINTER(c_int32), POINTER(c_int32), POINTER(c_uint8),
                                    c_int64, POINTER(c_int64)]
    L.bsa_plan_read_csr_transposed.argtypes = L.bsa_plan_read_csr.argtypes
    L.bsa_forward.argtypes = [c_void_p, c_void_p, c_void_p, P, c_void_p, c_void_p, c_void_p]
    L.bsa_plan_csr_transposed.argtypes = [P, c_int32, POINTER(POINTER(c_int32)), POINTER(POINTER(c_int32)),
                                          POINTER(POINTER(c_uint8)), POINTER(c_int64)]
    L.bsa_plan_work_kv.argtypes = [P, POINTER(POINTER(c_int32)), POINTER(c_int64)]
    L.bsa_plan_read_work.argtypes = [P, c_void_p, c_int64, POINTER(c_int64)]
    L.bsa_plan_read_work_kv.argtypes = [P, c_void_p, c_int64, POINTER(c_int64), POINTER(c_int64)]
    L.bsa_backward.argtypes = [c_void_p] * 6 + [P] + [c_void_p] * 5
    L.bsa_backward_noalloc.argtypes = [c_void_p] * 6 + [P] + [c_void_p] * 4
    L.bsa_forward_varlen.argtypes = [c_void_p, c_void_p, c_void_p, P, c_void_p, c_void_p, c_void_p, c_void_p]
    L.bsa_backward_varlen.argtypes = [c_void_p] * 6 + [P] + [c_void_p] * 6
    L.bsa_lse_merge.argtypes = [c_int32, c_int64, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                c_void_p]
    L.bsa_status_string.argtypes = [c_int32]
    L.bsa_status_string.restype = c_char_p
    L.bsa_last_error.argtypes = []
    L.bsa_last_error.restype = c_char_p
    L.bsa_abi_version.restype = c_int32
    for name in ("bsa_plan", "bsa_plan_host", "bsa_plan_csr", "bsa_plan_get_info", "bsa_plan_work",
                 "bsa_plan_dynamic", "bsa_plan_set_bitmap", "bsa_plan_read_csr", "bsa_plan_read_csr_transposed",
                 "bsa_forward", "bsa_plan_csr_transposed", "bsa_plan_work_kv", "bsa_plan_read_work", "bsa_plan_read_work_kv", "bsa_backward", "bsa_forward_varlen",
                 "bsa_backward_varlen", "bsa_lse_merge"):
        getattr(L, name).restype = c_int32
    _lib = L
    return L


def _status_name(status: int) -> str:
    try:
        return lib().bsa_status_string(status).decode()
    except Exception:  # pragma: no cover - library not loadable
        return f"status {status}"


def _check(status: int):
    if status != OK:
        raise BsaError(status, lib().bsa_last_error().decode())


def _dtype_code(dtype) -> int:
    import torch
    if dtype in (torch.bfloat16, "bf16", BF16):
        return BF16
    if dtype in (torch.float32, "f32", F32):
        return F32
    raise ValueError(f"unsupported dtype {dtype}")


def make_layout(layout: Dict):
    """Layout dict -> (ctypes Layout, keep-alive bitmap array)."""
    bm = layout.get("bitmap")
    arr = None
    lay = Layout()
    lay.causal = 1 if layout["causal"] else 0
    lay.unit = {"tokens": UNIT_TOKENS, "blocks": UNIT_BLOCKS}[layout["unit"]]
    lay.window_left = int(layout["window_left"])
    lay.window_right = int(layout["window_right"])
    lay.global_keys = int(layout["global_keys"])
    lay.global_queries = int(layout["global_queries"])
    if bm is not None:
        if hasattr(bm, "numpy"):
            bm = bm.detach().cpu().numpy()
        arr = np.ascontiguousarray(np.asarray(bm) != 0, dtype=np.uint8)
        if arr.ndim != 3:
            raise ValueError("bitmap must have shape [bitmap_heads, nb, nb]")
        lay.bitmap = arr.ctypes.data_as(POINTER(c_uint8))
        lay.bitmap_heads = arr.shape[0]
    else:
        lay.bitmap = None
        lay.bitmap_heads = 0
    return lay, arr


class Plan:
    """Owns a bsa_plan_t; freed on close() or garbage collection."""

    def __init__(self, handle: int, problem: Problem, host_only: bool):
        self._h = c_void_p(handle)
        self.problem = problem
        self.host_only = host_only
        info = PlanInfo()
        _check(lib().bsa_plan_get_info(self._h, ctypes.byref(info)))
        self.info = {name: getattr(info, name) for name, _ in PlanInfo._fields_}

    @property
    def handle(self):
        if self._h is None or not self._h.value:
            raise RuntimeError("plan has been destroyed")
        return self._h

    def csr(self, layout_head: int = 0):
        rp, ci, fl = POINTER(c_int32)(), POINTER(c_int32)(), POINTER(c_uint8)()
        nnz = c_int64()
        _check(lib().bsa_plan_csr(self.handle, layout_head, ctypes.byref(rp), ctypes.byref(ci),
                                  ctypes.byref(fl), ctypes.byref(nnz)))
        nb = self.info["num_blocks"]
        n = nnz.value
        return {"row_ptr": np.ctypeslib.as_array(rp, (nb + 1,)).copy(),
                "col_idx": np.ctypeslib.as_array(ci, (n,)).copy() if n else np.zeros(0, np.int32),
                "flags": np.ctypeslib.as_array(fl, (n,)).copy() if n else np.zeros(0, np.uint8)}

    def set_bitmap(self, bitmap, nnz=None):
        """bsa_plan_set_bitmap on torch.cuda.current_stream(): bitmap is a contiguous uint8
        CUDA tensor [layout_heads, nb, nb]; nnz, if given, a one-element int64 CUDA tensor
        that receives the entry count."""
        import torch
        nb, lh = self.info["num_blocks"], self.info["layout_heads"]
        if (not bitmap.is_cuda or bitmap.dtype != torch.uint8 or not bitmap.is_contiguous()
                or tuple(bitmap.shape) != (lh, nb, nb)):
            raise ValueError(f"bitmap must be a contiguous uint8 CUDA tensor of shape {(lh, nb, nb)}")
        if nnz is not None and (not nnz.is_cuda or nnz.dtype != torch.int64 or nnz.numel() != 1):
            raise ValueError("nnz must be a one-element int64 CUDA tensor")
        with torch.cuda.device(bitmap.device):
            stream = torch.cuda.current_stream().cuda_stream
            _check(lib().bsa_plan_set_bitmap(self.handle, bitmap.data_ptr(),
                                             nnz.data_ptr() if nnz is not None else None,
                                             c_void_p(stream)))

    def read_csr(self, layout_head: int = 0):
        """bsa_plan_read_csr: the device CSR of a dynamic plan, in the format of csr()."""
        rp, ci, fl = self._read_device(lib().bsa_plan_read_csr, layout_head)
        return {"row_ptr": rp, "col_idx": ci, "flags": fl}

    def read_csr_transposed(self, layout_head: int = 0):
        """bsa_plan_read_csr_transposed: the device-built transposed lists of a
        dynamic plan, in the format of csr_transposed()."""
        cp, ri, fl = self._read_device(lib().bsa_plan_read_csr_transposed, layout_head)
        return {"col_ptr": cp, "row_idx": ri, "flags": fl}

    def _read_device(self, fn, layout_head):
        nb = self.info["num_blocks"]
        ptr = np.zeros(nb + 1, np.int32)
        n = c_int64()
        cap = nb * nb
        idx = np.zeros(max(cap, 1), np.int32)
        fl = np.zeros(max(cap, 1), np.uint8)
        _check(fn(self.handle, layout_head, ptr.ctypes.data_as(POINTER(c_int32)), idx.ctypes.data_as(POINTER(c_int32)),
                  fl.ctypes.data_as(POINTER(c_uint8)), cap, ctypes.byref(n)))
        return ptr, idx[:n.value].copy(), fl[:n.value].copy()

    def work(self):
        w = POINTER(c_int32)()
        n = c_int64()
        _check(lib().bsa_plan_work(self.handle, ctypes.byref(w), ctypes.byref(n)))
        return np.ctypeslib.as_array(w, (n.value,)).copy() if n.value else np.zeros(0, np.int32)

    def csr_transposed(self, layout_head: int = 0):
        """bsa_plan_csr_transposed: per k-block, the q-blocks whose lists hold it."""
        cp, ri, fl = POINTER(c_int32)(), POINTER(c_int32)(), POINTER(c_uint8)()
        nnz = c_int64()
        _check(lib().bsa_plan_csr_transposed(self.handle, layout_head, ctypes.byref(cp), ctypes.byref(ri),
                                             ctypes.byref(fl), ctypes.byref(nnz)))
        nb = self.info["num_blocks"]
        n = nnz.value
        return {"col_ptr": np.ctypeslib.as_array(cp, (nb + 1,)).copy(),
                "row_idx": np.ctypeslib.as_array(ri, (n,)).copy() if n else np.zeros(0, np.int32),
                "flags": np.ctypeslib.as_array(fl, (n,)).copy() if n else np.zeros(0, np.uint8)}

    def work_kv(self):
        """bsa_plan_work_kv: launch order of the dK/dV kernel."""
        w = POINTER(c_int32)()
        n = c_int64()
        _check(lib().bsa_plan_work_kv(self.handle, ctypes.byref(w), ctypes.byref(n)))
        return np.ctypeslib.as_array(w, (n.value,)).copy() if n.value else np.zeros(0, np.int32)

    def read_work(self):
        """bsa_plan_read_work: the forward's launch order as the device holds it
        (for a dynamic plan, as the last set_bitmap left it)."""
        n = len(self.work())
        w = np.zeros(max(n, 1), np.int32)
        slots = c_int64()
        _check(lib().bsa_plan_read_work(self.handle, w.ctypes.data, n, ctypes.byref(slots)))
        return w[:slots.value]

    def read_work_kv(self):
        """bsa_plan_read_work_kv: the dK/dV launch descriptors on the device, an
        int32 [slots, 4] array {item, begin, end, partial}, and the number of
        split columns."""
        n = len(self.work_kv())
        desc = np.zeros((max(n, 1), 4), np.int32)
        slots, splits = c_int64(), c_int64()
        _check(lib().bsa_plan_read_work_kv(self.handle, desc.ctypes.data, n, ctypes.byref(slots),
                                           ctypes.byref(splits)))
        return desc[:slots.value], int(splits.value)

    def active_blocks(self) -> int:
        return int(lib().bsa_plan_active_blocks(self.handle))

    def flops(self) -> float:
        """Active-tile FLOPs of one forward: 2 GEMMs of block^2 x head_dim per tile."""
        p = self.problem
        return 4.0 * p.block_size * p.block_size * p.head_dim * self.active_blocks()

    def close(self):
        if self._h is not None and self._h.value:
            lib().bsa_plan_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def make_problem(batch, num_heads, num_kv_heads, seq_len, head_dim, block_size, dtype,
                 scale=0.0, schedule=SCHEDULE_DEFAULT) -> Problem:
    pr = Problem()
    pr.batch, pr.num_heads, pr.num_kv_heads, pr.head_dim = batch, num_heads, num_kv_heads, head_dim
    pr.seq_len, pr.block_size, pr.dtype = seq_len, block_size, _dtype_code(dtype)
    pr.scale, pr.schedule = float(scale), int(schedule)
    return pr


def plan(batch: int, num_heads: int, num_kv_heads: int, seq_len: int, head_dim: int,
         block_size: int, dtype, layout: Dict, scale: float = 0.0,
         schedule: int = SCHEDULE_DEFAULT, host_only: bool = False) -> Plan:
    """bsa_plan (or bsa_plan_host) on the current HIP device."""
    pr = make_problem(batch, num_heads, num_kv_heads, seq_len, head_dim, block_size, dtype,
                      scale, schedule)
    lay, keep = make_layout(layout)
    h = c_void_p()
    fn = lib().bsa_plan_host if host_only else lib().bsa_plan
    _check(fn(ctypes.byref(pr), ctypes.byref(lay), ctypes.byref(h)))
    del keep
    return Plan(h.value, pr, host_only)


def plan_dynamic(batch: int, num_heads: int, num_kv_heads: int, seq_len: int, head_dim: int,
                 block_size: int, dtype, causal: bool, bitmap_heads: int, scale: float = 0.0,
                 schedule: int = SCHEDULE_DEFAULT) -> Plan:
    """bsa_plan_dynamic on the current HIP device; feed it bitmaps with Plan.set_bitmap."""
    pr = make_problem(batch, num_heads, num_kv_heads, seq_len, head_dim, block_size, dtype,
                      scale, schedule)
    lay = Layout()
    lay.causal, lay.unit = int(bool(causal)), UNIT_BLOCKS
    lay.window_left, lay.window_right, lay.global_keys, lay.global_queries = -1, -1, 0, 0
    lay.bitmap, lay.bitmap_heads = None, int(bitmap_heads)
    h = c_void_p()
    _check(lib().bsa_plan_dynamic(ctypes.byref(pr), ctypes.byref(lay), ctypes.byref(h)))
    return Plan(h.value, pr, False)


def forward(q, k, v, p: Plan, out=None, lse=None):
    """bsa_forward on torch.cuda.current_stream(); returns (out, lse)."""
    import torch
    pr = p.problem
    B, H, Hk, N, D = pr.batch, pr.num_heads, pr.num_kv_heads, pr.seq_len, pr.head_dim
    dt = torch.bfloat16 if pr.dtype == BF16 else torch.float32
    if not q.is_cuda:
        raise ValueError(f"q must be a CUDA tensor, got one on {q.device}")
    if out is None:
        out = torch.empty((B, H, N, D), dtype=dt, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    for name, t, shape, tdt in (("q", q, (B, H, N, D), dt), ("k", k, (B, Hk, N, D), dt), ("v", v, (B, Hk, N, D), dt),
                                ("out", out, (B, H, N, D), dt), ("lse", lse, (B, H, N), torch.float32)):
        _require(name, t, shape, tdt, q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream().cuda_stream
        _check(lib().bsa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), p.handle,
                                 out.data_ptr(), lse.data_ptr(), c_void_p(stream)))
    return out, lse


def backward(q, k, v, out, lse, dout, p: Plan, dq=None, dk=None, dv=None, delta=None):
    """bsa_backward on torch.cuda.current_stream(); returns (dq, dk, dv).

    out and lse are the forward's outputs for these inputs and this plan;
    delta (float32 [B, H, N]) is the library's workspace for <dO, O>.
    """
    return _backward(q, k, v, out, lse, dout, p, None, dq, dk, dv, delta)


def backward_varlen(q, k, v, out, lse, dout, p: Plan, seq_lens, dq=None, dk=None, dv=None, delta=None):
    """bsa_backward_varlen on torch.cuda.current_stream(): the backward of
    forward_varlen with the same seq_lens (int32 CUDA tensor [batch]); rows of
    dq, dk, dv beyond an entry's length come out zero.  Returns (dq, dk, dv)."""
    import torch
    B = p.problem.batch
    if (not seq_lens.is_cuda or seq_lens.dtype != torch.int32 or tuple(seq_lens.shape) != (B,)
            or not seq_lens.is_contiguous()):
        raise ValueError(f"seq_lens must be a contiguous int32 CUDA tensor of shape ({B},)")
    return _backward(q, k, v, out, lse, dout, p, seq_lens, dq, dk, dv, delta)


def backward_noalloc(q, k, v, out, lse, dout, p: Plan, dq=None, dk=None, dv=None):
    """bsa_backward_noalloc on torch.cuda.current_stream(): bsa_backward with
    its workspace in the library's static per-GPU array (no device allocation
    by the library; pass dq, dk and dv to allocate nothing at all).  Calls
    that overlap on one GPU race.  Returns (dq, dk, dv)."""
    return _backward(q, k, v, out, lse, dout, p, None, dq, dk, dv, None, noalloc=True)


def _backward(q, k, v, out, lse, dout, p, seq_lens, dq, dk, dv, delta, noalloc=False):
    import torch
    pr = p.problem
    B, H, Hk, N, D = pr.batch, pr.num_heads, pr.num_kv_heads, pr.seq_len, pr.head_dim
    dt = torch.bfloat16 if pr.dtype == BF16 else torch.float32
    qs, ks = (B, H, N, D), (B, Hk, N, D)
    if not q.is_cuda:
        raise ValueError(f"q must be a CUDA tensor, got one on {q.device}")
    dev = q.device
    if dq is None:
        dq = torch.empty(qs, dtype=dt, device=dev)
    if dk is None:
        dk = torch.empty(ks, dtype=dt, device=dev)
    if dv is None:
        dv = torch.empty(ks, dtype=dt, device=dev)
    if delta is None and not noalloc:
        delta = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    checks = [("q", q, qs, dt), ("k", k, ks, dt), ("v", v, ks, dt), ("out", out, qs, dt),
              ("lse", lse, (B, H, N), torch.float32), ("dout", dout, qs, dt),
              ("dq", dq, qs, dt), ("dk", dk, ks, dt), ("dv", dv, ks, dt)]
    if not noalloc:
        checks.append(("delta", delta, (B, H, N), torch.float32))
    for name, t, shape, tdt in checks:
        _require(name, t, shape, tdt, dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream().cuda_stream
        if noalloc:
            st = lib().bsa_backward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                            lse.data_ptr(), dout.data_ptr(), p.handle, dq.data_ptr(),
                                            dk.data_ptr(), dv.data_ptr(), c_void_p(stream))
        elif seq_lens is None:
            st = lib().bsa_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                    dout.data_ptr(), p.handle, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                    delta.data_ptr(), c_void_p(stream))
        else:
            st = lib().bsa_backward_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                           lse.data_ptr(), dout.data_ptr(), p.handle, seq_lens.data_ptr(),
                                           dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                                           c_void_p(stream))
        _check(st)
    return dq, dk, dv


def _require(name, t, shape, dtype, device):
    """Raise ValueError unless t is a contiguous CUDA tensor of this shape and
    dtype on `device` (checked before any call into the library)."""
    if (not t.is_cuda or t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous()
            or t.device != device):
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor of shape {tuple(shape)} on "
                         f"{device}, got {tuple(t.shape)} {t.dtype} on {t.device}"
                         f"{'' if t.is_contiguous() else ' (not contiguous)'}")


def forward_varlen(q, k, v, p: Plan, seq_lens, out=None, lse=None):
    """bsa_forward_varlen on torch.cuda.current_stream(): batch entry b uses its
    first seq_lens[b] positions (seq_lens: int32 CUDA tensor [batch]); rows
    beyond come out as empty rows (O = 0, LSE = -inf).  Returns (out, lse)."""
    import torch
    pr = p.problem
    B, H, Hk, N, D = pr.batch, pr.num_heads, pr.num_kv_heads, pr.seq_len, pr.head_dim
    dt = torch.bfloat16 if pr.dtype == BF16 else torch.float32
    if not q.is_cuda:
        raise ValueError(f"q must be a CUDA tensor, got one on {q.device}")
    dev = q.device
    if out is None:
        out = torch.empty((B, H, N, D), dtype=dt, device=dev)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    for name, t, shape, tdt in (("q", q, (B, H, N, D), dt), ("k", k, (B, Hk, N, D), dt),
                                ("v", v, (B, Hk, N, D), dt), ("seq_lens", seq_lens, (B,), torch.int32),
                                ("out", out, (B, H, N, D), dt), ("lse", lse, (B, H, N), torch.float32)):
        _require(name, t, shape, tdt, dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream().cuda_stream
        _check(lib().bsa_forward_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), p.handle, seq_lens.data_ptr(),
                                        out.data_ptr(), lse.data_ptr(), c_void_p(stream)))
    return out, lse


def lse_merge(o_parts, lse_parts, out=None, lse=None):
    """bsa_lse_merge on torch.cuda.current_stream(): o_parts [P, ..., D] (bf16
    or float32) and lse_parts [P, ...] (float32) of P partial results over
    disjoint key sets of the same rows; returns (out [..., D], lse [...])."""
    import torch
    if o_parts.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"o_parts must be bfloat16 or float32, got {o_parts.dtype}")
    if not o_parts.is_cuda:
        raise ValueError(f"o_parts must be a CUDA tensor, got one on {o_parts.device}")
    P, D = int(o_parts.shape[0]), int(o_parts.shape[-1])
    row_shape = tuple(o_parts.shape[1:-1])
    dev = o_parts.device
    if out is None:
        out = torch.empty(row_shape + (D,), dtype=o_parts.dtype, device=dev)
    if lse is None:
        lse = torch.empty(row_shape, dtype=torch.float32, device=dev)
    for name, t, shape, tdt in (("o_parts", o_parts, tuple(o_parts.shape), o_parts.dtype),
                                ("lse_parts", lse_parts, (P,) + row_shape, torch.float32),
                                ("out", out, row_shape + (D,), o_parts.dtype),
                                ("lse", lse, row_shape, torch.float32)):
        _require(name, t, shape, tdt, dev)
    rows = 1
    for x in row_shape:
        rows *= int(x)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream().cuda_stream
        _check(lib().bsa_lse_merge(P, rows, D, BF16 if o_parts.dtype == torch.bfloat16 else F32,
                                   o_parts.data_ptr(), lse_parts.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                   c_void_p(stream)))
    return out, lse
