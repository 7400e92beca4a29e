"""Seeded synthetic workloads: problem shapes, layout specs and input tensors.

This module only describes problems and draws random inputs; it holds none of
the attention arithmetic.  Both the HIP path (through the tests and the
benchmark) and the CPU oracle consume the tensors it produces.

A layout is a plain dict (the same keys the oracle and the binding take):
    causal, unit ("tokens" | "blocks"), window_left, window_right,
    global_keys, global_queries, bitmap (None or bool tensor [Hl, nb, nb]).

Input recipe: values are iid N(0, 1) drawn in float32 with a generator seeded
per workload, in the order Q, K, V at their full shapes (K and V with the KV
head count), then rounded to nearest even in the compute dtype; the 256K GQA
workload then halves K (exact in bfloat16).  Small problems are drawn on the
CPU; full-size problems are drawn on the GPU (same recipe with a device
generator) because CPU normal sampling of ~1e9 values takes tens of seconds.
The random block bitmap is Bernoulli(0.10) per (head, q-block, k-block) from
torch.rand on a CPU generator with the workload seed, diagonal forced on.

The workloads stand in for the long-document inputs the pages benchmark on
(no dataset is used): a 512-token causal window at 16K, a 64-block window
plus a few global blocks at 128K, a random ~10% block layout, and a 4K window
with 8 global tokens at 256K.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    kv_heads: int
    seq_len: int
    head_dim: int
    block: int
    dtype: torch.dtype
    seed: int
    layout: Dict
    k_scale: float = 1.0
    bitmap_density: Optional[float] = None     # random bitmap recipe

    @property
    def num_blocks(self) -> int:
        return self.seq_len // self.block

    def with_shape(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def spec(causal, unit, wl=-1, wr=-1, gk=0, gq=0):
    return dict(causal=bool(causal), unit=unit, window_left=int(wl), window_right=int(wr),
                global_keys=int(gk), global_queries=int(gq), bitmap=None)


# The five workloads.  Window distances are inclusive: "0 <= q - k < 512" is
# window_left = 511; "i - j < 64" is window_left = 63 (blocks).
WORKLOADS = {
    # 16x16 block grid, block (i, j) active iff |i-j| <= 2 or i == 0 or j == 0.
    "tiny_f32": Workload("tiny_f32", 1, 2, 2, 1024, 64, 64, torch.float32, 0,
                         spec(False, "blocks", 2, 2, gk=1, gq=1)),
    # token-exact causal window of 512 keys.
    "window16k": Workload("window16k", 1, 32, 32, 16384, 128, 128, torch.bfloat16, 1,
                          spec(True, "tokens", 511, 0)),
    # causal, blocks j <= i with i - j < 64 or j < 4; rows i < 4 see every j <= i.
    "winglobal128k": Workload("winglobal128k", 1, 32, 32, 131072, 128, 128, torch.bfloat16, 2,
                              spec(True, "blocks", 63, 0, gk=4, gq=4)),
    # per-head Bernoulli(0.10) block bitmap, diagonal on, non-causal.
    "random32k": Workload("random32k", 2, 16, 16, 32768, 128, 128, torch.bfloat16, 3,
                          spec(False, "blocks"), bitmap_density=0.10),
    # GQA 32/8, causal, k <= q and (q - k < 4096 or k < 8).
    "gqa256k": Workload("gqa256k", 1, 32, 8, 262144, 128, 128, torch.bfloat16, 4,
                        spec(True, "tokens", 4095, 0, gk=8), k_scale=0.5),
    # same shape with a dense causal mask: the full-attention comparator.
    "dense256k": Workload("dense256k", 1, 32, 8, 262144, 128, 128, torch.bfloat16, 4,
                          spec(True, "tokens", -1, 0), k_scale=0.5),
}


def make_bitmap(w: Workload) -> Optional[torch.Tensor]:
    """Random block bitmap [heads, nb, nb] (bool, CPU) or None."""
    if w.bitmap_density is None:
        return None
    g = torch.Generator().manual_seed(w.seed)
    nb = w.num_blocks
    bm = torch.rand((w.heads, nb, nb), generator=g) < w.bitmap_density
    r = torch.arange(nb)
    bm[:, r, r] = True
    return bm


def layout_of(w: Workload) -> Dict:
    """The workload's layout dict, with its bitmap filled in when it has one."""
    lay = dict(w.layout)
    lay["bitmap"] = make_bitmap(w)
    return lay


def make_qkv(w: Workload, device="cpu"):
    """Seeded Q [B,H,N,D], K, V [B,Hkv,N,D] in the workload dtype on `device`."""
    dev = torch.device(device)
    g = torch.Generator(device=dev).manual_seed(w.seed)
    B, H, Hk, N, D = w.batch, w.heads, w.kv_heads, w.seq_len, w.head_dim

    def draw(shape):
        return torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(w.dtype)

    q = draw((B, H, N, D))
    k = draw((B, Hk, N, D))
    v = draw((B, Hk, N, D))
    if w.k_scale != 1.0:
        k = (k.float() * w.k_scale).to(w.dtype)
    return q, k, v


def make_dout(w: Workload, device="cpu"):
    """Seeded upstream gradient dO [B,H,N,D] for the backward: iid N(0, 1)
    drawn in float32 from a generator seeded (workload seed + 1000), rounded
    to the workload dtype."""
    dev = torch.device(device)
    g = torch.Generator(device=dev).manual_seed(w.seed + 1000)
    shape = (w.batch, w.heads, w.seq_len, w.head_dim)
    return torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(w.dtype)


def small_variant(w: Workload, seq_len: int, heads: Optional[int] = None,
                  kv_heads: Optional[int] = None, batch: Optional[int] = None) -> Workload:
    """Same layout rule at a size the oracle finishes in seconds."""
    heads = heads if heads is not None else min(w.heads, 2 * (w.heads // w.kv_heads))
    kv_heads = kv_heads if kv_heads is not None else max(1, heads // (w.heads // w.kv_heads))
    return w.with_shape(name=f"{w.name}@{seq_len}", seq_len=seq_len, heads=heads,
                        kv_heads=kv_heads, batch=batch if batch is not None else w.batch)
