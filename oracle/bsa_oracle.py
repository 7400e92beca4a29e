"""Reference oracle for block-sparse flash attention (forward and backward).

TEST INFRASTRUCTURE ONLY.  This module is a plain, slow, obviously-correct CPU
implementation used to check the HIP path.  Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it; the product path
(`block_sparse_flash_bsa_amd`) never does, and it shares no code with it.

What it computes (all arithmetic in float64 with numpy):

* `allowed_keys(layout, N, bs, h, q)` -- the set A(q) of keys query q of head h
  may attend to.  The layout is either a window/global/causal spec or a block
  bitmap.  Sources: section "How Does Flash-MSA Sparse Attention Work?" of
  "How Do Sparse Attention Kernels Work in GPU Clusters?" (a boolean mask of
  shape (N_blocks, N_blocks); whole blocks are in or out); the sliding-window
  mask |i-j| <= W and the causal window in "The Mechanics", and global tokens
  that both see and are seen by every position in "Global Tokens" under
  "Sparse Patterns Beyond Sliding Windows", both on "Flash MSA Sparse
  Attention vs Full Attention".
  Readings where the pages are silent or disagree (inclusive window distances,
  token vs block units, global keys and global queries as separate knobs,
  causal always token-exact) are listed in the design notes.

* `forward(Q, K, V, layout, block_size)` -- masked softmax attention written
  as its definition: for every (b, h, q), s_k = scale * <Q[q], K[k]> over
  k in A(q), m = max s_k, l = sum exp(s_k - m), O = sum exp(s_k - m) V[k] / l,
  LSE = m + ln l.  Attention formula: softmax(QK^T / sqrt(d_k)) V ("The
  Mechanics", Flash MSA Sparse Attention vs Full Attention; the naive masked
  version in "How Sparse Attention Kernels Actually Speed Up Inference" on
  "Sparse Attention Kernels vs Full Attention Performance").  The flash/online
  formulation on the pages reaches exactly this result (it only avoids
  materialising the scores), so the oracle is the definition, not the tiled
  algorithm.  An empty A(q) gives O = 0 and LSE = -inf (log of an empty sum).
  GQA: query head h reads KV head h // (H / Hkv).

* `forward_query_range(Qr, Kh, Vh, layout, block_size, h, q0)` -- the same
  definition for a run of consecutive queries of one head at once: masked
  softmax attention over the union of their allowed keys, every other key
  masked to -inf (so its weight is exactly 0).  It is what makes every-row
  checks of full-size problems affordable; its pins compare it with the
  per-query form and with library attention.

* `backward(Q, K, V, dO, layout, block_size)` -- the gradients dQ, dK, dV of
  sum(dO * O) by the chain rule through the forward above, per query over its
  allowed keys (softmax Jacobian ds = p * (dp - sum p dp)); `backward_dq_rows`
  and `backward_dkv_keys` evaluate sampled rows and keys of full-size
  problems, the latter through `allowed_queries`, the predicate evaluated
  for every query at a fixed key.

* `lse_merge(O_parts, L_parts)` -- partial results over disjoint key sets of
  the same queries combined into the result over their union: the softmax
  over A_1 U A_2 splits into the two partial softmaxes weighted by their
  normalisers, so LSE = ln(sum_p e^{L_p}) and O = sum_p e^{L_p} O_p / e^{LSE}
  (the online-softmax combination of local and remote partial attention in
  "How Do Sparse Attention Kernels Work in GPU Clusters?"); parts with L = -inf
  (no key) carry no weight, and a row empty in every part stays O = 0,
  LSE = -inf.  Its pins merge the oracle's own partial results over split
  layouts and compare with the oracle over the union.

* `plan(layout, N, bs)` -- the per-query-block list of key blocks (step three
  of "How Does Flash-MSA Sparse Attention Work?": a query block fetches only
  its active key blocks; a mask given as block indices in "The Architecture
  of Flash MSA Sparse Attention Kernels" on "Flash MSA Sparse Attention
  Kernels Explained"): for each
  (layout head, q-block i) the ascending key blocks j whose tile holds at
  least one allowed (q, k) pair, each flagged FULL when every pair of the tile
  is allowed and PARTIAL otherwise.  Counts are exact: brute force over the
  tile for small problems, per-query interval overlap otherwise.

Layout dictionary (plain Python, no dependency on the product package):
    causal          bool   -- token-exact k <= q
    unit            "tokens" | "blocks"  (units of the four fields below)
    window_left     int    -- q - k <= window_left  (-1: unbounded)
    window_right    int    -- k - q <= window_right (-1: unbounded)
    global_keys     int    -- keys  < global_keys  are visible to every query
    global_queries  int    -- queries < global_queries see every key
    bitmap          None or uint8/bool array [layout_heads, nb, nb]; when set
                    it replaces window/global (causal still applies)
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Tuple

import numpy as np

FULL = 0
PARTIAL = 1


# --------------------------------------------------------------------------
# Layout predicate
# --------------------------------------------------------------------------
def _num_layout_heads(layout) -> int:
    bm = layout.get("bitmap")
    return 1 if bm is None else int(np.asarray(bm).shape[0])


def _layout_head(layout, h: int) -> int:
    """Layout head used by query head h: a shared layout or one per head."""
    return 0 if _num_layout_heads(layout) == 1 else h


def _token_pieces(layout, N: int, q: int):
    """Allowed keys of query q for a token-unit spec as closed intervals.

    The allowed set is (window(q) U globals) n causal(q), returned as the two
    (possibly overlapping, possibly empty) intervals W n C and G n C, or the
    single interval C for a global query.  lo > hi means empty.
    """
    wl = layout["window_left"]
    wr = layout["window_right"]
    hi_c = q if layout["causal"] else N - 1          # causal: k <= q
    if q < layout["global_queries"]:                 # global query: every key
        return [(0, hi_c)]
    w_lo = 0 if wl < 0 else max(0, q - wl)
    w_hi = N - 1 if wr < 0 else min(N - 1, q + wr)
    return [(w_lo, min(w_hi, hi_c)), (0, min(layout["global_keys"] - 1, hi_c))]


def _intervals_tokens(layout, N: int, q: int):
    """Signed intervals whose overlap counts sum to |A(q) n block|.

    Inclusion-exclusion over the two pieces keeps every term an interval:
    |W u G| = |W| + |G| - |W n G|.  Returns (lo, hi, sign) triples.
    """
    pieces = _token_pieces(layout, N, q)
    if len(pieces) == 1:
        return [(pieces[0][0], pieces[0][1], 1)]
    (a0, b0), (a1, b1) = pieces
    return [(a0, b0, 1), (a1, b1, 1), (max(a0, a1), min(b0, b1), -1)]


def _blocks_active(layout, lh: int, i: int, js: np.ndarray) -> np.ndarray:
    """Block-level part of the predicate for block-unit specs and bitmaps:
    whether q-block i may see each key block in the int array js."""
    js = np.asarray(js, dtype=np.int64)
    bm = layout.get("bitmap")
    if bm is not None:
        return np.asarray(bm)[lh, i, js].astype(bool)
    wl = layout["window_left"]
    wr = layout["window_right"]
    in_w = np.ones(js.shape, dtype=bool)
    if wl >= 0:
        in_w &= (i - js) <= wl
    if wr >= 0:
        in_w &= (js - i) <= wr
    return in_w | (js < layout["global_keys"]) | (i < layout["global_queries"])


def allowed_keys(layout, N: int, bs: int, h: int, q: int) -> np.ndarray:
    """Sorted int64 array of the keys query q of head h may attend to."""
    if layout.get("bitmap") is None and layout["unit"] == "tokens":
        parts = [np.arange(lo, hi + 1) for lo, hi in _token_pieces(layout, N, q) if lo <= hi]
        if not parts:
            return np.zeros(0, dtype=np.int64)
        return np.unique(np.concatenate(parts)).astype(np.int64)
    nb = -(-N // bs)                     # a last, shorter block when bs does not divide N
    i = q // bs
    blocks = np.flatnonzero(_blocks_active(layout, _layout_head(layout, h), i, np.arange(nb)))
    keys = (blocks[:, None] * bs + np.arange(bs)[None, :]).ravel()
    keys = keys[keys < N]
    if layout["causal"]:
        keys = keys[keys <= q]
    return keys.astype(np.int64)


def allowed_count(layout, N: int, bs: int, h: int, q: int) -> int:
    return int(allowed_keys(layout, N, bs, h, q).size)


# --------------------------------------------------------------------------
# Forward: masked softmax attention, per query over its allowed keys
# --------------------------------------------------------------------------
def _f64(x) -> np.ndarray:
    """Exact upcast of a torch tensor (any float dtype) or array to float64."""
    try:
        import torch  # local import: the oracle also works on numpy inputs
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def attend_row(q_vec: np.ndarray, K_rows: np.ndarray, V_rows: np.ndarray,
               scale: float) -> Tuple[np.ndarray, float]:
    """One query against its allowed keys (already gathered), float64.

    Returns (o, lse).  With no keys: o = 0, lse = -inf.
    """
    D = V_rows.shape[1] if V_rows.ndim == 2 else q_vec.shape[0]
    if K_rows.shape[0] == 0:
        return np.zeros(D), -math.inf
    s = scale * (K_rows @ q_vec)
    m = s.max()
    w = np.exp(s - m)
    l = w.sum()
    o = (w @ V_rows) / l
    return o, float(m + math.log(l))


def kv_head(h: int, group: int) -> int:
    """KV head read by query head h when `group` consecutive query heads
    share one KV head (GQA; a reading, since the pages do not treat GQA)."""
    return h // group


def forward(Q, K, V, layout, block_size: int, scale: Optional[float] = None,
            rows: Optional[Iterable[Tuple[int, int, int]]] = None):
    """Oracle forward.

    Q: [B, H, N, D]; K, V: [B, Hkv, N, D]; numpy arrays or CPU torch tensors of
    any float dtype (upcast exactly to float64).
    rows: optional iterable of (b, h, q) to evaluate; default every row.  With
    rows given only the rows and keys they touch are upcast, so full-size
    inputs can be checked on a sample.
    Returns (O, LSE) as float64 arrays: [B,H,N,D] / [B,H,N] when rows is None,
    otherwise [R, D] / [R] in the order of `rows`.
    """
    B, H, N, D = (int(x) for x in Q.shape)
    Hkv = int(K.shape[1])
    assert H % Hkv == 0, "query heads must be a multiple of KV heads"
    group = H // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if rows is None:
        Qd, Kd, Vd = _f64(Q), _f64(K), _f64(V)
        O = np.zeros((B, H, N, D))
        L = np.full((B, H, N), -math.inf)
        for b in range(B):
            for h in range(H):
                hk = kv_head(h, group)
                for q in range(N):
                    keys = allowed_keys(layout, N, block_size, h, q)
                    O[b, h, q], L[b, h, q] = attend_row(
                        Qd[b, h, q], Kd[b, hk, keys], Vd[b, hk, keys], scale)
        return O, L
    rows = list(rows)
    O = np.zeros((len(rows), D))
    L = np.full(len(rows), -math.inf)
    for r, (b, h, q) in enumerate(rows):
        hk = kv_head(h, group)
        keys = allowed_keys(layout, N, block_size, h, q)
        O[r], L[r] = attend_row(_f64(Q[b, h, q]), _f64(K[b, hk][keys]),
                                _f64(V[b, hk][keys]), scale)
    return O, L


def forward_query_range(Qr, Kh, Vh, layout, block_size: int, h: int, q0: int,
                        scale: Optional[float] = None):
    """The same definition for the consecutive queries q0 .. q0+R-1 of one head.

    Qr: [R, D] the rows q0 .. q0+R-1 of query head h; Kh, Vh: [N, D] every
    row of its KV head (any float dtype; only the rows used are upcast to
    float64).  The queries are
    taken together as masked softmax attention over C, the union of their
    allowed key sets: S = scale * Q C^T, S[q, k] = -inf where k is not in
    A(q), then the row-wise softmax, O = P V_C / l and LSE = m + ln l.  Every
    key outside A(q) carries weight exactly 0, so each row equals its own
    per-query definition (up to the order of the float64 sums).  This is the
    naive masked formulation of "How Sparse Attention Kernels Actually Speed
    Up Inference" (Sparse Attention Kernels vs Full Attention Performance)
    restricted to the keys some row of the range may see.  A query with no
    allowed key gets O = 0 and LSE = -inf.
    Returns (O [R, D], LSE [R]) as float64.
    """
    R, D = int(Qr.shape[0]), int(Qr.shape[1])
    N = int(Kh.shape[0])
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    per_row = [allowed_keys(layout, N, block_size, h, q) for q in range(q0, q0 + R)]
    member = np.zeros(N, dtype=bool)
    for ks in per_row:
        member[ks] = True
    C = np.flatnonzero(member)
    O = np.zeros((R, D))
    L = np.full(R, -math.inf)
    if C.size == 0:
        return O, L
    col = np.full(N, -1, dtype=np.int64)
    col[C] = np.arange(C.size)
    M = np.zeros((R, C.size), dtype=bool)
    for r, ks in enumerate(per_row):
        M[r, col[ks]] = True
    Kc, Vc = _f64(Kh[C]), _f64(Vh[C])
    S = scale * (_f64(Qr) @ Kc.T)
    S[~M] = -math.inf
    m = S.max(axis=1)
    ok = np.isfinite(m)
    P = np.exp(S[ok] - m[ok, None])          # masked entries give exp(-inf) = 0
    l = P.sum(axis=1)
    O[ok] = (P @ Vc) / l[:, None]
    L[ok] = m[ok] + np.log(l)
    return O, L


# --------------------------------------------------------------------------
# Plan oracle: per-q-block CSR list of key blocks with FULL/PARTIAL flags
# --------------------------------------------------------------------------
def _tile_counts_bruteforce(layout, N: int, bs: int, h: int, i: int) -> np.ndarray:
    """Allowed-pair count of every tile (i, j) by enumerating A(q)."""
    nb = -(-N // bs)
    counts = np.zeros(nb, dtype=np.int64)
    for q in range(i * bs, min((i + 1) * bs, N)):
        keys = allowed_keys(layout, N, bs, h, q)
        counts += np.bincount(keys // bs, minlength=nb)
    return counts


def _tile_counts_intervals(layout, N: int, bs: int, i: int) -> np.ndarray:
    """Same counts for a token-unit spec, by interval overlap per query."""
    nb = -(-N // bs)
    counts = np.zeros(nb, dtype=np.int64)
    full_mid = np.zeros(nb + 1, dtype=np.int64)      # difference array of whole-block runs
    for q in range(i * bs, min((i + 1) * bs, N)):
        for lo, hi, sign in _intervals_tokens(layout, N, q):
            if lo > hi:
                continue
            ja, jb = lo // bs, hi // bs
            if ja == jb:
                counts[ja] += sign * (hi - lo + 1)
                continue
            counts[ja] += sign * ((ja + 1) * bs - lo)
            counts[jb] += sign * (hi - jb * bs + 1)
            if jb > ja + 1:
                full_mid[ja + 1] += sign * bs
                full_mid[jb] -= sign * bs
    counts += np.cumsum(full_mid)[:nb]
    return counts


def _tile_counts_blocks(layout, N: int, bs: int, h: int, i: int) -> np.ndarray:
    """Counts for block-unit specs and bitmaps: whole tiles, causal cuts the
    diagonal; a last, shorter block has only its rows below N."""
    nb = -(-N // bs)
    lh = _layout_head(layout, h)
    counts = np.zeros(nb, dtype=np.int64)
    rows_i = min(bs, N - i * bs)                     # queries of block i
    active = _blocks_active(layout, lh, i, np.arange(nb))
    for j in range(nb):
        if not active[j]:
            continue
        cols_j = min(bs, N - j * bs)                 # keys of block j
        if not layout["causal"] or j < i:
            counts[j] = rows_i * cols_j
        elif j == i:
            counts[j] = rows_i * (rows_i + 1) // 2   # pairs with k <= q inside the tile
    return counts


def tile_counts(layout, N: int, bs: int, h: int, i: int, brute: bool = False) -> np.ndarray:
    if brute:
        return _tile_counts_bruteforce(layout, N, bs, h, i)
    if layout.get("bitmap") is None and layout["unit"] == "tokens":
        return _tile_counts_intervals(layout, N, bs, i)
    return _tile_counts_blocks(layout, N, bs, h, i)


def plan(layout, N: int, bs: int, brute: Optional[bool] = None):
    """CSR plan per layout head.

    Returns a list (one per layout head) of dicts with int32 `row_ptr` [nb+1],
    int32 `col_idx` [nnz] and uint8 `flags` [nnz] (0 = FULL, 1 = PARTIAL).
    When bs does not divide N the last block is shorter; a tile is FULL only
    if all bs * bs of its pairs exist and are allowed, so tiles touching that
    block are PARTIAL.
    """
    nb = -(-N // bs)
    if brute is None:
        brute = N <= 1024
    out = []
    for lh in range(_num_layout_heads(layout)):
        row_ptr = [0]
        cols, flags = [], []
        for i in range(nb):
            c = tile_counts(layout, N, bs, lh, i, brute=brute)
            js = np.flatnonzero(c > 0)
            cols.extend(int(j) for j in js)
            flags.extend(FULL if c[j] == bs * bs else PARTIAL for j in js)
            row_ptr.append(len(cols))
        out.append({
            "row_ptr": np.asarray(row_ptr, dtype=np.int32),
            "col_idx": np.asarray(cols, dtype=np.int32),
            "flags": np.asarray(flags, dtype=np.uint8),
        })
    return out


# --------------------------------------------------------------------------
# Backward: gradients of masked softmax attention
# --------------------------------------------------------------------------
# For a scalar loss with upstream gradient dO = dLoss/dO, the chain rule
# through O_q = sum_k p_qk V_k with p_q = softmax(s_q) over A(q) and
# s_qk = scale * <Q_q, K_k> gives, per query q and allowed key k:
#     dV_k  += p_qk * dO_q
#     dp_qk  = <dO_q, V_k>
#     ds_qk  = p_qk * (dp_qk - sum_k' p_qk' dp_qk')      (softmax Jacobian)
#     dQ_q  += scale * ds_qk * K_k
#     dK_k  += scale * ds_qk * Q_q
# Keys shared by the query heads of a GQA group accumulate over the group.
# The pages treat the backward only through its cost ("Training Throughput"
# of "Sparse Attention Kernels vs Full Attention Performance"; forward and
# backward timings in the FAQ of "How Do Sparse Attention Kernels Work in GPU
# Clusters?"); the gradient itself is the derivative of the forward defined
# above, written out here.  sum_k' p_qk' dp_qk' equals <dO_q, O_q>.

def allowed_queries(layout, N: int, bs: int, h: int, k: int) -> np.ndarray:
    """Sorted int64 array of the queries q of head h with k in A(q).

    The layout predicate evaluated for every q at fixed k (the transpose of
    allowed_keys): causal_ok && (bitmap ? bitmap[hl][q/bs][k/bs]
    : in_window || key_global || query_global), in the spec's units.
    """
    q = np.arange(N, dtype=np.int64)
    bm = layout.get("bitmap")
    if bm is not None:
        ok = np.asarray(bm)[_layout_head(layout, h), q // bs, k // bs].astype(bool)
    else:
        if layout["unit"] == "tokens":
            qu, ku = q, k
        else:
            qu, ku = q // bs, k // bs
        wl, wr = layout["window_left"], layout["window_right"]
        in_w = np.ones(N, dtype=bool)
        if wl >= 0:
            in_w &= (qu - ku) <= wl
        if wr >= 0:
            in_w &= (ku - qu) <= wr
        ok = in_w | (ku < layout["global_keys"]) | (qu < layout["global_queries"])
    if layout["causal"]:
        ok &= k <= q
    return q[ok]


def grad_row(q_vec: np.ndarray, do_vec: np.ndarray, K_rows: np.ndarray,
             V_rows: np.ndarray, scale: float):
    """Softmax weights p and score gradients ds of one query over its keys.

    Returns (p, ds) over the gathered keys (float64); empty inputs give empty
    arrays.
    """
    if K_rows.shape[0] == 0:
        return np.zeros(0), np.zeros(0)
    s = scale * (K_rows @ q_vec)
    w = np.exp(s - s.max())
    p = w / w.sum()
    dp = V_rows @ do_vec
    ds = p * (dp - p @ dp)
    return p, ds


def backward(Q, K, V, dO, layout, block_size: int, scale: Optional[float] = None):
    """Oracle backward over every row: returns (dQ, dK, dV) as float64 arrays
    shaped like Q, K and V.  Inputs as for `forward`, plus dO shaped like Q."""
    B, H, N, D = (int(x) for x in Q.shape)
    Hkv = int(K.shape[1])
    group = H // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    Qd, Kd, Vd, dOd = _f64(Q), _f64(K), _f64(V), _f64(dO)
    dQ = np.zeros_like(Qd)
    dK = np.zeros_like(Kd)
    dV = np.zeros_like(Vd)
    for b in range(B):
        for h in range(H):
            hk = kv_head(h, group)
            for q in range(N):
                keys = allowed_keys(layout, N, block_size, h, q)
                p, ds = grad_row(Qd[b, h, q], dOd[b, h, q], Kd[b, hk, keys], Vd[b, hk, keys], scale)
                if keys.size == 0:
                    continue
                dQ[b, h, q] = scale * (ds @ Kd[b, hk, keys])
                dK[b, hk, keys] += scale * np.outer(ds, Qd[b, h, q])
                dV[b, hk, keys] += np.outer(p, dOd[b, h, q])
    return dQ, dK, dV


def backward_dq_rows(Q, K, V, dO, layout, block_size: int, rows, scale: Optional[float] = None):
    """dQ of the sampled rows (b, h, q) only: float64 [R, D]."""
    D = int(Q.shape[3])
    N = int(Q.shape[2])
    group = int(Q.shape[1]) // int(K.shape[1])
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rows = list(rows)
    out = np.zeros((len(rows), D))
    for r, (b, h, q) in enumerate(rows):
        keys = allowed_keys(layout, N, block_size, h, q)
        hk = kv_head(h, group)
        Kr = _f64(K[b, hk][keys])
        _, ds = grad_row(_f64(Q[b, h, q]), _f64(dO[b, h, q]), Kr, _f64(V[b, hk][keys]), scale)
        if keys.size:
            out[r] = scale * (ds @ Kr)
    return out


def backward_dkv_keys(Q, K, V, dO, layout, block_size: int, keys, scale: Optional[float] = None):
    """dK and dV of the sampled keys (b, hk, k) only: two float64 [R, D].

    Each key sums over every query of its GQA group's heads that may attend
    to it; each such query's softmax is formed over its own allowed keys.
    """
    H, N, D = (int(x) for x in Q.shape[1:])
    group = H // int(K.shape[1])
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    keys = list(keys)
    dK = np.zeros((len(keys), D))
    dV = np.zeros((len(keys), D))
    for r, (b, hk, k) in enumerate(keys):
        Kb, Vb = K[b, hk], V[b, hk]
        for h in range(hk * group, (hk + 1) * group):
            for q in allowed_queries(layout, N, block_size, h, k):
                ks = allowed_keys(layout, N, block_size, h, int(q))
                pos = int(np.searchsorted(ks, k))
                qv, dov = _f64(Q[b, h, q]), _f64(dO[b, h, q])
                p, ds = grad_row(qv, dov, _f64(Kb[ks]), _f64(Vb[ks]), scale)
                dK[r] += scale * ds[pos] * qv
                dV[r] += p[pos] * dov
    return dK, dV


# --------------------------------------------------------------------------
# Merging partial results over disjoint key sets
# --------------------------------------------------------------------------
def lse_merge(O_parts, L_parts):
    """Combine P partial results of the same query rows over disjoint key
    sets: O_parts [P, ..., D], L_parts [P, ...] (natural-log LSE, -inf for a
    part with no key).  Returns (O, LSE) over the union, in float64:
    LSE = ln(sum_p e^{L_p}), O = sum_p e^{L_p - LSE} O_p; rows with every
    L_p = -inf give O = 0 and LSE = -inf."""
    O = np.asarray(O_parts, dtype=np.float64)
    L = np.asarray(L_parts, dtype=np.float64)
    m = L.max(axis=0)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(L - m_safe[None])                       # e^{-inf} = 0 for empty parts
    s = w.sum(axis=0)
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, s)))
    out = (w[..., None] * O).sum(axis=0) / np.where(empty, 1.0, s)[..., None]
    out[empty] = 0.0
    return out, lse
