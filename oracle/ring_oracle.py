"""fp64 CPU oracle for one rank's share of ring attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module: only the tests, the smoke check and the bench's CPU-baseline leg
use it.  It shares no code with the HIP library.

Sources (web pages on ring attention; sections named as on the pages):
  [RA]  ai360xpert.com, "Ring Attention": "Sequence sharding and the ring
        topology", "Online softmax across ring steps", "Show Me the Code",
        "Watch Out For" (global-position causal masking).
  [NT]  instagit.com, "How to Implement Ring Attention for Long Sequences in
        Nanotron": "Forward Pass Implementation" (the per-step flash forward,
        the merge of block_out / block_lse, the causal rule "step <= rank"),
        "Backward Pass and Gradient Accumulation", "Numerically-Stable Output
        Fusion" (update_out_and_lse), "Calling the Ring Attention Function
        Directly" (bshd tensors, cu_seqlens, scaling=None -> 1/sqrt(head_dim)).
  [PF]  skillfed.io, "ring-flash-attn" fact sheet, "What it is and what it
        does": basic, zigzag, stripe and llama3-style variants, each in batch
        and varlen (packed, cu_seqlens) form.
  [IQ]  zenaique.com ring-attention question page: the online-softmax rescale
        by exp(old_max - new_max); "same exact math".

The method is exact ([RA] "Online softmax across ring steps"; [IQ]), so the
oracle is the plain definition of softmax attention over *global* token
positions, restricted to the rank's rows.  Readings taken where the pages are
silent (layout definitions of zigzag/stripe/varlen-ring and of the packed
zigzag/stripe forms, the sliding window, the LSE base, GQA head mapping,
fully-masked rows) are stated at each function.

Every function here is pinned by tests that do not re-type its formulas: the
pages' two-device example, ring == unblocked for every D and layout, brute
force with math.fsum, closed forms, finite differences and torch's fp64 SDPA
with autograd.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

BASIC, ZIGZAG, STRIPE, VARLEN_RING, LLAMA3, VARLEN_ZIGZAG, VARLEN_STRIPE = 0, 1, 2, 3, 4, 5, 6
# layouts over packed documents: masks also require the same document
PACKED = (VARLEN_RING, LLAMA3, VARLEN_ZIGZAG, VARLEN_STRIPE)


# ---------------------------------------------------------------------------
# Token positions held by each rank
# ---------------------------------------------------------------------------

def positions(layout: int, n: int, world: int, rank: int,
              cu_seqlens: Optional[Sequence[int]] = None) -> np.ndarray:
    """Global token index of every local row held by ``rank`` (int64, local order).

    BASIC   -- the sequence is cut into D equal consecutive blocks and rank d
               holds block d ([RA] "Sequence sharding and the ring topology").
    ZIGZAG  -- reading of the "more compute-balanced" variant ([PF]): the
               sequence is cut into 2D chunks of N/(2D); rank r holds chunk r
               followed by chunk 2D-1-r.
    STRIPE  -- plainest reading of the stripe variant ([PF]; Striped Attention
               on [IQ]): stripe width 1, token t belongs to rank t mod D, in
               increasing t.
    VARLEN_RING -- packed documents ([NT] cu_seqlens) with one cu_seqlens for q
               and kv: each document is split into D equal consecutive parts
               and rank r holds part r of every document, in document order.
    LLAMA3  -- the query shard is the BASIC block r of the packed stream; its
               KV is the gathered stream (see ``kv_positions``).
    VARLEN_ZIGZAG, VARLEN_STRIPE -- [PF] lists every variant in a packed
               form as well; read here as the ZIGZAG / STRIPE rule applied to
               the document-local token index inside every packed document,
               documents in order.
    """
    if layout in (BASIC, LLAMA3):
        s = n // world
        return rank * s + np.arange(s, dtype=np.int64)
    if layout == ZIGZAG:
        c = n // (2 * world)
        first = rank * c + np.arange(c, dtype=np.int64)
        second = (2 * world - 1 - rank) * c + np.arange(c, dtype=np.int64)
        return np.concatenate([first, second])
    if layout == STRIPE:
        return np.arange(rank, n, world, dtype=np.int64)
    if layout == VARLEN_RING:
        parts = []
        for a, b in zip(cu_seqlens[:-1], cu_seqlens[1:]):
            part = (b - a) // world
            parts.append(a + rank * part + np.arange(part, dtype=np.int64))
        return np.concatenate(parts) if parts else np.zeros(0, np.int64)
    if layout in (VARLEN_ZIGZAG, VARLEN_STRIPE):
        parts = []
        for a, b in zip(cu_seqlens[:-1], cu_seqlens[1:]):
            doc = positions(ZIGZAG if layout == VARLEN_ZIGZAG else STRIPE, b - a, world, rank)
            parts.append(a + doc)
        return np.concatenate(parts) if parts else np.zeros(0, np.int64)
    raise ValueError(f"unknown layout {layout}")


def kv_positions(layout: int, n: int, world: int, block: int,
                 cu_seqlens: Optional[Sequence[int]] = None) -> np.ndarray:
    """Global token index of every row of KV block ``block``.

    For the ring layouts, block j is exactly what rank j holds.  For LLAMA3
    there is one gathered block holding every token in global order.
    """
    if layout == LLAMA3:
        return np.arange(n, dtype=np.int64)
    return positions(layout, n, world, block, cu_seqlens)


def num_blocks(layout: int, world: int) -> int:
    return 1 if layout == LLAMA3 else world


def doc_index(pos: np.ndarray, cu_seqlens: Optional[Sequence[int]]) -> np.ndarray:
    """Document index of every global position (all zeros in batch mode)."""
    if cu_seqlens is None:
        return np.zeros(len(pos), dtype=np.int64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return np.searchsorted(cu, pos, side="right") - 1


def allowed(pos_q: np.ndarray, pos_k: np.ndarray, causal: bool,
            cu_seqlens: Optional[Sequence[int]] = None,
            window: Tuple[int, int] = (-1, -1)) -> np.ndarray:
    """Boolean [len(pos_q), len(pos_k)] mask on *global* positions.

    A key is visible to a query when it is not in the query's future (causal)
    and lies in the same packed document (varlen).  The mask is decided by
    global positions, not by positions inside a block ([RA] "Watch Out For").

    ``window`` = (left, right) is the sliding window of the call interface
    ([NT] "Calling the Ring Attention Function Directly" shows the argument,
    with (-1, -1) meaning an unbounded window).  Reading: a key at global
    position u is visible to the query at t only if t - left <= u (when
    left >= 0) and u <= t + right (when right >= 0), on top of the causal and
    document rules.
    """
    m = np.ones((len(pos_q), len(pos_k)), dtype=bool)
    if causal:
        m &= pos_k[None, :] <= pos_q[:, None]
    if cu_seqlens is not None:
        m &= doc_index(pos_k, cu_seqlens)[None, :] == doc_index(pos_q, cu_seqlens)[:, None]
    left, right = window
    if left >= 0:
        m &= pos_k[None, :] >= pos_q[:, None] - left
    if right >= 0:
        m &= pos_k[None, :] <= pos_q[:, None] + right
    return m


def kv_head_of(h: int, heads_q: int, heads_kv: int) -> int:
    """GQA reading (the pages never mention GQA): q head h uses KV head
    floor(h * Hkv / Hq), i.e. contiguous groups of Hq/Hkv query heads."""
    return (h * heads_kv) // heads_q


def default_scale(head_dim: int) -> float:
    """scaling=None means 1/sqrt(head_dim) ([NT] "Calling the Ring Attention
    Function Directly")."""
    return 1.0 / math.sqrt(head_dim)


# ---------------------------------------------------------------------------
# Softmax attention over explicit rows and keys (definition)
# ---------------------------------------------------------------------------

def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                   scale: float):
    """Softmax attention of query rows q [R, d] over keys k, v [M, d].

    out_t = sum_u softmax_u(scale * <q_t, k_u>) v_u over the visible keys,
    lse_t = ln sum_u exp(scale * <q_t, k_u>) (natural log of the *scaled*
    scores).  A row with no visible key has out 0 and lse -inf.
    Returns (out [R, d], lse [R]) in float64.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    s = scale * (q @ k.T)
    s = np.where(mask, s, -np.inf)
    has = mask.any(axis=1)
    m = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
    p = np.where(mask, np.exp(s - m[:, None]), 0.0)
    l = p.sum(axis=1)
    out = np.zeros((q.shape[0], v.shape[1]), np.float64)
    out[has] = (p[has] @ v) / l[has, None]
    lse = np.full(q.shape[0], -np.inf)
    lse[has] = m[has] + np.log(l[has])
    return out, lse


def _row_chunks(n_rows: int, n_keys: int, budget: int = 1 << 24):
    """Split rows into groups so that one [rows, keys] score matrix stays
    within ``budget`` elements.  Rows are independent, so grouping them does
    not change any row's arithmetic."""
    step = max(1, budget // max(1, n_keys))
    for a in range(0, n_rows, step):
        yield a, min(n_rows, a + step)


# ---------------------------------------------------------------------------
# O1/O2: the rank's share, computed directly over the global sequence
# ---------------------------------------------------------------------------

def rank_share_forward(q_glob, k_glob, v_glob, layout: int, world: int, rank: int,
                       causal: bool, cu_seqlens=None, scale: Optional[float] = None,
                       rows: Optional[np.ndarray] = None, heads: Optional[Sequence[int]] = None,
                       window: Tuple[int, int] = (-1, -1)):
    """Expected (out, lse) of rank ``rank``: plain attention of the rank's query
    rows over every key of the global sequence, with the global-position mask.

    q_glob [B, N, Hq, d], k_glob/v_glob [B, N, Hkv, d] in global order.
    Returns out [B, S, Hq, d] (local row order) and lse [B, Hq, S], float64.
    ``rows`` optionally restricts the computation to some local rows (then the
    returned arrays hold only those rows, in the given order); ``heads``
    restricts it to some q heads (the others are left at zero).
    """
    B, N, Hq, d = q_glob.shape
    Hkv = k_glob.shape[2]
    if scale is None:
        scale = default_scale(d)
    cu = cu_seqlens if layout in PACKED else None
    pos_q = positions(layout, N, world, rank, cu)
    if rows is not None:
        pos_q = pos_q[np.asarray(rows)]
    pos_k = np.arange(N, dtype=np.int64)
    S = len(pos_q)
    out = np.zeros((B, S, Hq, d), np.float64)
    lse = np.zeros((B, Hq, S), np.float64)
    for a, b in _row_chunks(S, N):
        mask = allowed(pos_q[a:b], pos_k, causal, cu, window)
        for bi in range(B):
            for h in (range(Hq) if heads is None else heads):
                hk = kv_head_of(h, Hq, Hkv)
                o, l = attention_rows(q_glob[bi, pos_q[a:b], h], k_glob[bi, :, hk],
                                      v_glob[bi, :, hk], mask, scale)
                out[bi, a:b, h] = o
                lse[bi, h, a:b] = l
    return out, lse


# ---------------------------------------------------------------------------
# A4: the LSE merge of two normalised partials
# ---------------------------------------------------------------------------

def lse_merge(out, lse, out_j, lse_j):
    """Fold a partial (out_j, lse_j) into a running (out, lse).

    Each partial is a normalised softmax average plus the log of its
    normaliser, so the union's normaliser is e^lse + e^lse_j and each partial
    enters with weight e^{lse - lse'} ([NT] "Numerically-Stable Output Fusion";
    the max shift is the online-softmax rescale of [IQ]).
      M    = max(lse, lse_j)
      lse' = M + ln(e^{lse - M} + e^{lse_j - M})
      out' = e^{lse - lse'} out + e^{lse_j - lse'} out_j
    A partial with lse = -inf (no visible key) is the identity.
    ``out`` is [..., R, d] with the row axis matching lse [..., R].
    """
    out = np.asarray(out, np.float64)
    out_j = np.asarray(out_j, np.float64)
    lse = np.asarray(lse, np.float64)
    lse_j = np.asarray(lse_j, np.float64)
    M = np.maximum(lse, lse_j)
    both_empty = np.isneginf(M)
    Ms = np.where(both_empty, 0.0, M)
    with np.errstate(divide="ignore"):
        new = Ms + np.log(np.exp(lse - Ms) + np.exp(lse_j - Ms))
    new = np.where(both_empty, -np.inf, new)
    w = np.where(both_empty, 0.0, np.exp(lse - np.where(both_empty, 0.0, new)))
    wj = np.where(both_empty, 0.0, np.exp(lse_j - np.where(both_empty, 0.0, new)))
    return w[..., None] * out + wj[..., None] * out_j, new


# ---------------------------------------------------------------------------
# O3: the ring-decomposed computation (a second route to the same numbers)
# ---------------------------------------------------------------------------

def ring_schedule(world: int, rank: int):
    """Ring order: the ring sends 0 -> 1 -> ... -> D-1 -> 0, so at step s rank r
    holds the block that started on rank (r - s) mod D ([RA] "Sequence sharding
    and the ring topology")."""
    return [(s, (rank - s) % world) for s in range(world)]


def ring_forward(q_glob, k_glob, v_glob, layout: int, world: int, rank: int,
                 causal: bool, cu_seqlens=None, scale: Optional[float] = None,
                 partial_out: Optional[list] = None, window: Tuple[int, int] = (-1, -1)):
    """Ring-decomposed (out, lse) of rank ``rank``: one partial attention per
    ring step against the block held at that step, folded in ring order with
    ``lse_merge`` ([NT] "Forward Pass Implementation").

    For the basic layout with a causal mask, steps with step > rank are skipped
    as the pages' rule states; other layouts run every step and a row with no
    visible key in a block contributes lse = -inf (identity under the merge).
    LLAMA3 has a single step over the gathered KV.
    """
    B, N, Hq, d = q_glob.shape
    Hkv = k_glob.shape[2]
    if scale is None:
        scale = default_scale(d)
    cu = cu_seqlens if layout in PACKED else None
    pos_q = positions(layout, N, world, rank, cu)
    S = len(pos_q)
    run_out = None
    run_lse = None
    steps = [(0, 0)] if layout == LLAMA3 else ring_schedule(world, rank)
    for s, j in steps:
        if layout == BASIC and causal and s > rank:
            continue
        pos_k = kv_positions(layout, N, world, j, cu)
        mask = allowed(pos_q, pos_k, causal, cu, window)
        o = np.zeros((B, Hq, S, d))
        l = np.zeros((B, Hq, S))
        for bi in range(B):
            for h in range(Hq):
                hk = kv_head_of(h, Hq, Hkv)
                o[bi, h], l[bi, h] = attention_rows(q_glob[bi, pos_q, h], k_glob[bi, pos_k, hk],
                                                    v_glob[bi, pos_k, hk], mask, scale)
        if partial_out is not None:
            partial_out.append((s, j, o.copy(), l.copy()))
        if run_out is None:
            run_out, run_lse = o, l
        else:
            run_out, run_lse = lse_merge(run_out, run_lse, o, l)
    return np.transpose(run_out, (0, 2, 1, 3)), run_lse


# ---------------------------------------------------------------------------
# O4: backward of the rank share (closed form of the softmax-attention gradient)
# ---------------------------------------------------------------------------

def rank_share_backward(q_glob, k_glob, v_glob, dout_local, layout: int, world: int,
                        rank: int, causal: bool, cu_seqlens=None,
                        scale: Optional[float] = None, rows: Optional[np.ndarray] = None,
                        heads: Optional[Sequence[int]] = None,
                        window: Tuple[int, int] = (-1, -1),
                        key_range: Optional[Tuple[int, int]] = None):
    """Gradients of  sum(dout * out)  over the rank's rows.

    With P_tu = exp(scale <q_t,k_u> - lse_t) on visible pairs (0 elsewhere) and
    Delta_t = <dout_t, out_t>:
      dV_u = sum_t P_tu dout_t
      dS_tu = P_tu (<dout_t, v_u> - Delta_t)
      dQ_t = scale sum_u dS_tu k_u,   dK_u = scale sum_t dS_tu q_t.
    Query heads of a GQA group add into their shared KV head.  ([NT] "Backward
    Pass and Gradient Accumulation": dq sums over steps; dk/dv of a block are
    summed over the ranks that visit it, so this rank's share is its
    contribution to every block.)

    dout_local [B, S, Hq, d] in the rank's local order.
    Returns dq [B, S, Hq, d] and dk, dv per KV block in block-major order,
    [nblocks, B, Skv, Hkv, d] (LLAMA3: one gathered block of N rows).
    ``rows`` (local row indices) and ``heads`` optionally restrict the sum to
    those query rows and heads: dq then holds those rows in the given order
    and dk, dv hold only their contribution (used to time a bounded sample).
    ``key_range`` = (k0, k1) runs the sums over the global keys [k0, k1) only.
    That changes no result when none of the rows sees a key outside the range,
    since an invisible key enters every sum with weight exactly 0; the function
    checks this and raises otherwise.  (Dropping invisible keys only saves
    time on long packed streams whose documents end far from the rank's rows.)
    """
    B, N, Hq, d = q_glob.shape
    Hkv = k_glob.shape[2]
    if scale is None:
        scale = default_scale(d)
    cu = cu_seqlens if layout in PACKED else None
    pos_q = positions(layout, N, world, rank, cu)
    local = np.arange(len(pos_q)) if rows is None else np.asarray(rows)
    pos_q = pos_q[local]
    S = len(pos_q)
    pos_k = np.arange(N, dtype=np.int64)
    if key_range is not None:
        k0, k1 = key_range
        for a, b in _row_chunks(S, N):
            vis = allowed(pos_q[a:b], pos_k, causal, cu, window)
            if vis[:, :k0].any() or vis[:, k1:].any():
                raise ValueError("key_range drops a visible key")
        pos_k = np.arange(k0, k1, dtype=np.int64)
    mask = allowed(pos_q, pos_k, causal, cu, window)
    nb = num_blocks(layout, world)
    blocks = [kv_positions(layout, N, world, j, cu) for j in range(nb)]
    dq = np.zeros((B, S, Hq, d))
    dk = np.zeros((nb, B, len(blocks[0]), Hkv, d))
    dv = np.zeros((nb, B, len(blocks[0]), Hkv, d))
    q_heads = list(range(Hq)) if heads is None else list(heads)
    for bi in range(B):
        for hk in sorted({kv_head_of(h, Hq, Hkv) for h in q_heads}):
            # gradients of every global key of KV head hk, summed over its q heads
            dk_h = np.zeros((N, d))
            dv_h = np.zeros((N, d))
            k = k_glob[bi, pos_k, hk].astype(np.float64)
            v = v_glob[bi, pos_k, hk].astype(np.float64)
            for h in q_heads:
                if kv_head_of(h, Hq, Hkv) != hk:
                    continue
                q = q_glob[bi, pos_q, h].astype(np.float64)
                do = dout_local[bi, local, h].astype(np.float64)
                out, lse = attention_rows(q, k, v, mask, scale)
                s = scale * (q @ k.T)
                finite = np.isfinite(lse)
                p = np.where(mask & finite[:, None],
                             np.exp(np.where(mask, s, 0.0) - np.where(finite, lse, 0.0)[:, None]), 0.0)
                delta = (do * out).sum(axis=1)
                dv_h[pos_k] += p.T @ do
                ds = p * (do @ v.T - delta[:, None])
                dq[bi, :, h] = scale * (ds @ k)
                dk_h[pos_k] += scale * (ds.T @ q)
            for j, pk in enumerate(blocks):
                dk[j, bi, :, hk] = dk_h[pk]
                dv[j, bi, :, hk] = dv_h[pk]
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Work counts (used for pins and for the bench's algorithmic flop count)
# ---------------------------------------------------------------------------

def step_pair_counts(layout: int, n: int, world: int, rank: int, causal: bool,
                     cu_seqlens=None, window: Tuple[int, int] = (-1, -1)):
    """Visible (query row, key) pairs of every ring step, per (batch, q-head):
    a list of (step, block, pairs) in ring order."""
    cu = cu_seqlens if layout in PACKED else None
    pos_q = positions(layout, n, world, rank, cu)
    steps = [(0, 0)] if layout == LLAMA3 else ring_schedule(world, rank)
    res = []
    for s, j in steps:
        pos_k = kv_positions(layout, n, world, j, cu)
        total = 0
        for a, b in _row_chunks(len(pos_q), len(pos_k)):
            total += int(allowed(pos_q[a:b], pos_k, causal, cu, window).sum())
        res.append((s, j, total))
    return res
