"""Plain float64 reference for fused causal grouped-query attention and paged decode.

TEST INFRASTRUCTURE ONLY.  This module is the oracle that the HIP library is
checked against.  Only the tests, the package smoke check and the benchmark's
CPU-baseline leg may import it; the library and its binding never do.  It
shares no code with the GPU path.

What it computes is the unfused ("MATH") attention that the pages describe as
the fallback that materialises the full S x S score matrix (page "Gemma4 FFPA
attention backend support for accelerating Gemma4-family training", operator
table and section Debugging notes; page "Root cause analysis: Gemma4
sliding-window BF16 cuDNN SDPA NaN on H100", operator table under "Why cuDNN
SDPA is the affected path"), carried out in float64 as the global FP32 upcast
of the second page suggests (section Summary, "Proposed fix"), one
(batch, head) unit at a time with explicit matrix products, exp, max and sum.
No attention routine of any library is called.

Readings adopted where the pages are silent (each is listed in the design notes):
* grouped-query heads follow the repeat-KV path of the first page (Debugging
  notes): query head h reads key/value head h // (Hq // Hkv);
* a 2D bool padding mask selects the variable-length path (first page,
  Integration): row b holds len_b valid tokens as a prefix; padded queries do
  not exist and padded keys are invisible;
* the sliding window admits key j for query i when i - W < j <= i;
* a query row with no visible key returns O = 0 and LSE = 0 rather than NaN
  (fourth page, "What broke correctness and had to be dropped": rows whose
  mask is all False must stay safe);
* LSE is the natural-log log-sum-exp of the scaled scores of the visible keys;
* the paged decode query sits at position ctx_b - 1 and sees every cached
  token t < ctx_b (fourth page, Architecture notes: PagedKVCache + PageTable);
* a paged prefill step (fourth page, "What's left on the table": prefill and decode
  rows in one step) gives sequence b n_b new query rows, the newest of its ctx_b
  cached tokens: row i sits at position ctx_b - n_b + i and sees the cached tokens
  at or before it (and inside the window); a row at a negative position sees none
  and returns O = 0, LSE = 0;
* a chunk pair of the ring path (first page, Integration) places query i at position
  q_pos0 + i and key j at k_pos0 + j; a row that sees no key of the chunk has LSE = -inf
  (the identity of the log-sum-exp merge) and O = 0;
* the softcap that the first page's gate sends to the eager path (Integration) is the tanh
  soft-capping of the scaled scores, s -> cap * tanh(s / cap), applied before masking;
  cap <= 0 means none.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "visibility", "lengths_from_pad_mask", "lengths_from_cu_seqlens",
    "scores", "unit_forward", "unit_backward", "unit_forward_backward",
    "attention_forward", "attention_backward", "attention_forward_head", "attention_backward_group", "attention_group",
    "attention_forward_packed", "attention_backward_packed",
    "gather_pages", "paged_append", "paged_decode", "paged_decode_one", "attention_rows",
    "chunk_visibility", "attention_forward_chunk", "attention_backward_chunk", "lse_merge",
    "paged_prefill",
]


# ---------------------------------------------------------------------------
# Which keys a query sees
# ---------------------------------------------------------------------------
def visibility(n: int, causal: bool, window: int) -> np.ndarray:
    """(n, n) bool over the valid prefix of one sequence: entry (i, j) is True when query i sees key j.

    Causal keeps j <= i; a window W > 0 keeps j > i - W.  Positions at or past
    the sequence's length are not part of the block at all: padded queries do
    not exist and padded keys are invisible.
    """
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    vis = np.ones((n, n), dtype=bool)
    if causal:
        vis &= j <= i
    if window > 0:
        vis &= j > i - window
    return vis


def lengths_from_pad_mask(mask: np.ndarray) -> np.ndarray:
    """(B, S) bool/uint8 right-padded mask -> (B,) valid lengths; rejects a mask that is not a prefix."""
    mask = np.asarray(mask).astype(bool)
    lengths = mask.sum(axis=1)
    S = mask.shape[1]
    expect = np.arange(S)[None, :] < lengths[:, None]
    if not np.array_equal(mask, expect):
        raise ValueError("padding mask is not a right-padded prefix mask")
    return lengths.astype(np.int64)


def lengths_from_cu_seqlens(cu: np.ndarray) -> np.ndarray:
    cu = np.asarray(cu, dtype=np.int64)
    if cu[0] != 0 or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0 and be non-decreasing")
    return np.diff(cu)


# ---------------------------------------------------------------------------
# One (batch, head) unit
# ---------------------------------------------------------------------------
def scores(q, k, scale, softcap=0.0):
    """Scaled scores scale * q k^T, soft-capped to cap * tanh(s / cap) when cap = softcap > 0.
    Returns the scores and their derivative with respect to the uncapped scaled score
    (1 - tanh^2, or 1 without a cap)."""
    s = scale * (q @ k.T)
    if softcap > 0:
        t = np.tanh(s / softcap)
        return softcap * t, 1.0 - t * t
    return s, np.ones_like(s)


def unit_forward(q, k, v, scale, vis, softcap=0.0):
    """One head: q (n, D), k (n, D), v (n, D) float64 and vis (n, n).

    Returns O (n, D), LSE (n,) and the probabilities P (n, n).  Every key row
    passed in must be finite: invisible keys get probability exactly 0, which
    removes a finite value but not a NaN.
    S = scale * q k^T (soft-capped when softcap > 0) with invisible entries at -inf;
    P = row softmax of S; O = P v; LSE = rowmax + ln(sum exp(S - rowmax)).
    """
    s, _ = scores(q, k, scale, softcap)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    live = np.isfinite(m)
    m0 = np.where(live, m, 0.0)
    e = np.exp(s - m0[:, None])          # exp(-inf) = 0 on invisible entries
    l = e.sum(axis=1)
    l_safe = np.where(live, l, 1.0)
    p = e / l_safe[:, None]
    o = p @ v
    lse = np.where(live, m0 + np.log(l_safe), 0.0)
    return o, lse, p


def unit_forward_backward(q, k, v, do, scale, vis, softcap=0.0):
    """Forward and gradients of sum(O * dO) for one head from one evaluation of the softmax:
    returns O, LSE, dQ, dK, dV (this head's share of dK, dV).

    dP = dO v^T; delta_i = sum_j P_ij dP_ij; dS = P * (dP - delta), times the cap's
    derivative 1 - tanh^2 under a softcap; dQ = scale dS k; dK = scale dS^T q; dV = P^T dO.
    """
    o, lse, p = unit_forward(q, k, v, scale, vis, softcap)
    _, deriv = scores(q, k, scale, softcap)
    dp = do @ v.T
    delta = (p * dp).sum(axis=1)
    ds = p * (dp - delta[:, None]) * deriv
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    dv = p.T @ do
    return o, lse, dq, dk, dv


def unit_backward(q, k, v, do, scale, vis, softcap=0.0):
    """Gradients of sum(O * dO) for one head; returns dQ, dK, dV (this head's share of dK, dV)."""
    return unit_forward_backward(q, k, v, do, scale, vis, softcap)[2:]


# ---------------------------------------------------------------------------
# Batched layouts: q, o, dO (B, S, Hq, D); k, v (B, S, Hkv, D); LSE (B, Hq, S)
# ---------------------------------------------------------------------------
def _lengths(B, S, lengths):
    if lengths is None:
        return np.full(B, S, dtype=np.int64)
    return np.asarray(lengths, dtype=np.int64)


def attention_forward_head(q, k, v, b, h, scale, causal=True, window=0, lengths=None, softcap=0.0):
    """O (S, D) and LSE (S,) of one (batch, query-head) unit; rows at or past the length are 0."""
    B, S, Hq, D = q.shape
    r = Hq // k.shape[2]
    n = int(_lengths(B, S, lengths)[b])
    o = np.zeros((S, D))
    lse = np.zeros(S)
    if n > 0:
        o[:n], lse[:n], _ = unit_forward(q[b, :n, h], k[b, :n, h // r], v[b, :n, h // r], scale,
                                         visibility(n, causal, window), softcap)
    return o, lse


def attention_forward(q, k, v, scale, causal=True, window=0, lengths=None, softcap=0.0):
    """Returns O (B, S, Hq, D) float64 and LSE (B, Hq, S) float64."""
    B, S, Hq, D = q.shape
    o = np.zeros((B, S, Hq, D))
    lse = np.zeros((B, Hq, S))
    for b in range(B):
        for h in range(Hq):
            o[b, :, h], lse[b, h] = attention_forward_head(q, k, v, b, h, scale, causal, window, lengths,
                                                           softcap)
    return o, lse


def attention_backward_group(q, k, v, do, b, g, scale, causal=True, window=0, lengths=None, softcap=0.0):
    """dQ (S, r, D) for the r query heads of kv-head g, and dK, dV (S, D) summed over them.

    Rows of dQ and keys of dK, dV at or past the sequence length are 0.
    """
    B, S, Hq, D = q.shape
    r = Hq // k.shape[2]
    n = int(_lengths(B, S, lengths)[b])
    dq = np.zeros((S, r, D))
    dk = np.zeros((S, D))
    dv = np.zeros((S, D))
    if n == 0:
        return dq, dk, dv
    vis = visibility(n, causal, window)
    for i in range(r):                   # fixed head order
        h = g * r + i
        dqh, dkh, dvh = unit_backward(q[b, :n, h], k[b, :n, g], v[b, :n, g], do[b, :n, h], scale, vis, softcap)
        dq[:n, i] = dqh
        dk[:n] += dkh
        dv[:n] += dvh
    return dq, dk, dv


def attention_group(q, k, v, do, b, g, scale, causal=True, window=0, lengths=None, softcap=0.0):
    """Everything one (batch, kv head) unit produces, from one softmax evaluation per query head:
    O (S, r, D) and LSE (r, S) of the r query heads of kv head g, their dQ (S, r, D), and dK, dV
    (S, D) summed over them in head order.  Rows and keys at or past the length are 0."""
    B, S, Hq, D = q.shape
    r = Hq // k.shape[2]
    n = int(_lengths(B, S, lengths)[b])
    o = np.zeros((S, r, D))
    lse = np.zeros((r, S))
    dq = np.zeros((S, r, D))
    dk = np.zeros((S, D))
    dv = np.zeros((S, D))
    if n == 0:
        return o, lse, dq, dk, dv
    vis = visibility(n, causal, window)
    for i in range(r):                   # fixed head order
        h = g * r + i
        oh, lh, dqh, dkh, dvh = unit_forward_backward(q[b, :n, h], k[b, :n, g], v[b, :n, g], do[b, :n, h], scale,
                                                      vis, softcap)
        o[:n, i], lse[i, :n], dq[:n, i] = oh, lh, dqh
        dk[:n] += dkh
        dv[:n] += dvh
    return o, lse, dq, dk, dv


def attention_backward(q, k, v, do, scale, causal=True, window=0, lengths=None, softcap=0.0):
    """Returns dQ (B, S, Hq, D), dK and dV (B, S, Hkv, D), float64."""
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    r = Hq // Hkv
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(B):
        for g in range(Hkv):
            gq, gk, gv = attention_backward_group(q, k, v, do, b, g, scale, causal, window, lengths, softcap)
            dq[b, :, g * r:(g + 1) * r] = gq
            dk[b, :, g] = gk
            dv[b, :, g] = gv
    return dq, dk, dv


def attention_rows(q, k, v, do, b, h, rows, scale, causal=True, window=0, lengths=None, softcap=0.0):
    """O, LSE and dQ of selected query rows of one (batch, head), one row at a time.

    Everything a query row needs is row-local: its visible keys, its softmax, and for
    the gradient delta_i = sum_j P_ij dP_ij.  Rows at or past the length give zeros.
    do may be None (then dQ is not computed).  Returns arrays indexed like `rows`.
    """
    B, S, Hq, D = q.shape
    r = Hq // k.shape[2]
    g = h // r
    n = int(_lengths(B, S, lengths)[b])
    rows = np.asarray(rows)
    o = np.zeros((len(rows), D))
    lse = np.zeros(len(rows))
    dq = np.zeros((len(rows), D))
    for x, i in enumerate(rows):
        i = int(i)
        if i >= n:
            continue
        vis = visibility(n, causal, window)[i][None, :]
        kk, vv = k[b, :n, g], v[b, :n, g]
        oi, li, p = unit_forward(q[b, i, h][None, :], kk, vv, scale, vis, softcap)
        o[x], lse[x] = oi[0], li[0]
        if do is not None:
            _, deriv = scores(q[b, i, h][None, :], kk, scale, softcap)
            dp = do[b, i, h][None, :] @ vv.T
            delta = (p * dp).sum(axis=1)
            ds = p * (dp - delta[:, None]) * deriv
            dq[x] = scale * (ds @ kk)[0]
    return o, lse, dq


# Packed rows (cu_seqlens): q, o, dO (T, Hq, D); k, v (T, Hkv, D); LSE (Hq, T).
def attention_forward_packed(q, k, v, cu_seqlens, scale, causal=True, window=0, softcap=0.0):
    lengths = lengths_from_cu_seqlens(cu_seqlens)
    T, Hq, D = q.shape
    r = Hq // k.shape[1]
    o = np.zeros(q.shape)
    lse = np.zeros((Hq, T))
    for b, n in enumerate(lengths):
        s0 = int(cu_seqlens[b])
        n = int(n)
        if n == 0:
            continue
        vis = visibility(n, causal, window)
        for h in range(Hq):
            o[s0:s0 + n, h], lse[h, s0:s0 + n], _ = unit_forward(
                q[s0:s0 + n, h], k[s0:s0 + n, h // r], v[s0:s0 + n, h // r], scale, vis, softcap)
    return o, lse


def attention_backward_packed(q, k, v, do, cu_seqlens, scale, causal=True, window=0, softcap=0.0):
    lengths = lengths_from_cu_seqlens(cu_seqlens)
    T, Hq, D = q.shape
    r = Hq // k.shape[1]
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b, n in enumerate(lengths):
        s0 = int(cu_seqlens[b])
        n = int(n)
        if n == 0:
            continue
        vis = visibility(n, causal, window)
        for h in range(Hq):
            g = h // r
            a, bk, bv = unit_backward(q[s0:s0 + n, h], k[s0:s0 + n, g], v[s0:s0 + n, g],
                                      do[s0:s0 + n, h], scale, vis, softcap)
            dq[s0:s0 + n, h] = a
            dk[s0:s0 + n, g] += bk
            dv[s0:s0 + n, g] += bv
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Chunks of a sequence: the unit of ring context parallelism.  The first page routes the
# full-attention chunks of its ring path through the fused kernel (section Integration:
# dense or varlen per chunk); a chunk pair is a query chunk against one key/value chunk at
# known positions, and the partial results of a row over its key chunks are combined by
# their log-sum-exp.
# ---------------------------------------------------------------------------
def chunk_visibility(nq: int, nk: int, q_pos0: int, k_pos0: int, causal: bool, window: int) -> np.ndarray:
    """(nq, nk) bool: query i sits at position q_pos0 + i and key j at k_pos0 + j; the key is
    visible when k_pos <= q_pos (causal) and k_pos > q_pos - W (window W > 0)."""
    qp = q_pos0 + np.arange(nq)[:, None]
    kp = k_pos0 + np.arange(nk)[None, :]
    vis = np.ones((nq, nk), dtype=bool)
    if causal:
        vis &= kp <= qp
    if window > 0:
        vis &= kp > qp - window
    return vis


def attention_forward_chunk(q, k, v, scale, causal, window, q_pos0, k_pos0, softcap=0.0):
    """Partial attention of a query chunk q (B, Sq, Hq, D) against one key/value chunk k, v
    (B, Sk, Hkv, D): O (B, Sq, Hq, D) and LSE (B, Hq, Sq) over the chunk's visible keys.  A row
    that sees no key of the chunk gets O = 0 and LSE = -inf, the identity of lse_merge."""
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    r = Hq // Hkv
    vis = chunk_visibility(Sq, Sk, q_pos0, k_pos0, causal, window)
    live = vis.any(axis=1)
    o = np.zeros((B, Sq, Hq, D))
    lse = np.full((B, Hq, Sq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            ob, lb, _ = unit_forward(q[b, :, h], k[b, :, h // r], v[b, :, h // r], scale, vis, softcap)
            o[b, :, h] = ob
            lse[b, h] = np.where(live, lb, -np.inf)
    return o, lse


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Combine two partial results of the same rows over disjoint key sets:
    L = ln(e^La + e^Lb), O = e^(La - L) O_a + e^(Lb - L) O_b.  A partial with LSE = -inf adds
    nothing; two of them give O = 0, LSE = -inf.  o: (B, S, H, D), lse: (B, H, S)."""
    m = np.maximum(lse_a, lse_b)
    live = np.isfinite(m)
    m0 = np.where(live, m, 0.0)
    wa = np.exp(lse_a - m0)              # exp(-inf) = 0
    wb = np.exp(lse_b - m0)
    tot = wa + wb
    lse = np.where(live, m0 + np.log(np.where(live, tot, 1.0)), -np.inf)
    tot_safe = np.where(live, tot, 1.0)
    fa = np.transpose(wa / tot_safe, (0, 2, 1))[..., None]   # (B, S, H, 1)
    fb = np.transpose(wb / tot_safe, (0, 2, 1))[..., None]
    return fa * o_a + fb * o_b, lse


def attention_backward_chunk(q, k, v, o, lse, do, scale, causal, window, q_pos0, k_pos0, softcap=0.0):
    """Gradient contributions of one (query chunk, key chunk) pair, given the rows' final O
    (B, Sq, Hq, D) and LSE (B, Hq, Sq) over all their keys: P = exp(scale q k^T - LSE) on the
    chunk's visible entries, delta = rowsum(dO * O), dS = P (dP - delta), dQ = scale dS k,
    dK = scale dS^T q and dV = P^T dO (dK, dV summed over the group's query heads).  Summing
    dQ over a row's key chunks, and dK, dV over a key chunk's query chunks, gives the full
    gradients."""
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    r = Hq // Hkv
    vis = chunk_visibility(Sq, Sk, q_pos0, k_pos0, causal, window)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(B):
        for h in range(Hq):
            g = h // r
            s, deriv = scores(q[b, :, h], k[b, :, g], scale, softcap)
            live = np.isfinite(lse[b, h])[:, None]       # a row that sees no key has no gradient
            arg = np.where(vis & live, s - np.where(live, lse[b, h][:, None], 0.0), -np.inf)
            p = np.exp(arg)
            dp = do[b, :, h] @ v[b, :, g].T
            delta = (do[b, :, h] * o[b, :, h]).sum(axis=1)
            ds = p * (dp - delta[:, None]) * deriv
            dq[b, :, h] = scale * (ds @ k[b, :, g])
            dk[b, :, g] += scale * (ds.T @ q[b, :, h])
            dv[b, :, g] += p.T @ do[b, :, h]
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Paged decode: q (B, Hq, D); caches (num_pages, page_size, Hkv, D); table (B, max_pages)
# ---------------------------------------------------------------------------
def gather_pages(cache, table_row, ctx, page_size):
    """Logical tokens 0..ctx-1 of one sequence, (ctx, Hkv, D): token t lives in page
    table_row[t // page_size] at slot t % page_size."""
    t = np.arange(int(ctx))
    return cache[np.asarray(table_row)[t // page_size], t % page_size]


def paged_append(cache, block_table, ctx_lens, new, page_size=16):
    """A copy of cache (num_pages, page_size, Hkv, D) with the n newest tokens of each sequence
    written in: new[b, i] (new is (B, n, Hkv, D)) goes to logical position ctx_b - n + i, i.e. to
    slot (pos % page_size) of page block_table[b][pos // page_size] (the page-table mapping of the
    fourth page, Architecture notes).  Positions below 0 or at or past the table's end, and table
    entries outside [0, num_pages), are skipped.  Works on any dtype (it only moves values)."""
    out = np.array(cache, copy=True)
    B, n = new.shape[0], new.shape[1]
    num_pages, table_cols = cache.shape[0], block_table.shape[1]
    for b in range(B):
        ctx = int(min(max(int(ctx_lens[b]), 0), table_cols * page_size))
        for i in range(n):
            pos = ctx - n + i
            if pos < 0:
                continue
            page = int(block_table[b, pos // page_size])
            if 0 <= page < num_pages:
                out[page, pos % page_size] = new[b, i]
    return out


def paged_decode_one(q, k_cache, v_cache, block_table, ctx_lens, scale, b, page_size=16, softcap=0.0):
    """O (Hq, D) for one sequence's single query token, placed at position ctx_b - 1."""
    Hq, D = q.shape[1], q.shape[2]
    Hkv = k_cache.shape[2]
    r = Hq // Hkv
    ctx = int(ctx_lens[b])
    out = np.zeros((Hq, D))
    if ctx == 0:
        return out
    kk = gather_pages(k_cache, block_table[b], ctx, page_size)
    vv = gather_pages(v_cache, block_table[b], ctx, page_size)
    vis = np.ones((1, ctx), dtype=bool)
    for h in range(Hq):
        o, _, _ = unit_forward(q[b, h][None, :], kk[:, h // r], vv[:, h // r], scale, vis, softcap)
        out[h] = o[0]
    return out


def paged_prefill(q, k_cache, v_cache, block_table, cu_q, ctx_lens, scale, window=0, page_size=16, softcap=0.0):
    """New query rows of several sequences against their paged caches, causal.  q (T, Hq, D) holds
    sequence b's n_b = cu_q[b+1] - cu_q[b] rows from cu_q[b] on; they are the newest of the ctx_b
    tokens in its cache, at positions ctx_b - n_b .. ctx_b - 1.  The sequence's tokens are read
    through its page-table row (gather_pages) and its rows computed as a chunk pair with the
    queries from q_pos0 = ctx_b - n_b and the keys from k_pos0 = 0.  Returns O (T, Hq, D) and
    LSE (Hq, T); a row that sees no token has O = 0 and LSE = 0."""
    T, Hq, D = q.shape
    o = np.zeros((T, Hq, D))
    lse = np.zeros((Hq, T))
    for b in range(len(cu_q) - 1):
        lo, hi = int(cu_q[b]), int(cu_q[b + 1])
        ctx = int(ctx_lens[b])
        if hi == lo or ctx == 0:
            continue
        kk = gather_pages(k_cache, block_table[b], ctx, page_size)[None]
        vv = gather_pages(v_cache, block_table[b], ctx, page_size)[None]
        ob, lb = attention_forward_chunk(q[None, lo:hi], kk, vv, scale, True, window, ctx - (hi - lo), 0, softcap)
        o[lo:hi] = ob[0]
        lse[:, lo:hi] = np.where(np.isfinite(lb[0]), lb[0], 0.0)
    return o, lse


def paged_decode(q, k_cache, v_cache, block_table, ctx_lens, scale, page_size=16, softcap=0.0):
    """O (B, Hq, D) float64."""
    B = q.shape[0]
    return np.stack([paged_decode_one(q, k_cache, v_cache, block_table, ctx_lens, scale, b, page_size, softcap)
                     for b in range(B)])
