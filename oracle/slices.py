"""Slice-list masks -- TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

"03 · 长文负载均衡", section 4.4 (MagiAttention): an irregular mask is written as a
list of slices, each a query range, a key range and a mask type on that rectangle;
the types are FULL, CAUSAL, INV-CAUSAL and BI-CAUSAL, and slices combine to express
anything from varlen causal to varlen block-causal masks.  The mask of the list is
the union of its slices' masks.

Readings where the page is silent:
* CAUSAL on a rectangle of Lq query rows and Lk keys is aligned at the bottom-right
  corner: row r (0-based in the slice) sees keys 0 .. r + (Lk - Lq) of the slice, so
  the last row sees every key (for Lq = Lk this is the usual causal triangle);
* INV-CAUSAL is aligned at the top-left corner: row r sees keys r .. Lk - 1; BI-CAUSAL
  is both at once, keys r .. r + (Lk - Lq) (a band; a sliding window of w keys over
  rows q0.. is the BI-CAUSAL rectangle of those rows against keys q0 - w + 1 ..);
* slices over the same query range must cover disjoint key ranges (the union is then
  a plain sum of their pairs), and two different query ranges must not overlap;
* a query row covered by no slice sees nothing: lse = -inf, out = 0 here.

A slice is (q_start, q_len, k_start, k_len, kind) with kind 0 = FULL, 1 = CAUSAL,
2 = INV-CAUSAL, 3 = BI-CAUSAL.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import ROW_BLOCK, _as_f64, attend

FULL, CAUSAL, INV_CAUSAL, BI_CAUSAL = 0, 1, 2, 3
FAR = 1 << 30  # a bound offset that no position reaches: no bound on that side


def visible(slices, n_q, n_k):
    """The explicit boolean mask [n_q, n_k] of a slice list."""
    m = np.zeros((n_q, n_k), dtype=bool)
    for (qs, ql, ks, kl, kind) in slices:
        r = np.arange(ql)[:, None]
        c = np.arange(kl)[None, :]
        blk = np.ones((ql, kl), dtype=bool)
        if kind in (CAUSAL, BI_CAUSAL):
            blk &= c <= r + (kl - ql)
        if kind in (INV_CAUSAL, BI_CAUSAL):
            blk &= c >= r
        m[qs:qs + ql, ks:ks + kl] |= blk
    return m


def slices_attention(q, k, v, slices, heads, kv_heads, scale=None):
    """out [n_q,H,d] and lse [H,n_q] of q [n_q,H,d] against k/v [n_k,H_kv,d] under the mask."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    n_q, H, d = q.shape
    n_k = k.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    vis = visible(slices, n_q, n_k)
    G = heads // kv_heads
    out = np.zeros((n_q, H, v.shape[2]))
    lse = np.full((H, n_q), -np.inf)
    for b in range(0, n_q, ROW_BLOCK):
        rows = np.arange(b, min(n_q, b + ROW_BLOCK))
        cols = np.nonzero(vis[rows].any(axis=0))[0]
        for h in range(H):
            o, l = attend(q[rows, h], k[cols, h // G], v[cols, h // G], vis[np.ix_(rows, cols)], scale)
            out[rows, h] = o
            lse[h, rows] = l
    return out, lse


def fragments(slices, n_q=None):
    """Planner fragments of a slice list (query ranges in order, each with the key spans of
    its slices): (q_start, q_len, q_pos0, [span, ...]) with query positions from 0 in the
    range.  A span (k_start, k_len, k_pos0) makes key j visible to row r iff
    k_pos0 + j <= r: CAUSAL at k_pos0 = q_len - k_len, FULL far below.  Kinds with a lower
    bound add k_lo, (k_start, k_len, k_pos0, k_lo), with key j visible only if k_lo + j >= r:
    INV-CAUSAL (k_pos0 far below, k_lo = 0) and BI-CAUSAL (both).  Rows no slice covers
    form fragments with no span (their lse is -inf): before and between the ranges, and,
    given the query count n_q, after the last one."""
    frags = []
    end = 0  # rows before `end` belong to a fragment already
    for (qs, ql, ks, kl, kind) in slices:
        hi = (ql - kl) if kind in (CAUSAL, BI_CAUSAL) else -FAR
        span = (ks, kl, hi) if kind in (FULL, CAUSAL) else (ks, kl, hi, 0)
        if frags and frags[-1][0] == qs and frags[-1][1] == ql:
            frags[-1][3].append(span)
        else:
            if qs > end:  # rows no slice covers: a fragment without keys (lse = -inf)
                frags.append((end, qs - end, 0, []))
            frags.append((qs, ql, 0, [span]))
            end = qs + ql
    if n_q is not None and end < n_q:
        frags.append((end, n_q - end, 0, []))
    return frags


def block_causal_slices(lengths, frame):
    """Varlen block-causal (MAGI-1's mask in section 4.4): every document is cut into frames
    of ``frame`` tokens; a frame's rows see every key of their document up to the frame's
    end.  One FULL slice per frame."""
    out = []
    start = 0
    for n in lengths:
        for f0 in range(0, n, frame):
            fl = min(frame, n - f0)
            out.append((start + f0, fl, start, f0 + fl, FULL))
        start += n
    return out


def sliding_window_slices(lengths, window, rows=64):
    """Per-document causal sliding window: row i of a document sees its keys i - window + 1
    .. i.  Rows go in ranges of ``rows``; a range starting at q0 is the BI-CAUSAL band
    against keys q0 - window + 1 .. q0 + rows - 1, cut at the document start (where it
    becomes CAUSAL against keys 0 .. q0 + rows - 1 of the document, while q0 + rows - 1 <
    window; the rows near the start see every earlier key)."""
    out, start = [], 0
    for n in lengths:
        for q0 in range(0, n, rows):
            ql = min(rows, n - q0)
            k0 = q0 - window + 1
            if k0 >= 0:
                out.append((start + q0, ql, start + k0, ql + window - 1, BI_CAUSAL))
            elif q0 + ql - 1 - window + 1 <= 0:  # no row of the range loses a key: plain causal
                out.append((start + q0, ql, start, q0 + ql, CAUSAL))
            else:  # mixed: row by row
                for r in range(ql):
                    i = q0 + r
                    lo = max(0, i - window + 1)
                    out.append((start + i, 1, start + lo, i - lo + 1, FULL))
        start += n
    return out


def varlen_causal_slices(lengths):
    """The per-document causal mask as slices: one square CAUSAL slice per document."""
    out, start = [], 0
    for n in lengths:
        if n:
            out.append((start, n, start, n, CAUSAL))
        start += n
    return out


def shared_question_slices(lengths):
    """The shared-question mask as slices: the question causal on itself; every answer FULL
    on the question and CAUSAL on itself."""
    Q = lengths[0]
    out = [(0, Q, 0, Q, CAUSAL)] if Q else []
    start = Q
    for n in lengths[1:]:
        if n:
            if Q:
                out.append((start, n, 0, Q, FULL))
            out.append((start, n, start, n, CAUSAL))
        start += n
    return out
