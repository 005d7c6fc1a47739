"""Reference tile enumerator -- TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The method skips attention blocks whose mask is all zero: only (query block,
key block) pairs with at least one visible pair become work ("03 · 长文负载均衡",
section 3.2, DCP's computation blocks), the work of a block is billed as its
exact count of visible (query, key) pairs (same section, Libra TAP), a mask is
described as rectangles of full or causal kind ("03 · 长文负载均衡", section 4.4,
MagiAttention's AttnSlice), and work is handed out longest first by an
estimate of its time ("03 · 长文负载均衡", section 2.1, VRSP; "数据并行负载均衡",
sections 4.3-4.4, LPT over costs from a fitted model).  The estimate here is
the number of key blocks a tile sweeps: a kernel spends a block's time whatever
share of the block is visible, and a short query block is billed as a whole
tile ("03 · 长文负载均衡", section 3.3).

Tiling rule written out here (the plan the library must reproduce exactly):

1. Query *fragments*.  Varlen causal: one fragment per document, query
   positions counted from 0 inside the document.  Shared question: the
   question is a fragment with positions from 0; answer a is a fragment whose
   positions start at Q (the question length), so the question lies wholly
   "before" every answer.  Block step: maximal runs of tokens with equal
   document id and consecutive global positions.
2. Key *spans* of a fragment (start index, length, position of its first key).
   Varlen causal: the document itself.  Shared question: the question (for
   the question and every answer) and, for an answer, the answer itself with
   positions from Q.  Block step: every key/value run (same run rule) of the
   same document, in key order.  Key j of a span is visible to query i of the
   fragment iff pos(j) <= pos(i).
3. *Tiles*: each fragment is cut into tiles of BM query rows anchored at the
   fragment start (the last tile may be shorter).  A tile keeps each span
   clipped to the keys its last row can see; spans clipped to nothing are
   dropped.  Tiles with no span remain (the kernel writes lse = -inf there).
4. *Cost* of a tile = its exact number of visible (query, key) pairs for one
   head, counted row by row.  *Blocks* of a tile = sum over its spans of
   ceil(keys kept / BLOCK_KEYS), the key blocks of BLOCK_KEYS keys it sweeps.
5. *Order*: blocks descending, ties by natural order (fragment order, then
   tile order inside the fragment).
"""
from __future__ import annotations

import numpy as np

BLOCK_KEYS = 64  # keys per block the attention kernel steps through


def fragments_varlen(cu_seqlens, mask="causal_doc"):
    """List of (q_start, q_len, q_pos0, [(k_start, k_len, k_pos0), ...])."""
    cu = [int(x) for x in cu_seqlens]
    frags = []
    if mask == "causal_doc":
        for s in range(len(cu) - 1):
            n = cu[s + 1] - cu[s]
            if n > 0:
                frags.append((cu[s], n, 0, [(cu[s], n, 0)]))
    elif mask == "shared_question":
        Q = cu[1] - cu[0]
        if Q > 0:
            frags.append((cu[0], Q, 0, [(cu[0], Q, 0)]))
        for s in range(1, len(cu) - 1):
            n = cu[s + 1] - cu[s]
            if n == 0:
                continue
            spans = [(cu[0], Q, 0)] if Q > 0 else []
            spans.append((cu[s], n, Q))
            frags.append((cu[s], n, Q, spans))
    else:
        raise ValueError(mask)
    return frags


def runs(pos, doc):
    """Maximal runs of equal doc id and consecutive positions: (start, len, pos0, doc)."""
    pos = [int(x) for x in pos]
    doc = [int(x) for x in doc]
    out = []
    for i in range(len(pos)):
        if i == 0 or doc[i] != doc[i - 1] or pos[i] != pos[i - 1] + 1:
            out.append([i, 1, pos[i], doc[i]])
        else:
            out[-1][1] += 1
    return [tuple(r) for r in out]


def fragments_block(q_pos, q_doc, kv_pos, kv_doc):
    q_runs = runs(q_pos, q_doc)
    kv_runs = runs(kv_pos, kv_doc)
    frags = []
    for (qs, ql, qp0, qd) in q_runs:
        spans = [(ks, kl, kp0) for (ks, kl, kp0, kd) in kv_runs if kd == qd]
        frags.append((qs, ql, qp0, spans))
    return frags


def visible_in_span(row_pos, k_len, k_pos0):
    """Number of keys of a span visible to one query at position row_pos."""
    return max(0, min(k_len, row_pos - k_pos0 + 1))


def tiles(frags, bm):
    """Tiles in natural order: dicts with q_start, q_len, q_pos0, spans, cost."""
    out = []
    for (qs, ql, qp0, spans) in frags:
        for t0 in range(0, ql, bm):
            n = min(bm, ql - t0)
            p0 = qp0 + t0
            last = p0 + n - 1
            kept = []
            for (ks, kl, kp0) in spans:
                keep = min(kl, last - kp0 + 1)
                if keep > 0:
                    kept.append((ks, keep, kp0))
            cost = 0
            for r in range(n):
                for (ks, kl, kp0) in kept:
                    cost += visible_in_span(p0 + r, kl, kp0)
            blocks = sum(-(-kl // BLOCK_KEYS) for (ks, kl, kp0) in kept)
            out.append(dict(q_start=qs + t0, q_len=n, q_pos0=p0, spans=kept, cost=cost, blocks=blocks))
    return out


def lpt_order(tile_list, key="blocks"):
    """Indices of tiles, `key` descending, ties in natural order."""
    return sorted(range(len(tile_list)), key=lambda i: (-tile_list[i][key], i))


def plan(frags, bm):
    """The full reference plan: tiles in longest-first order."""
    t = tiles(frags, bm)
    return [t[i] for i in lpt_order(t)]


def total_pairs(plan_tiles):
    return sum(t["cost"] for t in plan_tiles)
