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
5. *Order*: estimated time descending, ties by natural order (fragment order,
   then tile order inside the fragment).  The estimate is the block count, or a
   weighted sum of blocks and pairs (``lpt_order_weighted``); either is scaled
   to 15 bits as ``quantised`` states before ordering.  The documents order
   (``documents_order``) applies the same longest-first rule to fragments: a
   fragment's estimate is the largest of its tiles', fragments go out largest
   first, and each one's tiles together, from its last tile back to its first.

Transposed tiling, for the key/value gradients of the backward (each key block
gathers the query rows that see it):

1. Key *fragments*.  Varlen causal: one per document, positions from 0.
   Shared question: the question's keys (positions from 0) and each answer's
   keys (positions from Q).  Block step: the runs of the key/value metadata.
2. Query spans of a key fragment.  Varlen causal: the document's rows.  Shared
   question: the question's keys are seen by the question's own later rows and
   by every answer row, so their span is every row from the question's start
   to the end of the pack, positions counted from the question's start (an
   answer row's index is at least Q, past every question key); an answer's
   keys are seen by that answer's rows only, positions from Q.  Block step:
   every query run of the same document, in query order.  Query i of a span
   sees key j of the fragment iff pos(j) <= pos(i).
3. Tiles of BM keys anchored at the fragment start; a tile keeps each span
   from its first row that sees the tile's first key (pos(row) >= pos of that
   key); spans clipped to nothing are dropped.
4. Cost = the tile's exact visible pairs, counted key by key; blocks = sum over
   its spans of ceil(rows kept / BLOCK_KEYS).
5. Order: as above.
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


FAR = 1 << 30  # a position offset no real position reaches


def fragments_block(q_pos, q_doc, kv_pos, kv_doc, shared_doc=None):
    """Query runs with the key runs of their document.  With ``shared_doc``, a run of any
    other document also gets that document's key runs, wholly visible: their positions are
    taken as lying far below every row (a FULL span); FULL runs next to each other in the
    key buffer make one span.  Spans keep the key runs' order."""
    q_runs = runs(q_pos, q_doc)
    kv_runs = runs(kv_pos, kv_doc)
    frags = []
    for (qs, ql, qp0, qd) in q_runs:
        spans = []
        for (ks, kl, kp0, kd) in kv_runs:
            if kd == qd:
                spans.append((ks, kl, kp0))
            elif shared_doc is not None and kd == shared_doc and qd != shared_doc:
                add_full_span(spans, ks, kl, -FAR)
        frags.append((qs, ql, qp0, spans))
    return frags


def add_full_span(spans, start, length, pos0):
    """Appends a FULL span, or lengthens the last span when that one is FULL too and ends
    where this one starts in the buffer: a FULL span's positions are never looked at, so the
    two cover the same pairs as one."""
    if spans and spans[-1][2] == pos0 and spans[-1][0] + spans[-1][1] == start:
        s, n, p = spans[-1]
        spans[-1] = (s, n + length, p)
    else:
        spans.append((start, length, pos0))


def visible_in_span(row_pos, k_len, k_pos0):
    """Number of keys of a span visible to one query at position row_pos."""
    return max(0, min(k_len, row_pos - k_pos0 + 1))


def visible_in_span_lo(row_pos, k_len, k_pos0, k_lo):
    """Keys of a span visible to one query with both bounds: k_pos0 + j <= row_pos <= k_lo + j."""
    return sum(1 for j in range(k_len) if k_pos0 + j <= row_pos <= k_lo + j)


def tiles(frags, bm):
    """Tiles in natural order: dicts with q_start, q_len, q_pos0, spans, cost.

    A span with a lower bound, (k_start, k_len, k_pos0, k_lo), first loses the keys below
    the bound of the tile's first row (k_lo + j < first position: no row of the tile sees
    them), then is clipped like the others."""
    out = []
    for (qs, ql, qp0, spans) in frags:
        for t0 in range(0, ql, bm):
            n = min(bm, ql - t0)
            p0 = qp0 + t0
            last = p0 + n - 1
            kept = []
            for sp in spans:
                ks, kl, kp0 = sp[:3]
                if len(sp) == 4:
                    c = max(0, p0 - sp[3])
                    ks, kl, kp0, klo = ks + c, kl - c, kp0 + c, sp[3] + c
                keep = min(kl, last - kp0 + 1)
                if keep > 0:
                    kept.append((ks, keep, kp0) if len(sp) == 3 else (ks, keep, kp0, klo))
            cost = 0
            for r in range(n):
                for sp in kept:
                    cost += visible_in_span(p0 + r, sp[1], sp[2]) if len(sp) == 3 else \
                        visible_in_span_lo(p0 + r, sp[1], sp[2], sp[3])
            blocks = sum(-(-sp[1] // BLOCK_KEYS) for sp in kept)
            out.append(dict(q_start=qs + t0, q_len=n, q_pos0=p0, spans=kept, cost=cost, blocks=blocks))
    return out


def fragments_varlen_t(cu_seqlens, mask="causal_doc"):
    """Key fragments of the transposed tiling: (k_start, k_len, k_pos0, [(q_start, q_len, q_pos0), ...])."""
    cu = [int(x) for x in cu_seqlens]
    frags = []
    if mask == "causal_doc":
        return fragments_varlen(cu, mask)  # a document's keys and its rows: the same ranges
    if mask != "shared_question":
        raise ValueError(mask)
    Q = cu[1] - cu[0]
    if Q > 0:
        frags.append((cu[0], Q, 0, [(cu[0], cu[-1] - cu[0], 0)]))
    for s in range(1, len(cu) - 1):
        n = cu[s + 1] - cu[s]
        if n > 0:
            frags.append((cu[s], n, Q, [(cu[s], n, Q)]))
    return frags


def fragments_block_t(q_pos, q_doc, kv_pos, kv_doc, shared_doc=None):
    """Key runs with the query runs of their document; a run of ``shared_doc`` also gets every
    other document's query runs, which see all of it: their positions taken far above every
    key, and runs next to each other in the query buffer (of any documents) make one span."""
    q_runs = runs(q_pos, q_doc)
    frags = []
    for (ks, kl, kp0, kd) in runs(kv_pos, kv_doc):
        spans = []
        for (qs, ql, qp0, qd) in q_runs:
            if qd == kd:
                spans.append((qs, ql, qp0))
            elif shared_doc is not None and kd == shared_doc and qd != shared_doc:
                add_full_span(spans, qs, ql, FAR)
        frags.append((ks, kl, kp0, spans))
    return frags


def tiles_t(frags, bm):
    """Key tiles of the transposed tiling, in the same dict form as ``tiles`` (q_* fields
    describe the tile's keys, spans are query rows)."""
    out = []
    for (ks, kl, kp0, spans) in frags:
        for t0 in range(0, kl, bm):
            n = min(bm, kl - t0)
            p0 = kp0 + t0  # position of the tile's first key
            kept = []
            for (qs, ql, qp0) in spans:
                c = max(0, p0 - qp0)  # rows before the first key's position see none of the tile
                if ql - c > 0:
                    kept.append((qs + c, ql - c, qp0 + c))
            cost = 0
            for j in range(n):  # key at position p0 + j: rows of each span at or after it
                for (qs, ql, qp0) in kept:
                    cost += sum(1 for r in range(ql) if qp0 + r >= p0 + j)
            blocks = sum(-(-ql // BLOCK_KEYS) for (qs, ql, qp0) in kept)
            out.append(dict(q_start=ks + t0, q_len=n, q_pos0=p0, spans=kept, cost=cost, blocks=blocks))
    return out


# Orders are taken on costs of at most COST_MAX: every cost is divided by the least power of
# two 2^s that brings the largest cost to COST_MAX or below, rounding up.  (Reading: the
# pages fix no resolution for the estimate; the order only needs to put the longest tiles
# first, and the planner's 32-bit sort key holds 15 bits of cost.  Rounding up keeps every
# tile with work ahead of every tile without.)
COST_MAX = (1 << 15) - 1


def quantised(costs):
    """Non-negative integer costs scaled to at most COST_MAX: ceil(c / 2^s), least such s."""
    m = max(costs, default=0)
    s = 0
    while -(-m // (1 << s)) > COST_MAX:
        s += 1
    return [-(-c // (1 << s)) for c in costs]


def order_by_cost(costs):
    """Indices by quantised cost descending, ties in natural order."""
    q = quantised(costs)
    return sorted(range(len(q)), key=lambda i: (-q[i], i))


def lpt_order(tile_list, key="blocks"):
    """Indices of tiles, `key` descending (after quantisation), ties in natural order."""
    return order_by_cost([t[key] for t in tile_list])


def weighted_cost(t, block_weight, pair_weight, group):
    """A tile's time estimate: a linear load model in its key blocks and in the visible
    (query, key) pairs of the `group` query heads one item serves ("数据并行负载均衡",
    section 4.2: the load is fitted as a linear model of the work terms; the per-item
    constant of such a fit is dropped, as it moves every item alike)."""
    return block_weight * t["blocks"] + pair_weight * group * t["cost"]


def lpt_order_weighted(tile_list, block_weight, pair_weight, group):
    """LPT order on the weighted estimate ("数据并行负载均衡", section 4.4)."""
    return order_by_cost([weighted_cost(t, block_weight, pair_weight, group) for t in tile_list])


# The documents order groups a fragment's tiles so that the items running at one time share
# that fragment's keys and values (a cache effect: every order computes the same results).
# Reading: the pages order work longest first and say nothing of the order of items of
# equal standing; taking the longest-first rule at the level of documents, with a document's
# estimate its largest tile's, keeps the long items first and the short ones last.  Beyond
# GROUP_CAP segments or GROUP_TILE_CAP tiles the plan keeps the tile-level order (a capacity
# rule of the planner's shared memory, stated so that the two agree).
GROUP_CAP = 4096
GROUP_TILE_CAP = 16384


def documents_order(tile_list, frags, bm, costs, n_segments):
    """Indices of tiles: fragments by their largest quantised cost descending, ties later
    fragment first; inside a fragment, tiles in descending natural order; tiles without
    blocks (no key span) after all others, in descending natural order.  Falls back to
    ``order_by_cost`` beyond the capacities above."""
    n = len(tile_list)
    if n_segments > GROUP_CAP or n > GROUP_TILE_CAP:
        return order_by_cost(costs)
    q = quantised(costs)
    frag_of = []
    for f, (_, q_len, _, _) in enumerate(frags):
        frag_of += [f] * (-(-q_len // bm))
    assert len(frag_of) == n
    top = {}
    for i in range(n):
        if tile_list[i]["blocks"] > 0:
            top[frag_of[i]] = max(top.get(frag_of[i], 0), q[i])
    group = [top[frag_of[i]] if tile_list[i]["blocks"] > 0 else 0 for i in range(n)]
    return sorted(range(n), key=lambda i: (-group[i], -i))


def plan_documents(frags, bm, block_weight, pair_weight, group, n_segments):
    """The plan with tiles in the documents order of the weighted estimate."""
    t = tiles(frags, bm)
    costs = [weighted_cost(x, block_weight, pair_weight, group) for x in t]
    return [t[i] for i in documents_order(t, frags, bm, costs, n_segments)]


def plan(frags, bm):
    """The full reference plan: tiles in longest-first order."""
    t = tiles(frags, bm)
    return [t[i] for i in lpt_order(t)]


def plan_weighted(frags, bm, block_weight, pair_weight, group):
    """The plan with tiles in the order of the weighted estimate."""
    t = tiles(frags, bm)
    return [t[i] for i in lpt_order_weighted(t, block_weight, pair_weight, group)]


def merge_step_plans(plans):
    """One longest-first queue over several block steps' plans (the LPT rule of
    "数据并行负载均衡", section 4.4, applied to the union of the steps' items): the tiles that
    have key spans, by key blocks descending, ties by step and then by place in the step's own
    plan; after them every step's tiles without spans, step by step.  Each tile is tagged
    with its step."""
    work = [(-t["blocks"], s, i) for s, p in enumerate(plans) for i, t in enumerate(p) if t["spans"]]
    work.sort()
    out = [dict(plans[s][i], step=s) for (_, s, i) in work]
    out += [dict(t, step=s) for s, p in enumerate(plans) for t in p if not t["spans"]]
    return out


def total_pairs(plan_tiles):
    return sum(t["cost"] for t in plan_tiles)


FUSED_SPAN_CAP = 4  # key spans one query tile of a fused ring holds
FUSED_TILE_CAP = 4096  # query tiles one fused ring takes


def fuse_step_plans(natural_plans):
    """A ring's block steps fused per query tile: the steps cut the query shard into the same
    tiles (the tiling depends on the query side only), so query tile x gathers the key spans
    of tile x of every step, in step order, each span tagged with its step; its pairs and key
    blocks are the sums over the steps.  Its attention is then one online softmax over all
    the keys its rows see in any step: the rescale-and-sum of the steps' partials ("03 ·
    长文负载均衡", section 3.2, DCP) taken inside one tile instead of after the steps.  Tiles
    with key blocks go first, by key blocks descending (above COST_MAX as COST_MAX), ties in
    natural order; then the tiles without spans, in natural order (the LPT rule of
    "数据并行负载均衡", section 4.4, over whole query tiles).  ``natural_plans``: each step's
    tiles in natural order (``tiles``).  None when a tile would hold more than FUSED_SPAN_CAP
    spans, or there are more than FUSED_TILE_CAP tiles."""
    n = len(natural_plans[0])
    if any(len(p) != n for p in natural_plans):
        raise ValueError("the steps' plans cut the query shard differently")
    if n > FUSED_TILE_CAP:
        return None
    fused = []
    for x in range(n):
        first = natural_plans[0][x]
        spans, steps, cost, blocks = [], [], 0, 0
        for s, p in enumerate(natural_plans):
            t = p[x]
            if (t["q_start"], t["q_len"], t["q_pos0"]) != (first["q_start"], first["q_len"], first["q_pos0"]):
                raise ValueError("the steps' plans cut the query shard differently")
            spans += list(t["spans"])
            steps += [s] * len(t["spans"])
            cost += t["cost"]
            blocks += t["blocks"]
        if len(spans) > FUSED_SPAN_CAP:
            return None
        fused.append(dict(q_start=first["q_start"], q_len=first["q_len"], q_pos0=first["q_pos0"], spans=spans,
                          span_steps=steps, cost=cost, blocks=blocks))
    order = sorted(range(n), key=lambda x: (-min(fused[x]["blocks"], COST_MAX), x))
    return [fused[x] for x in order]
