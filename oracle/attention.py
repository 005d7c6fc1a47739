"""float64 explicit-mask attention -- TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What is computed, and where the pages fix it
--------------------------------------------
* Packed documents attend only inside their own document, so the attention
  work of a pack grows with the sum of squared document lengths, not with the
  square of the pack length ("03 · 长文负载均衡", section 1.1, the W_attn
  formula; "数据并行负载均衡", section 1, the flash_attn_varlen load model).
  Here: key j is visible to query i iff both lie in the same document and
  j <= i (the diagonal is included).
* Shared-question masks ("03 · 长文负载均衡", section 1.2): one question is
  followed by several answers; every answer sees the whole question and itself
  causally, never another answer; the question sees only itself, causally.
* Block attention of one context-parallel step ("03 · 长文负载均衡", section
  3.2, DCP computation blocks; "长序列训练与上下文并行", Ring Attention): a
  query shard against one key/value chunk, with global positions and document
  ids carried per token; key j is visible to query i iff they share a document
  and pos_k[j] <= pos_q[i].  Partial results are combined by the online-softmax
  rescale-and-sum, which is what ``lse_merge`` writes out.
* Zigzag sharding ("03 · 长文负载均衡", section 4.2): the sequence is cut into
  2*cp chunks and rank i holds chunks i and 2*cp-1-i.  Ring order
  ("长序列训练与上下文并行", Ring Attention): at step t a rank works on the
  key/value chunks that started on rank (r - t) mod cp.

Readings where the pages are silent: softmax scale 1/sqrt(d); lse is the
natural log of the sum of exp(scaled logits); query head h uses key/value head
h // (H / H_kv); a row that sees no key has lse = -inf and out = 0.

Everything is float64.  Rows are processed in blocks of at most ``ROW_BLOCK``
against the keys of their own unit (document, question + own answer, or the
same document in the key/value chunk); the explicit boolean mask is then
applied inside that unit, so the unit restriction only skips keys the mask
would hide anyway.
"""
from __future__ import annotations

import math

import numpy as np

ROW_BLOCK = 512


# --------------------------------------------------------------------------
# per-token metadata and visibility rules
# --------------------------------------------------------------------------
def doc_of_tokens(cu_seqlens) -> np.ndarray:
    """Index of the document (segment) each token belongs to."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    seg = np.zeros(int(cu[-1]), dtype=np.int64)
    for s in range(len(cu) - 1):
        seg[cu[s]:cu[s + 1]] = s
    return seg


def visible_causal_doc(seg, rows, cols) -> np.ndarray:
    rows = np.asarray(rows)[:, None]
    cols = np.asarray(cols)[None, :]
    return (seg[rows] == seg[cols]) & (cols <= rows)


def visible_shared_question(seg, rows, cols) -> np.ndarray:
    """Segment 0 is the question; later segments are answers."""
    rows = np.asarray(rows)[:, None]
    cols = np.asarray(cols)[None, :]
    same = seg[rows] == seg[cols]
    question_key = seg[cols] == 0
    return (cols <= rows) & (same | question_key)


def visible_block(q_pos, q_doc, kv_pos, kv_doc, rows, cols, shared_doc=None) -> np.ndarray:
    """Same document and key position <= query position; with ``shared_doc``, also every key
    of that document for the rows of every other document (the shared question of
    "03 · 长文负载均衡", section 1.2: answers see the whole question, the question does not
    see the answers)."""
    rows = np.asarray(rows)[:, None]
    cols = np.asarray(cols)[None, :]
    vis = (q_doc[rows] == kv_doc[cols]) & (kv_pos[cols] <= q_pos[rows])
    if shared_doc is not None:
        vis = vis | ((kv_doc[cols] == shared_doc) & (q_doc[rows] != shared_doc))
    return vis


# --------------------------------------------------------------------------
# the core: softmax attention of a row block under an explicit mask
# --------------------------------------------------------------------------
def attend(q_rows, k, v, visible, scale):
    """out[i] = sum_j softmax_j(scale*<q_i,k_j>, j visible) v_j ;  lse[i] = ln sum_j exp(...).

    q_rows [R,d], k [K,d], v [K,dv], visible [R,K] bool; float64 throughout.
    Rows with no visible key get out = 0 and lse = -inf.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    R = q_rows.shape[0]
    dv = v.shape[1]
    if k.shape[0] == 0:
        return np.zeros((R, dv)), np.full(R, -np.inf)
    s = scale * (q_rows @ np.asarray(k, dtype=np.float64).T)
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    p = np.exp(s - m_safe[:, None])
    l = p.sum(axis=1)
    l_safe = np.where(empty, 1.0, l)
    probs = p / l_safe[:, None]
    row_sum = probs.sum(axis=1)
    assert np.all(np.abs(row_sum[~empty] - 1.0) <= 1e-12), "softmax rows must sum to 1"
    out = probs @ np.asarray(v, dtype=np.float64)
    out[empty] = 0.0
    lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    return out, lse


def _as_f64(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:  # bfloat16 bits
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def _run_units(q, k, v, heads, kv_heads, units, scale):
    """units: list of (row_index_array, key_index_array, visible_fn(rows, cols)).

    Returns dict row -> (out [H,dv], lse [H]).
    """
    G = heads // kv_heads
    results = {}
    for rows_all, cols, vis_fn in units:
        for b in range(0, len(rows_all), ROW_BLOCK):
            rows = rows_all[b:b + ROW_BLOCK]
            visible = vis_fn(rows, cols)
            out = np.zeros((len(rows), heads, v.shape[2]))
            lse = np.zeros((heads, len(rows)))
            for h in range(heads):
                g = h // G
                o_h, l_h = attend(q[rows, h, :], k[cols, g, :], v[cols, g, :], visible, scale)
                out[:, h, :] = o_h
                lse[h, :] = l_h
            for i, r in enumerate(rows):
                results[int(r)] = (out[i], lse[:, i])
    return results


def _collect(results, rows, heads, dv):
    out = np.zeros((len(rows), heads, dv))
    lse = np.zeros((heads, len(rows)))
    for i, r in enumerate(rows):
        o, l = results[int(r)]
        out[i] = o
        lse[:, i] = l
    return out, lse


# --------------------------------------------------------------------------
# varlen forward (causal documents or shared question)
# --------------------------------------------------------------------------
def varlen_attention(q, k, v, cu_seqlens, heads, kv_heads, mask="causal_doc", rows=None, scale=None):
    """Varlen forward over a packed sequence in THD layout.

    q [T,H,d], k/v [T,H_kv,d] (float or bfloat16 bits).  ``mask`` is
    "causal_doc" or "shared_question" (segment 0 is the question).
    Returns out [R,H,d] and lse [H,R] for ``rows`` (default: every token).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    T, H, d = q.shape
    assert H == heads and k.shape[1] == kv_heads and heads % kv_heads == 0
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    seg = doc_of_tokens(cu)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    units = []
    for s in range(len(cu) - 1):
        r = rows[seg[rows] == s]
        if len(r) == 0:
            continue
        if mask == "causal_doc":
            cols = np.arange(cu[s], cu[s + 1])
            units.append((r, cols, lambda rr, cc: visible_causal_doc(seg, rr, cc)))
        elif mask == "shared_question":
            cols = np.arange(cu[0], cu[1]) if s == 0 else \
                np.concatenate([np.arange(cu[0], cu[1]), np.arange(cu[s], cu[s + 1])])
            units.append((r, cols, lambda rr, cc: visible_shared_question(seg, rr, cc)))
        else:
            raise ValueError(mask)
    res = _run_units(q, k, v, heads, kv_heads, units, scale)
    return _collect(res, rows, heads, v.shape[2])


# --------------------------------------------------------------------------
# block attention of one context-parallel step
# --------------------------------------------------------------------------
def block_attention(q, k, v, q_pos, kv_pos, q_doc, kv_doc, heads, kv_heads, rows=None, scale=None,
                    shared_doc=None):
    """Query shard [n_q,H,d] against one key/value chunk [n_kv,H_kv,d].

    Visible iff q_doc[i] == kv_doc[j] and kv_pos[j] <= q_pos[i], or (with ``shared_doc``)
    kv_doc[j] == shared_doc != q_doc[i].
    Returns out [R,H,d] (zeros on empty rows) and lse [H,R] (-inf on empty rows).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    n_q, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    kv_pos = np.asarray(kv_pos, dtype=np.int64)
    q_doc = np.asarray(q_doc, dtype=np.int64)
    kv_doc = np.asarray(kv_doc, dtype=np.int64)
    rows = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    units = []
    for doc in np.unique(q_doc[rows]):
        r = rows[q_doc[rows] == doc]
        sees = (kv_doc == doc) | ((kv_doc == shared_doc) if shared_doc is not None and doc != shared_doc else False)
        cols = np.nonzero(sees)[0]
        units.append((r, cols, lambda rr, cc: visible_block(q_pos, q_doc, kv_pos, kv_doc, rr, cc, shared_doc)))
    res = _run_units(q, k, v, heads, kv_heads, units, scale)
    return _collect(res, rows, heads, v.shape[2])


# --------------------------------------------------------------------------
# log-sum-exp merge of two partial results
# --------------------------------------------------------------------------
def lse_merge(out_a, lse_a, out_b, lse_b):
    """Online-softmax rescale-and-sum of two partials over disjoint key sets.

    out_* [R,H,d], lse_* [H,R].  With M = max(lse_a, lse_b):
      lse = M + ln(e^(lse_a-M) + e^(lse_b-M)),
      out = (e^(lse_a-M) out_a + e^(lse_b-M) out_b) / (e^(lse_a-M) + e^(lse_b-M)).
    A side whose lse is -inf contributes nothing (its out is never read).
    """
    out_a = np.asarray(out_a, dtype=np.float64)
    out_b = np.asarray(out_b, dtype=np.float64)
    la = np.asarray(lse_a, dtype=np.float64).T  # [R,H]
    lb = np.asarray(lse_b, dtype=np.float64).T
    out = np.array(out_a, copy=True)
    lse = np.array(la, copy=True)
    R, H = la.shape
    for r in range(R):
        for h in range(H):
            a, b = la[r, h], lb[r, h]
            if b == -np.inf:
                continue
            if a == -np.inf:
                out[r, h] = out_b[r, h]
                lse[r, h] = b
                continue
            M = max(a, b)
            wa, wb = math.exp(a - M), math.exp(b - M)
            out[r, h] = (wa * out_a[r, h] + wb * out_b[r, h]) / (wa + wb)
            lse[r, h] = M + math.log(wa + wb)
    return out, lse.T


# --------------------------------------------------------------------------
# zigzag context parallelism: chunk ownership, ring order, one rank's fold
# --------------------------------------------------------------------------
def zigzag_chunks_of_rank(rank: int, cp: int):
    """Chunks held by ``rank`` when the sequence is cut into 2*cp chunks."""
    return (rank, 2 * cp - 1 - rank)


def ring_source(rank: int, step: int, cp: int) -> int:
    """The rank whose key/value chunks ``rank`` processes at ring step ``step``."""
    return (rank - step) % cp


def pack_positions(lengths):
    """Global position and document id of every token of a pack."""
    lengths = list(lengths)
    T = int(sum(lengths))
    pos = np.arange(T, dtype=np.int64)
    doc = np.repeat(np.arange(len(lengths), dtype=np.int64), lengths)
    return pos, doc


def zigzag_rank_attention(get_chunk, lengths, chunk_tokens, rank, cp, heads, kv_heads, rows=None):
    """Fold the cp ring steps of one rank with ``lse_merge``.

    get_chunk(c) -> (q, k, v) of chunk c (any float dtype or bf16 bits).
    Returns (out [R,H,d], lse [H,R]) for the rank's query shard (its two
    chunks, in chunk order), plus the per-step partials.
    """
    pos, doc = pack_positions(lengths)
    qc = zigzag_chunks_of_rank(rank, cp)

    def span(c):
        return slice(c * chunk_tokens, (c + 1) * chunk_tokens)

    q_parts = [get_chunk(c)[0] for c in qc]
    q = np.concatenate([_as_f64(x) for x in q_parts])
    q_pos = np.concatenate([pos[span(c)] for c in qc])
    q_doc = np.concatenate([doc[span(c)] for c in qc])
    acc = None
    steps = []
    for t in range(cp):
        j = ring_source(rank, t, cp)
        kc = zigzag_chunks_of_rank(j, cp)
        k = np.concatenate([_as_f64(get_chunk(c)[1]) for c in kc])
        v = np.concatenate([_as_f64(get_chunk(c)[2]) for c in kc])
        kv_pos = np.concatenate([pos[span(c)] for c in kc])
        kv_doc = np.concatenate([doc[span(c)] for c in kc])
        o, l = block_attention(q, k, v, q_pos, kv_pos, q_doc, kv_doc, heads, kv_heads, rows=rows)
        steps.append((o, l))
        acc = (o, l) if acc is None else lse_merge(acc[0], acc[1], o, l)
    return acc[0], acc[1], steps
