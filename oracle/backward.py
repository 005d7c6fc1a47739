"""float64 backward of the masked attention -- TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The pages describe context-parallel systems that train, so the gradients of the
attention forward are carried too: "03 · 长文负载均衡", section 4.4 (MagiAttention)
reduces the partial key/value gradients of each block back to the rank that owns
the keys, and section 5 keeps key/value gradients with the states they belong to.
The pages give no formulas; the gradient is the plain definition, the derivative
of L = sum_i <dout_i, out_i> with out the forward of ``oracle.attention``, written
out with the chain rule through the softmax:

  P_ij  = exp(s_ij - lse_i) on visible pairs, 0 elsewhere, s_ij = scale <q_i, k_j>
  dv_j  = sum_i P_ij dout_i
  dP_ij = <dout_i, v_j>
  D_i   = sum_j P_ij dP_ij  (= <dout_i, out_i>)
  dS_ij = P_ij (dP_ij - D_i)
  dq_i  = scale sum_j dS_ij k_j
  dk_j  = scale sum_i dS_ij q_i

With grouped-query attention the key/value gradients of a kv head are the sums over
the query heads that share it.  One ring step of a context-parallel rank contributes
the same terms restricted to its key/value chunk, with lse and D of the whole
(merged) forward: summed over the steps they give the unsharded gradient, because
lse and D are the whole row's.  Rows that see no key have zero gradient.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import (ROW_BLOCK, _as_f64, doc_of_tokens, visible_block, visible_causal_doc,
                        visible_shared_question)


def row_dot(out, dout):
    """D [H,R] = sum_d out[r,h,d] dout[r,h,d] (float64)."""
    return np.einsum("rhd,rhd->hr", _as_f64(out), _as_f64(dout))


def attend_bwd(q_rows, k, v, dout_rows, visible, scale, lse_rows=None, d_rows=None):
    """Gradients of one row block of one head against its keys.

    q_rows [R,d], k [K,d], v [K,dv], dout_rows [R,dv], visible [R,K].  Without
    ``lse_rows`` / ``d_rows`` the softmax is taken over these keys (the whole row);
    with them (a ring step), P = exp(s - lse) and D are the given whole-row values.
    Returns dq_rows [R,d], dk [K,d], dv [K,dv].
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(dout_rows, dtype=np.float64)
    R, K = visible.shape
    if K == 0 or R == 0:
        return np.zeros_like(q_rows), np.zeros_like(k), np.zeros_like(v)
    s = scale * (q_rows @ k.T)
    if lse_rows is None:  # the row's own log-sum-exp over its visible keys
        s_vis = np.where(visible, s, -np.inf)
        m = s_vis.max(axis=1)
        seen = np.isfinite(m)
        m0 = np.where(seen, m, 0.0)
        total = np.exp(s_vis - m0[:, None]).sum(axis=1)
        lse_rows = np.full(R, -np.inf)
        lse_rows[seen] = m0[seen] + np.log(total[seen])
    lse_rows = np.asarray(lse_rows, dtype=np.float64)
    live = np.isfinite(lse_rows)
    p = np.where(visible & live[:, None], np.exp(s - np.where(live, lse_rows, 0.0)[:, None]), 0.0)
    dp = do @ v.T
    if d_rows is None:
        d_rows = (p * dp).sum(axis=1)
    ds = p * (dp - np.asarray(d_rows, dtype=np.float64)[:, None])
    return scale * (ds @ k), scale * (ds.T @ q_rows), p.T @ do


def _bwd_units(q, k, v, dout, heads, kv_heads, units, scale, lse=None, dvec=None):
    """units: (row_index_array, key_index_array, visible_fn).  Accumulates dq [T_q,H,d],
    dk/dv [T_k,H_kv,d]; lse/dvec [H,T_q] are whole-row values (ring steps) or None."""
    G = heads // kv_heads
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for rows_all, cols, vis_fn in units:
        for b in range(0, len(rows_all), ROW_BLOCK):
            rows = rows_all[b:b + ROW_BLOCK]
            visible = vis_fn(rows, cols)
            for h in range(heads):
                g = h // G
                gq, gk, gv = attend_bwd(q[rows, h], k[cols, g], v[cols, g], dout[rows, h], visible, scale,
                                        None if lse is None else lse[h, rows],
                                        None if dvec is None else dvec[h, rows])
                dq[rows, h] += gq
                dk[cols, g] += gk
                dv[cols, g] += gv
    return dq, dk, dv


def varlen_attention_bwd(q, k, v, dout, cu_seqlens, heads, kv_heads, mask="causal_doc", scale=None):
    """dq [T,H,d], dk and dv [T,H_kv,d] of the varlen forward (same masks as
    ``oracle.attention.varlen_attention``)."""
    q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    T, H, d = q.shape
    assert H == heads and k.shape[1] == kv_heads and heads % kv_heads == 0
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    seg = doc_of_tokens(cu)
    units = []
    for s in range(len(cu) - 1):
        r = np.arange(cu[s], cu[s + 1])
        if len(r) == 0:
            continue
        if mask == "causal_doc":
            units.append((r, r, lambda rr, cc: visible_causal_doc(seg, rr, cc)))
        elif mask == "shared_question":
            cols = r if s == 0 else np.concatenate([np.arange(cu[0], cu[1]), r])
            units.append((r, cols, lambda rr, cc: visible_shared_question(seg, rr, cc)))
        else:
            raise ValueError(mask)
    return _bwd_units(q, k, v, dout, heads, kv_heads, units, scale)


def block_attention_bwd(q, k, v, dout, lse, dvec, q_pos, kv_pos, q_doc, kv_doc, heads, kv_heads, scale=None,
                        shared_doc=None):
    """One ring step: the query shard's dq contribution [n_q,H,d] and the key/value chunk's
    dk, dv [n_kv,H_kv,d], from the whole-row lse and D [H,n_q] of the merged forward."""
    q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    n_q, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    q_pos, kv_pos = np.asarray(q_pos, dtype=np.int64), np.asarray(kv_pos, dtype=np.int64)
    q_doc, kv_doc = np.asarray(q_doc, dtype=np.int64), np.asarray(kv_doc, dtype=np.int64)
    units = []
    for doc in np.unique(q_doc):
        r = np.nonzero(q_doc == doc)[0]
        sees = (kv_doc == doc) | ((kv_doc == shared_doc) if shared_doc is not None and doc != shared_doc else False)
        cols = np.nonzero(sees)[0]
        units.append((r, cols, lambda rr, cc: visible_block(q_pos, q_doc, kv_pos, kv_doc, rr, cc, shared_doc)))
    return _bwd_units(q, k, v, dout, heads, kv_heads, units, scale,
                      np.asarray(lse, dtype=np.float64), np.asarray(dvec, dtype=np.float64))
