"""Pins of the oracle's backward (oracle/backward.py): torch autograd in float64, central
finite differences, closed forms, and the reassembly of ring-step partials."""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as A
from oracle import backward as B
from oracle import sharding as S


def rand(r, *shape):
    return r.standard_normal(shape)


def test_autograd_sdpa_causal_documents_with_gqa():
    """Per document, torch's scaled_dot_product_attention(is_causal=True) in float64 with the
    kv heads repeated per group, differentiated by autograd, equals the oracle."""
    r = np.random.default_rng(0)
    lengths = [7, 1, 30, 12]
    T, H, Hkv, d = sum(lengths), 4, 2, 16
    q, k, v, do = rand(r, T, H, d), rand(r, T, Hkv, d), rand(r, T, Hkv, d), rand(r, T, H, d)
    dq, dk, dv = B.varlen_attention_bwd(q, k, v, do, workloads.cu_from_lengths(lengths), H, Hkv)
    cu = workloads.cu_from_lengths(lengths)
    G = H // Hkv
    for s in range(len(lengths)):
        a, b = int(cu[s]), int(cu[s + 1])
        tq = torch.tensor(q[a:b], requires_grad=True)
        tk = torch.tensor(k[a:b], requires_grad=True)
        tv = torch.tensor(v[a:b], requires_grad=True)
        kk = tk.repeat_interleave(G, dim=1)
        vv = tv.repeat_interleave(G, dim=1)
        o = torch.nn.functional.scaled_dot_product_attention(tq.transpose(0, 1), kk.transpose(0, 1),
                                                             vv.transpose(0, 1), is_causal=True).transpose(0, 1)
        o.backward(torch.tensor(do[a:b]))
        assert np.max(np.abs(tq.grad.numpy() - dq[a:b])) < 1e-10
        assert np.max(np.abs(tk.grad.numpy() - dk[a:b])) < 1e-10
        assert np.max(np.abs(tv.grad.numpy() - dv[a:b])) < 1e-10


def test_finite_differences_shared_question():
    """Central differences of L = <dout, out(q, k, v)> through the oracle's own forward
    (shared-question mask: the answers see the whole question), on sampled coordinates."""
    r = np.random.default_rng(1)
    lengths = [6, 4, 5]
    T, H, Hkv, d = sum(lengths), 2, 1, 8
    cu = workloads.cu_from_lengths(lengths)
    q, k, v, do = rand(r, T, H, d), rand(r, T, Hkv, d), rand(r, T, Hkv, d), rand(r, T, H, d)
    grads = B.varlen_attention_bwd(q, k, v, do, cu, H, Hkv, mask="shared_question")

    def loss(qq, kk, vv):
        o, _ = A.varlen_attention(qq, kk, vv, cu, H, Hkv, mask="shared_question")
        return float(np.sum(o * do))

    eps = 1e-6
    for which, g in zip(range(3), grads):
        for _ in range(6):
            args = [q.copy(), k.copy(), v.copy()]
            idx = tuple(int(r.integers(0, n)) for n in args[which].shape)
            args[which][idx] += eps
            up = loss(*args)
            args[which][idx] -= 2 * eps
            down = loss(*args)
            fd = (up - down) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (which, idx, fd, g[idx])


def test_single_token_document_closed_form():
    # out = v exactly, so dv = dout, and the softmax has nothing to move: dq = dk = 0
    r = np.random.default_rng(2)
    q, k, v, do = rand(r, 1, 2, 8), rand(r, 1, 1, 8), rand(r, 1, 1, 8), rand(r, 1, 2, 8)
    dq, dk, dv = B.varlen_attention_bwd(q, k, v, do, [0, 1], 2, 1)
    assert np.all(dq == 0) and np.all(dk == 0)
    assert np.allclose(dv[0, 0], do[0, 0] + do[0, 1], atol=1e-15, rtol=0)


def test_softmax_invariants_per_document():
    """Every row's weights sum to 1 and shifting a row's logits leaves it unchanged, so per
    document and kv head: sum_j dk_j = 0 and sum_j dv_j = sum over the group's heads and the
    document's rows of dout."""
    r = np.random.default_rng(3)
    lengths = [40, 3, 17]
    T, H, Hkv, d = sum(lengths), 4, 2, 16
    cu = workloads.cu_from_lengths(lengths)
    q, k, v, do = rand(r, T, H, d), rand(r, T, Hkv, d), rand(r, T, Hkv, d), rand(r, T, H, d)
    dq, dk, dv = B.varlen_attention_bwd(q, k, v, do, cu, H, Hkv)
    for s in range(len(lengths)):
        a, b = int(cu[s]), int(cu[s + 1])
        for g in range(Hkv):
            assert np.max(np.abs(dk[a:b, g].sum(axis=0))) < 1e-12
            assert np.max(np.abs(dv[a:b, g].sum(axis=0) - do[a:b, 2 * g:2 * g + 2].sum(axis=(0, 1)))) < 1e-12


def test_row_dot_is_d():
    # D_i = <dout_i, out_i> = sum_j P_ij dP_ij: the two forms agree
    r = np.random.default_rng(4)
    lengths = [20, 9]
    T, H, Hkv, d = sum(lengths), 2, 2, 8
    cu = workloads.cu_from_lengths(lengths)
    q, k, v, do = rand(r, T, H, d), rand(r, T, Hkv, d), rand(r, T, Hkv, d), rand(r, T, H, d)
    out, lse = A.varlen_attention(q, k, v, cu, H, Hkv)
    dvec = B.row_dot(out, do)
    seg = A.doc_of_tokens(cu)
    for h in range(H):
        for i in range(T):
            cols = np.nonzero((seg == seg[i]) & (np.arange(T) <= i))[0]
            s = (q[i, h] @ k[cols, h].T) / math.sqrt(d)
            p = np.exp(s - lse[h, i])
            assert abs(np.sum(p * (v[cols, h] @ do[i, h])) - dvec[h, i]) < 1e-12


@pytest.mark.parametrize("rule", ["zigzag", "per_document", "dispatch"])
def test_ring_step_partials_reassemble_the_unsharded_gradient(rule):
    """Each rank's cp ring steps with the merged forward's lse and D: dq summed over its
    steps, and dk, dv of every shard summed over the ranks that attended to it, equal the
    unsharded gradients."""
    cp, H, Hkv, d = 4, 4, 2, 16
    r = np.random.default_rng(5)
    lengths = [37, 5, 90, 1, 59, 48]
    T = sum(lengths)
    if rule == "zigzag":
        lengths.append(2 * cp * 40 - T)
        T = sum(lengths)
    q, k, v, do = rand(r, T, H, d), rand(r, T, Hkv, d), rand(r, T, Hkv, d), rand(r, T, H, d)
    cu = workloads.cu_from_lengths(lengths)
    out, lse = A.varlen_attention(q, k, v, cu, H, Hkv)
    dvec = B.row_dot(out, do)
    ref = B.varlen_attention_bwd(q, k, v, do, cu, H, Hkv)
    tok = {"zigzag": lambda: S.zigzag_tokens(T, cp), "per_document": lambda: S.per_document_tokens(lengths, cp),
           "dispatch": lambda: S.dispatch_tokens(lengths, cp, 2 * cp)}[rule]()
    pos, doc = A.pack_positions(lengths)
    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for rank in range(cp):
        qi = tok[rank]
        for t in range(cp):
            ki = tok[A.ring_source(rank, t, cp)]
            gq, gk, gv = B.block_attention_bwd(q[qi], k[ki], v[ki], do[qi], lse[:, qi], dvec[:, qi], pos[qi], pos[ki],
                                               doc[qi], doc[ki], H, Hkv)
            dq[qi] += gq
            dk[ki] += gk
            dv[ki] += gv
    for got, want in zip((dq, dk, dv), ref):
        assert np.max(np.abs(got - want)) < 1e-11


def test_block_shared_doc_equals_varlen_shared_question():
    """One block step over a whole shared-question pack (document 0 shared), from the block
    forward's lse and D, gives the varlen shared-question gradient."""
    from oracle import attention as A
    r = np.random.default_rng(31)
    lengths = [20, 7, 1, 13]
    T, H, Hkv, d = sum(lengths), 4, 2, 8
    q, k, v = (r.standard_normal((T, h, d)) for h in (H, Hkv, Hkv))
    do = r.standard_normal((T, H, d))
    pos, doc = A.pack_positions(lengths)
    out, lse = A.block_attention(q, k, v, pos, pos, doc, doc, H, Hkv, shared_doc=0)
    dvec = B.row_dot(out, do)
    dq, dk, dv = B.block_attention_bwd(q, k, v, do, lse, dvec, pos, pos, doc, doc, H, Hkv, shared_doc=0)
    rq, rk, rv = B.varlen_attention_bwd(q, k, v, do, np.concatenate([[0], np.cumsum(lengths)]), H, Hkv,
                                        mask="shared_question")
    for got, want in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(got, want, atol=1e-10)
