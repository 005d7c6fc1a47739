"""Pins of the oracle's slice-list masks (oracle/slices.py): the varlen masks written as
slices give the varlen oracle's results, single slices match torch SDPA in float64 with
the explicit mask, and the tiles of a slice list count every visible pair once."""
import numpy as np
import pytest
import torch

import workloads
from oracle import attention as A
from oracle import plan as P
from oracle import slices as SL


def rand(r, *shape):
    return r.standard_normal(shape)


def test_varlen_causal_as_slices():
    r = np.random.default_rng(0)
    lengths = [5, 1, 40, 17]
    T, H, Hkv, d = sum(lengths), 4, 2, 16
    q, k, v = rand(r, T, H, d), rand(r, T, Hkv, d), rand(r, T, Hkv, d)
    o1, l1 = SL.slices_attention(q, k, v, SL.varlen_causal_slices(lengths), H, Hkv)
    o2, l2 = A.varlen_attention(q, k, v, workloads.cu_from_lengths(lengths), H, Hkv)
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12


def test_shared_question_as_slices():
    r = np.random.default_rng(1)
    lengths = [12, 7, 1, 9]
    T, H, Hkv, d = sum(lengths), 2, 1, 8
    q, k, v = rand(r, T, H, d), rand(r, T, Hkv, d), rand(r, T, Hkv, d)
    o1, l1 = SL.slices_attention(q, k, v, SL.shared_question_slices(lengths), H, Hkv)
    o2, l2 = A.varlen_attention(q, k, v, workloads.cu_from_lengths(lengths), H, Hkv, mask="shared_question")
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12


@pytest.mark.parametrize("lq,lk,kind", [(9, 20, SL.CAUSAL), (20, 9, SL.CAUSAL), (13, 13, SL.CAUSAL),
                                        (7, 30, SL.FULL), (9, 20, SL.INV_CAUSAL), (20, 9, SL.INV_CAUSAL),
                                        (9, 20, SL.BI_CAUSAL), (13, 13, SL.BI_CAUSAL)])
def test_single_slice_against_sdpa(lq, lk, kind):
    """A CAUSAL rectangle is the lower triangle aligned at its bottom-right corner (row r sees
    keys 0 .. r + lk - lq); INV-CAUSAL the upper one aligned at the top-left (keys r ..);
    BI-CAUSAL both; FULL sees everything.  torch SDPA with that explicit mask."""
    r = np.random.default_rng(lq * 100 + lk)
    d = 16
    q, k, v = rand(r, lq, 1, d), rand(r, lk, 1, d), rand(r, lk, 1, d)
    o, lse = SL.slices_attention(q, k, v, [(0, lq, 0, lk, kind)], 1, 1)
    mask = torch.ones(lq, lk, dtype=torch.bool)
    if kind in (SL.CAUSAL, SL.BI_CAUSAL):
        mask = mask.tril(diagonal=lk - lq)
    if kind in (SL.INV_CAUSAL, SL.BI_CAUSAL):
        mask = mask.triu(diagonal=0)
    rows = mask.any(dim=1).numpy()
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q[:, 0])[None], torch.tensor(k[:, 0])[None], torch.tensor(v[:, 0])[None], attn_mask=mask[None])
    assert np.max(np.abs(o[rows, 0] - ref[0].numpy()[rows])) < 1e-12
    assert np.all(lse[0, ~rows] == -np.inf) and np.all(o[~rows] == 0)


def test_block_causal_pairs_closed_form():
    """Frame f of a document (frames of F tokens) sees every key up to its own end: its rows
    see f0 + fl keys each, so the pairs are sum over frames of fl * (f0 + fl)."""
    lengths = [600, 1, 257, 256, 90]
    F = 128
    sl = SL.block_causal_slices(lengths, F)
    T = sum(lengths)
    want = sum(min(F, n - f0) * (f0 + min(F, n - f0)) for n in lengths for f0 in range(0, n, F))
    assert int(SL.visible(sl, T, T).sum()) == want
    tl = P.tiles(SL.fragments(sl), 64)
    assert sum(t["cost"] for t in tl) == want


def random_slices(r, n_q, n_k):
    out, q0 = [], 0
    while q0 < n_q:
        ql = int(min(n_q - q0, r.integers(1, 90)))
        if r.random() < 0.2:  # a query range no slice covers
            q0 += ql
            continue
        cuts = np.sort(r.choice(np.arange(1, n_k), size=int(r.integers(1, 4)), replace=False))
        bounds = [0] + cuts.tolist() + [n_k]
        picks = [(bounds[i], bounds[i + 1] - bounds[i]) for i in range(len(bounds) - 1) if r.random() < 0.6]
        for (ks, kl) in picks[:4]:
            out.append((q0, ql, ks, kl, int(r.integers(0, 4))))
        q0 += ql
    return out


@pytest.mark.parametrize("seed", range(5))
@pytest.mark.parametrize("bm", [16, 64])
def test_slice_tiles_count_every_pair_once(seed, bm):
    r = np.random.default_rng(seed)
    n_q, n_k = 300, 250
    sl = random_slices(r, n_q, n_k)
    V = SL.visible(sl, n_q, n_k)
    tl = P.tiles(SL.fragments(sl, n_q), bm)
    # every row is in exactly one tile; rows no slice covers are in tiles without a span
    rows = np.zeros(n_q, dtype=int)
    for t in tl:
        rows[t["q_start"]:t["q_start"] + t["q_len"]] += 1
        if not t["spans"]:
            assert not V[t["q_start"]:t["q_start"] + t["q_len"]].any()
    assert np.all(rows == 1)
    seen = np.zeros(V.shape, dtype=int)
    for t in tl:
        brute = 0
        for i in range(t["q_start"], t["q_start"] + t["q_len"]):
            for sp in t["spans"]:
                ks, kl = sp[0], sp[1]
                seen[i, ks:ks + kl] += V[i, ks:ks + kl]
                brute += int(V[i, ks:ks + kl].sum())
        assert t["cost"] == brute
    # a span may keep keys its tile's first rows do not see, but no visible pair is missed
    # or counted twice
    assert np.array_equal(seen, V.astype(int))


@pytest.mark.parametrize("window", [1, 5, 64, 100, 1000])
def test_sliding_window_slices(window):
    """The causal sliding window (row i sees keys i - window + 1 .. i of its document) as
    slices equals the band written out directly, and its tiles count every pair once."""
    lengths = [300, 1, 65, 129]
    T = sum(lengths)
    sl = SL.sliding_window_slices(lengths, window)
    seg = np.repeat(np.arange(len(lengths)), lengths)
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    band = (seg[:, None] == seg[None, :]) & (j <= i) & (j > i - window)
    assert np.array_equal(SL.visible(sl, T, T), band)
    tl = P.tiles(SL.fragments(sl), 64)
    assert sum(t["cost"] for t in tl) == int(band.sum())
