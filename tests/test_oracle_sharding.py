"""Pins of the oracle's context-parallel sharding rules and of the sharded ring fold."""
import numpy as np
import pytest

import workloads
from oracle import attention as A
from oracle import sharding as S


def random_lengths(r, n_docs, hi):
    return [int(x) for x in r.integers(1, hi, n_docs)]


def is_partition(tokens, total):
    cat = np.concatenate(tokens)
    return len(cat) == total and np.array_equal(np.sort(cat), np.arange(total))


@pytest.mark.parametrize("cp", [2, 4, 8])
@pytest.mark.parametrize("seed", range(4))
def test_per_document_is_a_partition_with_balanced_tokens(cp, seed):
    r = np.random.default_rng(seed)
    lengths = random_lengths(r, int(r.integers(1, 30)), 300)
    tok = S.per_document_tokens(lengths, cp)
    assert is_partition(tok, sum(lengths))
    counts = [len(t) for t in tok]
    assert max(counts) - min(counts) <= 1  # no padding; the remainder deal keeps ranks within one token
    for t in tok:
        assert np.all(np.diff(t) > 0)


@pytest.mark.parametrize("cp", [2, 4, 8])
def test_per_document_equal_area_closed_form(cp):
    """"03 · 长文负载均衡", section 4.3: every worker takes one symmetric chunk pair of every
    document and the areas (causal pairs) are equal.  With chunk length c per document,
    rank i holds positions i*c .. and (2cp-1-i)*c ..: pairs c^2 (2cp-1) + c (c+1)."""
    r = np.random.default_rng(cp)
    cs = [int(x) for x in r.integers(1, 40, 9)]
    lengths = [2 * cp * c for c in cs]
    tok = S.per_document_tokens(lengths, cp)
    pairs = S.rank_pairs(lengths, tok)
    expect = sum(c * c * (2 * cp - 1) + c * (c + 1) for c in cs)
    assert pairs == [expect] * cp


def test_per_document_remainder_is_dealt_round_robin():
    # cp = 2: 2cp = 4.  Doc 0 (len 6): chunks of 1 -> rank 0 {0, 3}, rank 1 {1, 2}; its tail
    # {4, 5} goes to ranks 0, 1.  Doc 1 (len 3, starting at 6): no chunks; tail 6, 7, 8 to
    # ranks 0, 1, 0 (the deal continues).  Doc 2 (len 1): token 9 to rank 1.
    tok = S.per_document_tokens([6, 3, 1], 2)
    assert tok[0].tolist() == [0, 3, 4, 6, 8]
    assert tok[1].tolist() == [1, 2, 5, 7, 9]


def test_zigzag_tokens_match_chunk_rule():
    T, cp = 64, 4
    tok = S.zigzag_tokens(T, cp)
    c = T // (2 * cp)
    for r in range(cp):
        a, b = A.zigzag_chunks_of_rank(r, cp)
        assert tok[r].tolist() == list(range(a * c, (a + 1) * c)) + list(range(b * c, (b + 1) * c))
    assert is_partition(tok, T)


def test_striped_tokens():
    tok = S.striped_tokens(20, 3, width=2)
    assert tok[0].tolist() == [0, 1, 6, 7, 12, 13, 18, 19]
    assert tok[1].tolist() == [2, 3, 8, 9, 14, 15]
    assert is_partition(tok, 20)
    assert S.striped_tokens(7, 2)[1].tolist() == [1, 3, 5]


def test_single_document_zigzag_and_per_document_agree():
    # one document of 2cp*c tokens: per-document sharding is the sequence zigzag
    cp, c = 4, 13
    assert all(np.array_equal(a, b) for a, b in zip(S.per_document_tokens([2 * cp * c], cp),
                                                       S.zigzag_tokens(2 * cp * c, cp)))


def test_rank_pairs_sum_to_the_pack():
    r = np.random.default_rng(5)
    lengths = random_lengths(r, 12, 200)
    for tok in (S.per_document_tokens(lengths, 4), S.striped_tokens(sum(lengths), 4, 3)):
        assert sum(S.rank_pairs(lengths, tok)) == sum(n * (n + 1) // 2 for n in lengths)


def test_packed_zigzag_is_imbalanced_per_document_is_not():
    """"03 · 长文负载均衡", sections 1.2 and 4.3: on a packed sequence the sequence-level zigzag
    leaves the ranks' attention work unequal; per-document sharding equalises it.  On the
    131072-token lognormal pack of seed 0 at cp = 8 the zigzag ranks carry
    [32.73M, 64.29M, 20.09M, 31.77M, 63.52M, 86.19M, 81.95M, 41.80M] pairs per head."""
    lengths = workloads.zigzag_pack_lengths(0)
    T, cp = sum(lengths), 8
    zz = S.rank_pairs(lengths, S.zigzag_tokens(T, cp))
    assert [round(x / 1e6, 2) for x in zz] == [32.73, 64.29, 20.09, 31.77, 63.52, 86.19, 81.95, 41.80]
    assert abs(max(zz) / np.mean(zz) - 1.633) < 1e-3
    pd = S.rank_pairs(lengths, S.per_document_tokens(lengths, cp))
    assert sum(pd) == sum(zz)
    assert max(pd) / np.mean(pd) < 1.001


@pytest.mark.parametrize("rule", ["zigzag", "per_document", "striped"])
def test_sharded_ring_reassembles_the_unsharded_result(rule):
    cp, H, Hkv, d = 4, 4, 2, 32
    r = np.random.default_rng(7)
    lengths = [37, 5, 90, 1, 59]
    T = sum(lengths)
    if rule == "zigzag":
        lengths = lengths + [2 * cp * 25 - T]  # pad the pack to a multiple of 2*cp with one more document
        T = sum(lengths)
    q, k, v = (r.standard_normal((T, h, d)) for h in (H, Hkv, Hkv))
    tok = {"zigzag": lambda: S.zigzag_tokens(T, cp), "per_document": lambda: S.per_document_tokens(lengths, cp),
           "striped": lambda: S.striped_tokens(T, cp, 3)}[rule]()
    full_o, full_l = A.varlen_attention(q, k, v, workloads.cu_from_lengths(lengths), H, Hkv)
    for rank in range(cp):
        o, l = S.sharded_rank_attention(q, k, v, lengths, tok, rank, H, Hkv)
        assert np.max(np.abs(o - full_o[tok[rank]])) < 1e-12
        assert np.max(np.abs(l - full_l[:, tok[rank]])) < 1e-12
