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


# --------------------------------------------------------------------------
# mask-area dispatch ("03 · 长文负载均衡", section 4.4, MagiAttention)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("cp", [2, 4, 8])
def test_dispatch_of_one_causal_document_is_zigzag(cp):
    """Section 4.4 places zigzag inside the dispatch solver's solution space as a hand-built
    symmetric point.  For one causal document cut into 2cp chunks of c tokens, chunk i has
    area c^2 i + c(c+1)/2 (strictly increasing), and the greedy puts chunks 2cp-1 .. cp on
    ranks 0 .. cp-1 and then chunk j < cp on rank j: exactly rank i <- {i, 2cp-1-i}."""
    c = 7
    areas = S.chunk_areas([2 * cp * c], 2 * cp)
    assert areas == [c * c * i + c * (c + 1) // 2 for i in range(2 * cp)]
    assert S.dispatch_chunks(areas, cp) == [[i, 2 * cp - 1 - i] for i in range(cp)]
    for a, b in zip(S.dispatch_tokens([2 * cp * c], cp, 2 * cp), S.zigzag_tokens(2 * cp * c, cp)):
        assert np.array_equal(a, b)


def test_dispatch_worked_example():
    # areas 5 5 3 3 1 1 into 3 buckets of 2: 0 -> b0, 1 -> b1, 2 -> b2 (loads 5 5 3);
    # 3 -> b2 (least, now full at 6); 4 -> b0 (tie 5 = 5, lower bucket); 5 -> b1
    assert S.dispatch_chunks([5, 5, 3, 3, 1, 1], 3) == [[0, 4], [1, 5], [2, 3]]
    # a chunk never goes to a full bucket even when that bucket is the least loaded
    assert S.dispatch_chunks([9, 1, 1, 1], 2) == [[0, 3], [1, 2]]


def test_chunk_areas_sum_to_the_pack_pairs():
    r = np.random.default_rng(3)
    lengths = random_lengths(r, 11, 90)
    lengths.append(16 * 40 - sum(lengths) % (16 * 40))  # pad to a multiple of 16 chunks
    areas = S.chunk_areas(lengths, 16)
    assert sum(areas) == sum(n * (n + 1) // 2 for n in lengths)
    tok = S.dispatch_tokens(lengths, 4, 16)
    assert is_partition(tok, sum(lengths))
    assert len({len(t) for t in tok}) == 1  # equal token counts: n / cp chunks each
    assert S.rank_pairs(lengths, tok) == [sum(areas[c] for c in h) for h in S.dispatch_chunks(areas, 4)]


@pytest.mark.parametrize("seed", range(6))
def test_dispatch_against_brute_force(seed):
    """Tiny cases against every assignment of 8 chunks to cp buckets of equal size: the
    greedy's assignment is feasible, and its busiest bucket is at or above the optimum and,
    on these cases, within one chunk's area of it."""
    import itertools
    r = np.random.default_rng(seed)
    areas = [int(x) for x in r.integers(1, 50, 8)]
    for cp in (2, 4):
        cap = 8 // cp
        best = None
        for labels in itertools.product(range(cp), repeat=8):
            if any(labels.count(b) != cap for b in range(cp)):
                continue
            mx = max(sum(a for a, l in zip(areas, labels) if l == b) for b in range(cp))
            best = mx if best is None else min(best, mx)
        held = S.dispatch_chunks(areas, cp)
        assert sorted(c for h in held for c in h) == list(range(8)) and all(len(h) == cap for h in held)
        got = max(sum(areas[c] for c in h) for h in held)
        assert best <= got <= best + max(areas)


def test_dispatch_balances_the_packed_pack():
    """On the 131072-token pack of seed 0 at cp = 8, where sequence zigzag leaves the busiest
    rank 1.633x the mean (section 1.2), the dispatch of 64 chunks of 2048 tokens brings it
    within 1% while every rank keeps 16384 tokens."""
    lengths = workloads.zigzag_pack_lengths(0)
    tok = S.dispatch_tokens(lengths, 8, 64)
    pairs = S.rank_pairs(lengths, tok)
    assert max(pairs) / np.mean(pairs) < 1.01
    assert all(len(t) == 16384 for t in tok)


@pytest.mark.parametrize("cp", [2, 4])
def test_dispatch_ring_reassembles_the_unsharded_result(cp):
    H, Hkv, d = 4, 2, 32
    r = np.random.default_rng(8)
    lengths = [37, 5, 90, 1, 59, 48]  # 240 tokens: 8 or 16 chunks
    T = sum(lengths)
    q, k, v = (r.standard_normal((T, h, d)) for h in (H, Hkv, Hkv))
    tok = S.dispatch_tokens(lengths, cp, 4 * cp)
    full_o, full_l = A.varlen_attention(q, k, v, workloads.cu_from_lengths(lengths), H, Hkv)
    for rank in range(cp):
        o, l = S.sharded_rank_attention(q, k, v, lengths, tok, rank, H, Hkv)
        assert np.max(np.abs(o - full_o[tok[rank]])) < 1e-12
        assert np.max(np.abs(l - full_l[:, tok[rank]])) < 1e-12
