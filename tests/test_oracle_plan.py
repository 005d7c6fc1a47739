"""Pins of the reference tile enumerator: brute force on tiny packs, closed
forms, and the worked examples the pages print."""
import json
import os

import numpy as np
import pytest

import workloads
from oracle import attention as A
from oracle import plan as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
with open(os.path.join(GOLDEN, "page_examples.json")) as f:
    PAGES = json.load(f)


def brute_check(tiles, visible, n_q):
    """Every tile's cost equals the explicit mask count of its rows, and its spans
    cover exactly the visible keys of each row (each key once)."""
    covered = np.zeros(n_q, dtype=bool)
    for t in tiles:
        rows = np.arange(t["q_start"], t["q_start"] + t["q_len"])
        assert not covered[rows].any()
        covered[rows] = True
        assert t["cost"] == int(visible[rows].sum())
        for i, r in enumerate(rows):
            got = np.zeros(visible.shape[1], dtype=int)
            for (ks, kl, kp0) in t["spans"]:
                n = P.visible_in_span(t["q_pos0"] + i, kl, kp0)
                got[ks:ks + n] += 1
            assert np.array_equal(got, visible[r].astype(int)), (t, r)
        # blocks: the fewest key blocks of BLOCK_KEYS, laid from each span's start, that hold
        # every key any row of the tile sees; each of them holds a key the last row sees
        seen = visible[rows].any(axis=0)
        swept = np.zeros(visible.shape[1], dtype=bool)
        n_blocks = 0
        for (ks, kl, kp0) in t["spans"]:
            for b0 in range(ks, ks + kl, P.BLOCK_KEYS):
                b1 = min(b0 + P.BLOCK_KEYS, ks + kl)
                assert visible[rows[-1], b0:b1].any(), (t, b0)
                swept[b0:b1] = True
                n_blocks += 1
        assert not (seen & ~swept).any(), t
        assert t["blocks"] == n_blocks, t
    assert covered.all()


def random_lengths(r, total):
    out = []
    while sum(out) < total:
        out.append(int(min(total - sum(out), r.integers(1, 60))))
    return out


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("bm", [16, 32, 64])
def test_causal_doc_brute_force(seed, bm):
    r = np.random.default_rng(seed)
    lengths = random_lengths(r, int(r.integers(1, 300)))
    cu = workloads.cu_from_lengths(lengths)
    T = int(cu[-1])
    seg = A.doc_of_tokens(cu)
    vis = A.visible_causal_doc(seg, np.arange(T), np.arange(T))
    tl = P.tiles(P.fragments_varlen(cu), bm)
    brute_check(tl, vis, T)
    assert P.total_pairs(tl) == sum(l * (l + 1) // 2 for l in lengths)


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("bm", [16, 64])
def test_shared_question_brute_force(seed, bm):
    r = np.random.default_rng(100 + seed)
    Q = int(r.integers(1, 90))
    ans = [int(r.integers(1, 70)) for _ in range(int(r.integers(0, 5)))]
    cu = workloads.cu_from_lengths([Q] + ans)
    T = int(cu[-1])
    seg = A.doc_of_tokens(cu)
    vis = A.visible_shared_question(seg, np.arange(T), np.arange(T))
    tl = P.tiles(P.fragments_varlen(cu, "shared_question"), bm)
    brute_check(tl, vis, T)
    closed = Q * (Q + 1) // 2 + sum(a * Q + a * (a + 1) // 2 for a in ans)
    assert P.total_pairs(tl) == closed


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("bm", [16, 32])
def test_block_brute_force(seed, bm):
    """Random zigzag-like shards: runs of positions cut from a packed sequence."""
    r = np.random.default_rng(200 + seed)
    cp = int(r.choice([2, 3, 4]))
    chunk = int(r.integers(4, 40))
    T = 2 * cp * chunk
    lengths = random_lengths(r, T)
    pos, doc = A.pack_positions(lengths)
    rank = int(r.integers(0, cp))
    src = int(r.integers(0, cp))
    qi = np.concatenate([np.arange(c * chunk, (c + 1) * chunk) for c in A.zigzag_chunks_of_rank(rank, cp)])
    ki = np.concatenate([np.arange(c * chunk, (c + 1) * chunk) for c in A.zigzag_chunks_of_rank(src, cp)])
    q_pos, q_doc, kv_pos, kv_doc = pos[qi], doc[qi], pos[ki], doc[ki]
    vis = A.visible_block(q_pos, q_doc, kv_pos, kv_doc, np.arange(len(qi)), np.arange(len(ki)))
    tl = P.tiles(P.fragments_block(q_pos, q_doc, kv_pos, kv_doc), bm)
    brute_check(tl, vis, len(qi))


def test_runs():
    assert P.runs([0, 1, 2, 7, 8, 9], [0, 0, 1, 1, 1, 2]) == [(0, 2, 0, 0), (2, 1, 2, 1), (3, 2, 7, 1), (5, 1, 9, 2)]


def test_lpt_order():
    cu = workloads.cu_from_lengths([100, 5, 300, 64, 64])
    tl = P.tiles(P.fragments_varlen(cu), 32)
    order = P.lpt_order(tl)
    blocks = [tl[i]["blocks"] for i in order]
    assert blocks == sorted(blocks, reverse=True)
    for a, b in zip(order, order[1:]):
        if tl[a]["blocks"] == tl[b]["blocks"]:
            assert a < b
    assert sorted(order) == list(range(len(tl)))
    # the two 64-token docs give equal tiles; the earlier document comes first
    p = P.plan(P.fragments_varlen(cu), 32)
    eq = [t["q_start"] for t in p if t["cost"] == 32 * 33 // 2 and t["q_len"] == 32]
    assert eq == sorted(eq)
    # ordering by pair count instead is still available to the caller
    by_cost = [tl[i]["cost"] for i in P.lpt_order(tl, key="cost")]
    assert by_cost == sorted(by_cost, reverse=True)


def test_quantised_costs_closed_form():
    """Costs up to 32767 order exactly; above, each is divided by the least power of two
    that brings the largest to 32767 or below, rounding up."""
    assert P.quantised([5, 32767, 0]) == [5, 32767, 0]
    assert P.quantised([32768]) == [16384]
    # 70000 / 2 = 35000 is still above 32767; / 4 rounds 69999 and 70000 up to 17500
    assert P.quantised([70000, 69999, 1, 0]) == [17500, 17500, 1, 0]
    assert P.order_by_cost([69999, 70000, 1, 0]) == [0, 1, 2, 3]  # equal after scaling: natural order
    # a tile with work never ties with one without, however large the plan's largest cost
    assert P.quantised([1 << 58, 1, 0]) == [1 << 14, 1, 0]
    assert P.order_by_cost([0, 1, 1 << 58]) == [2, 1, 0]
    assert P.quantised([]) == []


def test_weighted_order_default_is_blocks():
    """Weights (1, 0) give the block-count order, for any head grouping."""
    cu = workloads.cu_from_lengths([700, 3, 1, 257, 64, 129, 1000, 2])
    for mask in ("causal_doc", "shared_question"):
        tl = P.tiles(P.fragments_varlen(cu, mask), 64)
        for g in (1, 2, 4, 8):
            assert P.lpt_order_weighted(tl, 1, 0, g) == P.lpt_order(tl)


def test_weighted_order_pairs_break_block_ties():
    """A 256-token causal document in 32-row tiles: tile k holds rows 32k .. 32k + 31, sweeps
    ceil((32k + 32) / 64) blocks (1, 1, 2, 2, 3, 3, 4, 4) and holds sum of (r + 1) over its
    rows = 1024k + 528 pairs.  By blocks, the two tiles of each block count keep their natural
    order; with the fitted weights (41515 per block, 1 per pair) the later tile of each pair
    has 1024 more pairs and goes first.  Largest cost 4 * 41515 + 7696 = 173756 is scaled by
    2^3 (by 2^2 it would be 43439): tiles 7 and 6 become 21720 and 21592, still distinct."""
    tl = P.tiles(P.fragments_varlen([0, 256]), 32)
    assert [t["blocks"] for t in tl] == [1, 1, 2, 2, 3, 3, 4, 4]
    assert [t["cost"] for t in tl] == [1024 * k + 528 for k in range(8)]
    assert P.lpt_order(tl) == [6, 7, 4, 5, 2, 3, 0, 1]
    assert P.lpt_order_weighted(tl, 41515, 1, 1) == [7, 6, 5, 4, 3, 2, 1, 0]
    costs = [P.weighted_cost(t, 41515, 1, 1) for t in tl]
    assert costs[7] == 173756 and P.quantised(costs)[6:] == [21592, 21720]


def test_weighted_order_group_multiplies_pairs():
    """The pair term counts the query heads an item serves: tile A (2 blocks, 100 pairs) and
    tile B (1 block, 150 pairs) under weights (100, 1) cost 300 and 250 at G = 1 (A first),
    400 and 400 at G = 2 (a tie: natural order), 600 and 700 at G = 4 (B first)."""
    a = dict(blocks=2, cost=100)
    b = dict(blocks=1, cost=150)
    assert P.lpt_order_weighted([a, b], 100, 1, 1) == [0, 1]
    assert P.lpt_order_weighted([b, a], 100, 1, 2) == [0, 1]
    assert P.lpt_order_weighted([a, b], 100, 1, 2) == [0, 1]
    assert P.lpt_order_weighted([a, b], 100, 1, 4) == [1, 0]
    assert P.weighted_cost(b, 100, 1, 4) == 700


def test_documents_order_hand_worked():
    """Segments of 300, 100, 200, 0 and 10 tokens in 64-row tiles: 5 + 2 + 4 + 0 + 1 tiles,
    natural indices 0-4, 5-6, 7-10, 11.  A tile of rows a .. b sweeps ceil((b + 1) / 64)
    blocks of its document, so the documents' largest tiles sweep 5, 2, 4 and 1 blocks; at
    41515 per block the pair term (at most 4 * 64 * 300 = 76800 here, under two blocks) does
    not reorder them.  Documents longest first, each from its last tile back."""
    cu = [0, 300, 400, 600, 600, 610]
    frags = P.fragments_varlen(cu)
    tl = P.tiles(frags, 64)
    assert [t["blocks"] for t in tl] == [1, 2, 3, 4, 5, 1, 2, 1, 2, 3, 4, 1]
    costs = [P.weighted_cost(t, 41515, 1, 4) for t in tl]
    assert P.documents_order(tl, frags, 64, costs, len(cu) - 1) == [4, 3, 2, 1, 0, 10, 9, 8, 7, 6, 5, 11]
    assert [t["q_start"] for t in P.plan_documents(frags, 64, 41515, 1, 4, len(cu) - 1)] == \
        [256, 192, 128, 64, 0, 592, 528, 464, 400, 364, 300, 600]
    # the LPT order of the same estimates interleaves the documents
    assert P.order_by_cost(costs)[:4] == [4, 3, 10, 2]


def test_documents_order_ties_and_empty_tiles():
    """Fragments of equal largest cost: the later one first.  A tile without key blocks
    counts 0 for its fragment and goes after every tile with blocks, all such tiles in
    descending natural order."""
    frags = [(0, 128, 0, []), (128, 64, 0, []), (192, 128, 0, [])]
    tl = [dict(blocks=3), dict(blocks=0), dict(blocks=3), dict(blocks=1), dict(blocks=0)]
    costs = [3, 0, 3, 1, 0]
    assert P.documents_order(tl, frags, 64, costs, 3) == [2, 0, 3, 4, 1]


@pytest.mark.parametrize("mask", ["causal_doc", "shared_question"])
def test_documents_order_invariants(mask):
    """On random packs: a permutation; each document's tiles together, in descending natural
    order; documents by their largest quantised estimate, non-increasing; equal documents
    later first; a single document is its tiles from last to first."""
    rng = np.random.default_rng(3)
    for trial in range(6):
        lengths = [int(x) for x in rng.integers(1, 900, size=int(rng.integers(2, 12)))]
        cu = workloads.cu_from_lengths(lengths)
        frags = P.fragments_varlen(cu, mask)
        for bm, g in ((64, 4), (32, 8), (256, 1)):
            tl = P.tiles(frags, bm)
            costs = [P.weighted_cost(t, 41515, 1, g) for t in tl]
            order = P.documents_order(tl, frags, bm, costs, len(cu) - 1)
            assert sorted(order) == list(range(len(tl)))
            frag_of = [f for f, fr in enumerate(frags) for _ in range(-(-fr[1] // bm))]
            q = P.quantised(costs)
            top = {}
            for i, t in enumerate(tl):
                top[frag_of[i]] = max(top.get(frag_of[i], 0), q[i])
            seen, last_top, last_frag = set(), None, None
            for a, b in zip(order, order[1:]):
                if frag_of[a] == frag_of[b]:
                    assert a > b
            for i in order:
                f = frag_of[i]
                if f != last_frag:
                    assert f not in seen, "a document's tiles are split"
                    if last_top is not None:
                        assert top[f] < last_top or (top[f] == last_top and f < last_frag)
                    seen.add(f)
                    last_top, last_frag = top[f], f
    one = P.fragments_varlen([0, 1000], mask="causal_doc")
    tl = P.tiles(one, 64)
    costs = [P.weighted_cost(t, 41515, 1, 4) for t in tl]
    assert P.documents_order(tl, one, 64, costs, 1) == list(range(len(tl)))[::-1]


def test_documents_order_capacities():
    """Beyond 4096 segments or 16384 tiles the tile-level order applies."""
    frags = [(64 * i, 64, 0, []) for i in range(4097)]
    tl = [dict(blocks=1 + i % 5) for i in range(4097)]
    costs = [t["blocks"] for t in tl]
    assert P.documents_order(tl, frags, 64, costs, 4097) == P.order_by_cost(costs)
    assert P.documents_order(tl[:4096], frags[:4096], 64, costs[:4096], 4096) != P.order_by_cost(costs[:4096])
    frags = [(320 * i, 320, 0, []) for i in range(3300)]  # 16500 tiles of 64 rows
    tl = [dict(blocks=1 + i % 5) for i in range(16500)]
    costs = [t["blocks"] for t in tl]
    assert P.documents_order(tl, frags, 64, costs, 3300) == P.order_by_cost(costs)
    assert P.documents_order(tl[:16380], frags[:3276], 64, costs[:16380], 3276) != P.order_by_cost(costs[:16380])


def test_short_tile_is_billed_as_a_whole_tile():
    """"03 · 长文负载均衡", section 3.3: a query block shorter than one tile costs a whole
    tile.  A 4-row ragged tail of a 4100-token document sweeps 65 key blocks, more than
    any full tile of it, so it leads the queue although the next tile holds 16 times its pairs."""
    tl = P.tiles(P.fragments_varlen([0, 4100]), 64)
    p = P.plan(P.fragments_varlen([0, 4100]), 64)
    assert p[0]["q_len"] == 4 and p[0]["q_start"] == 4096 and p[0]["blocks"] == 65
    assert p[0]["cost"] == sum(pos + 1 for pos in range(4096, 4100)) == 16_394  # row at position p sees p + 1 keys
    assert p[1]["cost"] == sum(pos + 1 for pos in range(4032, 4096)) > 15 * p[0]["cost"]
    assert [t["blocks"] for t in p[1:]] == list(range(64, 0, -1))
    # tile k of a document covers query positions 64k .. 64k + 63: it sweeps k + 1 blocks
    assert all(t["blocks"] == t["q_start"] // 64 + 1 for t in tl[:-1])


def test_libra_ten_times_example():
    ex = PAGES["libra_pair_example"]
    a = P.total_pairs(P.tiles(P.fragments_varlen([0, ex["long_doc"]]), 64))
    b = P.total_pairs(P.tiles(P.fragments_varlen(workloads.cu_from_lengths(ex["short_docs"])), 64))
    assert sum(ex["short_docs"]) == ex["long_doc"]
    assert a == 838_881_280 and b == 83_906_560
    assert abs(a / b - ex["flop_ratio_approx"]) <= ex["ratio_tolerance"]
    # sum of squares proxy gives exactly 10
    assert ex["long_doc"] ** 2 / sum(l * l for l in ex["short_docs"]) == 10.0


def test_fixture_pair_counts():
    with open(os.path.join(GOLDEN, "oracle_pairs.json")) as f:
        fx = json.load(f)
    with open(os.path.join(GOLDEN, "workload_lengths.json")) as f:
        lens = json.load(f)
    for s in range(5):
        ls = lens[f"longtail_seed{s}"]
        assert fx[f"longtail_seed{s}"] == sum(l * (l + 1) // 2 for l in ls)
    Q, Al, m = 8192, 4096, 8
    assert fx["shared_question_pack"] == Q * (Q + 1) // 2 + m * (Al * Q + Al * (Al + 1) // 2)


# --------------------------------------------------------------------------
# zigzag / ring worked examples ("03 · 长文负载均衡", sections 4.2 and 4.4)
# --------------------------------------------------------------------------
def step_pairs(lengths, chunk, rank, cp, src, seq_chunks=None):
    pos, doc = A.pack_positions(lengths)
    qc = A.zigzag_chunks_of_rank(rank, cp) if seq_chunks is None else seq_chunks[0]
    kc = A.zigzag_chunks_of_rank(src, cp) if seq_chunks is None else seq_chunks[1]
    out = []
    for c in kc:
        qi = np.concatenate([np.arange(x * chunk, (x + 1) * chunk) for x in qc])
        ki = np.arange(c * chunk, (c + 1) * chunk)
        tl = P.tiles(P.fragments_block(pos[qi], doc[qi], pos[ki], doc[ki]), 16)
        out.append(P.total_pairs(tl))
    return out


def test_zigzag_rule_from_page():
    ex = PAGES["zigzag_rule"]
    assert list(A.zigzag_chunks_of_rank(ex["rank"], ex["cp"])) == ex["chunks"]


@pytest.mark.parametrize("cp", [2, 4, 8])
def test_zigzag_balances_a_single_document(cp):
    C = 8
    lengths = [2 * cp * C]
    per_rank = [sum(sum(step_pairs(lengths, C, r, cp, s)) for s in range(cp)) for r in range(cp)]
    assert per_rank == [(2 * cp - 1) * C * C + C * (C + 1)] * cp


@pytest.mark.parametrize("cp", [2, 4, 8])
def test_zigzag_causal_redundancy_is_a_quarter(cp):
    C = 4
    lengths = [2 * cp * C]
    useless = received = 0
    for r in range(cp):
        for t in range(1, cp):
            for pairs in step_pairs(lengths, C, r, cp, A.ring_source(r, t, cp)):
                received += 1
                useless += pairs == 0
    assert received == 2 * cp * (cp - 1)
    assert useless == cp * (cp - 1) // 2
    assert useless / received == PAGES["causal_ring_redundancy"]["fraction_approx"]


def test_sequential_ring_block_counts():
    ex = PAGES["sequential_ring_blocks"]
    cp, C = ex["cp"], 8
    lengths = [cp * C]
    counts = []
    for r in range(cp):
        n = 0
        for t in range(cp):
            src = A.ring_source(r, t, cp)
            n += step_pairs(lengths, C, r, cp, src, seq_chunks=([r], [src]))[0] > 0
        counts.append(n)
    assert counts == ex["blocks_per_rank"]


@pytest.mark.slow
def test_zigzag_rank3_step_pairs_match_explicit_mask():
    """Per-step visible pairs of rank 3 (cp=8, 8192-token chunks) by the span count
    and by an explicit mask count, on the 131072-token lognormal pack, seed 0."""
    lengths = workloads.zigzag_pack_lengths(0)
    pos, doc = A.pack_positions(lengths)
    C, cp, rank = 8192, 8, 3
    qi = np.concatenate([np.arange(c * C, (c + 1) * C) for c in A.zigzag_chunks_of_rank(rank, cp)])
    got = []
    for t in range(cp):
        src = A.ring_source(rank, t, cp)
        ki = np.concatenate([np.arange(c * C, (c + 1) * C) for c in A.zigzag_chunks_of_rank(src, cp)])
        tl = P.tiles(P.fragments_block(pos[qi], doc[qi], pos[ki], doc[ki]), 64)
        span_count = P.total_pairs(tl)
        explicit = 0
        for b in range(0, len(qi), 2048):
            rows = np.arange(b, b + 2048)
            explicit += int(A.visible_block(pos[qi], doc[qi], pos[ki], doc[ki], rows, np.arange(len(ki))).sum())
        assert span_count == explicit
        got.append(span_count)
    assert got == [20_319_978, 7_981_112, 0, 0, 0, 0, 0, 3_473_470]


# --------------------------------------------------------------------------
# transposed (key) tiling of the backward
# --------------------------------------------------------------------------
def brute_pairs_of_key_tile(t, visible):
    keys = range(t["q_start"], t["q_start"] + t["q_len"])
    rows = [r for (qs, ql, _) in t["spans"] for r in range(qs, qs + ql)]
    return sum(1 for j in keys for i in rows if visible(i, j))


@pytest.mark.parametrize("mask", ["causal_doc", "shared_question"])
@pytest.mark.parametrize("bm", [16, 32, 64])
def test_transposed_tiles_cover_every_visible_pair_once_varlen(mask, bm):
    r = np.random.default_rng(bm + (mask == "shared_question"))
    lengths = [int(x) for x in r.integers(1, 90, 7)]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    seg = A.doc_of_tokens(cu)
    T = int(cu[-1])
    vis = A.visible_causal_doc if mask == "causal_doc" else A.visible_shared_question
    V = vis(seg, np.arange(T), np.arange(T))
    tl = P.tiles_t(P.fragments_varlen_t(cu, mask), bm)
    seen = np.zeros((T, T), dtype=int)
    for t in tl:
        assert t["cost"] == brute_pairs_of_key_tile(t, lambda i, j: V[i, j])
        for j in range(t["q_start"], t["q_start"] + t["q_len"]):
            for (qs, ql, _) in t["spans"]:
                seen[qs:qs + ql, j] += V[qs:qs + ql, j]
    assert np.array_equal(seen, V.astype(int))  # every visible pair in exactly one (tile, span)
    assert sum(t["cost"] for t in tl) == int(V.sum())
    # the first row kept in every span sees the tile's first key
    for t in tl:
        for (qs, ql, _) in t["spans"]:
            assert V[qs, t["q_start"]]


@pytest.mark.parametrize("seed", range(4))
def test_transposed_tiles_cover_every_visible_pair_once_block(seed):
    r = np.random.default_rng(40 + seed)
    lengths = [int(x) for x in r.integers(1, 120, 6)]
    pos, doc = A.pack_positions(lengths)
    T = len(pos)
    perm = r.permutation(T)
    qi, ki = np.sort(perm[:T // 2]), np.sort(perm[T // 2:])
    qi = np.sort(np.concatenate([qi, ki[:T // 5]]))  # some tokens on both sides
    V = A.visible_block(pos[qi], doc[qi], pos[ki], doc[ki], np.arange(len(qi)), np.arange(len(ki)))
    tl = P.tiles_t(P.fragments_block_t(pos[qi], doc[qi], pos[ki], doc[ki]), 16)
    seen = np.zeros(V.shape, dtype=int)
    for t in tl:
        assert t["cost"] == brute_pairs_of_key_tile(t, lambda i, j: V[i, j])
        for j in range(t["q_start"], t["q_start"] + t["q_len"]):
            for (qs, ql, _) in t["spans"]:
                seen[qs:qs + ql, j] += V[qs:qs + ql, j]
    assert np.array_equal(seen, V.astype(int))
    # and the pair total equals the forward tiling's
    fwd = P.tiles(P.fragments_block(pos[qi], doc[qi], pos[ki], doc[ki]), 16)
    assert sum(t["cost"] for t in fwd) == sum(t["cost"] for t in tl) == int(V.sum())


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("bm", [16, 32])
@pytest.mark.parametrize("rule", ["zigzag", "per_document"])
def test_block_shared_doc_brute_force(seed, bm, rule):
    """Shards of a shared-question pack (document 0 shared), by sequence zigzag or per
    document (which cuts every document, the shared one too, into several runs per rank, so
    its FULL runs join): every tile's cost equals the explicit mask count, its spans cover
    each visible key once, and the transposed tiling covers every visible pair once."""
    from oracle import sharding as S
    r = np.random.default_rng(900 + seed)
    cp = int(r.choice([2, 3, 4]))
    chunk = int(r.integers(4, 40))
    T = 2 * cp * chunk
    lengths = random_lengths(r, T)
    pos, doc = A.pack_positions(lengths)
    rank, src = int(r.integers(0, cp)), int(r.integers(0, cp))
    if rule == "zigzag":
        qi = np.concatenate([np.arange(c * chunk, (c + 1) * chunk) for c in A.zigzag_chunks_of_rank(rank, cp)])
        ki = np.concatenate([np.arange(c * chunk, (c + 1) * chunk) for c in A.zigzag_chunks_of_rank(src, cp)])
    else:
        tok = S.per_document_tokens(lengths, cp)
        qi, ki = tok[rank], tok[src]
    vis = A.visible_block(pos[qi], doc[qi], pos[ki], doc[ki], np.arange(len(qi)), np.arange(len(ki)), 0)
    tl = P.tiles(P.fragments_block(pos[qi], doc[qi], pos[ki], doc[ki], shared_doc=0), bm)
    brute_check(tl, vis, len(qi))
    seen = np.zeros(vis.shape, dtype=int)
    for t in P.tiles_t(P.fragments_block_t(pos[qi], doc[qi], pos[ki], doc[ki], shared_doc=0), bm):
        assert t["cost"] == brute_pairs_of_key_tile(t, lambda i, j: vis[i, j])
        for j in range(t["q_start"], t["q_start"] + t["q_len"]):
            for (qs, ql, _) in t["spans"]:
                seen[qs:qs + ql, j] += vis[qs:qs + ql, j]
    assert np.array_equal(seen, vis.astype(int))


def test_block_shared_doc_pairs_closed_form():
    """Over a whole shared-question pack the tiles hold Q(Q+1)/2 + sum over answers of
    A*Q + A(A+1)/2 pairs, forward and transposed."""
    lengths = [300, 77, 1, 128, 64, 200]
    Q = lengths[0]
    want = Q * (Q + 1) // 2 + sum(a * Q + a * (a + 1) // 2 for a in lengths[1:])
    pos, doc = A.pack_positions(lengths)
    fwd = P.tiles(P.fragments_block(pos, doc, pos, doc, shared_doc=0), 64)
    bwd = P.tiles_t(P.fragments_block_t(pos, doc, pos, doc, shared_doc=0), 128)
    assert sum(t["cost"] for t in fwd) == want
    assert sum(t["cost"] for t in bwd) == want


def test_block_shared_doc_full_runs_join():
    """FULL runs next to each other in the buffer make one span; a run of the row's own
    document, or a gap in the buffer, starts a new one.  Spans written out by hand."""
    far = P.FAR
    # forward: a query run of document 1 against keys [doc 0 at 0..2 | doc 0 at 10..11 |
    # doc 1 at 0..1 | doc 0 at 20]
    q_pos, q_doc = np.arange(4), np.ones(4, dtype=int)
    kv_pos, kv_doc = np.array([0, 1, 2, 10, 11, 0, 1, 20]), np.array([0, 0, 0, 0, 0, 1, 1, 0])
    (f,) = P.fragments_block(q_pos, q_doc, kv_pos, kv_doc, shared_doc=0)
    assert f[3] == [(0, 5, -far), (5, 2, 0), (7, 1, -far)]
    # transposed: a key run of document 0 (positions 0..3) against query runs [doc 1 | doc 2 |
    # doc 0 at position 0 | doc 3]: documents 1 and 2 join, document 3 follows the own run
    q_pos, q_doc = np.array([0, 1, 0, 1, 2, 0, 0]), np.array([1, 1, 2, 2, 2, 0, 3])
    (f,) = P.fragments_block_t(q_pos, q_doc, np.arange(4), np.zeros(4, dtype=int), shared_doc=0)
    assert f[3] == [(0, 5, far), (5, 1, 0), (6, 1, far)]


def test_merge_step_plans_by_hand():
    """Two steps' plans with key blocks [5, 3, 1] and [4, 3, (no span)]: the merged queue,
    written out by hand, is 5, 4, 3 (step 0 first on the tie), 3, 1, then the spanless tile."""
    def t(blocks, tag):
        return dict(q_start=tag, q_len=1, q_pos0=0, spans=[(0, 1, 0)] if blocks else [], cost=blocks, blocks=blocks)
    a = [t(5, 0), t(3, 1), t(1, 2)]
    b = [t(4, 10), t(3, 11), t(0, 12)]
    got = [(x["step"], x["q_start"]) for x in P.merge_step_plans([a, b])]
    assert got == [(0, 0), (1, 10), (0, 1), (1, 11), (0, 2), (1, 12)]


@pytest.mark.parametrize("seed", range(4))
def test_merge_step_plans_keeps_each_step_and_sorts(seed):
    """The merged queue of the live steps of a zigzag rank: every step's tiles appear once and
    in that step's own order, the key blocks never increase over the tiles with spans, and
    spanless tiles come last."""
    r = np.random.default_rng(seed)
    cp, chunk = 4, 48
    T = 2 * cp * chunk
    lengths = random_lengths(r, T)
    pos, doc = A.pack_positions(lengths)
    rank = int(r.integers(0, cp))
    qi = np.concatenate([np.arange(c * chunk, (c + 1) * chunk) for c in A.zigzag_chunks_of_rank(rank, cp)])
    plans = []
    for src in range(cp):
        ki = np.concatenate([np.arange(c * chunk, (c + 1) * chunk) for c in A.zigzag_chunks_of_rank(src, cp)])
        plans.append(P.plan(P.fragments_block(pos[qi], doc[qi], pos[ki], doc[ki]), 16))
    merged = P.merge_step_plans(plans)
    assert len(merged) == sum(len(p) for p in plans)
    for s, p in enumerate(plans):
        mine = [{k: v for k, v in x.items() if k != "step"} for x in merged if x["step"] == s]
        assert [x for x in mine if x["spans"]] == [x for x in p if x["spans"]]
        assert [x for x in mine if not x["spans"]] == [x for x in p if not x["spans"]]
    n_work = sum(1 for x in merged if x["spans"])
    assert all(x["spans"] for x in merged[:n_work]) and not any(x["spans"] for x in merged[n_work:])
    blocks = [x["blocks"] for x in merged[:n_work]]
    assert blocks == sorted(blocks, reverse=True)


def test_fuse_step_plans_by_hand():
    """Three query tiles over two steps, written out by hand.  Step 0: tile 0 one span of 10
    keys (1 block), tile 1 none, tile 2 one span of 70 keys (2 blocks).  Step 1: tile 0 none,
    tile 1 one span of 5 keys (1 block), tile 2 two spans of 64 and 1 keys (2 blocks).  Fused:
    tile 2 (4 blocks, spans steps 0, 1, 1), then tiles 0 and 1 (1 block each, natural order)."""
    def t(x, spans, cost):
        return dict(q_start=16 * x, q_len=16, q_pos0=100 + 16 * x, spans=spans, cost=cost,
                    blocks=sum(-(-n // P.BLOCK_KEYS) for _, n, _ in spans))
    s0 = [t(0, [(0, 10, 0)], 7), t(1, [], 0), t(2, [(20, 70, 30)], 50)]
    s1 = [t(0, [], 0), t(1, [(3, 5, 9)], 4), t(2, [(0, 64, 0), (64, 1, 64)], 9)]
    got = P.fuse_step_plans([s0, s1])
    assert [g["q_start"] for g in got] == [32, 0, 16]
    assert got[0]["spans"] == [(20, 70, 30), (0, 64, 0), (64, 1, 64)] and got[0]["span_steps"] == [0, 1, 1]
    assert [(g["cost"], g["blocks"]) for g in got] == [(59, 4), (7, 1), (4, 1)]
    assert got[2]["span_steps"] == [1] and got[1]["span_steps"] == [0]


def test_fuse_step_plans_refuses_past_the_span_capacity():
    def t(n_spans):
        return dict(q_start=0, q_len=8, q_pos0=0, spans=[(64 * i, 8, 0) for i in range(n_spans)], cost=8 * n_spans,
                    blocks=n_spans)
    assert P.fuse_step_plans([[t(2)], [t(2)]]) is not None
    assert P.fuse_step_plans([[t(3)], [t(2)]]) is None


@pytest.mark.parametrize("seed", range(4))
def test_fuse_step_plans_against_explicit_masks(seed):
    """A zigzag rank's steps fused: each fused tile's spans of step s cover exactly the keys of
    step s that some row of the tile sees (brute force over the explicit block mask: same
    document, key position <= row position), its pairs are the visible pairs counted the same
    way, and the order is key blocks descending, spanless tiles last."""
    r = np.random.default_rng(100 + seed)
    cp, chunk, bm = 4, 48, 16
    T = 2 * cp * chunk
    lengths = random_lengths(r, T)
    pos, doc = A.pack_positions(lengths)
    rank = int(r.integers(0, cp))
    qi = np.concatenate([np.arange(c * chunk, (c + 1) * chunk) for c in A.zigzag_chunks_of_rank(rank, cp)])
    kis, plans = [], []
    for t in range(cp):
        src = (rank - t) % cp
        ki = np.concatenate([np.arange(c * chunk, (c + 1) * chunk) for c in A.zigzag_chunks_of_rank(src, cp)])
        kis.append(ki)
        plans.append(P.tiles(P.fragments_block(pos[qi], doc[qi], pos[ki], doc[ki]), bm))
    fused = P.fuse_step_plans(plans)
    if fused is None:  # more than FUSED_SPAN_CAP spans in some tile: nothing to check here
        pytest.skip("a tile past the span capacity")
    assert len(fused) == len(plans[0])
    rows_seen = set()
    for f in fused:
        rows = qi[f["q_start"]:f["q_start"] + f["q_len"]]
        rows_seen.update(range(f["q_start"], f["q_start"] + f["q_len"]))
        pairs = 0
        for s, ki in enumerate(kis):
            vis = (doc[rows][:, None] == doc[ki][None, :]) & (pos[ki][None, :] <= pos[rows][:, None])
            pairs += int(vis.sum())
            want = set(np.nonzero(vis.any(axis=0))[0].tolist())
            have = set()
            for (ks, kl, _), st in zip(f["spans"], f["span_steps"]):
                if st == s:
                    have.update(range(ks, ks + kl))
            assert have == want
        assert f["cost"] == pairs
    assert rows_seen == set(range(len(qi)))
    n_work = sum(1 for f in fused if f["blocks"] > 0)
    assert all(f["spans"] for f in fused[:n_work]) and not any(f["spans"] for f in fused[n_work:])
    blocks = [f["blocks"] for f in fused[:n_work]]
    assert blocks == sorted(blocks, reverse=True)
    empty_starts = [f["q_start"] for f in fused[n_work:]]
    assert empty_starts == sorted(empty_starts)
