"""GPU parity: the HIP library (through its C ABI) against the float64 oracle.

Tolerances (bf16 inputs, fp32 accumulation): out max |d| <= 2e-2 and mean
|d| <= 2e-3, lse max |d| <= 5e-3.  Plans (tiles, spans, exact pair costs and
longest-first order) must equal the oracle's enumerator bit for bit; the varlen
forward's queue follows the fitted estimate (41515 per key block, 1 per
query-head pair).
Large configurations are compared on sampled rows that the oracle computes
one by one; small ones on every row.
"""
import math
import sys

import numpy as np
import pytest
import torch

import load_balance_amd as lb
import workloads
from oracle import attention as OA
from oracle import plan as OP

pytestmark = pytest.mark.gpu

OUT_MAX, OUT_MEAN, LSE_MAX = 2e-2, 2e-3, 5e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bits_of(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def f32(bits):
    return workloads.bf16_bits_to_f32(bits)


def run_varlen(pack, mask_kind=lb.MASK_CAUSAL_DOC):
    say(f"  varlen_attn_fwd T={pack['tokens']} H={pack['heads']} Hkv={pack['kv_heads']} d={pack['d']} "
        f"docs={len(pack['lengths'])} mask={mask_kind}")
    q, k, v = dev_bf16(pack["q"]), dev_bf16(pack["k"]), dev_bf16(pack["v"])
    cu = torch.from_numpy(np.asarray(pack["cu_seqlens"], dtype=np.int32)).cuda()
    ws = lb.new_workspace(pack["tokens"], len(pack["lengths"]), pack["heads"], pack["kv_heads"])
    out, lse = lb.varlen_attn_fwd(q, k, v, cu, mask_kind=mask_kind, workspace=ws)
    torch.cuda.synchronize()
    assert lb.read_device_error(ws) == 0
    return out, lse, ws


def check(out_gpu, lse_gpu, out_ref, lse_ref, what=""):
    og = np.asarray(out_gpu, dtype=np.float64)
    lg = np.asarray(lse_gpu, dtype=np.float64)
    assert np.all(np.isfinite(og)), f"{what}: non-finite output"
    d_out = np.abs(og - out_ref)
    d_lse = np.abs(lg - lse_ref)
    say(f"  {what}: out max {d_out.max():.3e} mean {d_out.mean():.3e}  lse max {d_lse.max():.3e}")
    assert d_out.max() <= OUT_MAX, what
    assert d_out.mean() <= OUT_MEAN, what
    assert d_lse.max() <= LSE_MAX, what


def sample_rows(lengths, bm, n_random, seed, cap=None):
    cu = np.concatenate([[0], np.cumsum(lengths)])
    r = np.random.default_rng(seed)
    rows = set()
    for s in range(len(lengths)):
        a, b = int(cu[s]), int(cu[s + 1])
        if b <= a:
            continue
        rows.update([a, b - 1, min(b - 1, a + bm - 1), min(b - 1, a + bm)])
    rows.update(r.integers(0, int(cu[-1]), n_random).tolist())
    rows = sorted(rows)
    if cap is not None and len(rows) > cap:
        rows = sorted(r.choice(rows, cap, replace=False).tolist())
    return np.array(rows, dtype=np.int64)


def plan_ref_varlen(pack, mask="causal_doc"):
    return plan_ref_ordered(pack, lb.LPT_FIT_BLOCK_WEIGHT, lb.LPT_FIT_PAIR_WEIGHT, lb.ORDER_DOCUMENTS, mask)


def plan_ref_ordered(pack, block_weight, pair_weight, order, mask="causal_doc"):
    if order == lb.ORDER_LPT:
        return plan_ref_weighted(pack, block_weight, pair_weight, mask)
    bm = lb.tile_rows(pack["heads"], pack["kv_heads"], pack["d"])
    return OP.plan_documents(OP.fragments_varlen(pack["cu_seqlens"], mask), bm, block_weight, pair_weight,
                             pack["heads"] // pack["kv_heads"], len(pack["cu_seqlens"]) - 1)


def plan_ref_weighted(pack, block_weight, pair_weight, mask="causal_doc"):
    bm = lb.tile_rows(pack["heads"], pack["kv_heads"], pack["d"])
    return OP.plan_weighted(OP.fragments_varlen(pack["cu_seqlens"], mask), bm, block_weight, pair_weight,
                            pack["heads"] // pack["kv_heads"])


def assert_same_plan(gpu, ref, what):
    assert len(gpu) == len(ref), f"{what}: {len(gpu)} tiles vs {len(ref)}"
    for i, (a, b) in enumerate(zip(gpu, ref)):
        assert a == b, f"{what}: tile {i}: gpu {a} != oracle {b}"


# --------------------------------------------------------------------------
# fixtures: the five workloads
# --------------------------------------------------------------------------
@pytest.fixture(scope="module")
def tiny():
    return workloads.tiny_pack()


@pytest.fixture(scope="module")
def longtail():
    return workloads.longtail_pack(0)


@pytest.fixture(scope="module")
def pair():
    return workloads.pair_packs()


@pytest.fixture(scope="module")
def shared_q():
    return workloads.shared_question_packs()


# --------------------------------------------------------------------------
# config 1: tiny pack, every row
# --------------------------------------------------------------------------
def test_tiny_pack_full(tiny):
    out, lse, ws = run_varlen(tiny)
    ref_o, ref_l = OA.varlen_attention(tiny["q"], tiny["k"], tiny["v"], tiny["cu_seqlens"], 2, 2)
    check(out.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "tiny pack")
    assert_same_plan(lb.read_plan(ws), plan_ref_varlen(tiny), "tiny plan")
    # reported, not gated: distance to the unrounded fp32 inputs
    o32, l32 = OA.varlen_attention(tiny["q32"], tiny["k32"], tiny["v32"], tiny["cu_seqlens"], 2, 2)
    say(f"  vs unrounded fp32 inputs: out max {np.abs(out.float().cpu().numpy() - o32).max():.3e}")


@pytest.mark.parametrize("H,Hkv,d", [(2, 2, 64), (4, 2, 64), (8, 2, 128), (16, 2, 128), (32, 8, 128), (8, 8, 128)])
def test_random_pack_every_row(H, Hkv, d):
    """Several tiles per document, ragged tails, 1-token documents, all head groupings."""
    r = np.random.default_rng(H * 1000 + Hkv * 10 + d)
    lengths = [1, 700, 3, 1, 257, 64, 129, 1000, 2]
    T = sum(lengths)
    q, k, v = workloads.values(r, T, H, Hkv, d)
    pack = dict(lengths=lengths, cu_seqlens=workloads.cu_from_lengths(lengths), tokens=T, heads=H, kv_heads=Hkv,
                d=d, q=q, k=k, v=v)
    out, lse, ws = run_varlen(pack)
    ref_o, ref_l = OA.varlen_attention(q, k, v, pack["cu_seqlens"], H, Hkv)
    check(out.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, f"random pack H={H} Hkv={Hkv} d={d}")
    assert_same_plan(lb.read_plan(ws), plan_ref_varlen(pack), "random plan")


# --------------------------------------------------------------------------
# config 2: 32K long-tail pack, sampled rows
# --------------------------------------------------------------------------
def test_longtail_pack(longtail):
    p = longtail
    out, lse, ws = run_varlen(p)
    assert_same_plan(lb.read_plan(ws), plan_ref_varlen(p), "32K long-tail plan")
    rows = sample_rows(p["lengths"], 64, 96, 1, cap=256)
    ref_o, ref_l = OA.varlen_attention(p["q"], p["k"], p["v"], p["cu_seqlens"], 32, 8, rows=rows)
    check(out[rows].float().cpu().numpy(), lse[:, rows].cpu().numpy(), ref_o, ref_l, "32K long-tail (sampled)")
    recs = lb.read_worker_timing(ws)
    assert len(recs) == torch.cuda.get_device_properties(0).multi_processor_count
    plan = lb.read_plan(ws)
    assert sum(x["items"] for x in recs) == len(plan) * 8
    assert sum(x["pairs"] for x in recs) == 32 * 49_322_947
    assert sum(x["blocks"] for x in recs) == 8 * sum(t["blocks"] for t in plan)


@pytest.mark.timeout(900)
def test_longtail_pack_every_row(longtail, tmp_path):
    """All 32768 rows x 32 heads of the 32K long-tail pack, as the benchmark runs it (one
    launch over 256 persistent workgroups, 8 XCD queues, every item and every stolen tail),
    against the float64 oracle: the oracle's rows are split over a pool of CPU processes."""
    import oracle_pool
    out, lse, ws = run_varlen(longtail)
    st = oracle_pool.longtail_every_row(out.float().cpu().numpy(), lse.cpu().numpy(), 0, str(tmp_path), say)
    say(f"  32K long-tail every row: out max {st['out_max']:.3e} mean {st['out_mean']:.3e}  "
        f"lse max {st['lse_max']:.3e}")
    assert st["finite"] and st["n"] == 32768 * 32 * 128
    assert st["out_max"] <= OUT_MAX and st["out_mean"] <= OUT_MEAN and st["lse_max"] <= LSE_MAX


def test_longtail_is_deterministic(longtail):
    a, la, _ = run_varlen(longtail)
    b, lb_, _ = run_varlen(longtail)
    assert torch.equal(a, b) and torch.equal(la, lb_)


@pytest.mark.parametrize("seed", [1, 3])
def test_longtail_other_seeds_plan(seed):
    lengths = workloads.lognormal_lengths(32768, seed, 32768)
    T = 32768
    pack = dict(lengths=lengths, cu_seqlens=workloads.cu_from_lengths(lengths), tokens=T, heads=32, kv_heads=8,
                d=128, q=np.zeros((T, 32, 128), np.uint16), k=np.zeros((T, 8, 128), np.uint16),
                v=np.zeros((T, 8, 128), np.uint16))
    out, lse, ws = run_varlen(pack)
    assert_same_plan(lb.read_plan(ws), plan_ref_varlen(pack), f"seed {seed} plan")
    # zero inputs: every visible logit is 0, so exp(lse) counts the visible keys exactly
    n = np.concatenate([np.arange(1, l + 1) for l in lengths])
    got = np.rint(np.exp(lse[:, :].double().cpu().numpy())).astype(np.int64)
    assert np.array_equal(got, np.broadcast_to(n, got.shape))


@pytest.mark.parametrize("tokens,H,Hkv", [(1 << 20, 32, 8), (1 << 19, 64, 8)])
def test_plans_beyond_16k_tiles(tokens, H, Hkv):
    """Plans of more than 16384 tiles (the pages' long-context packs: Libra trains on 1M-token
    packed sequences, "03 · 长文负载均衡" section 1.3): a 1,048,576-token lognormal pack at 32 q
    / 8 kv heads (tiles of 64 rows) and a 524,288-token one at 64 q / 8 kv (tiles of 32 rows),
    planned on the device (bitonic order of 32-bit keys in LDS), equal the oracle's plan bit
    for bit."""
    lengths = workloads.lognormal_lengths(tokens, 11, tokens)
    pack = dict(lengths=lengths, cu_seqlens=workloads.cu_from_lengths(lengths), tokens=tokens, heads=H,
                kv_heads=Hkv, d=128)
    cu = torch.from_numpy(np.asarray(pack["cu_seqlens"], dtype=np.int32)).cuda()
    ws = lb.new_workspace(tokens, len(lengths), H, Hkv)
    lb.plan_varlen(cu, tokens, H, Hkv, 128, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    lb.plan_varlen(cu, tokens, H, Hkv, 128, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    assert lb.read_device_error(ws) == 0
    got = lb.read_plan(ws, max_tiles=1 << 16)
    say(f"  {tokens} tokens, {len(lengths)} documents, H={H}/{Hkv}: {len(got)} tiles planned in "
        f"{e0.elapsed_time(e1) * 1e3:.0f} us")
    assert len(got) > 16384
    assert_same_plan(got, plan_ref_varlen(pack), f"{tokens}-token plan")


# --------------------------------------------------------------------------
# queue order on a fitted time estimate (lb_plan_varlen_weighted)
# --------------------------------------------------------------------------
def run_weighted(pack, block_weight, pair_weight, mask_kind=lb.MASK_CAUSAL_DOC):
    T, H, Hkv, d = pack["tokens"], pack["heads"], pack["kv_heads"], pack["d"]
    say(f"  plan_varlen_weighted T={T} H={H} Hkv={Hkv} d={d} weights=({block_weight}, {pair_weight}) "
        f"mask={mask_kind}")
    q, k, v = dev_bf16(pack["q"]), dev_bf16(pack["k"]), dev_bf16(pack["v"])
    cu = torch.from_numpy(np.asarray(pack["cu_seqlens"], dtype=np.int32)).cuda()
    ws = lb.new_workspace(T, len(pack["lengths"]), H, Hkv)
    lb.plan_varlen_weighted(cu, T, H, Hkv, d, block_weight, pair_weight, mask_kind=mask_kind, workspace=ws)
    out = torch.empty((T, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
    lb.attn_run(q, k, v, out, lse, ws)
    torch.cuda.synchronize()
    assert lb.read_device_error(ws) == 0
    return out, lse, ws


def test_weighted_plan_longtail(longtail):
    """The 32K long-tail pack queued by key blocks alone (weights 1, 0) and by the fitted
    estimate through the explicit call: both orders equal the oracle's bit for bit, they
    differ (the pair term orders tiles of equal block count), lb_plan_varlen's documents order
    of the fitted estimate equals the oracle's too, and every order writes the same bits,
    since each item computes its own rows whatever its place in the queue."""
    p = longtail
    out_b, lse_b, ws_b = run_weighted(p, 1, 0)
    blocks_order = lb.read_plan(ws_b)
    assert_same_plan(blocks_order, plan_ref_weighted(p, 1, 0), "32K long-tail block-count plan")
    assert [t["blocks"] for t in blocks_order] == sorted((t["blocks"] for t in blocks_order), reverse=True)
    out_w, lse_w, ws_w = run_weighted(p, 41515, 1)
    fitted = lb.read_plan(ws_w)
    assert_same_plan(fitted, plan_ref_weighted(p, 41515, 1), "32K long-tail fitted plan")
    moved = sum(1 for a, b in zip(fitted, blocks_order) if a != b)
    say(f"  {moved} of {len(fitted)} queue positions differ between the two orders")
    assert moved > 0
    recs = lb.read_worker_timing(ws_b)
    assert sum(x["items"] for x in recs) == len(blocks_order) * 8
    assert sum(x["blocks"] for x in recs) == 8 * sum(t["blocks"] for t in blocks_order)
    out_d, lse_d, ws_d = run_varlen(p)
    assert_same_plan(lb.read_plan(ws_d), plan_ref_varlen(p), "32K long-tail documents plan")
    assert sorted(map(str, lb.read_plan(ws_d))) == sorted(map(str, fitted))  # the same tiles
    for o, l in ((out_w, lse_w), (out_d, lse_d)):
        assert torch.equal(o, out_b) and torch.equal(l, lse_b)


# --------------------------------------------------------------------------
# queue orders (lb_plan_varlen_ordered): LPT on tiles, or LPT on documents
# --------------------------------------------------------------------------
def plan_ordered(pack, order, weights=(41515, 1), mask_kind=lb.MASK_CAUSAL_DOC):
    T, H, Hkv, d = pack["tokens"], pack["heads"], pack["kv_heads"], pack["d"]
    say(f"  plan_varlen_ordered T={T} documents={len(pack['lengths'])} H={H} Hkv={Hkv} order={order} "
        f"weights={weights} mask={mask_kind}")
    cu = torch.from_numpy(np.asarray(pack["cu_seqlens"], dtype=np.int32)).cuda()
    ws = lb.new_workspace(T, len(pack["lengths"]), H, Hkv)
    lb.plan_varlen_ordered(cu, T, H, Hkv, d, weights[0], weights[1], order, mask_kind=mask_kind, workspace=ws)
    torch.cuda.synchronize()
    assert lb.read_device_error(ws) == 0
    return ws


def test_documents_order_longtail(longtail):
    """The 32K long-tail pack in both orders of the fitted estimate: each equals the oracle's
    bit for bit, the documents order keeps every document's tiles together (its last tile
    first) with documents by their largest estimate, lb_plan_varlen's plan is the documents
    order, and the attention outputs of both orders are the same bits."""
    p = longtail
    T, H, Hkv, d = p["tokens"], p["heads"], p["kv_heads"], p["d"]
    q, k, v = dev_bf16(p["q"]), dev_bf16(p["k"]), dev_bf16(p["v"])
    outs = []
    for order in (lb.ORDER_LPT, lb.ORDER_DOCUMENTS):
        ws = plan_ordered(p, order)
        got = lb.read_plan(ws)
        assert_same_plan(got, plan_ref_ordered(p, 41515, 1, order), f"32K long-tail order {order}")
        out = torch.empty((T, H, d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
        lb.attn_run(q, k, v, out, lse, ws)
        torch.cuda.synchronize()
        assert lb.read_device_error(ws) == 0
        outs.append((out, lse))
        if order == lb.ORDER_DOCUMENTS:
            cu = np.asarray(p["cu_seqlens"])
            doc = [int(np.searchsorted(cu, t["q_start"], side="right") - 1) for t in got]
            runs = [doc[0]] + [b for a, b in zip(doc, doc[1:]) if b != a]
            assert len(runs) == len(set(runs)), "a document's tiles are not together"
            assert all(got[i]["q_start"] < got[i - 1]["q_start"] for i in range(1, len(got)) if doc[i] == doc[i - 1])
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    _, _, ws_d = run_varlen(p)
    assert lb.read_plan(ws_d) == lb.read_plan(plan_ordered(p, lb.ORDER_DOCUMENTS))


@pytest.mark.parametrize("case", ["bitonic", "4096_documents", "4097_documents", "shared_question"])
def test_documents_order_capacities(case):
    """The documents order at the planner's limits, against the oracle bit for bit: a
    262,144-token pack (more than 2048 tiles: the bitonic sort with reversed tile indices),
    exactly 4096 documents (grouped), 4097 documents (the tile-level order), and a shared
    question pack."""
    r = np.random.default_rng(7)
    H, Hkv, d, mask = 32, 8, 128, "causal_doc"
    if case == "bitonic":
        lengths = workloads.lognormal_lengths(262144, 5, 262144)
    elif case == "4096_documents":
        lengths = [int(x) for x in r.integers(1, 40, size=4096)]
    elif case == "4097_documents":
        lengths = [int(x) for x in r.integers(1, 40, size=4097)]
    else:
        H, Hkv, mask = 16, 2, "shared_question"
        lengths = [900, 130, 7, 500, 64, 1, 260]
    T = sum(lengths)
    pack = dict(lengths=lengths, cu_seqlens=workloads.cu_from_lengths(lengths), tokens=T, heads=H,
                kv_heads=Hkv, d=d)
    kind = lb.MASK_CAUSAL_DOC if mask == "causal_doc" else lb.MASK_SHARED_QUESTION
    got = lb.read_plan(plan_ordered(pack, lb.ORDER_DOCUMENTS, mask_kind=kind), max_tiles=1 << 16)
    ref = plan_ref_ordered(pack, 41515, 1, lb.ORDER_DOCUMENTS, mask)
    assert_same_plan(got, ref, f"documents order, {case}")
    lpt = plan_ref_ordered(pack, 41515, 1, lb.ORDER_LPT, mask)
    if case == "4097_documents":
        assert ref == lpt
    else:
        assert ref != lpt
    if case == "bitonic":
        assert len(got) > 2048


@pytest.mark.parametrize("H,Hkv,d,weights,mask", [
    (8, 2, 128, (41515, 1), "causal_doc"),
    (2, 2, 64, (1, (1 << 16) - 1), "causal_doc"),
    (32, 8, 128, ((1 << 24) - 1, (1 << 16) - 1), "causal_doc"),
    (16, 2, 128, (1, 0), "shared_question"),
    (8, 8, 64, (41515, 1), "shared_question"),
])
def test_weighted_plan_every_row(H, Hkv, d, weights, mask):
    """Small packs with ragged tails and 1-token documents under weights from blocks alone to
    pairs dominating, and the largest weights the call accepts (largest costs, widest
    scaling): the plan equals the oracle's, every row equals the float64 oracle, and the
    outputs equal the block-count plan's bit for bit."""
    r = np.random.default_rng(H * 100 + Hkv * 10 + d + weights[1])
    lengths = [1, 700, 3, 1, 257, 64, 129, 1000, 2] if mask == "causal_doc" else [300, 41, 180, 7, 1]
    T = sum(lengths)
    q, k, v = workloads.values(r, T, H, Hkv, d)
    pack = dict(lengths=lengths, cu_seqlens=workloads.cu_from_lengths(lengths), tokens=T, heads=H, kv_heads=Hkv,
                d=d, q=q, k=k, v=v)
    kind = lb.MASK_CAUSAL_DOC if mask == "causal_doc" else lb.MASK_SHARED_QUESTION
    out, lse, ws = run_weighted(pack, *weights, mask_kind=kind)
    assert_same_plan(lb.read_plan(ws), plan_ref_weighted(pack, *weights, mask), f"weighted plan {weights}")
    ref_o, ref_l = OA.varlen_attention(q, k, v, pack["cu_seqlens"], H, Hkv, mask=mask)
    check(out.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, f"weighted {weights} H={H} Hkv={Hkv} d={d}")
    out_b, lse_b, _ = run_varlen(pack, kind)
    assert torch.equal(out, out_b) and torch.equal(lse, lse_b)


# --------------------------------------------------------------------------
# config 3: equal-token pair
# --------------------------------------------------------------------------
def test_pair_A_one_document(pair):
    p = pair[0]
    out, lse, ws = run_varlen(p)
    assert_same_plan(lb.read_plan(ws), plan_ref_varlen(p), "pair A plan")
    rows = np.array([0, 1, 63, 64, 65, 4095, 20000, 40894, 40895, 40959] +
                    np.random.default_rng(3).integers(0, 40960, 22).tolist())
    ref_o, ref_l = OA.varlen_attention(p["q"], p["k"], p["v"], p["cu_seqlens"], 32, 8, rows=rows)
    check(out[rows].float().cpu().numpy(), lse[:, rows].cpu().numpy(), ref_o, ref_l, "pair A (sampled)")


def test_pair_B_ten_documents(pair):
    p = pair[1]
    out, lse, ws = run_varlen(p)
    assert_same_plan(lb.read_plan(ws), plan_ref_varlen(p), "pair B plan")
    rows = sample_rows(p["lengths"], 64, 40, 4, cap=96)
    ref_o, ref_l = OA.varlen_attention(p["q"], p["k"], p["v"], p["cu_seqlens"], 32, 8, rows=rows)
    check(out[rows].float().cpu().numpy(), lse[:, rows].cpu().numpy(), ref_o, ref_l, "pair B (sampled)")


# --------------------------------------------------------------------------
# config 5: shared question, batch of 4 packs (one call per pack)
# --------------------------------------------------------------------------
def test_shared_question(shared_q):
    for i, p in enumerate(shared_q):
        out, lse, ws = run_varlen(p, lb.MASK_SHARED_QUESTION)
        assert_same_plan(lb.read_plan(ws), plan_ref_varlen(p, "shared_question"), f"shared question plan {i}")
        rows = sample_rows(p["lengths"], 64, 16, 10 + i, cap=40)
        ref_o, ref_l = OA.varlen_attention(p["q"], p["k"], p["v"], p["cu_seqlens"], 32, 8, mask="shared_question",
                                           rows=rows)
        check(out[rows].float().cpu().numpy(), lse[:, rows].cpu().numpy(), ref_o, ref_l, f"shared question pack {i}")


def test_shared_question_small_every_row():
    r = np.random.default_rng(77)
    lengths = [300, 129, 64, 1, 200]
    T = sum(lengths)
    q, k, v = workloads.values(r, T, 8, 2, 128)
    pack = dict(lengths=lengths, cu_seqlens=workloads.cu_from_lengths(lengths), tokens=T, heads=8, kv_heads=2, d=128,
                q=q, k=k, v=v)
    out, lse, ws = run_varlen(pack, lb.MASK_SHARED_QUESTION)
    ref_o, ref_l = OA.varlen_attention(q, k, v, pack["cu_seqlens"], 8, 2, mask="shared_question")
    check(out.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "shared question small")
    assert_same_plan(lb.read_plan(ws), plan_ref_varlen(pack, "shared_question"), "shared question small plan")


# --------------------------------------------------------------------------
# config 4: one zigzag rank's share at cp=8: 8 ring steps, a merge per live step after the first
# --------------------------------------------------------------------------
def test_zigzag_rank3_cp8():
    lengths = workloads.zigzag_pack_lengths(0)
    C, cp, rank = 8192, 8, 3
    cache = {}

    def get_chunk(c):
        if c not in cache:
            cache[c] = workloads.zigzag_chunk_values(c)
        return cache[c]

    say("  zigzag rank 3 of cp=8: building the share")
    share = lb.zigzag.RankShare(lengths, C, rank, cp, get_chunk)
    plans = {}

    def per_step(t, o, l):
        plans[t] = lb.read_plan(share.workspace)

    out, lse = share.run(per_step=per_step)
    torch.cuda.synchronize()
    assert lb.read_device_error(share.workspace) == 0
    # plans of every step against the oracle enumerator
    pos, doc = OA.pack_positions(lengths)
    qi = np.concatenate([np.arange(c * C, (c + 1) * C) for c in OA.zigzag_chunks_of_rank(rank, cp)])
    pairs = []
    for t in range(cp):
        ki = np.concatenate([np.arange(c * C, (c + 1) * C)
                             for c in OA.zigzag_chunks_of_rank(OA.ring_source(rank, t, cp), cp)])
        ref = OP.plan(OP.fragments_block(pos[qi], doc[qi], pos[ki], doc[ki]), 64)
        if t in share.live_steps:
            assert_same_plan(plans[t], ref, f"zigzag step {t}")
        else:  # a step that runs nothing: the oracle gives it no tile with a key span
            assert t not in plans and not any(x["spans"] for x in ref), t
        pairs.append(OP.total_pairs(ref))
    assert pairs == [20_319_978, 7_981_112, 0, 0, 0, 0, 0, 3_473_470]
    # output: oracle fold on sampled rows
    r = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 8191, 8192, 16383], r.integers(0, 2 * C, 60)]))
    ref_o, ref_l, _ = OA.zigzag_rank_attention(get_chunk, lengths, C, rank, cp, 32, 8, rows=rows)
    check(out[rows].cpu().numpy(), lse[:, rows].cpu().numpy(), ref_o, ref_l, "zigzag rank 3 (sampled)")


def test_zigzag_rank3_cp8_ring_launch():
    """Rank 3 of cp = 8 on the 131072-token pack, as the zigzag benchmark runs it: the live
    steps' plans merged into one longest-first queue and run by one attention launch with
    one queue per XCD, then the merges.  Same bits as the per-step launches, the merged
    queue equal to the oracle's, every item run once, and the oracle's fold on sampled
    rows."""
    lengths = workloads.zigzag_pack_lengths(0)
    C, cp, rank = 8192, 8, 3
    cache = {}

    def get_chunk(c):
        if c not in cache:
            cache[c] = workloads.zigzag_chunk_values(c)
        return cache[c]

    say("  zigzag rank 3 of cp=8: building the share")
    share = lb.zigzag.RankShare(lengths, C, rank, cp, get_chunk)
    assert share.live_steps == [0, 1, 7]
    out, lse = check_ring_against_steps(share, "zigzag rank 3 ring")
    r = np.random.default_rng(8)
    rows = np.unique(np.concatenate([[0, 1, 8191, 8192, 16383], r.integers(0, 2 * C, 60)]))
    ref_o, ref_l, _ = OA.zigzag_rank_attention(get_chunk, lengths, C, rank, cp, 32, 8, rows=rows)
    check(out[rows].cpu().numpy(), lse[:, rows].cpu().numpy(), ref_o, ref_l, "zigzag rank 3 ring (sampled)")


@pytest.mark.timeout(900)
def test_zigzag_rank3_cp8_ring_every_row(tmp_path):
    """All 16384 rows x 32 heads of rank 3's share, through the ring launch the zigzag
    benchmark times, against the oracle's fold of the 8 ring steps."""
    import oracle_pool
    lengths = workloads.zigzag_pack_lengths(0)
    C, cp, rank = 8192, 8, 3
    share = lb.zigzag.RankShare(lengths, C, rank, cp, workloads.zigzag_chunk_values)
    out, lse = share.run_ring()
    torch.cuda.synchronize()
    st = oracle_pool.zigzag_every_row(out.cpu().numpy(), lse.cpu().numpy(), 0, rank, cp, C, str(tmp_path), say)
    say(f"  zigzag rank 3 every row: out max {st['out_max']:.3e} mean {st['out_mean']:.3e}  "
        f"lse max {st['lse_max']:.3e}")
    assert st["finite"] and st["n"] == 2 * C * 32 * 128
    assert st["out_max"] <= OUT_MAX and st["out_mean"] <= OUT_MEAN and st["lse_max"] <= LSE_MAX


def test_zigzag_plans_made_up_front_equal_per_step_plans():
    """lb_plan_block_steps plans all 8 ring steps of rank 3 in one launch: every step's plan
    equals lb_plan_block's, and the run over them is bit-identical to the per-step calls."""
    lengths = workloads.zigzag_pack_lengths(0)
    C, cp, rank = 8192, 8, 3
    cache = {}

    def get_chunk(c):
        if c not in cache:
            cache[c] = workloads.zigzag_chunk_values(c)
        return cache[c]

    share = lb.zigzag.RankShare(lengths, C, rank, cp, get_chunk)
    # steps 2-6 of rank 3 hold no key its rows see (per-step pairs 20.3M, 8.0M, 0 x 5, 3.5M)
    assert share.live_steps == [0, 1, 7]
    say("  per-step plans and runs")
    ref_plans = {}
    out_ref, lse_ref = share.run(per_step=lambda t, o, l: ref_plans.update({t: lb.read_plan(share.workspace)}))
    out_ref, lse_ref = out_ref.clone(), lse_ref.clone()
    say("  all plans in one launch, then the runs")
    out, lse = share.run_planned()
    torch.cuda.synchronize()
    for t in share.live_steps:
        assert lb.read_device_error(share.step_workspaces[t]) == 0
        assert_same_plan(lb.read_plan(share.step_workspaces[t]), ref_plans[t], f"step {t}")
    assert torch.equal(out, out_ref) and torch.equal(lse, lse_ref)


def test_zigzag_graph_replays_equal_eager_runs():
    """The share captured in a HIP graph (1 planning launch, cp attention launches, cp - 1
    merges), replayed three times with eager runs and synchronisations in between: every
    replay is bit-identical to the eager result."""
    cp, C, H, Hkv, d = 4, 256, 8, 2, 128
    T = 2 * cp * C
    lengths = workloads.lognormal_lengths(T, 9, T)
    r = np.random.default_rng(13)
    q, k, v = workloads.values(r, T, H, Hkv, d)

    def get_chunk(c):
        sl = slice(c * C, (c + 1) * C)
        return q[sl], k[sl], v[sl]

    share = lb.zigzag.RankShare(lengths, C, 1, cp, get_chunk)
    out, lse = share.run_planned()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    say("  capturing the share")
    share.capture()
    for i in range(3):
        share.out.fill_(7.0)
        share.lse.fill_(7.0)
        out, lse = share.replay()
        torch.cuda.synchronize()
        say(f"  replay {i}")
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"replay {i}"
        out, lse = share.run_planned()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"eager run after replay {i}"
    for t in share.live_steps:
        assert lb.read_device_error(share.step_workspaces[t]) == 0


def test_zigzag_overlapped_steps_equal_the_serial_share():
    """The ring steps' attention launches spread over side streams (eager, then captured in
    one HIP graph and replayed three times with eager work in between) give the bits of the
    one-stream share: each step has its own partial buffers and the merges keep step order."""
    cp, C, H, Hkv, d = 4, 256, 8, 2, 128
    T = 2 * cp * C
    lengths = workloads.lognormal_lengths(T, 9, T)
    r = np.random.default_rng(14)
    q, k, v = workloads.values(r, T, H, Hkv, d)

    def get_chunk(c):
        sl = slice(c * C, (c + 1) * C)
        return q[sl], k[sl], v[sl]

    share = lb.zigzag.RankShare(lengths, C, 2, cp, get_chunk)
    out, lse = share.run_planned()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    streams = [torch.cuda.Stream() for _ in range(3)]
    out, lse = share.run_overlapped(streams)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), "eager overlapped"
    say("  capturing the overlapped share")
    share.capture(streams=streams)
    for i in range(3):
        share.out.fill_(7.0)
        share.lse.fill_(7.0)
        out, lse = share.replay()
        torch.cuda.synchronize()
        say(f"  replay {i}")
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"replay {i}"
        out, lse = share.run_planned()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"eager run after replay {i}"
    for t in share.live_steps:
        assert lb.read_device_error(share.step_workspaces[t]) == 0


def test_zigzag_reassembly_small():
    """All ranks of a reduced pack (cp=4, 16 chunks of 256... here 8 chunks of 256) against the unsharded oracle."""
    cp, C, H, Hkv, d = 4, 256, 8, 2, 128
    T = 2 * cp * C
    lengths = workloads.lognormal_lengths(T, 9, T)
    r = np.random.default_rng(12)
    q, k, v = workloads.values(r, T, H, Hkv, d)

    def get_chunk(c):
        sl = slice(c * C, (c + 1) * C)
        return q[sl], k[sl], v[sl]

    full_o, full_l = OA.varlen_attention(q, k, v, workloads.cu_from_lengths(lengths), H, Hkv)
    for rank in range(cp):
        share = lb.zigzag.RankShare(lengths, C, rank, cp, get_chunk)
        out, lse = share.run()
        rows = np.concatenate([np.arange(c * C, (c + 1) * C) for c in OA.zigzag_chunks_of_rank(rank, cp)])
        check(out.cpu().numpy(), lse.cpu().numpy(), full_o[rows], full_l[:, rows], f"reassembly rank {rank}")


@pytest.mark.parametrize("rule", ["per_document", "zigzag", "dispatch"])
def test_sharded_ranks_reassemble_the_unsharded_result(rule):
    """Every rank of a cp = 4 sharding (per document: "03 · 长文负载均衡", section 4.3;
    sequence zigzag; or the mask-area dispatch of section 4.4 over 16 chunks) runs its 4
    ring steps through block_attn_fwd + lse_merge; the ranks' rows together equal the
    unsharded oracle.  The plan-once path is bit-identical to the per-step calls."""
    from load_balance_amd import sharding as LS
    cp, H, Hkv, d = 4, 8, 2, 128
    r = np.random.default_rng(17)
    lengths = [1200, 37, 1, 650, 9, 301, 1900]  # remainders of every size
    if rule in ("zigzag", "dispatch"):
        lengths.append(2 * cp * 640 - sum(lengths))
    T = sum(lengths)
    q, k, v = workloads.values(r, T, H, Hkv, d)
    tok = LS.shard_tokens(rule, lengths, cp, n_chunks=4 * cp)
    if rule == "dispatch":
        assert LS.max_spans(lengths, tok) <= LS.MAX_SPANS
    shards = LS.build_shards(lengths, tok, lambda idx: (q[idx], k[idx], v[idx]))
    full_o, full_l = OA.varlen_attention(q, k, v, workloads.cu_from_lengths(lengths), H, Hkv)
    for rank in range(cp):
        say(f"  {rule} rank {rank}: {len(tok[rank])} tokens")
        share = LS.ShardedRank(shards, rank)
        out, lse = share.run()
        out_ref, lse_ref = out.clone(), lse.clone()
        out, lse = share.run_planned()
        torch.cuda.synchronize()
        assert torch.equal(out, out_ref) and torch.equal(lse, lse_ref)
        for t in share.live_steps:
            assert lb.read_device_error(share.step_workspaces[t]) == 0
        check(out.cpu().numpy(), lse.cpu().numpy(), full_o[tok[rank]], full_l[:, tok[rank]], f"{rule} rank {rank}")


@pytest.mark.parametrize("width,shared", [(1, False), (64, False), (3, True)])
def test_striped_ranks_reassemble_the_unsharded_result(width, shared):
    """Striped sharding ("03 · 长文负载均衡", section 4.2): stripes of `width` tokens dealt to
    cp = 4 ranks in turn.  A query stripe then meets a key run per earlier stripe of its
    document, more than the block planner's 4 spans, so those steps run as slice lists (the
    same mask over local indices); per step (run, run_planned) and as one ring launch
    (run_ring), every rank's rows equal the unsharded oracle (with a shared question:
    document 0 shared)."""
    from load_balance_amd import sharding as LS
    cp, H, Hkv, d = 4, 8, 2, 128
    r = np.random.default_rng(70 + width)
    lengths = [2600, 37, 1, 650, 9, 301, 1350]  # 2600 tokens: 10 stripes of 64 per rank
    T = sum(lengths)
    q, k, v = workloads.values(r, T, H, Hkv, d)
    tok = LS.shard_tokens("striped", lengths, cp, width=width)
    assert LS.max_spans(lengths, tok, 0 if shared else -1) > LS.MAX_SPANS
    shards = LS.build_shards(lengths, tok, lambda idx: (q[idx], k[idx], v[idx]))
    full_o, full_l = OA.varlen_attention(q, k, v, workloads.cu_from_lengths(lengths), H, Hkv,
                                         mask="shared_question" if shared else "causal_doc")
    for rank in range(cp):
        share = LS.ShardedRank(shards, rank, shared_doc=0 if shared else -1)
        n_sl = sum(1 for t in share.live_steps if "slices" in share.steps[t])
        say(f"  striped w={width} rank {rank}: {len(tok[rank])} tokens, live steps {share.live_steps}, "
            f"{n_sl} as slice lists")
        assert n_sl > 0
        for name, fn in (("run", share.run), ("run_planned", share.run_planned), ("run_ring", share.run_ring)):
            out, lse = fn()
            torch.cuda.synchronize()
            for t in share.live_steps:
                if share.step_workspaces is not None and share.step_workspaces[t] is not None:
                    assert lb.read_device_error(share.step_workspaces[t]) == 0
            check(out.cpu().numpy(), lse.cpu().numpy(), full_o[tok[rank]], full_l[:, tok[rank]],
                  f"striped w={width} rank {rank} {name}")


# --------------------------------------------------------------------------
# block path edge cases
# --------------------------------------------------------------------------
def run_block(q, k, v, q_pos, kv_pos, q_doc, kv_doc):
    n_q, H, d = q.shape
    n_kv, Hkv = k.shape[0], k.shape[1]
    say(f"  block_attn_fwd n_q={n_q} n_kv={n_kv} H={H} Hkv={Hkv} d={d}")
    kv = torch.stack([dev_bf16(k), dev_bf16(v)]) if n_kv else torch.zeros((2, 0, Hkv, d), dtype=torch.bfloat16,
                                                                            device="cuda")
    i32 = lambda x: torch.from_numpy(np.asarray(x, dtype=np.int32)).cuda()
    out, lse = lb.block_attn_fwd(dev_bf16(q), kv.contiguous(), i32(q_pos), i32(kv_pos), i32(q_doc), i32(kv_doc))
    torch.cuda.synchronize()
    return out, lse


def test_block_random_shards_every_row():
    r = np.random.default_rng(31)
    H, Hkv, d = 8, 2, 128
    T = 2048
    lengths = workloads.lognormal_lengths(T, 4, T)
    pos, doc = OA.pack_positions(lengths)
    q, k, v = workloads.values(r, T, H, Hkv, d)
    qi = np.r_[256:512, 1536:1792]
    ki = np.r_[0:384, 1400:2048]
    out, lse = run_block(q[qi], k[ki], v[ki], pos[qi], pos[ki], doc[qi], doc[ki])
    ref_o, ref_l = OA.block_attention(q[qi], k[ki], v[ki], pos[qi], pos[ki], doc[qi], doc[ki], H, Hkv)
    lse_g = lse.cpu().numpy()
    empty = ref_l == -np.inf
    assert np.array_equal(lse_g == -np.inf, empty)
    rows_ok = ~empty[0]
    check(out.cpu().numpy()[rows_ok], lse_g[:, rows_ok], ref_o[rows_ok], ref_l[:, rows_ok], "block random shards")


def test_block_no_keys_gives_minus_inf():
    r = np.random.default_rng(2)
    q, _, _ = workloads.values(r, 300, 4, 4, 64)
    out, lse = run_block(q, np.zeros((0, 4, 64), np.uint16), np.zeros((0, 4, 64), np.uint16), np.arange(300),
                         [], np.zeros(300), [])
    assert torch.all(lse == -math.inf)
    k, v = workloads.values(r, 50, 4, 4, 64)[1:]
    out, lse = run_block(q, k, v, np.arange(300), np.arange(50), np.zeros(300), np.ones(50))  # other document
    assert torch.all(lse == -math.inf)


def test_block_plan_many_rounds_ragged_and_unaligned():
    """Run detection over more than 16384 tokens per side, with a ragged tail and broken
    runs, from 16-byte aligned and from unaligned metadata pointers: the plan equals the
    oracle's either way."""
    H, Hkv, d = 32, 8, 128
    T = 40_003
    lengths = workloads.lognormal_lengths(T, 6, 6000)
    pos, doc = OA.pack_positions(lengths)
    qi = np.concatenate([np.arange(s, min(s + 700, T)) for s in range(0, T, 1000)])  # gaps break runs
    ki = np.arange(T)
    ref = OP.plan(OP.fragments_block(pos[qi], doc[qi], pos[ki], doc[ki]), lb.tile_rows(H, Hkv, d))

    def dev(x, shift):
        buf = torch.zeros(len(x) + shift, dtype=torch.int32, device="cuda")
        buf[shift:] = torch.from_numpy(np.asarray(x, dtype=np.int32)).cuda()
        return buf[shift:]

    for shift in (0, 1, 3):
        say(f"  block plan n_q={len(qi)} n_kv={len(ki)} pointer shift {shift} ints")
        ws = lb.new_workspace(T, 256, H, Hkv)
        lb.plan_block(dev(pos[qi], shift), dev(doc[qi], shift), dev(pos[ki], shift), dev(doc[ki], shift),
                      H, Hkv, d, ws)
        torch.cuda.synchronize()
        assert lb.read_device_error(ws) == 0
        assert_same_plan(lb.read_plan(ws), ref, f"block plan, shift {shift}")


# --------------------------------------------------------------------------
# special cases fixed by the mathematics
# --------------------------------------------------------------------------
def test_single_token_documents_return_their_value():
    r = np.random.default_rng(8)
    lengths = [1, 90, 1, 1, 130, 1]
    T = sum(lengths)
    H, Hkv, d = 8, 2, 128
    q, k, v = workloads.values(r, T, H, Hkv, d)
    pack = dict(lengths=lengths, cu_seqlens=workloads.cu_from_lengths(lengths), tokens=T, heads=H, kv_heads=Hkv,
                d=d, q=q, k=k, v=v)
    out, lse, _ = run_varlen(pack)
    ob = bits_of(out)
    scale = 1 / math.sqrt(d)
    for t in (0, 91, 92, 223):
        for h in range(H):
            assert np.array_equal(ob[t, h], v[t, h // 4]), (t, h)
            expect = scale * float(f32(q[t, h]).astype(np.float64) @ f32(k[t, h // 4]).astype(np.float64))
            assert abs(float(lse[h, t]) - expect) < 1e-4


def test_zero_query_counts_visible_keys_exactly():
    r = np.random.default_rng(9)
    lengths = [5, 17, 42, 1000, 3, 2000]
    T = sum(lengths)
    _, k, v = workloads.values(r, T, 4, 4, 64)
    pack = dict(lengths=lengths, cu_seqlens=workloads.cu_from_lengths(lengths), tokens=T, heads=4, kv_heads=4, d=64,
                q=np.zeros((T, 4, 64), np.uint16), k=k, v=v)
    _, lse, _ = run_varlen(pack)
    n = np.concatenate([np.arange(1, l + 1) for l in lengths])
    got = np.rint(np.exp(lse.double().cpu().numpy())).astype(np.int64)
    assert np.array_equal(got, np.broadcast_to(n, got.shape))


def test_constant_value_is_returned():
    r = np.random.default_rng(10)
    lengths = [333, 1, 64, 700]
    T = sum(lengths)
    q, k, _ = workloads.values(r, T, 8, 2, 128)
    v = workloads.f32_to_bf16_bits(np.full((T, 2, 128), 0.75, np.float32))
    pack = dict(lengths=lengths, cu_seqlens=workloads.cu_from_lengths(lengths), tokens=T, heads=8, kv_heads=2,
                d=128, q=q, k=k, v=v)
    out, _, _ = run_varlen(pack)
    assert (out.float() - 0.75).abs().max().item() <= OUT_MAX


def test_bad_cu_seqlens_sets_device_error():
    T = 128
    q = torch.zeros((T, 4, 64), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 100, 50, T], dtype=torch.int32, device="cuda")
    lse = torch.full((4, T), 12345.0, device="cuda")
    ws = lb.new_workspace(T, 3, 4, 4)
    lb.varlen_attn_fwd(q, q, q, cu, lse=lse, workspace=ws)
    assert lb.read_device_error(ws) == lb.DEVERR_CU_SEQLENS
    assert torch.all(lse == 12345.0)
    cu = torch.tensor([0, 100, 120, T - 1], dtype=torch.int32, device="cuda")
    lb.varlen_attn_fwd(q, q, q, cu, lse=lse, workspace=ws)
    assert lb.read_device_error(ws) == lb.DEVERR_CU_SEQLENS


# --------------------------------------------------------------------------
# split entry points: one plan, several runs
# --------------------------------------------------------------------------
def test_plan_once_run_many_equals_fused():
    r = np.random.default_rng(21)
    lengths = [300, 5, 1200, 77]
    T, H, Hkv, d = sum(lengths), 32, 8, 128
    q, k, v = workloads.values(r, T, H, Hkv, d)
    pack = dict(lengths=lengths, cu_seqlens=workloads.cu_from_lengths(lengths), tokens=T, heads=H, kv_heads=Hkv,
                d=d, q=q, k=k, v=v)
    ref_out, ref_lse, _ = run_varlen(pack)
    cu = torch.from_numpy(pack["cu_seqlens"]).cuda()
    ws = lb.plan_varlen(cu, T, H, Hkv, d)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    for _ in range(3):  # the queue rewinds itself after every run
        out = torch.empty_like(qd)
        lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
        lb.attn_run(qd, kd, vd, out, lse, ws)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    assert lb.read_device_error(ws) == 0


def test_run_against_wrong_plan_does_nothing():
    T, H, Hkv, d = 256, 8, 2, 64
    qd = torch.zeros((T, H, d), dtype=torch.bfloat16, device="cuda")
    kd = torch.zeros((T, Hkv, d), dtype=torch.bfloat16, device="cuda")
    out = torch.full((T, H, d), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((H, T), 7.0, device="cuda")
    ws = torch.zeros(lb.workspace_bytes(T, 4, H, Hkv), dtype=torch.uint8, device="cuda")  # never planned
    lb.attn_run(qd, kd, kd, out, lse, ws)
    assert lb.read_device_error(ws) & lb.DEVERR_PLAN
    cu = torch.tensor([0, 100, 200], dtype=torch.int32, device="cuda")
    lb.plan_varlen(cu, 200, H, Hkv, d, workspace=ws)  # plan for 200 tokens, run with 256
    lb.attn_run(qd, kd, kd, out, lse, ws)
    assert lb.read_device_error(ws) & lb.DEVERR_PLAN
    assert torch.all(out == 3.0) and torch.all(lse == 7.0)


# --------------------------------------------------------------------------
# lse_merge
# --------------------------------------------------------------------------
@pytest.mark.parametrize("d", [64, 128])
def test_lse_merge_matches_oracle(d):
    r = np.random.default_rng(d)
    R, H = 777, 6
    oa, ob = r.standard_normal((R, H, d)), r.standard_normal((R, H, d))
    la, lb_ = r.standard_normal((H, R)) * 3, r.standard_normal((H, R)) * 3
    la[r.random((H, R)) < 0.2] = -np.inf
    lb_[r.random((H, R)) < 0.2] = -np.inf
    ref_o, ref_l = OA.lse_merge(oa, la, ob, lb_)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    ga, gla = t(oa), t(la)
    gb = t(ob)
    gb[torch.from_numpy((lb_ == -np.inf).T.copy())] = float("nan")  # never read where lse_b = -inf
    # nor out_a where lse_a = -inf and lse_b is finite: the first partial never wrote it
    ga[torch.from_numpy(((la == -np.inf) & (lb_ != -np.inf)).T.copy())] = float("nan")
    lb.lse_merge(ga, gla, gb, t(lb_))
    torch.cuda.synchronize()
    go, gl = ga.cpu().numpy(), gla.cpu().numpy()
    both_inf = (la == -np.inf) & (lb_ == -np.inf)
    assert np.all(gl[both_inf] == -np.inf)
    fin = ~both_inf
    assert np.abs(gl[fin] - ref_l[fin]).max() <= 1e-5
    rows_fin = fin.T
    assert np.abs(go[rows_fin] - ref_o[rows_fin]).max() <= 1e-5
    keep = (lb_ == -np.inf).T
    assert np.array_equal(go[keep], np.float32(oa)[keep])
    assert np.all(np.isfinite(go[rows_fin]))


@pytest.mark.parametrize("n_parts,d", [(2, 128), (3, 128), (5, 64), (16, 128)])
def test_lse_merge_parts_equals_pairwise_merges(n_parts, d):
    """lb_lse_merge_parts against n_parts - 1 lb_lse_merge calls in sequence: the same bits,
    on partials with -inf rows in every part (rows no part touches, rows only part 0 holds,
    rows whose first writer is a later part), NaN in every row a partial never wrote (so a
    read of one shows), and rows touched by several parts; the result also against the
    float64 oracle's merges in step order."""
    r = np.random.default_rng(100 + n_parts)
    R, H = 1000, 4
    outs = [r.standard_normal((R, H, d)) for _ in range(n_parts)]
    lses = [r.standard_normal((H, R)) * 3 for _ in range(n_parts)]
    for i in range(n_parts):
        lses[i][r.random((H, R)) < (0.3 if i == 0 else 0.7)] = -np.inf
    lses[0][:, :64] = -np.inf  # a whole row group first written by a later part
    for i in range(n_parts):
        lses[i][:, 64:100] = -np.inf  # rows no part touches
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    def poisoned():
        go = [t(o) for o in outs]
        for o, l in zip(go, lses):
            o[torch.from_numpy((l == -np.inf).T.copy())] = float("nan")
        return go, [t(l) for l in lses]
    seq_o, seq_l = poisoned()
    for i in range(1, n_parts):
        lb.lse_merge(seq_o[0], seq_l[0], seq_o[i], seq_l[i])
    one_o, one_l = poisoned()
    lb.lse_merge_parts(one_o, one_l)
    torch.cuda.synchronize()
    assert torch.equal(one_l[0], seq_l[0])
    a, b = one_o[0].cpu().numpy(), seq_o[0].cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))  # NaN rows (never written) included
    ref_o, ref_l = outs[0], lses[0]
    for i in range(1, n_parts):
        ref_o, ref_l = OA.lse_merge(ref_o, ref_l, outs[i], lses[i])
    fin = ref_l != -np.inf
    assert np.array_equal(one_l[0].cpu().numpy() == -np.inf, ~fin)
    assert np.abs(one_l[0].cpu().numpy()[fin] - ref_l[fin]).max() <= 1e-5
    assert np.abs(a[fin.T] - ref_o[fin.T]).max() <= 1e-5


# --------------------------------------------------------------------------
# the shared-question mask on the block path (a shared document)
# --------------------------------------------------------------------------
def test_block_shared_question_whole_pack():
    """Document 0 shared over a whole shared-question pack: every row against the varlen
    shared-question oracle, and the plan (FULL spans for the question's keys) against the
    oracle's enumerator bit for bit."""
    lengths = [700, 300, 1, 128, 90, 64]
    T, H, Hkv, d = sum(lengths), 8, 2, 128
    r = np.random.default_rng(61)
    q, k, v = workloads.values(r, T, H, Hkv, d)
    pos, doc = OA.pack_positions(lengths)
    i32 = lambda x: torch.from_numpy(np.asarray(x, dtype=np.int32)).cuda()
    say(f"  block_attn_fwd, shared question, T={T}")
    kv = torch.stack([dev_bf16(k), dev_bf16(v)]).contiguous()
    ws = lb.new_workspace(T, T, H, Hkv)
    out, lse = lb.block_attn_fwd(dev_bf16(q), kv, i32(pos), i32(pos), i32(doc), i32(doc), workspace=ws, shared_doc=0)
    torch.cuda.synchronize()
    assert lb.read_device_error(ws) == 0
    ref_o, ref_l = OA.varlen_attention(q, k, v, workloads.cu_from_lengths(lengths), H, Hkv, mask="shared_question")
    check(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "block path, shared question")
    ref_plan = OP.plan(OP.fragments_block(pos, doc, pos, doc, shared_doc=0), lb.tile_rows(H, Hkv, d))
    assert_same_plan(lb.read_plan(ws), ref_plan, "shared question plan")


@pytest.mark.parametrize("rule", ["zigzag", "per_document"])
def test_sharded_shared_question_reassembles(rule):
    """A shared-question pack sharded over cp = 4 ranks: each rank's ring with document 0
    shared (steps without visible pairs run nothing) reassembles the unsharded oracle; the
    plan-once path is bit-identical to the per-step calls."""
    from load_balance_amd import sharding as LS
    cp, H, Hkv, d, C = 4, 8, 2, 128, 256
    r = np.random.default_rng(62)
    lengths = [700, 300, 1, 128, 90, 333]
    lengths.append(2 * cp * C - sum(lengths))
    T = sum(lengths)
    q, k, v = workloads.values(r, T, H, Hkv, d)
    tok = LS.shard_tokens(rule, lengths, cp)
    shards = LS.build_shards(lengths, tok, lambda idx: (q[idx], k[idx], v[idx]))
    full_o, full_l = OA.varlen_attention(q, k, v, workloads.cu_from_lengths(lengths), H, Hkv, mask="shared_question")
    for rank in range(cp):
        share = LS.ShardedRank(shards, rank, shared_doc=0)
        say(f"  {rule} rank {rank}: live steps {share.live_steps}")
        out, lse = share.run()
        out_ref, lse_ref = out.clone(), lse.clone()
        out, lse = share.run_planned()
        torch.cuda.synchronize()
        assert torch.equal(out, out_ref) and torch.equal(lse, lse_ref)
        for t in share.live_steps:
            assert lb.read_device_error(share.step_workspaces[t]) == 0
        check(out.cpu().numpy(), lse.cpu().numpy(), full_o[tok[rank]], full_l[:, tok[rank]],
              f"{rule} rank {rank}, shared question")


# --------------------------------------------------------------------------
# one attention launch over every live ring step (ring workspace)
# --------------------------------------------------------------------------
def ring_share(cp=4, C=256, rank=2, seed=9, H=8, Hkv=2, d=128, with_inputs=False):
    T = 2 * cp * C
    lengths = workloads.lognormal_lengths(T, seed, T)
    r = np.random.default_rng(14 + seed)
    q, k, v = workloads.values(r, T, H, Hkv, d)

    def get_chunk(c):
        sl = slice(c * C, (c + 1) * C)
        return q[sl], k[sl], v[sl]

    share = lb.zigzag.RankShare(lengths, C, rank, cp, get_chunk)
    return (share, (lengths, q, k, v)) if with_inputs else share


def ring_oracle_plan(share):
    """The oracle's merged queue over the share's live steps."""
    n_q, H, d = share.q.shape
    Hkv = share.steps[0]["kv"].shape[2]
    bm = lb.tile_rows(H, Hkv, d)
    qp, qd = share.q_pos.cpu().numpy(), share.q_doc.cpu().numpy()
    shared = None if share.shared_doc < 0 else share.shared_doc
    plans = [OP.plan(OP.fragments_block(qp, qd, share.steps[t]["kv_pos"].cpu().numpy(),
                                        share.steps[t]["kv_doc"].cpu().numpy(), shared_doc=shared), bm)
             for t in share.live_steps]
    return OP.merge_step_plans(plans)


def check_ring_against_steps(share, what):
    out, lse = share.run_planned()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    out, lse = share.run_ring()
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"{what}: ring launch != per-step launches"
    assert lb.read_device_error(share.ring_workspace) == 0
    want = ring_oracle_plan(share)
    assert_same_plan(lb.read_plan(share.ring_workspace, with_step=True), want, f"{what}: ring plan")
    # the workgroups' records cover every item once
    n_q, H, d = share.q.shape
    Hkv = share.steps[0]["kv"].shape[2]
    recs = lb.read_worker_timing(share.ring_workspace)
    work = [t for t in want if t["spans"]]
    assert sum(x["items"] for x in recs) == len(work) * Hkv
    assert sum(x["blocks"] for x in recs) == sum(t["blocks"] for t in work) * Hkv
    assert sum(x["pairs"] for x in recs) == sum(t["cost"] for t in work) * H
    return ref_out, ref_lse


@pytest.mark.parametrize("rank", [0, 2, 3])
@pytest.mark.parametrize("H,Hkv,d", [(8, 2, 128), (4, 4, 64), (8, 1, 64), (16, 2, 128), (32, 8, 128), (16, 8, 128),
                                     (8, 8, 64)])
def test_ring_launch_equals_the_step_launches(rank, H, Hkv, d):
    """A zigzag rank's live steps run from one merged queue in one launch: the same bits as
    one launch per step, the merged queue equal to the oracle's (every step's tiles, key
    blocks descending, ties by step), every item run once, and the merged result equal to
    the unsharded oracle on every row of the rank; every head grouping and head size the
    ring kernel is built for, with one queue (kv heads 1, 2, 4) and one per XCD (8)."""
    cp, C = 4, 256
    share, (lengths, q, k, v) = ring_share(cp=cp, C=C, rank=rank, H=H, Hkv=Hkv, d=d, with_inputs=True)
    say(f"  zigzag cp=4 rank {rank} H={H} Hkv={Hkv} d={d}: live steps {share.live_steps}")
    out, lse = check_ring_against_steps(share, f"rank {rank} H={H} Hkv={Hkv} d={d}")
    rows = np.concatenate([np.arange(c * C, (c + 1) * C) for c in lb.zigzag.chunks_of_rank(rank, cp)])
    ref_o, ref_l = OA.varlen_attention(q, k, v, workloads.cu_from_lengths(lengths), H, Hkv, rows=rows)
    check(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, f"ring rank {rank} H={H}/{Hkv} d={d} vs oracle")


def test_ring_graph_replays_equal_eager_runs():
    """The ring share captured in one HIP graph (plans, merged queue, one attention launch,
    merges) and replayed three times with eager work in between gives the eager bits."""
    share = ring_share(rank=1, seed=5)
    ref_out, ref_lse = check_ring_against_steps(share, "graph share")
    say("  capturing the ring share")
    share.capture(ring=True)
    for i in range(3):
        share.out.fill_(7.0)
        share.lse.fill_(7.0)
        out, lse = share.replay()
        torch.cuda.synchronize()
        say(f"  replay {i}")
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"replay {i}"
        out, lse = share.run_planned()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"eager run after replay {i}"


@pytest.mark.parametrize("rule,H,Hkv", [("per_document", 8, 2), ("dispatch", 8, 2), ("per_document", 32, 8)])
def test_ring_launch_on_sharded_ranks(rule, H, Hkv):
    """Every rank of a cp = 4 sharding with a shared question (document 0): the ring launch
    gives the bits of the per-step launches and the ranks reassemble the unsharded oracle."""
    from load_balance_amd import sharding as LS
    cp, d = 4, 128
    r = np.random.default_rng(65)
    lengths = [700, 300, 1, 128, 90, 333]
    lengths.append(2 * cp * 256 - sum(lengths))
    T = sum(lengths)
    q, k, v = workloads.values(r, T, H, Hkv, d)
    tok = LS.shard_tokens(rule, lengths, cp, n_chunks=4 * cp)
    assert LS.max_spans(lengths, tok, 0) <= LS.MAX_SPANS
    shards = LS.build_shards(lengths, tok, lambda idx: (q[idx], k[idx], v[idx]))
    full_o, full_l = OA.varlen_attention(q, k, v, workloads.cu_from_lengths(lengths), H, Hkv, mask="shared_question")
    for rank in range(cp):
        share = LS.ShardedRank(shards, rank, shared_doc=0)
        say(f"  {rule} rank {rank}: live steps {share.live_steps}")
        out, lse = check_ring_against_steps(share, f"{rule} rank {rank}")
        check(out.cpu().numpy(), lse.cpu().numpy(), full_o[tok[rank]], full_l[:, tok[rank]],
              f"{rule} rank {rank}, ring")


def test_ring_made_for_other_steps_runs_nothing():
    """A ring merged for other key/value counts is refused on the device: LB_DEVERR_PLAN,
    no partial written."""
    share = ring_share(rank=2)
    share.run_ring()
    torch.cuda.synchronize()
    live = [share.steps[t] for t in share.live_steps]
    assert len(live) >= 2
    ks = [st["kv"][0] for st in live]
    vs = [st["kv"][1] for st in live]
    ks[1], vs[1] = ks[1][:-1], vs[1][:-1]  # one token fewer than the ring was made for
    outs = [torch.full_like(share.out, 7.0) for _ in live]
    lses = [torch.full_like(share.lse, 7.0) for _ in live]
    lb.ring_attn_run(share.q, ks, vs, outs, lses, share.ring_workspace)
    torch.cuda.synchronize()
    assert lb.read_device_error(share.ring_workspace) & lb.DEVERR_PLAN
    for o, l in zip(outs, lses):
        assert torch.all(o == 7.0) and torch.all(l == 7.0)


def test_ring_too_small_for_the_steps_runs_nothing():
    """A ring workspace with room for two tiles: the merge flags LB_DEVERR_CAPACITY, the
    ring holds no work, and a launch over it writes no partial."""
    share = ring_share(rank=2)
    share.run_ring()
    torch.cuda.synchronize()
    live = [share.steps[t] for t in share.live_steps]
    n_q, H, d = share.q.shape
    Hkv = live[0]["kv"].shape[2]
    header_and_records = 256 + 2048 * 40  # the ring's tiles start after the worker records
    small = torch.empty(header_and_records + 2 * 96, dtype=torch.uint8, device="cuda")
    lb.plan_ring([share.step_workspaces[t] for t in share.live_steps], [st["kv"].shape[1] for st in live], n_q, H,
                 Hkv, d, small)
    outs = [torch.full_like(share.out, 7.0) for _ in live]
    lses = [torch.full_like(share.lse, 7.0) for _ in live]
    lb.ring_attn_run(share.q, [st["kv"][0] for st in live], [st["kv"][1] for st in live], outs, lses, small)
    torch.cuda.synchronize()
    assert lb.read_device_error(small) & lb.DEVERR_CAPACITY
    assert lb.read_plan(small) == []
    for o, l in zip(outs, lses):
        assert torch.all(o == 7.0) and torch.all(l == 7.0)
