"""GPU parity of the backward (dq, dk, dv) through the C ABI against the float64 oracle.

The library runs its own forward and then its backward from the forward's bf16 out and
fp32 lse; the oracle differentiates the exact forward from q, k, v and dout alone.
Tolerances, per tensor, relative to the reference's scale: max |d| <= GRAD_MAX * max|ref|
and mean |d| <= GRAD_MEAN * mean|ref|.  The kernels feed P and dS to the matrix cores
in bf16 (relative rounding 2^-9) and take D = <dout, out> from the bf16 out (relative
2^-9 of |out|), and every gradient is a sum of such terms with mixed signs, so errors of
a few parts in a thousand of the gradients' scale are expected; the bounds allow about
5x that.  Plans (key tiles and their query spans) equal the oracle's bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import load_balance_amd as lb
import workloads
from oracle import backward as OB
from oracle import plan as OP

pytestmark = pytest.mark.gpu

GRAD_MAX, GRAD_MEAN = 2e-2, 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to64(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_grad(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    d = np.abs(got - ref)
    scale_max, scale_mean = np.abs(ref).max(), np.abs(ref).mean()
    say(f"  {what}: max |d| {d.max():.3e} (scale {scale_max:.3e}, ratio {d.max() / scale_max:.2e})  "
        f"mean |d| {d.mean():.3e} (ratio {d.mean() / scale_mean:.2e})")
    assert d.max() <= GRAD_MAX * scale_max, what
    assert d.mean() <= GRAD_MEAN * scale_mean, what


def varlen_case(lengths, H, Hkv, d, seed, mask="causal_doc"):
    r = np.random.default_rng(seed)
    T = int(sum(lengths))
    q, k, v = workloads.values(r, T, H, Hkv, d)
    do = workloads.f32_to_bf16_bits(r.standard_normal((T, H, d)).astype(np.float32))
    cu = workloads.cu_from_lengths(lengths)
    mk = lb.MASK_CAUSAL_DOC if mask == "causal_doc" else lb.MASK_SHARED_QUESTION
    say(f"  varlen bwd T={T} H={H} Hkv={Hkv} d={d} docs={len(lengths)} mask={mask}")
    tq, tk, tv, tdo = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(do)
    tcu = torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    out, lse = lb.varlen_attn_fwd(tq, tk, tv, tcu, mask_kind=mk)
    ws = torch.empty(lb.bwd_workspace_bytes(T, len(lengths), H, Hkv), dtype=torch.uint8, device="cuda")
    dq, dk, dv = lb.varlen_attn_bwd(tq, tk, tv, out, tdo, lse, tcu, mask_kind=mk, workspace=ws)
    torch.cuda.synchronize()
    off = lb.bwd_key_plan_offset(False, T, T, len(lengths), H, Hkv, ws.numel())
    assert lb.read_device_error(ws) == 0 and lb.read_device_error(ws[off:]) == 0
    ref = OB.varlen_attention_bwd(q, k, v, do, cu, H, Hkv, mask=mask)
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_grad(to64(got), want, f"{name} T={T} H={H}/{Hkv} d={d} {mask}")
    return ws, off, cu


@pytest.mark.parametrize("H,Hkv,d", [(8, 2, 128), (4, 4, 64), (4, 2, 64), (8, 1, 64), (32, 8, 128), (16, 8, 128),
                                     (8, 8, 64)])
def test_varlen_backward_every_element(H, Hkv, d):
    lengths = [1, 150, 37, 64, 1, 200, 3]
    varlen_case(lengths, H, Hkv, d, seed=H * 10 + Hkv + d)


@pytest.mark.parametrize("H,Hkv,d", [(32, 8, 128), (16, 8, 128)])
def test_varlen_backward_eight_queues_many_items(H, Hkv, d):
    """8 kv heads: the dQ and dK/dV kernels take one queue per XCD, and with documents of up
    to 1000 tokens every queue holds several items of both kernels, stolen across queues."""
    lengths = [1, 700, 3, 1, 257, 64, 129, 1000, 2]
    varlen_case(lengths, H, Hkv, d, seed=H + Hkv + d)


def test_varlen_backward_shared_question():
    varlen_case([96, 70, 33, 1, 64], 8, 2, 128, seed=3, mask="shared_question")


@pytest.mark.parametrize("mask", ["causal_doc", "shared_question"])
def test_key_tile_plan_equals_oracle(mask):
    """The key-tile (transposed) plan of the backward, in queue order, equals the oracle's
    transposed enumerator bit for bit; the query-tile plan equals the forward enumerator at
    the backward's tile height.  Both are in the documents order of key blocks."""
    lengths = [300, 1, 64, 65, 129, 2, 90]
    H, Hkv, d = 8, 2, 128
    ws, off, cu = varlen_case(lengths, H, Hkv, d, seed=11, mask=mask)
    G = H // Hkv
    q_rows = 256 // G  # the forward's tile height
    k_rows = 128
    n_seg = len(cu) - 1
    ref_q = OP.plan_documents(OP.fragments_varlen(cu, mask), q_rows, 1, 0, G, n_seg)
    frags_t = OP.fragments_varlen_t(cu, mask)
    ref_k_tiles = OP.tiles_t(frags_t, k_rows)
    ref_k = [ref_k_tiles[i] for i in OP.documents_order(ref_k_tiles, frags_t, k_rows,
                                                        [t["blocks"] for t in ref_k_tiles], n_seg)]
    for got, want, what in ((lb.read_plan(ws), ref_q, "query tiles"), (lb.read_plan(ws[off:]), ref_k, "key tiles")):
        assert len(got) == len(want), what
        for i, (a, b) in enumerate(zip(got, want)):
            assert (a["q_start"], a["q_len"], a["q_pos0"], a["cost"], a["blocks"]) == \
                   (b["q_start"], b["q_len"], b["q_pos0"], b["cost"], b["blocks"]), (what, i)
            assert [tuple(s) for s in a["spans"]] == [tuple(s) for s in b["spans"]], (what, i)
    # the workgroups' records account for every item: pairs per query head, and the blocks
    # swept (dQ: 64-key blocks per kv head; dK/dV: 64-row query stages per query head)
    for w, want, per in ((ws, ref_q, Hkv), (ws[off:], ref_k, H)):
        recs = lb.read_worker_timing(w)
        assert sum(x["pairs"] for x in recs) == H * sum(t["cost"] for t in want)
        assert sum(x["blocks"] for x in recs) == per * sum(t["blocks"] for t in want)


def test_single_token_documents():
    """out = v, so dv is the sum of the group's dout rows, and dq = dk = 0: P = 1 is rebuilt
    from the saved lse up to one rounding, so dq and dk stay below 1e-5 where the inputs are
    of order 1."""
    lengths = [1] * 40
    H, Hkv, d = 4, 2, 128
    r = np.random.default_rng(5)
    q, k, v = workloads.values(r, 40, H, Hkv, d)
    do = workloads.f32_to_bf16_bits(r.standard_normal((40, H, d)).astype(np.float32))
    tq, tk, tv, tdo = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(do)
    tcu = torch.from_numpy(np.asarray(workloads.cu_from_lengths(lengths), dtype=np.int32)).cuda()
    out, lse = lb.varlen_attn_fwd(tq, tk, tv, tcu)
    dq, dk, dv = lb.varlen_attn_bwd(tq, tk, tv, out, tdo, lse, tcu)
    torch.cuda.synchronize()
    assert torch.equal(out, tv.repeat_interleave(2, dim=1))
    assert to64(dq).__abs__().max() < 1e-5 and to64(dk).__abs__().max() < 1e-5
    want = workloads.bf16_bits_to_f32(do).astype(np.float64).reshape(40, Hkv, 2, d).sum(axis=2)
    check_grad(to64(dv), want, "single-token dv")


@pytest.mark.parametrize("rule,H,Hkv", [("zigzag", 8, 2), ("dispatch", 8, 2), ("zigzag", 32, 8)])
def test_ring_backward_reassembles_the_unsharded_gradient(rule, H, Hkv):
    """Every rank of a cp = 4 sharding: the forward ring (block steps + merges) gives out and
    lse; D comes from the merged out; each step's backward adds its dq and returns the
    source chunk's partial dk, dv.  Summed per owner, they equal the unsharded gradient."""
    from load_balance_amd import sharding as LS
    cp, d = 4, 128
    r = np.random.default_rng(21)
    lengths = [700, 37, 1, 260, 9, 301]
    lengths.append(2 * cp * 256 - sum(lengths))
    T = sum(lengths)
    q, k, v = workloads.values(r, T, H, Hkv, d)
    do = workloads.f32_to_bf16_bits(r.standard_normal((T, H, d)).astype(np.float32))
    tok = LS.shard_tokens(rule, lengths, cp, n_chunks=4 * cp)
    shards = LS.build_shards(lengths, tok, lambda idx: (q[idx], k[idx], v[idx]))
    ref = OB.varlen_attention_bwd(q, k, v, do, workloads.cu_from_lengths(lengths), H, Hkv)
    dk_sum = [torch.zeros((2, len(t), Hkv, d), dtype=torch.float32, device="cuda") for t in tok]
    dq_all = np.zeros((T, H, d))
    for rank in range(cp):
        say(f"  {rule} rank {rank}: {len(tok[rank])} tokens")
        share = LS.ShardedRank(shards, rank)
        out, lse = share.run_planned()
        tdo = dev_bf16(do[tok[rank]])
        dvec = lb.attn_bwd_rowdot(out, tdo)
        dq = torch.zeros_like(out)
        for t, st in enumerate(share.steps):
            _, dkv = lb.block_attn_bwd(share.q, st["kv"], tdo, lse, dvec, share.q_pos, st["kv_pos"], share.q_doc,
                                       st["kv_doc"], dq)
            dk_sum[st["source"]] += dkv
        torch.cuda.synchronize()
        dq_all[tok[rank]] = to64(dq)
    dk_all = np.zeros((T, Hkv, d))
    dv_all = np.zeros((T, Hkv, d))
    for s in range(cp):
        dk_all[tok[s]] = to64(dk_sum[s][0])
        dv_all[tok[s]] = to64(dk_sum[s][1])
    for name, got, want in zip(("dq", "dk", "dv"), (dq_all, dk_all, dv_all), ref):
        check_grad(got, want, f"{rule} ring {name}")


def test_block_backward_leaves_unseen_rows_and_zeroes_unseen_keys():
    """A step whose chunk holds another document's keys: dq is left as it was and every dk,
    dv row is written zero."""
    H, Hkv, d = 4, 2, 128
    r = np.random.default_rng(2)
    n = 64
    q, k, v = workloads.values(r, 2 * n, H, Hkv, d)
    do = workloads.f32_to_bf16_bits(r.standard_normal((n, H, d)).astype(np.float32))
    i32 = lambda x: torch.from_numpy(np.asarray(x, dtype=np.int32)).cuda()
    q_pos, q_doc = i32(np.arange(n)), i32(np.zeros(n))
    kv_pos, kv_doc = i32(np.arange(n)), i32(np.ones(n))
    kv = torch.stack([dev_bf16(k[n:]), dev_bf16(v[n:])]).contiguous()
    lse = torch.zeros((H, n), dtype=torch.float32, device="cuda")
    dvec = torch.zeros((H, n), dtype=torch.float32, device="cuda")
    dq = torch.full((n, H, d), 3.0, dtype=torch.float32, device="cuda")
    dkv = torch.full((2, n, Hkv, d), 5.0, dtype=torch.float32, device="cuda")
    lb.block_attn_bwd(dev_bf16(q[:n]), kv, dev_bf16(do), lse, dvec, q_pos, kv_pos, q_doc, kv_doc, dq, dkv)
    torch.cuda.synchronize()
    assert torch.all(dq == 3.0) and torch.all(dkv == 0.0)


def test_block_backward_shared_question_whole_pack():
    """One block step over a whole shared-question pack with document 0 shared: dq, dk, dv
    against the varlen shared-question oracle gradient; the key-tile plan (the question's
    keys with every answer's rows) against the oracle's transposed enumerator."""
    lengths = [300, 120, 1, 64, 90]
    T, H, Hkv, d = sum(lengths), 8, 2, 128
    r = np.random.default_rng(63)
    q, k, v = workloads.values(r, T, H, Hkv, d)
    do = workloads.f32_to_bf16_bits(r.standard_normal((T, H, d)).astype(np.float32))
    pos = np.arange(T, dtype=np.int32)
    doc = np.repeat(np.arange(len(lengths), dtype=np.int32), lengths)
    i32 = lambda x: torch.from_numpy(np.asarray(x, dtype=np.int32)).cuda()
    say(f"  block bwd, shared question, T={T}")
    tq, tdo = dev_bf16(q), dev_bf16(do)
    kv = torch.stack([dev_bf16(k), dev_bf16(v)]).contiguous()
    out, lse = lb.block_attn_fwd(tq, kv, i32(pos), i32(pos), i32(doc), i32(doc), shared_doc=0)
    dvec = lb.attn_bwd_rowdot(out, tdo)
    dq = torch.zeros((T, H, d), dtype=torch.float32, device="cuda")
    half = lb.workspace_bytes(T, T, H, Hkv)
    ws = torch.empty(2 * half + 512, dtype=torch.uint8, device="cuda")
    _, dkv = lb.block_attn_bwd(tq, kv, tdo, lse, dvec, i32(pos), i32(pos), i32(doc), i32(doc), dq, workspace=ws,
                               shared_doc=0)
    torch.cuda.synchronize()
    ref = OB.varlen_attention_bwd(q, k, v, do, workloads.cu_from_lengths(lengths), H, Hkv, mask="shared_question")
    for name, got, want in zip(("dq", "dk", "dv"), (to64(dq), to64(dkv[0]), to64(dkv[1])), ref):
        check_grad(got, want, f"{name} block path, shared question")
    off = lb.bwd_key_plan_offset(True, T, T, T, H, Hkv, ws.numel())
    ref_k_tiles = OP.tiles_t(OP.fragments_block_t(pos, doc, pos, doc, shared_doc=0), 128)
    ref_k = [ref_k_tiles[i] for i in OP.lpt_order(ref_k_tiles)]
    got = lb.read_plan(ws[off:])
    assert len(got) == len(ref_k)
    for i, (a, b) in enumerate(zip(got, ref_k)):
        assert (a["q_start"], a["q_len"], a["q_pos0"], a["cost"], a["blocks"]) == \
               (b["q_start"], b["q_len"], b["q_pos0"], b["cost"], b["blocks"]), i
        assert [tuple(s) for s in a["spans"]] == [tuple(s) for s in b["spans"]], i


@pytest.mark.parametrize("H,Hkv", [(8, 2), (32, 8)])
@pytest.mark.parametrize("ring", [False, True])
def test_ring_backward_shared_question_reassembles(ring, H, Hkv):
    """A shared-question pack sharded by sequence zigzag over cp = 4 ranks, document 0
    shared: each rank's forward ring and ring backward (steps no row sees send nothing back;
    with ring=True the steps' dK/dV items in one launch), summed per owner, equal the
    unsharded shared-question gradient."""
    from load_balance_amd import sharding as LS
    cp, d = 4, 128
    r = np.random.default_rng(64)
    lengths = [500, 37, 1, 260, 9, 301]
    lengths.append(2 * cp * 256 - sum(lengths))
    T = sum(lengths)
    q, k, v = workloads.values(r, T, H, Hkv, d)
    do = workloads.f32_to_bf16_bits(r.standard_normal((T, H, d)).astype(np.float32))
    tok = LS.shard_tokens("zigzag", lengths, cp)
    shards = LS.build_shards(lengths, tok, lambda idx: (q[idx], k[idx], v[idx]))
    ref = OB.varlen_attention_bwd(q, k, v, do, workloads.cu_from_lengths(lengths), H, Hkv, mask="shared_question")
    dk_sum = [torch.zeros((2, len(t), Hkv, d), dtype=torch.float32, device="cuda") for t in tok]
    dq_all = np.zeros((T, H, d))
    for rank in range(cp):
        share = LS.ShardedRank(shards, rank, shared_doc=0)
        say(f"  zigzag rank {rank}, shared question: live steps {share.live_steps}")
        share.run_planned()
        dq, dkvs = share.backward(dev_bf16(do[tok[rank]]), ring=ring)
        for st, dkv in zip(share.steps, dkvs):
            if dkv is not None:
                dk_sum[st["source"]] += dkv
        torch.cuda.synchronize()
        dq_all[tok[rank]] = to64(dq)
    dk_all = np.zeros((T, Hkv, d))
    dv_all = np.zeros((T, Hkv, d))
    for s in range(cp):
        dk_all[tok[s]] = to64(dk_sum[s][0])
        dv_all[tok[s]] = to64(dk_sum[s][1])
    for name, got, want in zip(("dq", "dk", "dv"), (dq_all, dk_all, dv_all), ref):
        check_grad(got, want, f"zigzag ring {name}, shared question, H={H}/{Hkv}")


@pytest.mark.parametrize("rank", [1, 3])
@pytest.mark.parametrize("H,Hkv,d", [(8, 2, 128), (4, 4, 64), (8, 1, 64), (32, 8, 128), (16, 8, 128)])
def test_ring_dkv_launch_equals_the_step_backwards(rank, H, Hkv, d):
    """A zigzag rank's ring backward with every live step's dK/dV items in one launch: dq and
    every step's partial dk, dv have the bits of the per-step backward; the merged key-tile
    queue equals the oracle's (each step's transposed plan, merged longest first); the
    workgroups' records cover every item once; summed per owner over all ranks the
    gradients equal the oracle's."""
    from load_balance_amd import zigzag as LZ
    cp, C = 4, 256
    T = 2 * cp * C
    lengths = workloads.lognormal_lengths(T, 3, T)
    r = np.random.default_rng(66 + rank)
    q, k, v = workloads.values(r, T, H, Hkv, d)
    do_all = workloads.f32_to_bf16_bits(r.standard_normal((T, H, d)).astype(np.float32))

    def get_chunk(c):
        sl = slice(c * C, (c + 1) * C)
        return q[sl], k[sl], v[sl]

    share = LZ.RankShare(lengths, C, rank, cp, get_chunk)
    say(f"  zigzag cp=4 rank {rank} H={H} Hkv={Hkv} d={d}: live steps {share.live_steps}")
    share.run_planned()
    rows = np.concatenate([np.arange(c * C, (c + 1) * C) for c in LZ.chunks_of_rank(rank, cp)])
    dout = dev_bf16(do_all[rows])
    dq, dkvs = share.backward(dout)
    torch.cuda.synchronize()
    ref_dq, ref_dkv = dq.clone(), {t: x.clone() for t, x in enumerate(dkvs) if x is not None}
    dq, dkvs = share.backward(dout, ring=True)
    torch.cuda.synchronize()
    assert torch.equal(dq, ref_dq), "dq"
    for t, x in ref_dkv.items():
        assert torch.equal(dkvs[t], x), f"dkv of step {t}"
    assert lb.read_device_error(share.bwd_ring_workspace) == 0
    # the merged key-tile queue against the oracle's
    qp, qd = share.q_pos.cpu().numpy(), share.q_doc.cpu().numpy()
    plans = []
    for t in share.live_steps:
        st = share.steps[t]
        tl = OP.tiles_t(OP.fragments_block_t(qp, qd, st["kv_pos"].cpu().numpy(), st["kv_doc"].cpu().numpy()), 128)
        plans.append([tl[i] for i in OP.lpt_order(tl)])
    want = OP.merge_step_plans(plans)
    got = lb.read_plan(share.bwd_ring_workspace, with_step=True)
    assert len(got) == len(want)
    for i, (a, b) in enumerate(zip(got, want)):
        assert (a["q_start"], a["q_len"], a["q_pos0"], a["cost"], a["blocks"], a["step"]) == \
               (b["q_start"], b["q_len"], b["q_pos0"], b["cost"], b["blocks"], b["step"]), i
        assert [tuple(s) for s in a["spans"]] == [tuple(s) for s in b["spans"]], i
    recs = lb.read_worker_timing(share.bwd_ring_workspace)
    assert sum(x["items"] for x in recs) == sum(1 for t in want if t["spans"]) * Hkv
    # the rank's dq against the oracle (every rank's dq rows are its own)
    ref = OB.varlen_attention_bwd(q, k, v, do_all, workloads.cu_from_lengths(lengths), H, Hkv)
    check_grad(to64(dq), ref[0][rows], f"rank {rank} ring dq")
