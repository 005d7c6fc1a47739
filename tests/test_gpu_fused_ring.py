"""GPU parity of the fused ring (lb_plan_ring_fused + lb_ring_attn_run_fused): a rank's live
ring steps run as one item per query tile and kv head, each against the keys of every step in
one online softmax, writing the merged result with no partials and no merges.

The plan is compared bit for bit with the oracle's ``fuse_step_plans`` over the steps' natural
tile orders; the result with the float64 oracle (the unsharded attention of the rank's rows)
at the tolerances of the other parity tests, and with the unfused ring to the rounding of the
bf16 softmax weights."""
import numpy as np
import pytest
import torch

import load_balance_amd as lb
import workloads
from oracle import attention as OA
from oracle import plan as OP
from test_gpu_parity import LSE_MAX, OUT_MAX, OUT_MEAN, assert_same_plan, check, ring_share, say

pytestmark = pytest.mark.gpu


def fused_oracle_plan(share):
    """The oracle's fused tiles over the share's live steps, with each span's step."""
    n_q, H, d = share.q.shape
    Hkv = share.steps[0]["kv"].shape[2]
    bm = lb.tile_rows(H, Hkv, d)
    qp, qd = share.q_pos.cpu().numpy(), share.q_doc.cpu().numpy()
    shared = None if share.shared_doc < 0 else share.shared_doc
    plans = [OP.tiles(OP.fragments_block(qp, qd, share.steps[t]["kv_pos"].cpu().numpy(),
                                         share.steps[t]["kv_doc"].cpu().numpy(), shared_doc=shared), bm)
             for t in share.live_steps]
    return OP.fuse_step_plans(plans)


def read_fused_plan(ring_workspace):
    """The ring's tiles with the step of every span decoded from `reserved` (4 bits a span)."""
    tiles = lb.read_plan(ring_workspace, with_step=True)
    for t in tiles:
        packed = t.pop("step")
        t["span_steps"] = [(packed >> (4 * s)) & 15 for s in range(len(t["spans"]))]
    return tiles


def check_fused(share, what):
    """run_fused() against the oracle's fused plan and the unfused ring; returns (out, lse)."""
    assert share.fusable, f"{what}: the share should fuse"
    out, lse = share.run_ring()
    torch.cuda.synchronize()
    ring_out, ring_lse = out.clone(), lse.clone()
    share.out.fill_(7.0)
    share.lse.fill_(7.0)
    out, lse = share.run_fused()
    torch.cuda.synchronize()
    assert lb.read_device_error(share.ring_workspace) == 0, what
    want = fused_oracle_plan(share)
    assert want is not None
    assert_same_plan(read_fused_plan(share.ring_workspace), want, f"{what}: fused plan")
    # every item run once: the workgroups' records add up to the plan's work
    n_q, H, d = share.q.shape
    Hkv = share.steps[0]["kv"].shape[2]
    recs = lb.read_worker_timing(share.ring_workspace)
    work = [t for t in want if t["spans"]]
    assert sum(x["items"] for x in recs) == len(work) * Hkv
    assert sum(x["blocks"] for x in recs) == sum(t["blocks"] for t in work) * Hkv
    assert sum(x["pairs"] for x in recs) == sum(t["cost"] for t in work) * H
    # The same rows see no key on both paths.  Elsewhere both round the softmax weights to bf16
    # before the PV product, each against its own running maximum (a step's, or every step's
    # at once), so they agree to that rounding: within the tolerances both meet against the
    # float64 oracle (the check that decides).
    assert torch.equal(torch.isinf(lse), torch.isinf(ring_lse)), f"{what}: rows without keys differ"
    seen = ~torch.isinf(ring_lse)
    d_lse = (lse - ring_lse)[seen].abs().max().item() if seen.any() else 0.0
    rows_seen = seen.all(dim=0)
    d_out = (out - ring_out)[rows_seen].abs().max().item() if rows_seen.any() else 0.0
    say(f"  {what}: fused vs ring: out max {d_out:.2e}, lse max {d_lse:.2e}")
    assert d_out <= OUT_MAX and d_lse <= LSE_MAX, what
    return out, lse


@pytest.mark.parametrize("rank", [0, 2, 3])
@pytest.mark.parametrize("H,Hkv,d", [(8, 2, 128), (4, 4, 64), (8, 1, 64), (32, 8, 128), (16, 8, 128), (8, 8, 64)])
def test_fused_ring_equals_oracle(rank, H, Hkv, d):
    """A zigzag rank of cp = 4 as a fused ring, for every head grouping and head size the
    kernel is built for, with one queue (kv heads 1, 2, 4) and one per XCD (8): the plan is
    the oracle's, every item runs once, and every row of the rank equals the unsharded
    oracle."""
    cp, C = 4, 256
    share, (lengths, q, k, v) = ring_share(cp=cp, C=C, rank=rank, H=H, Hkv=Hkv, d=d, with_inputs=True)
    say(f"  fused ring: zigzag cp=4 rank {rank} H={H} Hkv={Hkv} d={d}: live steps {share.live_steps}")
    out, lse = check_fused(share, f"rank {rank} H={H}/{Hkv} d={d}")
    rows = np.concatenate([np.arange(c * C, (c + 1) * C) for c in lb.zigzag.chunks_of_rank(rank, cp)])
    ref_o, ref_l = OA.varlen_attention(q, k, v, workloads.cu_from_lengths(lengths), H, Hkv, rows=rows)
    check(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, f"fused rank {rank} H={H}/{Hkv} d={d} vs oracle")


def test_fused_ring_graph_replays_equal_eager_runs():
    """The fused share captured in one HIP graph (step plans, fused ring, one attention launch)
    and replayed three times with eager work in between gives the eager bits."""
    share = ring_share(rank=1, seed=5)
    out, lse = share.run_fused()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    say("  capturing the fused share")
    share.capture(fused=True)
    for i in range(3):
        share.out.fill_(7.0)
        share.lse.fill_(7.0)
        out, lse = share.replay()
        torch.cuda.synchronize()
        say(f"  replay {i}")
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"replay {i}"
        share.run_planned()
        out, lse = share.run_fused()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"eager run after replay {i}"


def test_rings_of_the_other_kind_run_nothing():
    """A fused ring given to the unfused ring kernel, and an unfused ring given to the fused
    one, are refused on the device: LB_DEVERR_PLAN, nothing written."""
    share = ring_share(rank=2)
    live = [share.steps[t] for t in share.live_steps]
    assert len(live) >= 2
    ks, vs = [st["kv"][0] for st in live], [st["kv"][1] for st in live]
    share.run_fused()
    outs = [torch.full_like(share.out, 7.0) for _ in live]
    lses = [torch.full_like(share.lse, 7.0) for _ in live]
    lb.ring_attn_run(share.q, ks, vs, outs, lses, share.ring_workspace)
    torch.cuda.synchronize()
    assert lb.read_device_error(share.ring_workspace) & lb.DEVERR_PLAN
    for o, l in zip(outs, lses):
        assert torch.all(o == 7.0) and torch.all(l == 7.0)
    share.run_ring()
    out, lse = torch.full_like(share.out, 7.0), torch.full_like(share.lse, 7.0)
    lb.ring_attn_run_fused(share.q, ks, vs, out, lse, share.ring_workspace)
    torch.cuda.synchronize()
    assert lb.read_device_error(share.ring_workspace) & lb.DEVERR_PLAN
    assert torch.all(out == 7.0) and torch.all(lse == 7.0)


def test_fused_ring_past_the_span_capacity_runs_nothing():
    """Per-document shards of cp = 4: each step's query runs meet few key runs, but over all
    live steps together a query tile meets more than LB_MAX_SPANS, so the share does not fuse
    (judged on the host); fused on the device anyway, the ring flags LB_DEVERR_SPANS and a
    launch over it writes nothing."""
    from load_balance_amd import sharding as LS
    cp, H, Hkv, d = 4, 8, 2, 128
    r = np.random.default_rng(66)
    lengths = [2 * cp * 256]
    q, k, v = workloads.values(r, lengths[0], H, Hkv, d)
    tok = LS.shard_tokens("per_document", lengths, cp)
    shards = LS.build_shards(lengths, tok, lambda idx: (q[idx], k[idx], v[idx]))
    share = LS.ShardedRank(shards, 1)
    assert not share.fusable
    live = [share.steps[t] for t in share.live_steps]
    assert all("slices" not in st for st in live)
    n_q = share.q.shape[0]
    share.plan_all()
    ring = lb.new_ring_workspace(len(live), *share._ws_shape[:4])
    lb.plan_ring([share.step_workspaces[t] for t in share.live_steps], [st["kv"].shape[1] for st in live], n_q, H,
                 Hkv, d, ring, fused=True)
    out, lse = torch.full_like(share.out, 7.0), torch.full_like(share.lse, 7.0)
    lb.ring_attn_run_fused(share.q, [st["kv"][0] for st in live], [st["kv"][1] for st in live], out, lse, ring)
    torch.cuda.synchronize()
    assert lb.read_device_error(ring) & lb.DEVERR_SPANS
    assert lb.read_plan(ring) == []
    assert torch.all(out == 7.0) and torch.all(lse == 7.0)
    with pytest.raises(ValueError):
        share.run_fused()


def zigzag_rank3():
    lengths = workloads.zigzag_pack_lengths(0)
    C, cp, rank = 8192, 8, 3
    cache = {}

    def get_chunk(c):
        if c not in cache:
            cache[c] = workloads.zigzag_chunk_values(c)
        return cache[c]

    say("  zigzag rank 3 of cp=8: building the share")
    return lb.zigzag.RankShare(lengths, C, rank, cp, get_chunk), get_chunk, lengths


def test_fused_ring_zigzag_rank3_cp8():
    """Rank 3 of cp = 8 on the 131072-token pack, as the zigzag benchmark runs it: the fused
    plan equal to the oracle's, every item run once, agreement with the unfused ring, and the
    oracle's fold on sampled rows."""
    share, get_chunk, lengths = zigzag_rank3()
    assert share.live_steps == [0, 1, 7] and share.fusable
    out, lse = check_fused(share, "zigzag rank 3 fused")
    r = np.random.default_rng(18)
    rows = np.unique(np.concatenate([[0, 1, 8191, 8192, 16383], r.integers(0, 2 * 8192, 60)]))
    ref_o, ref_l, _ = OA.zigzag_rank_attention(get_chunk, lengths, 8192, 3, 8, 32, 8, rows=rows)
    check(out[rows].cpu().numpy(), lse[:, rows].cpu().numpy(), ref_o, ref_l, "zigzag rank 3 fused (sampled)")


@pytest.mark.timeout(900)
def test_fused_ring_zigzag_rank3_cp8_every_row(tmp_path):
    """All 16384 rows x 32 heads of rank 3's share through the fused ring against the
    oracle's fold of the 8 ring steps."""
    import oracle_pool
    lengths = workloads.zigzag_pack_lengths(0)
    C, cp, rank = 8192, 8, 3
    share = lb.zigzag.RankShare(lengths, C, rank, cp, workloads.zigzag_chunk_values)
    out, lse = share.run_fused()
    torch.cuda.synchronize()
    assert lb.read_device_error(share.ring_workspace) == 0
    st = oracle_pool.zigzag_every_row(out.cpu().numpy(), lse.cpu().numpy(), 0, rank, cp, C, str(tmp_path), say)
    say(f"  zigzag rank 3 fused every row: out max {st['out_max']:.3e} mean {st['out_mean']:.3e}  "
        f"lse max {st['lse_max']:.3e}")
    assert st["finite"] and st["n"] == 2 * C * 32 * 128
    assert st["out_max"] <= OUT_MAX and st["out_mean"] <= OUT_MEAN and st["lse_max"] <= LSE_MAX


def check_fused_bwd(share, what):
    """The ring backward with the dQ side fused (lb_block_attn_bwd_ring_fused) against the
    unfused ring backward: dk, dv bit for bit (the same dK/dV launch), dq to fp32 rounding
    (one sum over every step's key blocks instead of a sum per step added into dq)."""
    n_q, H, d = share.q.shape
    r = np.random.default_rng(31)
    dout = torch.from_numpy(workloads.f32_to_bf16_bits(r.standard_normal((n_q, H, d)).astype(np.float32))
                            .view(np.int16)).view(torch.bfloat16).cuda()
    share.run_fused()
    dq, dkv = share.backward(dout, ring=True)
    torch.cuda.synchronize()
    dq_ref, dkv_ref = dq.clone(), [None if x is None else x.clone() for x in dkv]
    dq, dkv = share.backward(dout, ring=True, fused=True)
    torch.cuda.synchronize()
    assert lb.read_device_error(share.bwd_q_ring_workspace) == 0, what
    for a, b in zip(dkv, dkv_ref):
        assert (a is None) == (b is None)
        if a is not None:
            assert torch.equal(a, b), f"{what}: dk/dv differ"
    scale = dq_ref.abs().max().item()
    diff = (dq - dq_ref).abs().max().item()
    say(f"  {what}: fused dQ vs per-step dQ: max |diff| {diff:.2e} (max |dq| {scale:.2e})")
    assert diff <= 1e-4 * scale, what


@pytest.mark.parametrize("rank,H,Hkv,d", [(0, 8, 2, 128), (3, 32, 8, 128), (2, 8, 1, 64)])
def test_fused_dq_ring_backward(rank, H, Hkv, d):
    share = ring_share(cp=4, C=256, rank=rank, H=H, Hkv=Hkv, d=d)
    check_fused_bwd(share, f"bwd rank {rank} H={H}/{Hkv} d={d}")


def test_fused_dq_ring_backward_zigzag_rank3_cp8():
    share, _, _ = zigzag_rank3()
    check_fused_bwd(share, "zigzag rank 3 backward")
