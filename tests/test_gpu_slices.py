"""GPU parity of slice-list masks ("03 · 长文负载均衡", section 4.4) through the C ABI.

The same tolerances as the forward (out max |d| <= 2e-2, mean <= 2e-3; lse max <= 5e-3);
plans equal the oracle's enumerator bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import load_balance_amd as lb
import workloads
from oracle import plan as OP
from oracle import slices as SL

pytestmark = pytest.mark.gpu

OUT_MAX, OUT_MEAN, LSE_MAX = 2e-2, 2e-3, 5e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def check(out, lse, ref_o, ref_l, what):
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    seen = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(l), seen), f"{what}: rows with no key differ"
    rows = seen.all(axis=0)
    d_o = np.abs(o[rows] - ref_o[rows])
    d_l = np.abs(l[seen] - ref_l[seen])
    say(f"  {what}: out max {d_o.max():.3e} mean {d_o.mean():.3e}  lse max {d_l.max():.3e}")
    assert d_o.max() <= OUT_MAX and d_o.mean() <= OUT_MEAN and d_l.max() <= LSE_MAX, what


def run(slices, n_q, n_k, H, Hkv, d, seed):
    r = np.random.default_rng(seed)
    q, _, _ = workloads.values(r, n_q, H, Hkv, d)
    _, k, v = workloads.values(r, n_k, H, Hkv, d)
    say(f"  slices_attn_fwd n_q={n_q} n_kv={n_k} H={H}/{Hkv} d={d} slices={len(slices)}")
    ws = lb.new_workspace(n_q, 2 * len(slices) + 1, H, Hkv)
    out, lse = lb.slices_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), slices, workspace=ws)
    torch.cuda.synchronize()
    assert lb.read_device_error(ws) == 0
    return (q, k, v), out, lse, ws


def test_varlen_causal_as_slices_is_the_varlen_forward_bit_for_bit():
    lengths = [1, 300, 64, 65, 2, 700]
    T, H, Hkv, d = sum(lengths), 8, 2, 128
    (q, k, v), out, lse, ws = run(SL.varlen_causal_slices(lengths), T, T, H, Hkv, d, seed=1)
    cu = torch.from_numpy(np.asarray(workloads.cu_from_lengths(lengths), dtype=np.int32)).cuda()
    out2, lse2 = lb.varlen_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), cu)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("frame", [64, 200])
@pytest.mark.parametrize("H,Hkv", [(8, 2), (32, 8)])
def test_block_causal(frame, H, Hkv):
    lengths = [900, 1, 257, 333, 64]
    T, d = sum(lengths), 128
    sl = SL.block_causal_slices(lengths, frame)
    (q, k, v), out, lse, ws = run(sl, T, T, H, Hkv, d, seed=frame)
    ref_o, ref_l = SL.slices_attention(q, k, v, sl, H, Hkv)
    check(out, lse, ref_o, ref_l, f"block-causal frames of {frame} H={H}/{Hkv}")
    plan = lb.read_plan(ws)
    t = OP.tiles(SL.fragments(sl), lb.tile_rows(H, Hkv, d))
    ref = [t[i] for i in OP.lpt_order(t)]
    assert [(a["q_start"], a["q_len"], a["q_pos0"], a["cost"], a["blocks"], [tuple(x) for x in a["spans"]]) for a in plan] \
        == [(b["q_start"], b["q_len"], b["q_pos0"], b["cost"], b["blocks"], [tuple(x) for x in b["spans"]]) for b in ref]


def test_shared_question_as_slices():
    lengths = [300, 128, 1, 77, 128]
    T, H, Hkv, d = sum(lengths), 8, 2, 128
    sl = SL.shared_question_slices(lengths)
    (q, k, v), out, lse, ws = run(sl, T, T, H, Hkv, d, seed=4)
    ref_o, ref_l = SL.slices_attention(q, k, v, sl, H, Hkv)
    check(out, lse, ref_o, ref_l, "shared question as slices")


@pytest.mark.parametrize("seed", range(3))
def test_random_slice_lists(seed):
    """Rectangles of all four kinds with unequal sides, several per query range, and query
    ranges no slice covers (lse = -inf there)."""
    r = np.random.default_rng(50 + seed)
    n_q, n_k = 700, 520
    sl, q0 = [], 0
    while q0 < n_q:
        ql = int(min(n_q - q0, r.integers(1, 150)))
        if r.random() < 0.15:
            q0 += ql
            continue
        cuts = np.sort(r.choice(np.arange(1, n_k), size=int(r.integers(1, 4)), replace=False))
        bounds = [0] + cuts.tolist() + [n_k]
        picks = [(bounds[i], bounds[i + 1] - bounds[i]) for i in range(len(bounds) - 1) if r.random() < 0.6]
        for (ks, kl) in picks[:4]:
            sl.append((q0, ql, ks, kl, int(r.integers(0, 4))))
        q0 += ql
    H, Hkv, d = 4, 2, 64 if seed == 1 else 128
    (q, k, v), out, lse, ws = run(sl, n_q, n_k, H, Hkv, d, seed=seed)
    ref_o, ref_l = SL.slices_attention(q, k, v, sl, H, Hkv)
    check(out, lse, ref_o, ref_l, f"random slices seed {seed}")
    # the plan, the fragments of rows no slice covers included, equals the oracle's
    t = OP.tiles(SL.fragments(sl, n_q), lb.tile_rows(H, Hkv, d))
    ref = [t[i] for i in OP.lpt_order(t)]
    plan = lb.read_plan(ws)
    assert [(a["q_start"], a["q_len"], a["q_pos0"], a["cost"], a["blocks"], [tuple(x) for x in a["spans"]]) for a in plan] \
        == [(b["q_start"], b["q_len"], b["q_pos0"], b["cost"], b["blocks"], [tuple(x) for x in b["spans"]]) for b in ref]


@pytest.mark.parametrize("bad", ["overlap", "kind", "range"])
def test_malformed_slice_lists_run_nothing(bad):
    H, Hkv, d, n = 4, 2, 128, 64
    sl = {"overlap": [(0, 32, 0, 32, 1), (16, 32, 0, 32, 1)],
          "kind": [(0, 32, 0, 32, 7)],
          "range": [(0, 32, 0, 100, 0)]}[bad]
    r = np.random.default_rng(0)
    q, k, v = workloads.values(r, n, H, Hkv, d)
    ws = lb.new_workspace(n, 2 * len(sl) + 1, H, Hkv)
    out = torch.full((n, H, d), 3.0, dtype=torch.bfloat16, device="cuda")
    lb.slices_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), sl, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert lb.read_device_error(ws) & lb.DEVERR_SLICES
    assert torch.all(out == 3.0)


@pytest.mark.parametrize("window,H,Hkv", [(1, 8, 2), (100, 8, 2), (4096, 8, 2), (100, 32, 8), (1024, 16, 8)])
def test_sliding_window(window, H, Hkv):
    """The causal sliding window as slices (BI-CAUSAL bands) against the oracle; the plan,
    spans with their lower bounds included, equals the oracle's bit for bit.  With 8 kv
    heads the bounded kernel takes one queue per XCD."""
    lengths = [1500, 1, 700, 64]
    T, d = sum(lengths), 128
    sl = SL.sliding_window_slices(lengths, window)
    (q, k, v), out, lse, ws = run(sl, T, T, H, Hkv, d, seed=window)
    ref_o, ref_l = SL.slices_attention(q, k, v, sl, H, Hkv)
    check(out, lse, ref_o, ref_l, f"sliding window {window} H={H}/{Hkv}")
    plan = lb.read_plan(ws)
    t = OP.tiles(SL.fragments(sl), lb.tile_rows(H, Hkv, d))
    ref = [t[i] for i in OP.lpt_order(t)]
    assert [(a["q_start"], a["q_len"], a["q_pos0"], a["cost"], a["blocks"], [tuple(x) for x in a["spans"]]) for a in plan] \
        == [(b["q_start"], b["q_len"], b["q_pos0"], b["cost"], b["blocks"], [tuple(x) for x in b["spans"]]) for b in ref]


def test_plain_run_refuses_a_plan_with_lower_bounds():
    """lb_attn_run keeps the key loop without a lower bound: given a plan with one it flags
    LB_DEVERR_PLAN and writes nothing; lb_attn_run_lower runs it."""
    H, Hkv, d, n = 4, 2, 128, 96
    sl = [(0, 96, 0, 96, lb.SLICE_BI_CAUSAL)]
    r = np.random.default_rng(3)
    q, k, v = (dev_bf16(x) for x in workloads.values(r, n, H, Hkv, d))
    ws = lb.plan_slices(sl, n, n, H, Hkv, d)
    out = torch.full((n, H, d), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((H, n), 3.0, dtype=torch.float32, device="cuda")
    lb.attn_run(q, k, v, out, lse, ws)
    torch.cuda.synchronize()
    assert lb.read_device_error(ws) & lb.DEVERR_PLAN
    assert torch.all(out == 3.0) and torch.all(lse == 3.0)
    ws = lb.plan_slices(sl, n, n, H, Hkv, d)
    lb.attn_run_lower(q, k, v, out, lse, ws)
    torch.cuda.synchronize()
    assert lb.read_device_error(ws) == 0
    assert torch.all(torch.isfinite(lse))  # the band keeps the diagonal: every row sees its own key
