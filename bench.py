#!/usr/bin/env python3
"""Effective masked-attention TFLOP/s on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload longtail]

A step is one pass of the hot path over one batch: the planning kernel
(fragments, key spans, exact pair costs, longest-first order) and the
persistent attention kernel, i.e. exactly lb_varlen_attn_fwd split into its
two halves so that HIP events can time each kernel on the stream they run
on.  Inputs are resident in HBM before timing starts.

Effective FLOPs count only unmasked work: 4 * d * H * (visible query-key
pairs), with pairs = sum over documents of l(l+1)/2 (diagonal included).

Prints one JSON line.  Extra workloads (--workload pairA|pairB|zigzag|
shared_question|tiny) print the same fields for their own configuration.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective masked-attn TFLOP/s (Σℓ² FLOPs) & % bf16 MFMA peak, 32K varlen pack"
PEAK_BF16_TFLOPS = 2500.0           # MI355X published dense bf16 MFMA peak (2.5 PFLOP/s)
PEAK_BF16_AT_2400MHZ = 256 * 2.4e9 * 4096 / 1e12   # 256 CUs x 2.4 GHz x 4096 FLOP/clk/CU = 2516.6
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_longtail32k_traffic.json")
TRAFFIC_SOURCE = ("profiles/attn_fwd_longtail32k_traffic.json: rocprofv3 FETCH_SIZE and WRITE_SIZE passes of this "
                  "kernel and planner source and queue order, copy-calibrated; read from that file, not measured "
                  "in this run")
# the attention kernel's and the planner's source files (the queue order decides which reads hit
# in L2): the traffic file applies while their joint hash and the run's queue order match it
KERNEL_SOURCES = [os.path.join(ROOT, "load_balance_amd", "csrc", f) for f in ("attn_fwd.hip", "lds_staging.h",
                                                                              "plan.hip")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def causal_pairs(lengths):
    return int(sum(int(l) * (int(l) + 1) // 2 for l in lengths))


def to_dev(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


# ----------------------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------------------
class VarlenStep:
    """plan + attention over one packed sequence (per-document causal or shared question)."""

    def __init__(self, packs, mask_kind, name, torch, lb):
        self.torch, self.lb = torch, lb
        self.name = name
        self.mask_kind = mask_kind
        self.lpt_weights = None  # (block, pair) weights of the queue order; None: lb_plan_varlen's fitted ones
        self.queue_order = None  # lb.ORDER_LPT or lb.ORDER_DOCUMENTS; None: lb_plan_varlen's (documents)
        self.items = []
        for p in packs:
            T, H, Hkv, d = p["tokens"], p["heads"], p["kv_heads"], p["d"]
            it = dict(T=T, H=H, Hkv=Hkv, d=d,
                      q=to_dev(p["q"], torch), k=to_dev(p["k"], torch), v=to_dev(p["v"], torch),
                      cu=torch.from_numpy(np.asarray(p["cu_seqlens"], np.int32)).cuda())
            it["out"] = torch.empty_like(it["q"])
            it["lse"] = torch.empty((H, T), dtype=torch.float32, device="cuda")
            it["ws"] = lb.new_workspace(T, len(p["lengths"]), H, Hkv)
            self.items.append(it)
        self.H, self.d = packs[0]["heads"], packs[0]["d"]
        if mask_kind == lb.MASK_CAUSAL_DOC:
            self.pairs = sum(causal_pairs(p["lengths"]) for p in packs)
        else:
            self.pairs = 0
            for p in packs:
                Q, ans = p["lengths"][0], p["lengths"][1:]
                self.pairs += Q * (Q + 1) // 2 + sum(a * Q + a * (a + 1) // 2 for a in ans)
        self.flops = 4 * self.d * self.H * self.pairs

    def n_launches(self):
        return len(self.items)

    def run(self, evs=None):
        """evs: optional [launch][3] events recorded before the plan, between plan and attention, after."""
        lb = self.lb
        for i, it in enumerate(self.items):
            ev = None if evs is None else evs[i]
            if ev is not None:
                ev[0].record()
            if self.lpt_weights is None and self.queue_order is None:
                lb.plan_varlen(it["cu"], it["T"], it["H"], it["Hkv"], it["d"], self.mask_kind, workspace=it["ws"])
            else:
                weights = self.lpt_weights or (lb.LPT_FIT_BLOCK_WEIGHT, lb.LPT_FIT_PAIR_WEIGHT)
                order = lb.ORDER_LPT if self.queue_order is None else self.queue_order
                lb.plan_varlen_ordered(it["cu"], it["T"], it["H"], it["Hkv"], it["d"], *weights, order,
                                       mask_kind=self.mask_kind, workspace=it["ws"])
            if ev is not None:
                ev[1].record()
            lb.attn_run(it["q"], it["k"], it["v"], it["out"], it["lse"], it["ws"])
            if ev is not None:
                ev[2].record()

    def plan_pairs(self):
        return sum(sum(t["cost"] for t in self.lb.read_plan(it["ws"])) for it in self.items)

    def worker_ws(self):  # the workspace whose worker records and plan the bench reports
        return self.items[-1]["ws"]


class VarlenBwdStep:
    """The backward of one packed sequence: lb_varlen_attn_bwd (both plans, the D pass, the
    dq kernel and the dk/dv kernel) from the forward's out and lse and a seeded dout, all
    resident before the timed region.  Effective FLOPs: the five products of the gradient
    (S recomputed, dP, dV, dQ, dK) at 2 * d per visible pair each, 10 * d * H * pairs,
    2.5x the forward's count; the kernels compute S and dP in both passes (7 products)."""

    def __init__(self, pack, mask_kind, name, torch, lb):
        self.torch, self.lb = torch, lb
        self.name = name
        T, H, Hkv, d = pack["tokens"], pack["heads"], pack["kv_heads"], pack["d"]
        self.q, self.k, self.v = to_dev(pack["q"], torch), to_dev(pack["k"], torch), to_dev(pack["v"], torch)
        self.cu = torch.from_numpy(np.asarray(pack["cu_seqlens"], np.int32)).cuda()
        self.mask_kind = mask_kind
        self.out, self.lse = lb.varlen_attn_fwd(self.q, self.k, self.v, self.cu, mask_kind=mask_kind)
        r = np.random.default_rng(2000)
        import workloads
        self.dout = to_dev(workloads.f32_to_bf16_bits(r.standard_normal((T, H, d)).astype(np.float32)), torch)
        self.dq, self.dk, self.dv = torch.empty_like(self.q), torch.empty_like(self.k), torch.empty_like(self.v)
        self.ws = torch.empty(lb.bwd_workspace_bytes(T, len(pack["lengths"]), H, Hkv), dtype=torch.uint8,
                              device="cuda")
        self.key_plan = lb.bwd_key_plan_offset(False, T, T, len(pack["lengths"]), H, Hkv, self.ws.numel())
        self.H, self.d = H, d
        self.pairs = causal_pairs(pack["lengths"])
        self.flops = 10 * d * H * self.pairs
        self.kernel_name = "backward call (plans, D, bwd_dq_kernel<128,1,false>, bwd_dkv_kernel<128,false,false>)"

    def n_launches(self):
        return 1

    def run(self, evs=None):
        if evs is not None:
            evs[0][0].record()
            evs[0][1].record()
        self.lb.varlen_attn_bwd(self.q, self.k, self.v, self.out, self.dout, self.lse, self.cu,
                                mask_kind=self.mask_kind, dq=self.dq, dk=self.dk, dv=self.dv, workspace=self.ws)
        if evs is not None:
            evs[0][2].record()

    def plan_pairs(self):
        return sum(t["cost"] for t in self.lb.read_plan(self.ws[self.key_plan:]))

    def worker_ws(self):  # the workspace whose worker records and plan the bench reports
        return self.ws[self.key_plan:]


class SlicesStep:
    """plan + attention of one pack under a slice-list mask (lb_plan_slices + lb_attn_run)."""

    def __init__(self, pack, slices, name, torch, lb):
        self.torch, self.lb = torch, lb
        self.name = name
        # lower-bounded slices (INV-CAUSAL, BI-CAUSAL) run on the bounded kernel
        self.lower = any(x[4] in (lb.SLICE_INV_CAUSAL, lb.SLICE_BI_CAUSAL) for x in slices)
        T, H, Hkv, d = pack["tokens"], pack["heads"], pack["kv_heads"], pack["d"]
        self.T, self.H, self.Hkv, self.d = T, H, Hkv, d
        self.q, self.k, self.v = to_dev(pack["q"], torch), to_dev(pack["k"], torch), to_dev(pack["v"], torch)
        self.sl = torch.tensor([list(x) for x in slices], dtype=torch.int32, device="cuda")
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
        self.ws = lb.new_workspace(T, 2 * len(slices) + 1, H, Hkv)
        # visible pairs, rectangle by rectangle: row r sees keys lo .. hi of its slice (CAUSAL
        # and BI-CAUSAL bound hi at r + kl - ql, INV-CAUSAL and BI-CAUSAL bound lo at r)
        pairs = 0
        for (qs, ql, ks, kl, kind) in slices:
            r = np.arange(ql)
            hi = np.minimum(kl - 1, r + kl - ql) if kind in (lb.SLICE_CAUSAL, lb.SLICE_BI_CAUSAL) else np.full(ql, kl - 1)
            lo = r if kind in (lb.SLICE_INV_CAUSAL, lb.SLICE_BI_CAUSAL) else np.zeros(ql, dtype=np.int64)
            pairs += int(np.maximum(0, hi - lo + 1).sum())
        self.pairs = pairs
        self.flops = 4 * d * H * pairs

    def n_launches(self):
        return 1

    def run(self, evs=None):
        lb = self.lb
        if evs is not None:
            evs[0][0].record()
        lb.plan_slices(self.sl, self.T, self.T, self.H, self.Hkv, self.d, workspace=self.ws)
        if evs is not None:
            evs[0][1].record()
        (lb.attn_run_lower if self.lower else lb.attn_run)(self.q, self.k, self.v, self.out, self.lse, self.ws)
        if evs is not None:
            evs[0][2].record()

    def plan_pairs(self):
        return sum(t["cost"] for t in self.lb.read_plan(self.ws))

    def worker_ws(self):  # the workspace whose worker records and plan the bench reports
        return self.ws


class ZigzagStep:
    """one zigzag rank's share: cp block steps (plan + attention each) and cp-1 merges."""

    def __init__(self, torch, lb, workloads, rank=3, cp=8, chunk=8192, seed=0, graph=True, overlap=4, ring=True,
                 fused=True):
        self.torch, self.lb = torch, lb
        self.ring = ring
        lengths = workloads.zigzag_pack_lengths(seed)
        cache = {}

        def get_chunk(c):
            if c not in cache:
                cache[c] = workloads.zigzag_chunk_values(c, chunk)
            return cache[c]

        self.share = lb.zigzag.RankShare(lengths, chunk, rank, cp, get_chunk)
        self.share.plan_all()  # allocates the per-step workspaces outside the timed region
        # fused: the live steps as one item per query tile and kv head, no partials, no merges
        self.fused = ring and fused and self.share.fusable
        # the share is replayed from one HIP graph: with ring, the live steps' plans, their
        # merged queue, one attention launch and the merges; without, the per-step attention
        # launches spread over `overlap` streams so that the steps overlap (none: one stream);
        # per-kernel events need eager launches one at a time (run_eager)
        self.streams = [torch.cuda.Stream() for _ in range(overlap)] if overlap and not ring else None
        if self.fused:
            self.share.plan_ring_fused()
        elif ring:
            self.share.plan_ring()
        if not graph:
            self.graph = None
        elif self.fused:
            self.graph = self.share.capture(fused=True)
        else:
            self.graph = self.share.capture(ring=True) if ring else self.share.capture(streams=self.streams)
        if self.fused:
            self.kernel_name = ("attn_kernel<128,true,false,true,true> (persistent, one LPT queue of query tiles, "
                                "each against the keys of every live step; the merged result, no partials)")
        else:
            self.kernel_name = ("attn_kernel<128,true,false,true,false> (persistent, one LPT queue over the live "
                                "steps; fp32 partials)" if ring else
                                "attn_kernel<128,true,false,false,false> (persistent, LPT queue; fp32 partials)")
        self.H, self.d = 32, 128
        # pairs: positions and document ids of the rank's rows against each step's chunks
        pos, doc = lb.zigzag.token_meta(lengths)
        total = 0
        qc = lb.zigzag.chunks_of_rank(rank, cp)
        for t in range(cp):
            kc = lb.zigzag.chunks_of_rank(lb.zigzag.ring_source(rank, t, cp), cp)
            for a in qc:
                for b in kc:
                    qs, ks = slice(a * chunk, (a + 1) * chunk), slice(b * chunk, (b + 1) * chunk)
                    total += int(np.sum((doc[qs][:, None] == doc[ks][None, :]) &
                                        (pos[ks][None, :] <= pos[qs][:, None])))
        self.pairs = total
        self.flops = 4 * self.d * self.H * self.pairs
        self.name = f"zigzag cp={cp} rank {rank}"

    def n_launches(self):
        return 1 if self.ring else len(self.share.live_steps)

    def run(self, evs=None):
        if self.graph is not None and evs is None:
            self.share.replay()
            return
        self.run_eager(evs)

    def run_eager(self, evs=None):
        # one planning launch for all steps (their key/value metadata is known up front),
        # then per step the attention launch and, from step 1 on, the merge; in ring mode
        # the plans are merged and one attention launch runs every step
        lb, sh = self.lb, self.share
        if self.fused:
            if evs is not None:
                evs[0][0].record()
            sh.plan_ring_fused()
            if evs is not None:
                evs[0][1].record()
            live = [sh.steps[t] for t in sh.live_steps]
            lb.ring_attn_run_fused(sh.q, [st["kv"][0] for st in live], [st["kv"][1] for st in live], sh.out, sh.lse,
                                   sh.ring_workspace)
            if evs is not None:
                evs[0][2].record()
            return
        if self.ring:
            if evs is not None:
                evs[0][0].record()
            sh.plan_ring()
            if evs is not None:
                evs[0][1].record()
            sh.ring_attention()
            if evs is not None:
                evs[0][2].record()
            sh.merge_partials()
            return
        if evs is not None:
            evs[0][0].record()
        sh.plan_all()
        if evs is not None:
            evs[0][1].record()
        for i, t in enumerate(sh.live_steps):
            st = sh.steps[t]
            out = sh.out if i == 0 else sh.step_out
            lse = sh.lse if i == 0 else sh.step_lse
            ev = None if evs is None else evs[i]
            if ev is not None and i > 0:
                ev[0].record()
                ev[1].record()
            lb.attn_run(sh.q, st["kv"][0], st["kv"][1], out, lse, sh.step_workspaces[t])
            if ev is not None:
                ev[2].record()
            if i > 0:
                lb.lse_merge(sh.out, sh.lse, sh.step_out, sh.step_lse)

    def plan_pairs(self):
        return None

    def worker_ws(self):  # the workspace whose worker records and plan the bench reports
        if self.ring:
            return self.share.ring_workspace
        return self.share.step_workspaces[self.share.live_steps[0]]


class ZigzagBwdStep(ZigzagStep):
    """The ring backward of the zigzag rank's share: D from the merged forward output, then
    per step the block backward (dq added, the source chunk's partial dk, dv written).
    Effective FLOPs 10 * d * H * pairs, 2.5x the forward's."""

    def __init__(self, torch, lb, workloads, seed=0, ring=True, fused=True):
        super().__init__(torch, lb, workloads, seed=seed, graph=False, overlap=0, ring=False, fused=False)
        self.bwd_ring = ring
        # the dQ side fused per query tile (one launch over every live step) when the share fuses
        self.bwd_fused = ring and fused and self.share.fusable
        sh = self.share
        sh.run_planned()
        r = np.random.default_rng(2001)
        n_q = sh.q.shape[0]
        self.dout = to_dev(workloads.f32_to_bf16_bits(r.standard_normal((n_q, self.H, self.d)).astype(np.float32)),
                           torch)
        sh.backward(self.dout, ring=ring, fused=self.bwd_fused)  # allocates its buffers outside the timed region
        torch.cuda.synchronize()
        self.flops = 10 * self.d * self.H * self.pairs
        self.kernel_name = ("ring backward (D; all steps' plans in one launch, their key-tile plans merged and their "
                            "query-tile plans fused; one bwd_dq_kernel<128,1,true,fused> over every step; one "
                            "bwd_dkv_kernel<128,true,ring> over every step)" if self.bwd_fused else
                            "ring backward (D; all steps' plans in one launch, their key-tile plans merged; "
                            "bwd_dq_kernel<128,1,true> per step; one bwd_dkv_kernel<128,true,ring> over every step)"
                            if ring else "ring backward (D, then per step: plans, bwd_dq_kernel<128,1,true>, "
                            "bwd_dkv_kernel<128,true,false>)")
        self.graph = None

    def n_launches(self):
        return 1

    def run(self, evs=None):
        if evs is not None:
            evs[0][0].record()
            evs[0][1].record()
        self.share.backward(self.dout, ring=self.bwd_ring, fused=self.bwd_fused)
        if evs is not None:
            evs[0][2].record()

    def worker_ws(self):  # the workspace whose worker records and plan the bench reports
        if self.bwd_ring:
            return self.share.bwd_ring_workspace
        return self.share.bwd_buffers["ws"][self.share.live_steps[0]]


class CpJob:
    """Every rank's share of a context-parallel job at cp = 8 over the 131072-token pack,
    one after another on this GPU (each share replayed from its own HIP graph)."""

    def __init__(self, torch, lb, workloads, rule, cp=8, chunk=8192, seed=0, overlap=4, ring=True, fused=True):
        from load_balance_amd import sharding as LS
        self.torch, self.lb = torch, lb
        lengths = workloads.zigzag_pack_lengths(seed)
        parts = [workloads.zigzag_chunk_values(c, chunk) for c in range(2 * cp)]
        q, k, v = (np.concatenate([p[i] for p in parts]) for i in range(3))
        base, n_chunks = LS.parse_rule(rule)
        self.tokens = LS.shard_tokens(base, lengths, cp, n_chunks=n_chunks)
        shards = LS.build_shards(lengths, self.tokens, lambda idx: (q[idx], k[idx], v[idx]))
        self.shares = [LS.ShardedRank(shards, r) for r in range(cp)]
        streams = [torch.cuda.Stream() for _ in range(overlap)] if overlap and not ring else None
        self.ring = ring
        # with ring, a rank whose live steps fuse (ShardedRank.fusable) runs the fused ring
        self.fused_ranks = [r for r, s in enumerate(self.shares) if ring and fused and s.fusable]
        for r, s in enumerate(self.shares):
            if ring:
                s.capture(ring=True, fused=r in self.fused_ranks)
            else:
                s.capture(streams=streams)
        self.H, self.d = 32, 128
        pos_in_doc = np.concatenate([np.arange(n) for n in lengths])
        self.rank_pairs = [int(np.sum(pos_in_doc[t] + 1)) for t in self.tokens]
        self.pairs = sum(self.rank_pairs)
        self.flops = 4 * self.d * self.H * self.pairs
        best, cost = LS.choose_sharding(lengths, cp, 64, rules=CP_RULES)
        self.predicted = {"chosen": best,
                          "rank_us": {r: [round(x, 1) for x in c["us"]] for r, c in cost.items()}}
        self.kernel_name = "attn_kernel<128,true> (persistent, LPT queue; fp32 partials)"
        self.graph = None  # events go around each rank's replay

    def n_launches(self):
        return len(self.shares)

    def run(self, evs=None):
        for r, s in enumerate(self.shares):
            if evs is not None:
                evs[r][0].record()
                evs[r][1].record()
            s.replay()
            if evs is not None:
                evs[r][2].record()

    def plan_pairs(self):
        return None

    def worker_ws(self):  # the workspace whose worker records and plan the bench reports
        if self.ring:
            return self.shares[0].ring_workspace
        return self.shares[0].step_workspaces[self.shares[0].live_steps[0]]


CP_RULES = ("zigzag", "per_document", "dispatch/16", "dispatch/32", "dispatch/64", "dispatch/128")


def make_workload(name, seed, torch, lb, workloads, graph=True, rule="per_document", overlap=4, ring=True,
                  fused=True):
    if name == "longtail":
        p = workloads.longtail_pack(seed)
        w = VarlenStep([p], lb.MASK_CAUSAL_DOC, name, torch, lb)
        w.config = {"workload": f"32K long-tail varlen pack: lognormal lengths (median 644, sigma 1.6), seed {seed}, "
                                "per-document causal mask",
                    "tokens": p["tokens"], "documents": len(p["lengths"]), "max_doc": max(p["lengths"]),
                    "heads": 32, "kv_heads": 8, "head_dim": 128, "seed": seed}
        w.packs = [p]
        return w
    if name in ("pairA", "pairB"):
        a, b = workloads.pair_packs()
        p = a if name == "pairA" else b
        w = VarlenStep([p], lb.MASK_CAUSAL_DOC, name, torch, lb)
        w.config = {"workload": "equal-token pair, " + ("A: one 40960-token document" if name == "pairA"
                                                        else "B: ten 4096-token documents"),
                    "tokens": 40960, "documents": len(p["lengths"]), "heads": 32, "kv_heads": 8, "head_dim": 128}
        w.packs = [p]
        return w
    if name == "shared_question":
        packs = workloads.shared_question_packs()
        w = VarlenStep(packs, lb.MASK_SHARED_QUESTION, name, torch, lb)
        w.config = {"workload": "shared question: 4 packs of one 8192-token question + 8 answers of 4096",
                    "tokens": 4 * 40960, "heads": 32, "kv_heads": 8, "head_dim": 128}
        w.packs = packs
        return w
    if name == "tiny":
        p = workloads.tiny_pack()
        w = VarlenStep([p], lb.MASK_CAUSAL_DOC, name, torch, lb)
        w.config = {"workload": "tiny pack [5,17,42], 2 q heads = 2 kv heads, head_dim 64", "tokens": 64}
        w.packs = [p]
        return w
    if name == "zigzag":
        w = ZigzagStep(torch, lb, workloads, seed=seed, graph=graph, overlap=overlap, ring=ring, fused=fused)
        w.config = {"workload": "one zigzag CP rank's share at cp=8: rank 3 of a 131072-token lognormal pack "
                                f"(seed {seed}), 16 chunks of 8192, 8 ring steps"
                                + (", fused per query tile (each tile against the keys of every live step in one "
                                   "online softmax, the merged result written once)" if w.fused else
                                   " and a merge per step after the first")
                                + "; steps whose chunks hold no key the rank's rows see (5 of 8 here, found on "
                                "the host from positions and document ids) run nothing",
                    "tokens": 16384, "heads": 32, "kv_heads": 8, "head_dim": 128,
                    "launch": ("one HIP graph: the live steps' plans (one launch) fused per query tile into one "
                               "longest-first queue, one attention launch" if w.fused else
                               "one HIP graph: the live steps' plans (one launch) merged into one longest-first "
                               "queue, one attention launch over every live step, merges in step order" if ring else
                               f"one HIP graph: plan, the live steps' attention launches on {overlap} streams, merges "
                               "in step order" if overlap else "one HIP graph, one stream") if graph else "eager"}
        return w
    if name == "blockcausal":
        p = workloads.longtail_pack(seed)
        frame = 256
        sl, start = [], 0
        for n in p["lengths"]:  # every document cut into frames that see it up to their own end
            for f0 in range(0, n, frame):
                fl = min(frame, n - f0)
                sl.append((start + f0, fl, start, f0 + fl, lb.SLICE_FULL))
            start += n
        w = SlicesStep(p, sl, name, torch, lb)
        w.config = {"workload": f"varlen block-causal mask as a slice list: the 32K long-tail pack (seed {seed}), "
                                f"every document in frames of {frame} tokens that see their document up to their "
                                "own end (one FULL slice per frame)",
                    "tokens": p["tokens"], "documents": len(p["lengths"]), "frame": frame, "slices": len(sl),
                    "heads": 32, "kv_heads": 8, "head_dim": 128, "seed": seed}
        return w
    if name == "slidingwindow":
        p = workloads.longtail_pack(seed)
        window, rows = 1024, 64
        sl, start = [], 0
        for n in p["lengths"]:  # causal sliding window per document, as BI-CAUSAL bands of 64 rows
            for q0 in range(0, n, rows):
                ql = min(rows, n - q0)
                k0 = q0 - window + 1
                if k0 >= 0:
                    sl.append((start + q0, ql, start + k0, ql + window - 1, lb.SLICE_BI_CAUSAL))
                elif q0 + ql - window <= 0:
                    sl.append((start + q0, ql, start, q0 + ql, lb.SLICE_CAUSAL))
                else:
                    for i in range(q0, q0 + ql):
                        lo = max(0, i - window + 1)
                        sl.append((start + i, 1, start + lo, i - lo + 1, lb.SLICE_FULL))
            start += n
        w = SlicesStep(p, sl, name, torch, lb)
        w.config = {"workload": f"causal sliding window of {window} keys per document, as a slice list (BI-CAUSAL "
                                f"bands of {rows} rows): the 32K long-tail pack (seed {seed})",
                    "tokens": p["tokens"], "documents": len(p["lengths"]), "window": window, "slices": len(sl),
                    "heads": 32, "kv_heads": 8, "head_dim": 128, "seed": seed}
        w.kernel_name = "attn_kernel<128,false,lower bound> (persistent, LPT queue)"
        return w
    if name == "longtail_bwd":
        p = workloads.longtail_pack(seed)
        w = VarlenBwdStep(p, lb.MASK_CAUSAL_DOC, name, torch, lb)
        w.config = {"workload": f"backward (dq, dk, dv) of the 32K long-tail varlen pack, seed {seed}: "
                                "lb_varlen_attn_bwd from the forward's out and lse and a seeded dout",
                    "tokens": p["tokens"], "documents": len(p["lengths"]), "heads": 32, "kv_heads": 8,
                    "head_dim": 128, "seed": seed, "flop_convention": "10*d*H*pairs (2.5x the forward's)"}
        return w
    if name == "zigzag_bwd":
        w = ZigzagBwdStep(torch, lb, workloads, seed=seed, ring=ring, fused=fused)
        w.config = {"workload": "ring backward of one zigzag CP rank's share at cp=8: rank 3 of a 131072-token "
                                f"lognormal pack (seed {seed}), a block-step backward per step with visible pairs "
                                "(3 of 8: dq accumulated, per-step partial dk, dv) after the forward's merged out and "
                                "lse" + ("; the steps' dK/dV items in one launch from one longest-first queue" if ring
                                         else "; one dK/dV launch per step"),
                    "tokens": 16384, "heads": 32, "kv_heads": 8, "head_dim": 128,
                    "flop_convention": "10*d*H*pairs (2.5x the forward's)"}
        return w
    if name == "cp_job":
        w = CpJob(torch, lb, workloads, rule, seed=seed, overlap=overlap, ring=ring, fused=fused)
        w.config = {"workload": f"context-parallel job at cp=8 over a 131072-token lognormal pack (seed {seed}), "
                                f"{rule} sharding: all 8 ranks' shares (8 ring steps + 7 merges each) in turn",
                    "tokens": 131072, "heads": 32, "kv_heads": 8, "head_dim": 128, "sharding": rule,
                    "rank_pairs_per_head": w.rank_pairs, "fused_ring_ranks": w.fused_ranks,
                    "time_model_prediction": w.predicted}
        return w
    raise SystemExit(f"unknown workload {name}")


# ----------------------------------------------------------------------------------------
# CPU baseline: the oracle, on a bounded sample of the same workload
# ----------------------------------------------------------------------------------------
def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _blas_info():
    try:
        from threadpoolctl import threadpool_info
        return ", ".join(f"{x.get('internal_api')} {x.get('version')}" for x in threadpool_info()
                         if x.get("user_api") == "blas") or None
    except Exception:  # pragma: no cover
        return None


def cpu_baseline(w, seconds, seed=0):
    """The float64 oracle on the host cores, on a bounded sample of the same pack: blocks of up
    to 32 rows of one document (all heads), in a random order that starts over once every
    block has been handed out, fed to a pool of processes, one per core with one BLAS thread
    each, until `seconds` have elapsed; blocks still running then are not counted."""
    import concurrent.futures as cf
    import itertools
    import multiprocessing as mp
    import tempfile
    from oracle import timing as OT
    p = w.packs[0]
    lengths = np.asarray(p["lengths"])
    cu = np.concatenate([[0], np.cumsum(lengths)])
    seg = np.repeat(np.arange(len(lengths)), lengths)
    pos_in_doc = np.arange(p["tokens"]) - cu[seg]
    cores = len(os.sched_getaffinity(0))
    n_proc = max(1, min(cores, 16))  # a GPU machine shares its host: at most 16 processes per GPU
    rb = 32  # rows per task, inside one document
    tasks = [(int(cu[d]), int(lengths[d]), r0, min(r0 + rb, int(lengths[d])))
             for d in range(len(lengths)) for r0 in range(0, int(lengths[d]), rb)]
    order = itertools.cycle(np.random.default_rng(seed).permutation(len(tasks)).tolist())
    done = []
    with tempfile.TemporaryDirectory(dir="/tmp") as tmp:
        paths = {}
        for k in ("q", "k", "v"):
            paths[k] = os.path.join(tmp, k + ".npy")
            np.save(paths[k], p[k])
        meta = dict(cu_seqlens=np.asarray(p["cu_seqlens"]), heads=p["heads"], kv_heads=p["kv_heads"])
        # a worker that fails to start breaks the pool (an error here) rather than being respawned
        with cf.ProcessPoolExecutor(n_proc, mp_context=mp.get_context("spawn"), initializer=OT.init_worker,
                                    initargs=(paths, meta)) as ex:
            list(ex.map(OT.ready, range(n_proc)))  # workers up before the clock starts
            t0 = time.perf_counter()
            inflight = {ex.submit(OT.run_block, *tasks[next(order)]) for _ in range(4 * n_proc)}
            while True:
                finished, inflight = cf.wait(inflight, return_when=cf.FIRST_COMPLETED)
                if time.perf_counter() - t0 >= seconds:
                    break
                for f in finished:
                    done.append(f.result())
                    inflight.add(ex.submit(OT.run_block, *tasks[next(order)]))
            el = time.perf_counter() - t0
            for f in inflight:
                f.cancel()
    pairs = int(sum(np.sum(pos_in_doc[a:a + n] + 1) for a, n in done))
    rows = int(sum(n for _, n in done))
    flops = 4 * p["d"] * p["heads"] * pairs
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(n_proc), "kind": "oracle",
            "host_cpus": cores, "cpu_model": _cpu_model(), "numpy": np.__version__, "blas": _blas_info(),
            "sample": f"{len(done)} blocks of up to {rb} query rows of one document (all {p['heads']} heads) of the "
                      f"{p['tokens']}-token pack, in a random order repeated once exhausted: {rows} rows, "
                      f"{pairs} visible pairs per head = {pairs / causal_pairs(lengths):.2f} x the pack's, "
                      f"float64 numpy, {n_proc} processes x 1 BLAS thread, {el:.1f} s"}


def traffic_entry(config):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they match this kernel,
    planner and queue order."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        h = hashlib.sha256()
        for path in KERNEL_SOURCES:
            with open(path, "rb") as f:
                h.update(f.read())
        if t.get("source_sha256") != h.hexdigest():
            return None
        if t.get("queue_order") != config.get("queue_order") or t.get("lpt_weights") != config.get("lpt_weights"):
            return None
        return t.get("hbm_bytes_per_launch")
    except Exception:
        return None


def cu_balance(recs):
    """Busy time per compute unit from the workgroups' records.  A workgroup's compute unit
    is (XCC_ID, SE_ID, SH_ID, CU_ID) from its HW_ID and XCC_ID registers (gfx9 HW_ID fields:
    CU_ID bits 8-11, SH_ID bit 12, SE_ID bits 13-15); workgroups that shared one compute
    unit add up."""
    per_cu = {}
    for r in recs:
        hw = int(r["hw_id"])
        key = (int(r["xcc_id"]) & 0xF, (hw >> 13) & 0x7, (hw >> 12) & 0x1, (hw >> 8) & 0xF)
        per_cu.setdefault(key, []).append(float(r["t_end"] - r["t_start"]))
    if not per_cu:
        return {"max_over_mean": None}
    busy = np.array([sum(v) for v in per_cu.values()])
    return {"max_over_mean": round(float(busy.max() / busy.mean()), 4) if busy.mean() > 0 else None,
            "compute_units": len(per_cu), "workgroups": len(recs),
            "max_workgroups_on_one_cu": max(len(v) for v in per_cu.values()),
            "unit": "per compute unit, from s_memrealtime stamps"}


def cp_job_fields(w, per_launch):
    """For the context-parallel job: each rank's share time, the makespan if the ranks ran on
    their own GPUs, and the per-GPU throughput that makespan gives."""
    if not isinstance(w, CpJob):
        return {}
    rank_ms = [pl[1] for pl in per_launch]
    makespan = max(rank_ms)
    return {"cp_rank_ms": rank_ms, "cp_makespan_ms": round(makespan, 4),
            "cp_busiest_over_mean": round(makespan / float(np.mean(rank_ms)), 4),
            "cp_tflops_per_gpu_if_parallel": round(w.flops / len(rank_ms) / (makespan / 1e3) / 1e12, 3)}


# ----------------------------------------------------------------------------------------
def dump_worker_records(path, name, w, recs, lb):
    """Per-workgroup busy ticks (100 MHz), pairs, key blocks and items of the last launch,
    with the items of its plan in queue order (the input of ``load_balance_amd.fit_item_cost``)."""
    plan = [dict(cost=int(t["cost"]), blocks=int(t["blocks"]), q_len=int(t["q_len"])) for t in lb.read_plan(w.worker_ws())]
    with open(path, "w") as f:
        json.dump({"workload": name, "config": w.config, "records": recs, "plan": plan}, f)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU needs some tens of launches to reach steady clocks: the first 10 launches of the
    # 32K pack run ~25% slower than launches 50+
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="longtail",
                    choices=["longtail", "pairA", "pairB", "zigzag", "shared_question", "tiny", "copy", "cp_job",
                             "longtail_bwd", "blockcausal", "slidingwindow", "zigzag_bwd"])
    ap.add_argument("--rule", default="per_document", choices=list(CP_RULES),
                    help="cp_job: how the pack is sharded over the ranks")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="zigzag: launch the kernels one by one, no HIP graph")
    ap.add_argument("--no-ring", action="store_true",
                    help="zigzag, cp_job, zigzag_bwd: one attention (dK/dV) launch per live step instead of one over all of them")
    ap.add_argument("--no-fuse", action="store_true",
                    help="zigzag: the ring with a partial per live step and the merges, instead of the ring fused per "
                         "query tile")
    ap.add_argument("--overlap", type=int, default=4,
                    help="zigzag, cp_job with --no-ring: streams the ring steps' attention launches are spread over "
                         "(0: one)")
    ap.add_argument("--lpt-weights", default=None, metavar="blocks|BLOCK,PAIR",
                    help="longtail, pairA, pairB, shared_question: queue the tiles by BLOCK * key blocks + "
                         "PAIR * G * pairs (lb_plan_varlen_weighted; 'blocks' is 1,0) instead of lb_plan_varlen's "
                         "fitted weights")
    ap.add_argument("--order", default=None, choices=["lpt", "documents"],
                    help="longtail, pairA, pairB, shared_question: queue order (lb_plan_varlen_ordered): the tiles "
                         "by their estimate (lpt) or the documents by their largest tile's, each document's tiles "
                         "together (documents, lb_plan_varlen's); with --lpt-weights the default is lpt")
    ap.add_argument("--worker-records", default=None, metavar="PATH",
                    help="write the last launch's per-workgroup records and its plan (JSON) to PATH")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build runs on a single MI355X and has no multi-GPU path "
              "(see DESIGN.md for how the attention would shard). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.workload == "copy":
        # calibration for rocprofv3's FETCH_SIZE / WRITE_SIZE: a plain 1 GiB device copy
        a = torch.ones(1 << 28, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"workload": "copy", "bytes_per_copy": a.numel() * 4, "copies": 3}), flush=True)
        return
    import load_balance_amd as lb
    import workloads

    lb.lib()
    log(f"bench: building workload {args.workload}")
    w = make_workload(args.workload, args.seed, torch, lb, workloads, graph=not args.eager, rule=args.rule,
                      overlap=args.overlap, ring=not args.no_ring, fused=not args.no_fuse)
    if args.lpt_weights is not None:
        if not isinstance(w, VarlenStep):
            sys.exit("--lpt-weights applies to the varlen forward workloads")
        bw, pw = (1, 0) if args.lpt_weights == "blocks" else map(int, args.lpt_weights.split(","))
        w.lpt_weights = (bw, pw)
    if args.order is not None:
        if not isinstance(w, VarlenStep):
            sys.exit("--order applies to the varlen forward workloads")
        w.queue_order = lb.ORDER_LPT if args.order == "lpt" else lb.ORDER_DOCUMENTS
    if isinstance(w, VarlenStep):
        order = w.queue_order if w.queue_order is not None else (lb.ORDER_LPT if w.lpt_weights else lb.ORDER_DOCUMENTS)
        w.config = dict(w.config, lpt_weights=list(w.lpt_weights or (lb.LPT_FIT_BLOCK_WEIGHT, lb.LPT_FIT_PAIR_WEIGHT)),
                        queue_order="documents" if order == lb.ORDER_DOCUMENTS else "lpt")
    graphed = getattr(w, "graph", None) is not None
    torch.cuda.synchronize()

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        w.run()
    torch.cuda.synchronize()
    if w.plan_pairs() is not None:
        assert w.plan_pairs() == w.pairs, "plan pair count differs from the closed form"

    n_launch = w.n_launches()
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_launch)]
           for _ in range(args.steps)]
    log(f"bench: timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        w.run(None if graphed else evs[s])
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms_per_step = el / args.steps * 1e3
    eager_ms_per_step = None
    if graphed:
        # per-kernel times come from more passes of eager launches, outside the timed region: one
        # plain pass for the eager step time, then one with events, each step's launches queued
        # behind a short spin kernel so that the host's launch latency falls before the step's
        # first event rather than between its events (a share whose kernels finish faster than
        # the host enqueues them would otherwise show the host's time as the plan's)
        log(f"bench: {args.steps} eager steps, then {args.steps} with per-kernel events")
        t1 = time.perf_counter()
        for s in range(args.steps):
            w.run_eager(None)
        torch.cuda.synchronize()
        eager_ms_per_step = (time.perf_counter() - t1) / args.steps * 1e3
        for s in range(args.steps):
            torch.cuda._sleep(1_000_000)
            w.run_eager(evs[s])
        torch.cuda.synchronize()
    plan_ms = float(np.mean([sum(e[0].elapsed_time(e[1]) for e in step) for step in evs]))
    attn_ms = float(np.mean([sum(e[1].elapsed_time(e[2]) for e in step) for step in evs]))
    per_launch = [[round(float(np.mean([evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(args.steps)])), 4),
                   round(float(np.mean([evs[s][i][1].elapsed_time(evs[s][i][2]) for s in range(args.steps)])), 4)]
                  for i in range(n_launch)]
    attn_ms_per_launch = attn_ms / n_launch

    recs = lb.read_worker_timing(w.worker_ws())
    if args.worker_records:
        dump_worker_records(args.worker_records, args.workload, w, recs, lb)
    busy = np.array([r["t_end"] - r["t_start"] for r in recs], dtype=np.float64)
    span_ticks = max(r["t_end"] for r in recs) - min(r["t_start"] for r in recs)
    cu = cu_balance(recs)

    value = w.flops / (ms_per_step / 1e3) / 1e12
    achieved = w.flops / (attn_ms / 1e3) / 1e12
    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": dict(w.config, pairs_per_head=w.pairs, effective_flops=w.flops),
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "pct_bf16_peak_at_2400mhz": round(100 * value / PEAK_BF16_AT_2400MHZ, 2),
        "kernels_ms": {"plan": round(plan_ms, 4), "attention": round(attn_ms, 4)},
        "kernels_ms_per_launch": per_launch if n_launch > 1 else None,
        "eager_ms_per_step": None if eager_ms_per_step is None else round(eager_ms_per_step, 4),
        **cp_job_fields(w, per_launch),
        "cu_busy_max_over_mean": cu["max_over_mean"],
        "cu_busy": cu,
        "attention_span_device_clock_ms": round(span_ticks / 1e5, 4),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_entry(w.config) if args.workload == "longtail" else None,
            "traffic_source": (TRAFFIC_SOURCE if args.workload == "longtail" and traffic_entry(w.config) is not None
                               else None),
            "kernel": getattr(w, "kernel_name", "attn_kernel<128,false,false,false> (persistent, longest-first queue)"),
            "launch_ms": round(attn_ms_per_launch, 4),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and hasattr(w, "packs"):
        log(f"bench: cpu baseline (~{args.cpu_seconds:.0f} s of the float64 oracle)")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
