"""Zigzag context-parallel step driver for one rank, on one GPU.

The pages' ring attention ("长序列训练与上下文并行", Ring Attention): each rank
keeps its query shard; at every step it receives the key/value chunks that
started on another rank, runs local attention on them, merges the result into
its running output with the online-softmax merge, and passes the chunks on.
Zigzag sharding ("03 · 长文负载均衡", section 4.2): the sequence is cut into
2*cp chunks and rank i holds chunks i and 2*cp-1-i.

Here one rank's share runs at its real shape on one GPU: the chunks a peer
would have sent are already resident in HBM, and each step is one
``block_attn_fwd`` call followed (from step 1 on) by ``lse_merge``.  No
collectives are involved.
"""
from __future__ import annotations

import numpy as np
import torch


def chunks_of_rank(rank: int, cp: int):
    return (rank, 2 * cp - 1 - rank)


def ring_source(rank: int, step: int, cp: int) -> int:
    """Rank whose chunks this rank works on at ``step`` (received from the previous rank)."""
    return (rank - step) % cp


def token_meta(lengths):
    """Global position and document id (int32) of every token of a packed sequence."""
    lengths = np.asarray(lengths, dtype=np.int64)
    total = int(lengths.sum())
    pos = np.arange(total, dtype=np.int32)
    doc = np.repeat(np.arange(len(lengths), dtype=np.int32), lengths)
    return pos, doc


class RankShare:
    """Device-resident inputs of one rank's cp ring steps.

    get_chunk(c) -> (q, k, v) of chunk c as bfloat16 bit arrays (uint16 numpy) or bf16 tensors.
    """

    def __init__(self, lengths, chunk_tokens, rank, cp, get_chunk, device="cuda"):
        self.cp, self.rank, self.chunk = cp, rank, chunk_tokens
        pos, doc = token_meta(lengths)
        assert len(pos) == 2 * cp * chunk_tokens, "pack length must be 2*cp*chunk_tokens"

        def bf16(x):
            if isinstance(x, torch.Tensor):
                return x.to(device=device, dtype=torch.bfloat16)
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)

        def span(c):
            return slice(c * chunk_tokens, (c + 1) * chunk_tokens)

        qc = chunks_of_rank(rank, cp)
        self.q_chunks = qc
        self.q = torch.cat([bf16(get_chunk(c)[0]) for c in qc]).contiguous()
        self.q_pos = torch.from_numpy(np.concatenate([pos[span(c)] for c in qc])).to(device)
        self.q_doc = torch.from_numpy(np.concatenate([doc[span(c)] for c in qc])).to(device)
        self.steps = []
        for t in range(cp):
            kc = chunks_of_rank(ring_source(rank, t, cp), cp)
            k = torch.cat([bf16(get_chunk(c)[1]) for c in kc])
            v = torch.cat([bf16(get_chunk(c)[2]) for c in kc])
            kv = torch.stack([k, v]).contiguous()
            self.steps.append(dict(
                chunks=kc, kv=kv,
                kv_pos=torch.from_numpy(np.concatenate([pos[span(c)] for c in kc])).to(device),
                kv_doc=torch.from_numpy(np.concatenate([doc[span(c)] for c in kc])).to(device)))
        n_q, H, d = self.q.shape
        self.out = torch.empty((n_q, H, d), dtype=torch.float32, device=device)
        self.lse = torch.empty((H, n_q), dtype=torch.float32, device=device)
        self.step_out = torch.empty_like(self.out)
        self.step_lse = torch.empty_like(self.lse)
        from . import new_workspace
        n_kv = self.steps[0]["kv"].shape[1]
        # runs per side: at most one per document piece in each of the two chunks
        runs = int(min(max(n_q, n_kv), 2 * len(lengths) + 2))
        self.workspace = new_workspace(max(n_q, n_kv), runs, H, self.steps[0]["kv"].shape[2], device)
        self._ws_shape = (max(n_q, n_kv), runs, H, self.steps[0]["kv"].shape[2], device)
        self.step_workspaces = None

    def run(self, stream=None, per_step=None):
        """All cp steps plus cp-1 merges; returns (out fp32 [n_q,H,d], lse [H,n_q])."""
        from . import block_attn_fwd, lse_merge
        for t, st in enumerate(self.steps):
            first = t == 0
            out = self.out if first else self.step_out
            lse = self.lse if first else self.step_lse
            block_attn_fwd(self.q, st["kv"], self.q_pos, st["kv_pos"], self.q_doc, st["kv_doc"], out=out, lse=lse,
                           workspace=self.workspace, stream=stream)
            if per_step is not None:
                per_step(t, out, lse)
            if not first:
                lse_merge(self.out, self.lse, self.step_out, self.step_lse, stream=stream)
        return self.out, self.lse

    def plan_all(self, stream=None):
        """Plans every ring step in one launch, one workspace per step: a step's key/value
        positions and document ids follow from the packing, before its chunk arrives."""
        from . import new_workspace, plan_block_steps
        if self.step_workspaces is None:
            self.step_workspaces = [new_workspace(*self._ws_shape) for _ in self.steps]
        n_q, H, d = self.q.shape
        plan_block_steps(self.q_pos, self.q_doc, [st["kv_pos"] for st in self.steps],
                         [st["kv_doc"] for st in self.steps], H, self.steps[0]["kv"].shape[2], d,
                         self.step_workspaces, stream=stream)

    def run_planned(self, stream=None, per_step=None):
        """run() with the plans of all steps made up front by plan_all(): one planning launch,
        then per step the attention launch and (from step 1 on) the merge."""
        from . import attn_run, lse_merge
        self.plan_all(stream)
        for t, st in enumerate(self.steps):
            first = t == 0
            out = self.out if first else self.step_out
            lse = self.lse if first else self.step_lse
            attn_run(self.q, st["kv"][0], st["kv"][1], out, lse, self.step_workspaces[t], stream=stream)
            if per_step is not None:
                per_step(t, out, lse)
            if not first:
                lse_merge(self.out, self.lse, self.step_out, self.step_lse, stream=stream)
        return self.out, self.lse

    def capture(self, stream=None):
        """Captures run_planned() -- one planning launch, cp attention launches and cp - 1
        merges -- into a HIP graph, so that replay() launches the whole share at once.
        Every kernel of the share is safe to replay: the planner resets the queue heads
        and the attention kernel rewinds them, and nothing in it clears memory with a
        memset node."""
        self.run_planned(stream=stream)  # allocates the step workspaces, caches the CU count
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run_planned()
        torch.cuda.synchronize()
        self.graph = g
        return g

    def replay(self):
        """One launch of the captured share; returns (out, lse), written in place."""
        self.graph.replay()
        return self.out, self.lse
