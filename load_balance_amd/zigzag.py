"""Zigzag context-parallel step driver for one rank, on one GPU.

The pages' ring attention ("长序列训练与上下文并行", Ring Attention): each rank
keeps its query shard; at every step it receives the key/value chunks that
started on another rank, runs local attention on them, merges the result into
its running output with the online-softmax merge, and passes the chunks on.
Zigzag sharding ("03 · 长文负载均衡", section 4.2): the sequence is cut into
2*cp chunks and rank i holds chunks i and 2*cp-1-i.

Here one rank's share runs at its real shape on one GPU: the chunks a peer
would have sent are already resident in HBM, and each step is one
``block_attn_fwd`` call followed (after the first) by ``lse_merge``; a step whose
chunks hold no key the rank's rows see runs nothing (``ShardedRank``).  No
collectives are involved.
"""
from __future__ import annotations

import numpy as np
import torch

from .sharding import ShardedRank, live_steps


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


class RankShare(ShardedRank):
    """Device-resident inputs of one rank's cp ring steps under sequence zigzag sharding,
    built chunk by chunk (only the chunks the rank needs are materialised).  The ring
    itself (run, plan_all, run_planned, capture, replay) is ShardedRank's.

    get_chunk(c) -> (q, k, v) of chunk c as bfloat16 bit arrays (uint16 numpy) or bf16 tensors.
    """

    def __init__(self, lengths, chunk_tokens, rank, cp, get_chunk, device="cuda"):
        self.cp, self.rank, self.chunk = cp, rank, chunk_tokens
        self.shared_doc = -1  # per-document causal mask
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
        qpos = np.concatenate([pos[span(c)] for c in qc])
        qdoc = np.concatenate([doc[span(c)] for c in qc])
        self.live_steps = live_steps(qpos, qdoc, [(np.concatenate([pos[span(c)] for c in st["chunks"]]),
                                                   np.concatenate([doc[span(c)] for c in st["chunks"]]))
                                                  for st in self.steps])
        self.step_workspaces = None
        self.graph = None
        self.overlap_buffers = None
        self._set_fusable(qpos, qdoc)
