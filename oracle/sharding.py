"""Context-parallel sharding rules and the sharded ring fold -- TEST INFRASTRUCTURE ONLY
(see ``oracle/__init__``).

Which query tokens each of cp ranks holds:

* Per-sequence zigzag ("03 · 长文负载均衡", section 4.2): the pack is cut into
  2*cp equal chunks and rank i holds chunks i and 2*cp-1-i.
* Per-document sharding ("03 · 长文负载均衡", section 4.3, WLB-LLM): every
  document on its own is cut into 2*cp chunks and rank i takes chunks i and
  2*cp-1-i of every document, so each rank holds the same number of tokens and
  the same causal area of each document; when a length is not a multiple of
  2*cp the remainder is dealt round-robin to the ranks (no padding).
* Striped ("03 · 长文负载均衡", section 4.2, Striped Attention; "长序列训练与上下文并行",
  the zigzag / striped remedy): the pack is dealt out in stripes, stripe s to
  rank s mod cp.
* Mask-area dispatch ("03 · 长文负载均衡", section 4.4, MagiAttention's dispatch
  solver): the pack is cut along the query axis into n equal chunks, each chunk's
  mask area (the (query, key) pairs its queries see) is computed, and the chunks go
  into cp buckets of exactly n/cp chunks each, largest area first, each into the
  bucket that currently holds the least area and is not yet full.

Readings where the pages leave a step open:
* per-document chunk length is floor(len / (2*cp)); the remainder is the last
  len mod 2*cp tokens of the document, and the round-robin deal continues from
  one document to the next (one counter over the whole pack) rather than
  restarting at rank 0, which keeps the ranks' token counts within one;
* the striped rule takes a stripe width (the pages' Striped Attention deals
  single tokens: width 1);
* inside a rank the tokens are kept in ascending global order (the layout of a
  shard does not change its result);
* dispatch ties: chunks of equal area go in chunk order, and of equally loaded
  buckets the lowest-numbered one is taken; the mask is the per-document causal
  one, so a chunk's area is the sum over its tokens of (position in document + 1).

A rank's attention over the whole ring: at step t it attends its query tokens
to the key/value tokens of rank (r - t) mod cp ("长序列训练与上下文并行", Ring
Attention) and folds the partial results with the online-softmax merge.
"""
from __future__ import annotations

import numpy as np

from .attention import _as_f64, block_attention, lse_merge, pack_positions, ring_source


def zigzag_tokens(total: int, cp: int):
    """Per rank, the global token indices of its two zigzag chunks (total divisible by 2*cp)."""
    assert total % (2 * cp) == 0
    c = total // (2 * cp)
    return [np.concatenate([np.arange(i * c, (i + 1) * c), np.arange((2 * cp - 1 - i) * c, (2 * cp - i) * c)])
            for i in range(cp)]


def per_document_tokens(lengths, cp: int):
    """Per rank, the global token indices it holds under per-document sharding."""
    owned = [[] for _ in range(cp)]
    start = 0
    deal = 0  # round-robin pointer for remainder tokens, carried across documents
    for n in lengths:
        n = int(n)
        c = n // (2 * cp)
        for i in range(cp):
            for j in (i, 2 * cp - 1 - i):
                owned[i].extend(range(start + j * c, start + (j + 1) * c))
        for t in range(start + 2 * cp * c, start + n):
            owned[deal].append(t)
            deal = (deal + 1) % cp
        start += n
    return [np.array(sorted(o), dtype=np.int64) for o in owned]


def striped_tokens(total: int, cp: int, width: int = 1):
    """Per rank, the global token indices of stripes r, r + cp, r + 2cp, ... of ``width`` tokens."""
    t = np.arange(total)
    stripe = t // width
    return [t[stripe % cp == r] for r in range(cp)]


def chunk_areas(lengths, n_chunks: int):
    """Mask area of each of n equal query chunks of the pack under the per-document causal
    mask: a token at position p of its document sees p + 1 keys."""
    total = int(sum(int(n) for n in lengths))
    assert total % n_chunks == 0
    size = total // n_chunks
    pos_in_doc = [p for n in lengths for p in range(int(n))]
    return [sum(pos_in_doc[t] + 1 for t in range(c * size, (c + 1) * size)) for c in range(n_chunks)]


def dispatch_chunks(areas, cp: int):
    """The greedy dispatch: per bucket (rank), the ascending list of chunk ids it gets."""
    n = len(areas)
    assert n % cp == 0
    capacity = n // cp
    load, held = [0] * cp, [[] for _ in range(cp)]
    for c in sorted(range(n), key=lambda c: (-areas[c], c)):
        open_buckets = [b for b in range(cp) if len(held[b]) < capacity]
        b = min(open_buckets, key=lambda b: (load[b], b))
        held[b].append(c)
        load[b] += areas[c]
    return [sorted(h) for h in held]


def dispatch_tokens(lengths, cp: int, n_chunks: int):
    """Per rank, the global token indices of the chunks the dispatch gives it."""
    total = int(sum(int(n) for n in lengths))
    size = total // n_chunks
    held = dispatch_chunks(chunk_areas(lengths, n_chunks), cp)
    return [np.concatenate([np.arange(c * size, (c + 1) * size) for c in h]).astype(np.int64) for h in held]


def rank_pairs(lengths, tokens):
    """Visible (query, key) pairs per rank over the whole ring: a query at position p of its
    document sees its document's keys at positions 0..p."""
    pos_in_doc = np.concatenate([np.arange(int(n)) for n in lengths]) if len(lengths) else np.zeros(0, int)
    return [int(np.sum(pos_in_doc[idx] + 1)) for idx in tokens]


def sharded_rank_attention(q, k, v, lengths, tokens, rank, heads, kv_heads, rows=None):
    """One rank's cp ring steps (block attention of its query tokens against every rank's
    key/value tokens in ring order), folded with the online-softmax merge.

    q [T,H,d], k/v [T,H_kv,d] (any float dtype or bf16 bits) of the whole pack; tokens: the
    per-rank index arrays.  Returns (out [n_r,H,d], lse [H,n_r]) in the order of tokens[rank].
    """
    pos, doc = pack_positions(lengths)
    cp = len(tokens)
    qi = tokens[rank]
    qq = _as_f64(q)[qi]
    kk, vv = _as_f64(k), _as_f64(v)
    acc = None
    for t in range(cp):
        ki = tokens[ring_source(rank, t, cp)]
        o, l = block_attention(qq, kk[ki], vv[ki], pos[qi], pos[ki], doc[qi], doc[ki], heads, kv_heads, rows=rows)
        acc = (o, l) if acc is None else lse_merge(acc[0], acc[1], o, l)
    return acc
