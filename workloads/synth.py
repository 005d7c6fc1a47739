"""Seeded generators for the five attention workloads.

Document lengths follow the long-tail picture drawn in "03 · 长文负载均衡"
(llm-infra-atlas), section 1.1: a production corpus with median length 644
tokens and a tail reaching far beyond it.  We model it as a lognormal with
median 644 and sigma 1.6, one integer draw at a time (round half to even,
at least 1, clipped at ``cap``), truncating the last draw so the pack holds
exactly ``total`` tokens.

Values are standard normal float32 drawn by numpy's PCG64 generator and
rounded to bfloat16 (round to nearest even).  Both the oracle and the HIP
path consume exactly these rounded values.

Nothing here computes attention, masks, tiles, costs or shards.
"""
from __future__ import annotations

import numpy as np

MEDIAN_LEN = 644
SIGMA = 1.6

CONFIGS = {
    1: "tiny pack: docs [5,17,42], 2 q heads = 2 kv heads, d 64",
    2: "32K long-tail pack: lognormal lengths, 32 q / 8 kv heads, d 128",
    3: "equal-token pair: A = 1x40960, B = 10x4096, 32 q / 8 kv heads, d 128",
    4: "zigzag cp=8 rank share of a 131072-token lognormal pack, 32 q / 8 kv heads, d 128",
    5: "shared question: 4 packs of 8192 question + 8x4096 answers, 32 q / 8 kv heads, d 128",
}


def lognormal_lengths(total: int, seed: int, cap: int) -> list[int]:
    """Document lengths summing to exactly ``total``."""
    rng = np.random.default_rng(seed)
    out: list[int] = []
    s = 0
    while s < total:
        x = rng.lognormal(np.log(MEDIAN_LEN), SIGMA)
        n = int(min(cap, max(1, np.rint(x))))
        n = min(n, total - s)
        out.append(n)
        s += n
    return out


def cu_from_lengths(lengths) -> np.ndarray:
    """Exclusive prefix sum of lengths as int32 ``cu_seqlens`` (n+1 entries)."""
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu.astype(np.int32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits.

    Inputs here are finite normals, so NaN payloads are not handled.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def values(rng: np.random.Generator, tokens: int, heads: int, kv_heads: int, d: int):
    """Draw q [T,H,d], k [T,Hkv,d], v [T,Hkv,d] in that order; bf16 bits (uint16)."""
    q = rng.standard_normal((tokens, heads, d), dtype=np.float32)
    k = rng.standard_normal((tokens, kv_heads, d), dtype=np.float32)
    v = rng.standard_normal((tokens, kv_heads, d), dtype=np.float32)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def _pack(lengths, rng, heads, kv_heads, d, **extra):
    tokens = int(sum(lengths))
    q, k, v = values(rng, tokens, heads, kv_heads, d)
    out = dict(lengths=list(lengths), cu_seqlens=cu_from_lengths(lengths), tokens=tokens,
               heads=heads, kv_heads=kv_heads, d=d, q=q, k=k, v=v)
    out.update(extra)
    return out


def tiny_pack():
    """3 documents [5,17,42], Hq = Hkv = 2, d = 64; float32 N(0,1) from seed 1001.

    Also returns the unrounded float32 values under ``q32/k32/v32``.
    """
    lengths = [5, 17, 42]
    rng = np.random.default_rng(1001)
    T = sum(lengths)
    q32 = rng.standard_normal((T, 2, 64), dtype=np.float32)
    k32 = rng.standard_normal((T, 2, 64), dtype=np.float32)
    v32 = rng.standard_normal((T, 2, 64), dtype=np.float32)
    return dict(lengths=lengths, cu_seqlens=cu_from_lengths(lengths), tokens=T,
                heads=2, kv_heads=2, d=64,
                q=f32_to_bf16_bits(q32), k=f32_to_bf16_bits(k32), v=f32_to_bf16_bits(v32),
                q32=q32, k32=k32, v32=v32, mask="causal_doc")


def longtail_pack(seed: int = 0, tokens: int = 32768, heads: int = 32, kv_heads: int = 8, d: int = 128):
    lengths = lognormal_lengths(tokens, seed, cap=tokens)
    return _pack(lengths, np.random.default_rng(1002), heads, kv_heads, d, mask="causal_doc", seed=seed)


def pair_packs(heads: int = 32, kv_heads: int = 8, d: int = 128, tokens: int = 40960, n_short: int = 10):
    """Pack A: one document of ``tokens``; pack B: ``n_short`` equal documents.

    A draws from default_rng([1003, 0]), B from default_rng([1003, 1]).
    """
    a = _pack([tokens], np.random.default_rng([1003, 0]), heads, kv_heads, d, mask="causal_doc")
    b = _pack([tokens // n_short] * n_short, np.random.default_rng([1003, 1]), heads, kv_heads, d,
              mask="causal_doc")
    return a, b


def zigzag_pack_lengths(seed: int = 0, tokens: int = 131072) -> list[int]:
    return lognormal_lengths(tokens, seed, cap=tokens)


def zigzag_chunk_values(chunk: int, chunk_tokens: int = 8192, heads: int = 32, kv_heads: int = 8,
                        d: int = 128):
    """q, k, v (bf16 bits) of one fixed-size chunk of the 131072-token pack.

    Each chunk has its own stream default_rng([1004, chunk]) so that only the
    chunks one rank touches need to be drawn.
    """
    return values(np.random.default_rng([1004, chunk]), chunk_tokens, heads, kv_heads, d)


def shared_question_packs(n_packs: int = 4, question: int = 8192, answers: int = 8, answer_len: int = 4096,
                          heads: int = 32, kv_heads: int = 8, d: int = 128):
    """Packs of one question followed by equal answers; one value stream for all packs."""
    lengths = [question] + [answer_len] * answers
    per = sum(lengths)
    rng = np.random.default_rng(1005)
    q, k, v = values(rng, n_packs * per, heads, kv_heads, d)
    packs = []
    for p in range(n_packs):
        sl = slice(p * per, (p + 1) * per)
        packs.append(dict(lengths=list(lengths), cu_seqlens=cu_from_lengths(lengths), tokens=per,
                          heads=heads, kv_heads=kv_heads, d=d, q=q[sl], k=k[sl], v=v[sl],
                          mask="shared_question"))
    return packs
