"""The oracle timed on the host cores: the CPU baseline the benchmark reports (test
infrastructure, like the rest of this package).

Worker processes each run the oracle (``attention.varlen_attention``, unchanged) on 256-row
blocks of one pack, one BLAS thread per process, the pack's arrays memory-mapped from .npy
files the parent wrote.  Nothing here computes attention itself.
"""
from __future__ import annotations

import numpy as np

_PACK = {}


def init_worker(paths, meta):
    """Process initializer: one BLAS thread, the pack's q, k, v memory-mapped."""
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)
    _PACK.update({k: np.load(v, mmap_mode="r") for k, v in paths.items()})
    _PACK.update(meta)


def ready(_=None):
    """A no-op the parent maps over the pool so that every worker has started."""
    return bool(_PACK)


def run_block(doc_start, doc_len, r0, r1):
    """The oracle on rows [r0, r1) of the document at [doc_start, doc_start + doc_len) of the
    pack, all heads: the document's own arrays with cu_seqlens [0, doc_len], which is the same
    computation as over the whole pack (a row sees only its own document)."""
    from .attention import varlen_attention
    p = _PACK
    sl = slice(doc_start, doc_start + doc_len)
    varlen_attention(p["q"][sl], p["k"][sl], p["v"][sl], np.array([0, doc_len]), p["heads"], p["kv_heads"],
                     rows=np.arange(r0, r1))
    return doc_start + r0, r1 - r0
