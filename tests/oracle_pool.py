"""Every-row parity at full size: the oracle's rows are split over a pool of CPU processes.

The GPU result is saved to .npy files; each worker regenerates the seeded workload itself
(nothing large crosses the pipe), computes the float64 oracle on its share of the rows and
compares them with the saved rows, returning only the error statistics.  Workers are
spawned (a fresh interpreter that never imports torch or touches the GPU).
"""
from __future__ import annotations

import multiprocessing as mp
import os
import time

import numpy as np


def _stats(out, lse, ref_o, ref_l):
    out = np.asarray(out, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    d = np.abs(out - ref_o)
    dl = np.abs(lse - ref_l)
    return dict(out_max=float(d.max()), out_sum=float(d.sum()), n=int(d.size), lse_max=float(dl.max()),
                finite=bool(np.isfinite(out).all() and np.isfinite(lse).all()))


_CACHE = {}  # per worker process: the regenerated workload, reused across its row ranges


def _longtail_rows(args):
    out_path, lse_path, seed, r0, r1 = args
    import workloads
    from oracle import attention as OA
    if ("longtail", seed) not in _CACHE:
        _CACHE[("longtail", seed)] = workloads.longtail_pack(seed)
    p = _CACHE[("longtail", seed)]
    rows = np.arange(r0, r1)
    ref_o, ref_l = OA.varlen_attention(p["q"], p["k"], p["v"], p["cu_seqlens"], p["heads"], p["kv_heads"], rows=rows)
    out = np.load(out_path, mmap_mode="r")[r0:r1]
    lse = np.load(lse_path, mmap_mode="r")[:, r0:r1]
    return r1 - r0, _stats(out, lse, ref_o, ref_l)


def _zigzag_rows(args):
    out_path, lse_path, seed, rank, cp, chunk, r0, r1 = args
    import workloads
    from oracle import attention as OA
    lengths = workloads.zigzag_pack_lengths(seed)

    def get_chunk(c):
        if ("zigzag", c, chunk) not in _CACHE:
            _CACHE[("zigzag", c, chunk)] = workloads.zigzag_chunk_values(c, chunk_tokens=chunk)
        return _CACHE[("zigzag", c, chunk)]

    rows = np.arange(r0, r1)
    ref_o, ref_l, _ = OA.zigzag_rank_attention(get_chunk, lengths, chunk, rank, cp, 32, 8, rows=rows)
    out = np.load(out_path, mmap_mode="r")[r0:r1]
    lse = np.load(lse_path, mmap_mode="r")[:, r0:r1]
    return r1 - r0, _stats(out, lse, ref_o, ref_l)


def _one_thread():
    """Each worker runs its BLAS on one thread; the pool supplies the parallelism."""
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def _run(fn, jobs, say):
    n_proc = max(1, min(16, len(os.sched_getaffinity(0)), len(jobs)))
    say(f"  oracle over {len(jobs)} row ranges on {n_proc} processes")
    ctx = mp.get_context("spawn")
    total = dict(out_max=0.0, out_sum=0.0, n=0, lse_max=0.0, finite=True)
    t0 = time.time()
    done_rows = 0
    with ctx.Pool(n_proc, initializer=_one_thread) as pool:
        for i, (nrows, st) in enumerate(pool.imap_unordered(fn, jobs)):
            done_rows += nrows
            total["out_max"] = max(total["out_max"], st["out_max"])
            total["out_sum"] += st["out_sum"]
            total["n"] += st["n"]
            total["lse_max"] = max(total["lse_max"], st["lse_max"])
            total["finite"] &= st["finite"]
            say(f"    {i + 1}/{len(jobs)} ranges ({done_rows} rows, {time.time() - t0:.0f} s): "
                f"out max {total['out_max']:.3e}, lse max {total['lse_max']:.3e}")
    total["out_mean"] = total["out_sum"] / max(total["n"], 1)
    return total


def balanced_ranges(lengths, n_ranges):
    """Row ranges of about equal oracle work: a row costs the length of its document (the
    oracle builds the explicit mask over the whole document for every row block)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cost = np.repeat(lengths, lengths).astype(np.float64)
    c = np.cumsum(cost)
    cuts = np.searchsorted(c, np.linspace(0, c[-1], n_ranges + 1)[1:-1])
    bounds = np.unique(np.concatenate([[0], cuts, [len(cost)]]))
    return [(int(a), int(b)) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]


def longtail_every_row(out, lse, seed, tmpdir, say):
    """out [T,H,d] (float32 numpy), lse [H,T]: every row of the 32K long-tail pack."""
    import workloads
    op, lp = os.path.join(tmpdir, "out.npy"), os.path.join(tmpdir, "lse.npy")
    np.save(op, np.ascontiguousarray(out, dtype=np.float32))
    np.save(lp, np.ascontiguousarray(lse, dtype=np.float32))
    lengths = workloads.lognormal_lengths(32768, seed, 32768)
    jobs = [(op, lp, seed, a, b) for a, b in balanced_ranges(lengths, 64)]
    return _run(_longtail_rows, jobs, say)


def zigzag_every_row(out, lse, seed, rank, cp, chunk, tmpdir, say):
    """out [n_q,H,d], lse [H,n_q] of one zigzag rank's share: every row."""
    op, lp = os.path.join(tmpdir, "out.npy"), os.path.join(tmpdir, "lse.npy")
    np.save(op, np.ascontiguousarray(out, dtype=np.float32))
    np.save(lp, np.ascontiguousarray(lse, dtype=np.float32))
    n_q = out.shape[0]
    step = 512
    jobs = [(op, lp, seed, rank, cp, chunk, a, min(a + step, n_q)) for a in range(0, n_q, step)]
    return _run(_zigzag_rows, jobs, say)

