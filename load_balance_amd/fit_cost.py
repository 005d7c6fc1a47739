"""Fits the rank time model of ``sharding.TIME_MODEL_US`` to measured rank shares.

    python -m load_balance_amd.fit_cost cp_per_document.json cp_zigzag.json

Each file is one ``bench.py --workload cp_job --rule <rule>`` line (its ``cp_rank_ms``
and sharding rule, on the 131072-token pack of the given seed at cp = 8).  The features
of every rank come from the library's own work estimate (``sharding.rank_work``); the
fit is least squares of rank microseconds on (blocks * kv_heads / CUs, items * kv_heads /
CUs, ring steps with work, 1).
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from load_balance_amd import sharding  # noqa: E402
import workloads  # noqa: E402


def fit(lines, n_cu=256, tile_rows=64):
    rows, times = [], []
    for d in lines:
        cfg = d["config"]
        lengths = workloads.zigzag_pack_lengths(int(cfg.get("seed", 0)))
        rule, n_chunks = sharding.parse_rule(cfg["sharding"])
        tokens = sharding.shard_tokens(rule, lengths, len(d["cp_rank_ms"]), n_chunks=n_chunks)
        for (b, i, s), ms in zip(sharding.rank_work(lengths, tokens, tile_rows), d["cp_rank_ms"]):
            rows.append([b * cfg["kv_heads"] / n_cu, i * cfg["kv_heads"] / n_cu, s, 1.0])
            times.append(ms * 1e3)
    X, y = np.array(rows), np.array(times)
    coef = np.linalg.lstsq(X, y, rcond=None)[0]
    err = float(np.max(np.abs(X @ coef - y) / y))
    return dict(per_block=coef[0], per_item=coef[1], per_step=coef[2], fixed=coef[3]), err


if __name__ == "__main__":
    lines = [json.loads(open(f).read().strip().splitlines()[-1]) for f in sys.argv[1:]]
    model, err = fit(lines)
    print(json.dumps({k: round(float(v), 3) for k, v in model.items()}), f"max relative error {err:.3f}")
