"""Fits the cost of one attention work item from the kernel's own per-workgroup records.

    python -m load_balance_amd.fit_item_cost records_longtail.json records_pairB.json ...

Each file is what ``bench.py --workload <name> --worker-records <file>`` writes: for every
persistent workgroup of the last launch its busy ticks (the 100 MHz device clock), the
query-head pairs, key blocks and items it ran, and the plan's items in queue order.

The kernel does a whole key block for any block the mask touches ("03 · 长文负载均衡",
section 3.3, a short block billed as a whole tile), so the key-block count carries most of
an item's time.  The pages sort by a time estimate from a fitted cost model ("数据并行负载
均衡", sections 4.2 to 4.4); this fits one to the kernel.  The fit is least squares of a
workgroup's busy microseconds on (pairs, blocks, items, 1): the per-pair term is the part
of the cost that the partial blocks on a causal diagonal save or not, the per-item term
the prologue and epilogue of an item, the constant the workgroup's start and drain.

Since every workgroup pops from a shared queue, a per-item constant shifts every item's
key alike and cannot change a longest-first order; only the ratio of the block and pair
terms can.  That ratio, as integer weights, is what lb_plan_varlen_weighted takes (the
library's default, LB_LPT_FIT_BLOCK_WEIGHT : LB_LPT_FIT_PAIR_WEIGHT = 41515 : 1, came from
this fit).  The report gives, per workload, the makespan over mean busy time predicted by
list scheduling under the fitted costs for the recorded plan's order and for the order by
the new fit, next to the measured max/mean of the workgroups' busy time.
"""
from __future__ import annotations

import heapq
import json
import sys

import numpy as np

TICKS_PER_US = 100.0
XCDS = 8


def features(rec):
    return [float(rec["pairs"]), float(rec["blocks"]), float(rec["items"]), 1.0]


def fit(files):
    X, y = [], []
    for d in files:
        for r in d["records"]:
            X.append(features(r))
            y.append((r["t_end"] - r["t_start"]) / TICKS_PER_US)
    X, y = np.array(X), np.array(y)
    coef, *_ = np.linalg.lstsq(X, y, rcond=None)
    pred = X @ coef
    ss_res = float(np.sum((y - pred) ** 2))
    ss_tot = float(np.sum((y - y.mean()) ** 2))
    return dict(per_pair_us=coef[0], per_block_us=coef[1], per_item_us=coef[2], per_workgroup_us=coef[3]), \
        dict(r2=1.0 - ss_res / ss_tot if ss_tot > 0 else 1.0, max_rel_err=float(np.max(np.abs(pred - y) / y)))


def list_schedule(times, workers):
    """Makespan and mean load when ``workers`` take items in the given order, each taking the
    next item when it becomes free (the persistent kernel's queue)."""
    free = [0.0] * workers
    heapq.heapify(free)
    for t in times:
        heapq.heappush(free, heapq.heappop(free) + t)
    return max(free), sum(times) / workers


def compare_orders(d, m):
    """Predicted max/mean busy under the plan's order and under the fitted-cost order.  Every
    XCD's queue holds the plan once per kv head it serves and is drained by that XCD's
    workgroups; the per-workgroup constant is added to every workgroup."""
    n_wg = len(d["records"])
    kv_heads = int(d["config"].get("kv_heads", XCDS))
    per_xcd_wg = max(1, n_wg // XCDS) if kv_heads % XCDS == 0 else n_wg
    reps = kv_heads // XCDS if kv_heads % XCDS == 0 else kv_heads
    group = int(d["config"].get("heads", kv_heads)) // kv_heads
    cost = [m["per_pair_us"] * t["cost"] * group + m["per_block_us"] * t["blocks"]
            + m["per_item_us"] for t in d["plan"]]
    out = {}
    for name, order in (("plan", list(range(len(cost)))),
                        ("fitted", sorted(range(len(cost)), key=lambda i: -cost[i]))):
        times = [cost[i] for i in order for _ in range(reps)]
        mk, mean = list_schedule(times, per_xcd_wg)
        out[name] = (mk + m["per_workgroup_us"]) / (mean + m["per_workgroup_us"])
    busy = np.array([(r["t_end"] - r["t_start"]) for r in d["records"]], dtype=np.float64)
    out["measured"] = float(busy.max() / busy.mean())
    out["reordered_items"] = sum(1 for a, b in zip(range(len(cost)), sorted(range(len(cost)), key=lambda i: -cost[i]))
                                 if a != b)
    return out


if __name__ == "__main__":
    files = [json.load(open(f)) for f in sys.argv[1:]]
    model, quality = fit(files)
    print(json.dumps({k: round(float(v), 5) for k, v in model.items()}),
          f"R^2 {quality['r2']:.4f}, max relative error {quality['max_rel_err']:.3f}")
    if model["per_pair_us"] > 0:
        print(f"LPT weights (block, pair): ({round(model['per_block_us'] / model['per_pair_us'])}, 1)")
    for f, d in zip(sys.argv[1:], files):
        c = compare_orders(d, model)
        print(f"{d['workload']:>16}: max/mean busy measured {c['measured']:.4f}, predicted plan order "
              f"{c['plan']:.4f}, order by this fit {c['fitted']:.4f} ({c['reordered_items']} items move)")
