"""Writes the stored fixtures under tests/golden/ that are not page numbers.

Calls only the seeded input generators (``workloads``) and the oracle.
Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import workloads  # noqa: E402
from oracle import plan  # noqa: E402


def main():
    lengths = {f"longtail_seed{s}": workloads.lognormal_lengths(32768, s, 32768) for s in range(5)}
    lengths["zigzag_pack_seed0"] = workloads.zigzag_pack_lengths(0)
    with open(os.path.join(HERE, "workload_lengths.json"), "w") as f:
        json.dump({"_about": "document lengths drawn by workloads.lognormal_lengths (inputs, not results)",
                   **lengths}, f, indent=1)

    pairs = {}
    for name, ls in lengths.items():
        if name.startswith("longtail"):
            pairs[name] = plan.total_pairs(plan.tiles(plan.fragments_varlen(workloads.cu_from_lengths(ls)), 64))
    pairs["pair_A"] = plan.total_pairs(plan.tiles(plan.fragments_varlen([0, 40960]), 64))
    pairs["pair_B"] = plan.total_pairs(plan.tiles(
        plan.fragments_varlen(workloads.cu_from_lengths([4096] * 10)), 64))
    sq = workloads.cu_from_lengths([8192] + [4096] * 8)
    pairs["shared_question_pack"] = plan.total_pairs(plan.tiles(plan.fragments_varlen(sq, "shared_question"), 64))
    with open(os.path.join(HERE, "oracle_pairs.json"), "w") as f:
        json.dump({"_about": "visible (query, key) pairs per head, from oracle.plan", **pairs}, f, indent=1)


if __name__ == "__main__":
    main()
