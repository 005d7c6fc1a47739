"""Host-side helpers of bench.py (no GPU): per-compute-unit balance from worker records."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def rec(xcc, se, sh, cu, busy):
    return dict(hw_id=(se << 13) | (sh << 12) | (cu << 8) | 5, xcc_id=xcc, t_start=100, t_end=100 + busy)


def test_cu_balance_adds_workgroups_that_share_a_compute_unit():
    b = _bench()
    recs = [rec(0, 0, 0, 1, 10), rec(0, 0, 0, 1, 10), rec(1, 0, 0, 1, 20), rec(0, 1, 0, 1, 20)]
    c = b.cu_balance(recs)
    # three compute units, each busy 20 ticks: two workgroups of 10 share (xcc 0, se 0, sh 0, cu 1)
    assert c["compute_units"] == 3 and c["workgroups"] == 4
    assert c["max_workgroups_on_one_cu"] == 2
    assert c["max_over_mean"] == 1.0


def test_cu_balance_ratio():
    b = _bench()
    c = b.cu_balance([rec(x, 0, 0, 0, busy) for x, busy in enumerate([10, 10, 10, 30])])
    assert c["max_over_mean"] == 2.0 and c["compute_units"] == 4
