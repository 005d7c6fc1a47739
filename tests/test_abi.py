"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before anything reaches a GPU (no device needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import load_balance_amd as lb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lbattn.h")
LB_OK, LB_EINVAL, LB_EUNSUPPORTED, LB_EWORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x100000)  # aligned, never dereferenced by the host checks


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(lb.LIB_PATH):
        from load_balance_amd import build
        build.build()
    return lb.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lb_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert {"lb_varlen_attn_fwd", "lb_block_attn_fwd", "lb_lse_merge"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", lb.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (lb_\w+)", out))
    assert set(names) <= exported, set(names) - exported
    for n in names:
        getattr(L, n)


def test_struct_sizes_match_header(L):
    # the library asserts the same sizes (lbattn_internal.h): 96 and 40 bytes
    assert ctypes.sizeof(lb.PlanTile) == 96
    assert lb.PlanTile.k_lo.offset == lb.PlanTile.k_start.offset + 12 * lb.MAX_SPANS
    assert ctypes.sizeof(lb.WorkerRecord) == 40


def test_status_strings(L):
    assert L.lb_status_string(0) == b"ok"
    assert b"workspace" in L.lb_status_string(3)
    assert L.lb_status_string(99) == b"unknown status"


def test_tile_rows(L):
    assert L.lb_tile_rows(32, 8, 128) == 64
    assert L.lb_tile_rows(2, 2, 64) == 256
    assert L.lb_tile_rows(16, 8, 128) == 128
    assert L.lb_tile_rows(64, 8, 128) == 32
    assert L.lb_tile_rows(24, 8, 128) == -1   # G = 3
    assert L.lb_tile_rows(32, 8, 96) == -1


def test_workspace_bytes(L):
    a = L.lb_workspace_bytes(32768, 30, 32, 8)
    b = L.lb_workspace_bytes(65536, 30, 32, 8)
    c = L.lb_workspace_bytes(32768, 300, 32, 8)
    assert 0 < a < b and a < c and a % 256 == 0
    assert L.lb_workspace_bytes(-1, 1, 32, 8) == 0
    assert L.lb_workspace_bytes(10, 0, 32, 8) == 0
    assert L.lb_workspace_bytes(10, 1, 30, 8) == 0


def varlen(L, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, cu=FAKE, n_seg=3, T=64, H=2, Hkv=2, d=64, mask=0, out=FAKE, lse=FAKE,
                ws=FAKE, ws_bytes=1 << 20, stream=None)
    args.update(kw)
    return L.lb_varlen_attn_fwd(args["q"], args["k"], args["v"], args["cu"], args["n_seg"], args["T"], args["H"],
                                args["Hkv"], args["d"], args["mask"], args["out"], args["lse"], args["ws"],
                                args["ws_bytes"], args["stream"])


def test_varlen_host_checks(L):
    assert varlen(L, q=None) == LB_EINVAL
    assert varlen(L, cu=None) == LB_EINVAL
    assert varlen(L, ws=None) == LB_EINVAL
    assert varlen(L, n_seg=0) == LB_EINVAL
    assert varlen(L, T=-1) == LB_EINVAL
    assert varlen(L, H=3, Hkv=2) == LB_EINVAL
    assert varlen(L, mask=2) == LB_EINVAL
    assert varlen(L, d=96) == LB_EUNSUPPORTED
    assert varlen(L, H=6, Hkv=2) == LB_EUNSUPPORTED
    assert varlen(L, q=ctypes.c_void_p(0x100008)) == LB_EINVAL          # 16-byte alignment
    assert varlen(L, ws=ctypes.c_void_p(0x100010)) == LB_EWORKSPACE     # 256-byte alignment
    need = L.lb_workspace_bytes(64, 3, 2, 2)
    assert varlen(L, ws_bytes=need - 1) == LB_EWORKSPACE
    assert varlen(L, T=1 << 22, n_seg=1, H=32, Hkv=8, d=128, ws_bytes=1 << 30) == LB_EUNSUPPORTED  # > sort capacity
    assert varlen(L, T=0, ws_bytes=need) == LB_OK                        # nothing to do, nothing enqueued


def test_noalloc_host_checks(L):
    """The allocation-free forward's host checks: nothing reaches the device (there is none)."""
    def call(n_seg=3, T=64, H=2, Hkv=2, d=64):
        return L.lb_varlen_attn_fwd_noalloc(FAKE, FAKE, FAKE, FAKE, n_seg, T, H, Hkv, d, 0, FAKE, FAKE, None)
    assert call(n_seg=0) == LB_EINVAL
    assert call(T=-1) == LB_EINVAL
    assert call(H=3, Hkv=2) == LB_EINVAL
    assert call(d=96) == LB_EUNSUPPORTED
    assert call(T=1 << 22, n_seg=1, H=32, Hkv=8, d=128) == LB_EUNSUPPORTED  # > sort capacity
    # every plan within the sort capacity fits the scratch array
    assert L.lb_workspace_bytes(32768 * 64, 32768, 32, 8) <= lb.NOALLOC_SCRATCH_BYTES


def test_block_host_checks(L):
    def call(**kw):
        a = dict(q=FAKE, n_q=128, kv=FAKE, n_kv=128, qp=FAKE, kp=FAKE, qd=FAKE, kd=FAKE, H=32, Hkv=8, d=128,
                 shared=-1, out=FAKE, lse=FAKE, ws=FAKE, ws_bytes=1 << 20)
        a.update(kw)
        return L.lb_block_attn_fwd(a["q"], a["n_q"], a["kv"], a["n_kv"], a["qp"], a["kp"], a["qd"], a["kd"], a["H"],
                                   a["Hkv"], a["d"], a["shared"], a["out"], a["lse"], a["ws"], a["ws_bytes"], None)
    assert call(q=None) == LB_EINVAL
    assert call(shared=-2) == LB_EINVAL
    assert call(kv=None) == LB_EINVAL
    assert call(n_q=-1) == LB_EINVAL
    assert call(d=80) == LB_EUNSUPPORTED
    assert call(ws_bytes=100) == LB_EWORKSPACE
    assert call(n_q=0) == LB_OK
    assert call(n_q=0, kv=None, n_kv=0) == LB_OK


def test_lse_merge_parts_host_checks(L):
    """Argument errors of lb_lse_merge_parts, all caught on the host before any launch."""
    P = ctypes.c_void_p
    arr = lambda *xs: (P * len(xs))(*xs)
    A, B = 0x100000, 0x200000  # aligned, never dereferenced by the host checks
    outs, lses = arr(A, B), arr(A + 0x1000, B + 0x1000)
    M = L.lb_lse_merge_parts
    assert M(outs, lses, 1, 100, 4, 128, None) == LB_EINVAL
    assert M(outs, lses, 17, 100, 4, 128, None) == LB_EINVAL
    assert M(None, lses, 2, 100, 4, 128, None) == LB_EINVAL
    assert M(arr(A, A), lses, 2, 100, 4, 128, None) == LB_EINVAL  # one buffer twice
    assert M(arr(A, None), lses, 2, 100, 4, 128, None) == LB_EINVAL
    assert M(outs, lses, 2, 100, 4, 6, None) == LB_EUNSUPPORTED
    assert M(arr(A, B + 4), lses, 2, 100, 4, 128, None) == LB_EINVAL  # misaligned
    assert M(outs, lses, 2, -1, 4, 128, None) == LB_EINVAL
    assert M(outs, lses, 2, 0, 4, 128, None) == LB_OK  # nothing to merge, nothing launched


def test_split_host_checks(L):
    n = 64
    need = L.lb_workspace_bytes(n, 3, 2, 2)
    assert L.lb_plan_varlen(None, 3, n, 2, 2, 64, 0, FAKE, need, None) == LB_EINVAL
    assert L.lb_plan_varlen(FAKE, 3, n, 2, 2, 64, 5, FAKE, need, None) == LB_EINVAL
    assert L.lb_plan_varlen(FAKE, 3, n, 2, 2, 64, 0, FAKE, need - 1, None) == LB_EWORKSPACE
    assert L.lb_plan_varlen(FAKE, 3, n, 2, 2, 48, 0, FAKE, need, None) == LB_EUNSUPPORTED
    W = L.lb_plan_varlen_weighted
    assert W(FAKE, 3, n, 2, 2, 64, 0, 0, 0, FAKE, need, None) == LB_EINVAL  # block weight 0
    assert W(FAKE, 3, n, 2, 2, 64, 0, 1 << 24, 0, FAKE, need, None) == LB_EINVAL
    assert W(FAKE, 3, n, 2, 2, 64, 0, 1, 1 << 16, FAKE, need, None) == LB_EINVAL
    assert W(None, 3, n, 2, 2, 64, 0, 1, 0, FAKE, need, None) == LB_EINVAL
    assert W(FAKE, 3, n, 2, 2, 64, 0, 41515, 1, FAKE, need - 1, None) == LB_EWORKSPACE
    assert W(FAKE, 3, n, 2, 2, 48, 0, 41515, 1, FAKE, need, None) == LB_EUNSUPPORTED
    O = L.lb_plan_varlen_ordered
    for order in (-1, 2):
        assert O(FAKE, 3, n, 2, 2, 64, 0, 41515, 1, order, FAKE, need, None) == LB_EINVAL
    assert O(FAKE, 3, n, 2, 2, 64, 0, 0, 1, 1, FAKE, need, None) == LB_EINVAL  # block weight 0
    assert O(FAKE, 3, n, 2, 2, 64, 0, 1, 1 << 16, 0, FAKE, need, None) == LB_EINVAL
    assert O(None, 3, n, 2, 2, 64, 0, 1, 0, 1, FAKE, need, None) == LB_EINVAL
    assert O(FAKE, 3, n, 2, 2, 64, 0, 41515, 1, 1, FAKE, need - 1, None) == LB_EWORKSPACE
    assert O(FAKE, 3, n, 2, 2, 48, 0, 41515, 1, 0, FAKE, need, None) == LB_EUNSUPPORTED
    assert L.lb_plan_block(None, FAKE, n, FAKE, FAKE, n, 2, 2, 64, -1, FAKE, need, None) == LB_EINVAL
    assert L.lb_plan_block(FAKE, FAKE, n, FAKE, FAKE, n, 2, 2, 64, -2, FAKE, need, None) == LB_EINVAL
    assert L.lb_plan_block(FAKE, FAKE, n, FAKE, FAKE, n, 2, 2, 64, -1, FAKE, 64, None) == LB_EWORKSPACE
    assert L.lb_attn_run(FAKE, FAKE, FAKE, n, n, 2, 2, 64, 0, None, FAKE, FAKE, need, None) == LB_EINVAL
    assert L.lb_attn_run(FAKE, None, FAKE, n, n, 2, 2, 64, 0, FAKE, FAKE, FAKE, need, None) == LB_EINVAL
    assert L.lb_attn_run(FAKE, FAKE, FAKE, n, n, 2, 2, 64, 0, FAKE, FAKE, FAKE, 100, None) == LB_EWORKSPACE
    assert L.lb_attn_run(FAKE, FAKE, FAKE, 0, n, 2, 2, 64, 0, FAKE, FAKE, FAKE, need, None) == LB_OK


def test_plan_steps_host_checks(L):
    n = 64
    need = L.lb_workspace_bytes(n, 3, 2, 2)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    arr = lambda t, xs: (t * len(xs))(*xs)
    two = [P(0x100000), P(0x200000)]

    def call(n_steps=2, ws=two, sizes=(need, need), kv=(FAKE, FAKE), n_kv=(n, n), d=64, q_pos=FAKE):
        return L.lb_plan_block_steps(q_pos, FAKE, n, arr(P, kv), arr(P, kv), arr(I32, n_kv), n_steps, 2, 2, d, -1,
                                     arr(P, ws), arr(SZ, sizes), None)
    assert call(n_steps=0) == LB_EINVAL
    assert call(n_steps=17) == LB_EINVAL           # more than LB_MAX_PLAN_STEPS
    assert call(ws=[FAKE, FAKE]) == LB_EINVAL      # one workspace for two steps
    assert call(sizes=(need, 64)) == LB_EWORKSPACE  # the second step's workspace is too small
    assert call(kv=(FAKE, None)) == LB_EINVAL
    assert call(q_pos=None) == LB_EINVAL
    assert call(d=48) == LB_EUNSUPPORTED
    assert L.lb_plan_block_steps(FAKE, FAKE, n, None, None, None, 1, 2, 2, 64, -1, None, None, None) == LB_EINVAL


def test_ring_host_checks(L):
    """lb_ring_workspace_bytes, lb_plan_ring and lb_ring_attn_run reject bad arguments on the
    host, before anything is enqueued."""
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    arr = lambda t, xs: (t * len(xs))(*xs)
    one = L.lb_ring_workspace_bytes(1, 64, 3, 2, 2)
    two = L.lb_ring_workspace_bytes(2, 64, 3, 2, 2)
    assert one > 0 and two > one and one % 256 == 0
    assert L.lb_ring_workspace_bytes(0, 64, 3, 2, 2) == 0
    assert L.lb_ring_workspace_bytes(17, 64, 3, 2, 2) == 0
    assert L.lb_ring_workspace_bytes(2, 64, 3, 3, 2) == 0
    ring = P(0x300000)
    wss = [P(0x100000), P(0x200000)]
    need = L.lb_workspace_bytes(64, 3, 2, 2)

    def plan(n_steps=2, ws=wss, sizes=(need, need), n_kv=(64, 64), d=64, ring=ring, ring_bytes=two):
        return L.lb_plan_ring(arr(P, ws), arr(SZ, sizes), arr(I32, n_kv), n_steps, 64, 2, 2, d, ring, ring_bytes, None)
    assert plan(n_steps=0) == LB_EINVAL
    assert plan(n_steps=17) == LB_EINVAL
    assert plan(ring=None) == LB_EINVAL
    assert plan(ring=P(0x300010)) == LB_EWORKSPACE       # not 256-byte aligned
    assert plan(ring_bytes=1024) == LB_EWORKSPACE        # no room for a tile
    assert plan(ws=[P(0x100000), ring]) == LB_EINVAL     # a step's workspace is the ring's
    assert plan(n_kv=(64, -1)) == LB_EINVAL
    assert plan(d=48) == LB_EUNSUPPORTED
    assert L.lb_plan_ring(None, None, None, 1, 64, 2, 2, 64, ring, two, None) == LB_EINVAL

    def run(n_steps=2, k=(FAKE, FAKE), n_kv=(64, 64), out=(P(0x400000), P(0x500000)),
            lse=(P(0x600000), P(0x700000)), n_q=0, d=64, ring=ring):
        return L.lb_ring_attn_run(FAKE, n_q, 2, 2, d, n_steps, arr(P, k), arr(P, k), arr(I32, n_kv), arr(P, out),
                                  arr(P, lse), ring, two, None)
    assert run() == LB_OK                                  # no query rows: nothing to launch
    assert run(n_steps=0) == LB_EINVAL
    assert run(out=(P(0x400000), P(0x400000))) == LB_EINVAL  # two steps into one partial
    assert run(k=(FAKE, None)) == LB_EINVAL
    assert run(n_kv=(64, -2)) == LB_EINVAL
    assert run(d=48) == LB_EUNSUPPORTED
    assert run(ring=P(0x300010)) == LB_EWORKSPACE



def test_fused_ring_host_checks(L):
    """lb_plan_ring_fused and lb_ring_attn_run_fused reject bad arguments on the host, before
    anything is enqueued, as their unfused counterparts do."""
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    arr = lambda t, xs: (t * len(xs))(*xs)
    two = L.lb_ring_workspace_bytes(2, 64, 3, 2, 2)
    ring = P(0x300000)
    wss = [P(0x100000), P(0x200000)]
    need = L.lb_workspace_bytes(64, 3, 2, 2)

    def plan(n_steps=2, ws=wss, n_kv=(64, 64), d=64, ring=ring, ring_bytes=two):
        return L.lb_plan_ring_fused(arr(P, ws), arr(SZ, (need, need)), arr(I32, n_kv), n_steps, 64, 2, 2, d, ring,
                                    ring_bytes, None)
    assert plan(n_steps=0) == LB_EINVAL
    assert plan(n_steps=17) == LB_EINVAL
    assert plan(ring=None) == LB_EINVAL
    assert plan(ring=P(0x300010)) == LB_EWORKSPACE
    assert plan(ring_bytes=1024) == LB_EWORKSPACE
    assert plan(ws=[P(0x100000), ring]) == LB_EINVAL
    assert plan(n_kv=(64, -1)) == LB_EINVAL
    assert plan(d=48) == LB_EUNSUPPORTED

    def run(n_steps=2, k=(FAKE, FAKE), n_kv=(64, 64), out=P(0x400000), lse=P(0x600000), n_q=0, d=64, ring=ring):
        return L.lb_ring_attn_run_fused(FAKE, n_q, 2, 2, d, n_steps, arr(P, k), arr(P, k), arr(I32, n_kv), out, lse,
                                        ring, two, None)
    assert run() == LB_OK                                  # no query rows: nothing to launch
    assert run(n_steps=0) == LB_EINVAL
    assert run(out=None) == LB_EINVAL
    assert run(lse=P(0x600002)) == LB_EINVAL               # lse not 4-byte aligned
    assert run(k=(FAKE, None)) == LB_EINVAL
    assert run(n_kv=(64, -2)) == LB_EINVAL
    assert run(d=48) == LB_EUNSUPPORTED
    assert run(ring=P(0x300010)) == LB_EWORKSPACE

def test_ring_backward_host_checks(L):
    """lb_block_attn_bwd_ring rejects bad arguments on the host, before anything is enqueued."""
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    arr = lambda t, xs: (t * len(xs))(*xs)
    n = 64
    ws_need = L.lb_bwd_workspace_bytes(n, 3, 2, 2) * 4
    ring = P(0x900000)
    ring_bytes = L.lb_ring_workspace_bytes(2, n, 3, 2, 2)

    def call(n_steps=2, n_kv=(n, n), dkv=(P(0x400000), P(0x500000)), ws=(P(0x100000), P(0x200000)), n_q=0, d=64,
             ring=ring):
        k = max(n_steps, 1)
        pad = lambda xs, fill: list(xs) + [fill] * (k - len(xs))
        return L.lb_block_attn_bwd_ring(FAKE, n_q, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, d, -1, n_steps,
                                        arr(P, pad([FAKE, FAKE], FAKE)), arr(I32, pad(n_kv, n)),
                                        arr(P, pad([FAKE, FAKE], FAKE)), arr(P, pad([FAKE, FAKE], FAKE)), FAKE,
                                        arr(P, pad(dkv, P(0x600000))), arr(P, pad(ws, P(0x700000))),
                                        arr(SZ, pad([ws_need, ws_need], ws_need)), ring, ring_bytes, None)
    assert call() == LB_OK                                   # no query rows: nothing to launch
    assert call(n_steps=0) == LB_EINVAL
    assert call(n_steps=9) == LB_EINVAL                      # two plans per step, at most LB_MAX_PLAN_STEPS
    assert call(n_kv=(n, 0)) == LB_EINVAL                    # a ring step has keys
    assert call(dkv=(P(0x400000), P(0x400000))) == LB_EINVAL  # two steps into one partial
    assert call(ws=(P(0x100000), P(0x100000))) == LB_EINVAL
    assert call(ws=(P(0x100000), ring)) == LB_EINVAL
    assert call(ring=P(0x900010)) == LB_EWORKSPACE
    assert call(d=48) == LB_EUNSUPPORTED


def test_merge_host_checks(L):
    assert L.lb_lse_merge(None, FAKE, FAKE, FAKE, 4, 2, 8, None) == LB_EINVAL
    assert L.lb_lse_merge(FAKE, FAKE, FAKE, FAKE, 4, 2, 6, None) == LB_EUNSUPPORTED
    assert L.lb_lse_merge(FAKE, FAKE, FAKE, FAKE, -1, 2, 8, None) == LB_EINVAL
    assert L.lb_lse_merge(FAKE, FAKE, FAKE, FAKE, 0, 2, 8, None) == LB_OK


def test_read_backs_reject_bad_arguments(L):
    n = ctypes.c_int32()
    assert L.lb_read_plan(FAKE, 1 << 20, None, 4, ctypes.byref(n), None) == LB_EINVAL
    assert L.lb_read_plan(None, 1 << 20, None, 0, ctypes.byref(n), None) == LB_EWORKSPACE
    assert L.lb_read_device_error(FAKE, 1 << 20, None, None) == LB_EINVAL


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(lb, "_lib", None)
    monkeypatch.setattr(lb, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "liblbattn.so"))
    with pytest.raises(lb.LBError, match="no CPU fallback"):
        lb.lib()


def test_product_and_oracle_share_no_code():
    pkg = os.path.join(ROOT, "load_balance_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, re.M), f
                assert "oracle/" not in text and "oracle." not in text, f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            text = open(os.path.join(ROOT, "oracle", f)).read()
            assert not re.search(r"^\s*(from|import)\s+load_balance_amd\b", text, re.M), f
            assert "liblbattn" not in text, f
