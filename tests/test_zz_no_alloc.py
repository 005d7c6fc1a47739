"""lb_varlen_attn_fwd_noalloc, the forward for callers that cannot allocate, through the C ABI.

It runs lb_varlen_attn_fwd's plan and kernels with the plan held in the library's per-GPU
scratch array, so on the same inputs its out and lse must be those of lb_varlen_attn_fwd
with a caller's workspace, bit for bit (the bar of the forward's parity tests is then met
by construction; the small call is also checked against the float64 oracle).  Two calls in
a row, the second on a smaller pack: it finds the first call's plan in the shared array and
must use none of it.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import load_balance_amd as lb
import workloads
from oracle import attention as OA

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def case(lengths, H, Hkv, d, seed):
    r = np.random.default_rng(seed)
    T = int(sum(lengths))
    q, k, v = workloads.values(r, T, H, Hkv, d)
    cu = np.asarray(workloads.cu_from_lengths(lengths), dtype=np.int32)
    return (q, k, v, cu), (dev_bf16(q), dev_bf16(k), dev_bf16(v), torch.from_numpy(cu).cuda())


def noalloc(q, k, v, cu, out, lse, mask):
    """The entry point itself, through ctypes (the binding's checks are not in the way)."""
    T, H, d = q.shape
    st = lb.lib().lb_varlen_attn_fwd_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
        ctypes.c_void_p(cu.data_ptr()), cu.numel() - 1, T, H, k.shape[1], d, mask, ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(lse.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


CASES = [  # the second is smaller than the first: it reuses the array the first call filled
    ([1, 700, 3, 1, 257, 64, 129, 1000, 2, 5000], 32, 8, 128, lb.MASK_CAUSAL_DOC, 1),
    ([300, 129, 64, 1, 200], 8, 2, 64, lb.MASK_SHARED_QUESTION, 2),
]


def test_noalloc_equals_the_workspace_entry_point_twice():
    for i, (lengths, H, Hkv, d, mask, seed) in enumerate(CASES):
        host, (q, k, v, cu) = case(lengths, H, Hkv, d, seed)
        T = q.shape[0]
        say(f"  call {i}: T={T} H={H}/{Hkv} d={d} mask={mask} docs={len(lengths)}")
        ws = lb.new_workspace(T, len(lengths), H, Hkv)
        ref_o, ref_l = lb.varlen_attn_fwd(q, k, v, cu, mask_kind=mask, workspace=ws)
        out = torch.full_like(q, float("nan"))
        lse = torch.full((H, T), float("nan"), dtype=torch.float32, device="cuda")
        assert noalloc(q, k, v, cu, out, lse, mask) == 0
        torch.cuda.synchronize()
        assert lb.read_device_error(ws) == 0
        assert torch.equal(out, ref_o), f"call {i}: out differs from lb_varlen_attn_fwd"
        assert torch.equal(lse, ref_l), f"call {i}: lse differs from lb_varlen_attn_fwd"
        if i == 1:  # the small call against the oracle as well
            o, l = OA.varlen_attention(*host[:3], host[3], H, Hkv,
                                       mask="shared_question" if mask == lb.MASK_SHARED_QUESTION else "causal_doc")
            d_o = np.abs(out.float().cpu().numpy() - o)
            d_l = np.abs(lse.cpu().numpy() - l)
            say(f"  call {i} vs oracle: out max {d_o.max():.3e} mean {d_o.mean():.3e}  lse max {d_l.max():.3e}")
            assert d_o.max() <= 2e-2 and d_o.mean() <= 2e-3 and d_l.max() <= 5e-3


def test_noalloc_binding_and_rejections():
    """The Python binding gives the same bits; calls beyond what the entry point supports
    return an error before anything is enqueued, leaving out and lse as they were."""
    lengths, H, Hkv, d = [100, 28], 4, 2, 64
    _, (q, k, v, cu) = case(lengths, H, Hkv, d, 3)
    T = q.shape[0]
    ref_o, ref_l = lb.varlen_attn_fwd(q, k, v, cu)
    out = torch.empty_like(q)
    lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
    lb.varlen_attn_fwd_noalloc(q, k, v, cu, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    out.fill_(3.0)
    lse.fill_(3.0)
    cu_bad = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    T_big = 1 << 22  # more tiles than one plan holds: refused on the host
    st = lb.lib().lb_varlen_attn_fwd_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
        ctypes.c_void_p(cu_bad.data_ptr()), 1, T_big, H, Hkv, d, 0, ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(lse.data_ptr()), None)
    assert st == 2  # LB_EUNSUPPORTED
    st = lb.lib().lb_varlen_attn_fwd_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
        ctypes.c_void_p(cu_bad.data_ptr()), 0, T, H, Hkv, d, 0, ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(lse.data_ptr()), None)
    assert st == 1  # LB_EINVAL
    torch.cuda.synchronize()
    assert torch.all(out == 3.0) and torch.all(lse == 3.0)
