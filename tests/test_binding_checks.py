"""The Python binding checks every operand before its pointer crosses the C ABI.

A host tensor, a wrong dtype or a wrong shape (a bf16 out where the kernel stores fp32, a
short lse, positions of another length than the rows) would hand a kernel a pointer it
overruns or a host address.  Every wrapper raises LBError instead, before any library
call: these run on the CPU, where a library call that launched a kernel could not succeed.
"""
import pytest
import torch

import load_balance_amd as lb

bf16, f32, i32, u8 = torch.bfloat16, torch.float32, torch.int32, torch.uint8


def z(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


T, H, HKV, D = 64, 8, 2, 128
WS = z(4096, u8)


def varlen_args(**kw):
    a = dict(q=z((T, H, D), bf16), k=z((T, HKV, D), bf16), v=z((T, HKV, D), bf16),
             cu_seqlens=torch.tensor([0, 10, T], dtype=i32), out=z((T, H, D), bf16), lse=z((H, T), f32), workspace=WS)
    a.update(kw)
    return a


def raises(match, fn, *args, **kw):
    with pytest.raises(lb.LBError, match=match):
        fn(*args, **kw)


def test_varlen_forward_checks():
    raises("GPU tensors", lb.varlen_attn_fwd, **varlen_args())
    raises("k has shape", lb.varlen_attn_fwd, **varlen_args(k=z((T - 1, HKV, D), bf16)))
    raises("v has shape", lb.varlen_attn_fwd, **varlen_args(k=z((T, HKV + 1, D), bf16)))
    raises("v has shape", lb.varlen_attn_fwd, **varlen_args(v=z((T - 1, HKV, D), bf16)))
    raises("v must be torch.bfloat16", lb.varlen_attn_fwd, **varlen_args(v=z((T, HKV, D), f32)))
    raises("out must be torch.bfloat16", lb.varlen_attn_fwd, **varlen_args(out=z((T, H, D), f32)))
    raises("lse has shape", lb.varlen_attn_fwd, **varlen_args(lse=z((T, H), f32)))
    raises("cu_seqlens must be torch.int32", lb.varlen_attn_fwd,
           **varlen_args(cu_seqlens=torch.tensor([0, T], dtype=torch.int64)))
    raises("q must be contiguous", lb.varlen_attn_fwd, **varlen_args(q=z((H, T, D), bf16).transpose(0, 1)))
    raises("workspace must be torch.uint8", lb.varlen_attn_fwd, **varlen_args(workspace=z(64, i32)))
    raises("must be a torch tensor", lb.varlen_attn_fwd, **varlen_args(lse=[0.0] * T))


def test_plan_varlen_checks():
    cu = torch.tensor([0, 10, T], dtype=i32)
    for fn, extra in ((lb.plan_varlen, ()), (lb.plan_varlen_weighted, (41515, 1)),
                      (lb.plan_varlen_ordered, (41515, 1, lb.ORDER_DOCUMENTS))):
        raises("GPU tensors", fn, cu, T, H, HKV, D, *extra, workspace=WS)
        raises("cu_seqlens must be torch.int32", fn, torch.tensor([0, T], dtype=torch.int64), T, H, HKV, D, *extra,
               workspace=WS)


def block_args(n_q=64, n_kv=128, **kw):
    a = dict(q_shard=z((n_q, H, D), bf16), kv_chunk=z((2, n_kv, HKV, D), bf16), q_pos=z(n_q, i32),
             kv_pos=z(n_kv, i32), q_doc=z(n_q, i32), kv_doc=z(n_kv, i32), out=z((n_q, H, D), f32),
             lse=z((H, n_q), f32), workspace=WS)
    a.update(kw)
    return a


def test_lse_merge_parts_checks():
    o, l = z((10, H, D), f32), z((H, 10), f32)
    raises("2 to 16 partials", lb.lse_merge_parts, [o], [l])
    raises("2 to 16 partials", lb.lse_merge_parts, [o, o], [l])
    raises("outs\\[1\\] has shape", lb.lse_merge_parts, [o, z((11, H, D), f32)], [l, l])
    raises("lses\\[1\\] must be torch.float32", lb.lse_merge_parts, [o, o], [l, z((H, 10), bf16)])
    raises("GPU tensors", lb.lse_merge_parts, [o, z((10, H, D), f32)], [l, z((H, 10), f32)])


def test_block_forward_checks():
    raises("GPU tensors", lb.block_attn_fwd, **block_args())
    raises("q_pos has shape", lb.block_attn_fwd, **block_args(q_pos=z(63, i32)))
    raises("kv_doc has shape", lb.block_attn_fwd, **block_args(kv_doc=z(64, i32)))
    raises("kv_pos must be torch.int32", lb.block_attn_fwd, **block_args(kv_pos=z(128, torch.int64)))
    raises("kv_chunk must be", lb.block_attn_fwd, **block_args(kv_chunk=z((128, HKV, D), bf16)))
    raises("out must be torch.float32", lb.block_attn_fwd, **block_args(out=z((64, H, D), bf16)))
    raises("lse has shape", lb.block_attn_fwd, **block_args(lse=z((H, 65), f32)))


def test_merge_checks():
    R = 32
    a = dict(out_a=z((R, H, D), f32), lse_a=z((H, R), f32), out_b=z((R, H, D), f32), lse_b=z((H, R), f32))
    raises("GPU tensors", lb.lse_merge, **a)
    raises("lse_b has shape", lb.lse_merge, **dict(a, lse_b=z((H, R + 1), f32)))
    raises("out_b has shape", lb.lse_merge, **dict(a, out_b=z((R, H, D // 2), f32)))
    raises("lse_a has shape", lb.lse_merge, **dict(a, lse_a=z((R, H), f32)))
    raises("out_a must be torch.float32", lb.lse_merge, **dict(a, out_a=z((R, H, D), bf16)))


def test_run_checks():
    a = dict(q=z((T, H, D), bf16), k=z((T, HKV, D), bf16), v=z((T, HKV, D), bf16), out=z((T, H, D), bf16),
             lse=z((H, T), f32), workspace=WS)
    raises("GPU tensors", lb.attn_run, **a)
    raises("out has shape", lb.attn_run, **dict(a, out=z((T, H, 64), bf16)))
    raises("out must be", lb.attn_run, **dict(a, out=z((T, H, D), torch.float16)))
    raises("lse must be torch.float32", lb.attn_run_lower, **dict(a, lse=z((H, T), bf16)))


def test_ring_run_checks():
    n_kv = 128
    ks = [z((n_kv, HKV, D), bf16) for _ in range(2)]
    outs = [z((T, H, D), f32), z((T, H, D), f32)]
    lses = [z((H, T), f32), z((H, T), f32)]
    raises("GPU tensors", lb.ring_attn_run, z((T, H, D), bf16), ks, ks, outs, lses, WS)
    raises(r"outs\[1\] has shape", lb.ring_attn_run, z((T, H, D), bf16), ks, ks, [outs[0], z((T, H, D + 1), f32)], lses,
           WS)
    raises("one entry per step", lb.ring_attn_run, z((T, H, D), bf16), ks, ks[:1], outs, lses, WS)


def test_backward_checks():
    a = dict(q=z((T, H, D), bf16), k=z((T, HKV, D), bf16), v=z((T, HKV, D), bf16), out=z((T, H, D), bf16),
             dout=z((T, H, D), bf16), lse=z((H, T), f32), cu_seqlens=torch.tensor([0, T], dtype=i32),
             dq=z((T, H, D), bf16), dk=z((T, HKV, D), bf16), dv=z((T, HKV, D), bf16), workspace=WS)
    raises("GPU tensors", lb.varlen_attn_bwd, **a)
    raises("dk has shape", lb.varlen_attn_bwd, **dict(a, dk=z((T, H, D), bf16)))
    raises("dout has shape", lb.varlen_attn_bwd, **dict(a, dout=z((T - 1, H, D), bf16)))
    b = dict(q_shard=z((T, H, D), bf16), kv_chunk=z((2, 128, HKV, D), bf16), dout=z((T, H, D), bf16),
             lse=z((H, T), f32), dvec=z((H, T), f32), q_pos=z(T, i32), kv_pos=z(128, i32), q_doc=z(T, i32),
             kv_doc=z(128, i32), dq=z((T, H, D), f32), dkv=z((2, 128, HKV, D), f32), workspace=WS)
    raises("GPU tensors", lb.block_attn_bwd, **b)
    raises("dvec has shape", lb.block_attn_bwd, **dict(b, dvec=z((T, H), f32)))
    raises("dkv has shape", lb.block_attn_bwd, **dict(b, dkv=z((2, 127, HKV, D), f32)))
    raises("dq must be torch.float32", lb.block_attn_bwd, **dict(b, dq=z((T, H, D), bf16)))
    raises("out has shape", lb.attn_bwd_rowdot, z((T, H, D + 1), f32), z((T, H, D), bf16))


def test_slices_and_read_back_checks():
    q = z((T, H, D), bf16)
    kv = z((T, HKV, D), bf16)
    raises("slices must be", lb.slices_attn_fwd, q, kv, kv, torch.zeros((1, 5), dtype=torch.int64), workspace=WS)
    raises("GPU tensors", lb.slices_attn_fwd, q, kv, kv, torch.tensor([[0, T, 0, T, 1]], dtype=i32), workspace=WS)
    raises("GPU tensors", lb.read_device_error, WS)
    raises("workspace must be torch.uint8", lb.read_plan, z(16, f32))
    raises("workspace must be 1-D", lb.read_worker_timing, z((4, 4), u8))
