"""MI355X-native document-masked varlen attention.

Thin ctypes binding over ``liblbattn.so`` (C ABI in ``include/lbattn.h``):
argument marshalling only -- every step of the computation runs in the HIP
kernels.  torch supplies device memory and the current stream.  There is no
CPU fallback: if the library is missing, every call raises.

Python names match the C entry points without their ``lb_`` prefix:
``varlen_attn_fwd``, ``block_attn_fwd``, ``lse_merge``, and the backward
``varlen_attn_bwd``, ``block_attn_bwd``, ``attn_bwd_rowdot``.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import zigzag  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblbattn.so")

MASK_CAUSAL_DOC = 0
MASK_SHARED_QUESTION = 1
NO_SHARED_DOC = -1  # block path: no document shared by the others
MAX_SPANS = 4
MAX_PLAN_STEPS = 16
NOALLOC_SCRATCH_BYTES = 16 << 20  # LB_NOALLOC_SCRATCH_BYTES

DEVERR_CU_SEQLENS = 1
DEVERR_CAPACITY = 2
DEVERR_SPANS = 4
DEVERR_PLAN = 8
DEVERR_SLICES = 16
SLICE_FULL = 0
SLICE_CAUSAL = 1
SLICE_INV_CAUSAL = 2
SLICE_BI_CAUSAL = 3
NO_LOWER_BOUND = 1 << 30


class LBError(RuntimeError):
    pass


class PlanTile(ctypes.Structure):
    _fields_ = [("q_start", ctypes.c_int32), ("q_len", ctypes.c_int32), ("q_pos0", ctypes.c_int32),
                ("n_spans", ctypes.c_int32), ("cost", ctypes.c_int64),
                ("k_start", ctypes.c_int32 * MAX_SPANS), ("k_len", ctypes.c_int32 * MAX_SPANS),
                ("k_pos0", ctypes.c_int32 * MAX_SPANS), ("k_lo", ctypes.c_int32 * MAX_SPANS),
                ("blocks", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class WorkerRecord(ctypes.Structure):
    _fields_ = [("hw_id", ctypes.c_uint32), ("xcc_id", ctypes.c_uint32), ("t_start", ctypes.c_uint64),
                ("t_end", ctypes.c_uint64), ("pairs", ctypes.c_int64), ("items", ctypes.c_int32),
                ("blocks", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LBError(f"{LIB_PATH} is missing: build it with `python -m load_balance_amd.build` "
                      "(there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.lb_tile_rows.argtypes = [I32, I32, I32]
    L.lb_tile_rows.restype = I32
    L.lb_workspace_bytes.argtypes = [I32, I32, I32, I32]
    L.lb_workspace_bytes.restype = SZ
    L.lb_varlen_attn_fwd.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, I32, P, P, P, SZ, P]
    L.lb_varlen_attn_fwd.restype = ctypes.c_int
    L.lb_varlen_attn_fwd_noalloc.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, I32, P, P, P]
    L.lb_varlen_attn_fwd_noalloc.restype = ctypes.c_int
    L.lb_block_attn_fwd.argtypes = [P, I32, P, I32, P, P, P, P, I32, I32, I32, I32, P, P, P, SZ, P]
    L.lb_block_attn_fwd.restype = ctypes.c_int
    L.lb_plan_varlen.argtypes = [P, I32, I32, I32, I32, I32, I32, P, SZ, P]
    L.lb_plan_varlen.restype = ctypes.c_int
    U32 = ctypes.c_uint32
    L.lb_plan_varlen_weighted.argtypes = [P, I32, I32, I32, I32, I32, I32, U32, U32, P, SZ, P]
    L.lb_plan_varlen_weighted.restype = ctypes.c_int
    L.lb_plan_varlen_ordered.argtypes = [P, I32, I32, I32, I32, I32, I32, U32, U32, I32, P, SZ, P]
    L.lb_plan_varlen_ordered.restype = ctypes.c_int
    L.lb_plan_block.argtypes = [P, P, I32, P, P, I32, I32, I32, I32, I32, P, SZ, P]
    L.lb_plan_block.restype = ctypes.c_int
    L.lb_plan_block_steps.argtypes = [P, P, I32, P, P, P, I32, I32, I32, I32, I32, P, P, P]
    L.lb_plan_block_steps.restype = ctypes.c_int
    L.lb_ring_workspace_bytes.argtypes = [I32, I32, I32, I32, I32]
    L.lb_ring_workspace_bytes.restype = SZ
    L.lb_plan_ring.argtypes = [P, P, P, I32, I32, I32, I32, I32, P, SZ, P]
    L.lb_plan_ring.restype = ctypes.c_int
    L.lb_ring_attn_run.argtypes = [P, I32, I32, I32, I32, I32, P, P, P, P, P, P, SZ, P]
    L.lb_ring_attn_run.restype = ctypes.c_int
    L.lb_plan_ring_fused.argtypes = [P, P, P, I32, I32, I32, I32, I32, P, SZ, P]
    L.lb_plan_ring_fused.restype = ctypes.c_int
    L.lb_ring_attn_run_fused.argtypes = [P, I32, I32, I32, I32, I32, P, P, P, P, P, P, SZ, P]
    L.lb_ring_attn_run_fused.restype = ctypes.c_int
    L.lb_attn_run.argtypes = [P, P, P, I32, I32, I32, I32, I32, I32, P, P, P, SZ, P]
    L.lb_attn_run.restype = ctypes.c_int
    L.lb_attn_run_lower.argtypes = [P, P, P, I32, I32, I32, I32, I32, I32, P, P, P, SZ, P]
    L.lb_attn_run_lower.restype = ctypes.c_int
    L.lb_lse_merge.argtypes = [P, P, P, P, I32, I32, I32, P]
    L.lb_lse_merge_parts.argtypes = [P, P, I32, I32, I32, I32, P]
    L.lb_lse_merge_parts.restype = ctypes.c_int
    L.lb_lse_merge.restype = ctypes.c_int
    L.lb_plan_slices.argtypes = [P, I32, I32, I32, I32, I32, I32, P, SZ, P]
    L.lb_plan_slices.restype = ctypes.c_int
    L.lb_slices_attn_fwd.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, I32, P, P, P, SZ, P]
    L.lb_slices_attn_fwd.restype = ctypes.c_int
    L.lb_bwd_workspace_bytes.argtypes = [I32, I32, I32, I32]
    L.lb_bwd_workspace_bytes.restype = SZ
    L.lb_bwd_key_plan_offset.argtypes = [I32, I32, I32, I32, I32, I32, SZ]
    L.lb_bwd_key_plan_offset.restype = SZ
    L.lb_attn_bwd_rowdot.argtypes = [P, I32, P, I32, I32, I32, P, P]
    L.lb_attn_bwd_rowdot.restype = ctypes.c_int
    L.lb_varlen_attn_bwd.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, P, P, P, P, SZ, P]
    L.lb_varlen_attn_bwd.restype = ctypes.c_int
    L.lb_block_attn_bwd.argtypes = [P, I32, P, I32, P, P, P, P, P, P, P, I32, I32, I32, I32, P, P, P, SZ, P]
    L.lb_block_attn_bwd.restype = ctypes.c_int
    L.lb_block_attn_bwd_ring.argtypes = [P, I32, P, P, P, P, P, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, P, P, SZ,
                                         P]
    L.lb_block_attn_bwd_ring_fused.argtypes = [P, I32, P, P, P, P, P, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, P,
                                               P, SZ, P, SZ, P]
    L.lb_block_attn_bwd_ring_fused.restype = ctypes.c_int
    L.lb_block_attn_bwd_ring.restype = ctypes.c_int
    L.lb_status_string.argtypes = [ctypes.c_int]
    L.lb_status_string.restype = ctypes.c_char_p
    L.lb_read_device_error.argtypes = [P, SZ, ctypes.POINTER(I32), P]
    L.lb_read_device_error.restype = ctypes.c_int
    L.lb_read_plan.argtypes = [P, SZ, ctypes.POINTER(PlanTile), I32, ctypes.POINTER(I32), P]
    L.lb_read_plan.restype = ctypes.c_int
    L.lb_read_worker_timing.argtypes = [P, SZ, ctypes.POINTER(WorkerRecord), I32, ctypes.POINTER(I32), P]
    L.lb_read_worker_timing.restype = ctypes.c_int
    del I64
    _lib = L
    return L


def _check(status: int, what: str):
    if status != 0:
        msg = lib().lb_status_string(status).decode()
        raise LBError(f"{what}: {msg} (status {status})")


def _dev(t, name, dtype, shape=None, device=None):
    """Checks one operand before its pointer crosses the C ABI: a contiguous tensor of the
    given dtype (or one of a tuple of dtypes), the exact shape when given, on `device` when
    given.  A wrong dtype or a short buffer would otherwise reach a kernel.  Every wrapper
    checks all its operands this way against its first one, then that one with _gpu, so a
    host tensor never reaches the library either."""
    if not isinstance(t, torch.Tensor):
        raise LBError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if device is not None and t.device != device:
        raise LBError(f"{name} is on {t.device}, the other operands on {device}")
    dtypes = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in dtypes:
        raise LBError(f"{name} must be {' or '.join(str(x) for x in dtypes)}, got {t.dtype}")
    if not t.is_contiguous():
        raise LBError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise LBError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    return t


def _gpu(t, name):
    """The operands share one device (checked by _dev); it must be a GPU."""
    if t.device.type != "cuda":
        raise LBError(f"{name} and the other operands must be GPU tensors, got {t.device}")


def _ws(t, name="workspace", device=None):
    """A workspace: a contiguous 1-D uint8 GPU tensor."""
    _dev(t, name, torch.uint8, device=device)
    if t.dim() != 1:
        raise LBError(f"{name} must be 1-D")
    return t


def _raise_device_error(workspace, what, stream=None):
    """For a call whose workspace the wrapper allocated (the caller cannot read it back):
    errors only the device sees (malformed cu_seqlens, too many key runs, a capacity
    overflow) leave out and lse unwritten, so they are read here and raised.  This waits
    for the stream; callers that pass their own workspace read it with read_device_error."""
    err = read_device_error(workspace, stream=stream)
    if err:
        names = [n for n, b in (("CU_SEQLENS", DEVERR_CU_SEQLENS), ("CAPACITY", DEVERR_CAPACITY),
                                ("SPANS", DEVERR_SPANS), ("PLAN", DEVERR_PLAN), ("SLICES", DEVERR_SLICES)) if err & b]
        raise LBError(f"{what}: the device rejected the call's metadata ({'|'.join(names) or err}); "
                      "nothing was computed")


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def tile_rows(heads: int, kv_heads: int, d: int) -> int:
    return int(lib().lb_tile_rows(heads, kv_heads, d))


def workspace_bytes(max_tokens: int, max_segments: int, heads: int, kv_heads: int) -> int:
    n = int(lib().lb_workspace_bytes(max_tokens, max_segments, heads, kv_heads))
    if n == 0:
        raise LBError("lb_workspace_bytes: invalid or unsupported arguments")
    return n


def new_workspace(max_tokens: int, max_segments: int, heads: int, kv_heads: int, device="cuda"):
    """A uint8 device tensor sized for the given bounds (torch's allocator aligns to 256 B or more)."""
    return torch.empty(workspace_bytes(max_tokens, max_segments, heads, kv_heads), dtype=torch.uint8,
                       device=device)


def varlen_attn_fwd(q, k, v, cu_seqlens, mask_kind=MASK_CAUSAL_DOC, out=None, lse=None, workspace=None,
                    stream=None):
    """out [T,H,d] bf16, lse [H,T] fp32 for q [T,H,d], k/v [T,H_kv,d] bf16 and int32 cu_seqlens."""
    _dev(q, "q", torch.bfloat16)
    if q.dim() != 3:
        raise LBError("q must be [T, H, d]")
    T, H, d = q.shape
    dev = q.device
    _dev(k, "k", torch.bfloat16, device=dev)
    if k.dim() != 3:
        raise LBError("k must be [T, H_kv, d]")
    Hkv = k.shape[1]
    _dev(k, "k", torch.bfloat16, (T, Hkv, d), dev)
    _dev(v, "v", torch.bfloat16, (T, Hkv, d), dev)
    _dev(cu_seqlens, "cu_seqlens", torch.int32, device=dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise LBError("cu_seqlens must be 1-D with at least two entries")
    n_seg = cu_seqlens.numel() - 1
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, T), dtype=torch.float32, device=dev)
    _dev(out, "out", torch.bfloat16, (T, H, d), dev)
    _dev(lse, "lse", torch.float32, (H, T), dev)
    owned = workspace is None
    workspace = new_workspace(T, max(1, n_seg), H, Hkv, dev) if owned else _ws(workspace, device=dev)
    _gpu(q, "q")
    st = lib().lb_varlen_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), n_seg, T, H, Hkv, d,
                                  int(mask_kind), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                  ctypes.c_void_p(_stream(stream)))
    _check(st, "lb_varlen_attn_fwd")
    if owned:
        _raise_device_error(workspace, "lb_varlen_attn_fwd", stream)
    return out, lse


def varlen_attn_fwd_noalloc(q, k, v, cu_seqlens, out, lse, mask_kind=MASK_CAUSAL_DOC, stream=None):
    """varlen_attn_fwd with the plan in the library's per-GPU scratch array: no workspace, and
    the library allocates nothing.  out [T,H,d] bf16 and lse [H,T] fp32 are the caller's.
    Calls that overlap in time on one GPU race (they share the array)."""
    _dev(q, "q", torch.bfloat16)
    if q.dim() != 3 or k.dim() != 3:
        raise LBError("q must be [T, H, d] and k, v [T, H_kv, d]")
    T, H, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    _dev(k, "k", torch.bfloat16, (T, Hkv, d), dev)
    _dev(v, "v", torch.bfloat16, (T, Hkv, d), dev)
    _dev(cu_seqlens, "cu_seqlens", torch.int32, device=dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise LBError("cu_seqlens must be 1-D with at least two entries")
    _dev(out, "out", torch.bfloat16, (T, H, d), dev)
    _dev(lse, "lse", torch.float32, (H, T), dev)
    _gpu(q, "q")
    _check(lib().lb_varlen_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), cu_seqlens.numel() - 1, T, H,
                                            Hkv, d, int(mask_kind), _ptr(out), _ptr(lse),
                                            ctypes.c_void_p(_stream(stream))), "lb_varlen_attn_fwd_noalloc")
    return out, lse


def block_attn_fwd(q_shard, kv_chunk, q_pos, kv_pos, q_doc, kv_doc, out=None, lse=None, workspace=None,
                   max_runs=None, stream=None, shared_doc=NO_SHARED_DOC):
    """One ring step: q_shard [n_q,H,d] bf16 against kv_chunk [2,n_kv,H_kv,d] bf16 (K then V).
    shared_doc: a document whose keys every other document's rows see in full (the shared
    question), or NO_SHARED_DOC.

    Returns out [n_q,H,d] fp32 (rows with no visible key left unwritten) and lse [H,n_q] fp32.
    """
    _dev(q_shard, "q_shard", torch.bfloat16)
    if q_shard.dim() != 3:
        raise LBError("q_shard must be [n_q, H, d]")
    n_q, H, d = q_shard.shape
    dev = q_shard.device
    _dev(kv_chunk, "kv_chunk", torch.bfloat16, device=dev)
    if kv_chunk.dim() != 4 or kv_chunk.shape[0] != 2 or kv_chunk.shape[3] != d:
        raise LBError("kv_chunk must be [2, n_kv, H_kv, d] (K then V)")
    _, n_kv, Hkv, _ = kv_chunk.shape
    _meta(q_pos, q_doc, n_q, "q", dev)
    _meta(kv_pos, kv_doc, n_kv, "kv", dev)
    if out is None:
        out = torch.empty((n_q, H, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((H, n_q), dtype=torch.float32, device=dev)
    _dev(out, "out", torch.float32, (n_q, H, d), dev)
    _dev(lse, "lse", torch.float32, (H, n_q), dev)
    owned = workspace is None
    if owned:
        runs = max_runs if max_runs is not None else max(n_q, n_kv, 1)
        workspace = new_workspace(max(n_q, n_kv), runs, H, Hkv, dev)
    else:
        _ws(workspace, device=dev)
    _gpu(q_shard, "q_shard")
    st = lib().lb_block_attn_fwd(_ptr(q_shard), n_q, _ptr(kv_chunk), n_kv, _ptr(q_pos), _ptr(kv_pos),
                                 _ptr(q_doc), _ptr(kv_doc), H, Hkv, d, int(shared_doc), _ptr(out), _ptr(lse),
                                 _ptr(workspace),
                                 workspace.numel(), ctypes.c_void_p(_stream(stream)))
    _check(st, "lb_block_attn_fwd")
    if owned:
        _raise_device_error(workspace, "lb_block_attn_fwd", stream)
    return out, lse


def _meta(pos, doc, n, side, device):
    """Positions and document ids of one side of a block step: int32 [n] each."""
    _dev(pos, f"{side}_pos", torch.int32, (n,), device)
    _dev(doc, f"{side}_doc", torch.int32, (n,), device)


def _plan_varlen_args(cu_seqlens, total_tokens, heads, kv_heads, workspace):
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise LBError("cu_seqlens must be 1-D with at least two entries")
    n_seg = cu_seqlens.numel() - 1
    if workspace is None:
        workspace = new_workspace(total_tokens, max(1, n_seg), heads, kv_heads, cu_seqlens.device)
    _ws(workspace, device=cu_seqlens.device)
    _gpu(cu_seqlens, "cu_seqlens")
    return n_seg, workspace


def plan_varlen(cu_seqlens, total_tokens, heads, kv_heads, d, mask_kind=MASK_CAUSAL_DOC, workspace=None,
                stream=None):
    """First half of varlen_attn_fwd: writes the tile plan into ``workspace`` (returned), its
    queue in the documents order (ORDER_DOCUMENTS) of the fitted estimate (LPT_FIT_BLOCK_WEIGHT,
    LPT_FIT_PAIR_WEIGHT)."""
    n_seg, workspace = _plan_varlen_args(cu_seqlens, total_tokens, heads, kv_heads, workspace)
    _check(lib().lb_plan_varlen(_ptr(cu_seqlens), n_seg, total_tokens, heads, kv_heads, d, int(mask_kind),
                                _ptr(workspace), workspace.numel(), ctypes.c_void_p(_stream(stream))),
           "lb_plan_varlen")
    return workspace


# The per-item cost fitted to the attention kernel on MI355X, as LPT weights: 1.37 us per
# key block against 3.3e-5 us per query-head pair.
LPT_FIT_BLOCK_WEIGHT = 41515
LPT_FIT_PAIR_WEIGHT = 1


def plan_varlen_weighted(cu_seqlens, total_tokens, heads, kv_heads, d, block_weight, pair_weight,
                         mask_kind=MASK_CAUSAL_DOC, workspace=None, stream=None):
    """plan_varlen with the queue ordered by block_weight * blocks + pair_weight * G * pairs
    ("数据并行负载均衡", sections 4.2 and 4.4: LPT on a fitted load estimate); (1, 0) orders by
    key blocks alone."""
    n_seg, workspace = _plan_varlen_args(cu_seqlens, total_tokens, heads, kv_heads, workspace)
    _check(lib().lb_plan_varlen_weighted(_ptr(cu_seqlens), n_seg, total_tokens, heads, kv_heads, d,
                                         int(mask_kind), int(block_weight), int(pair_weight), _ptr(workspace),
                                         workspace.numel(), ctypes.c_void_p(_stream(stream))),
           "lb_plan_varlen_weighted")
    return workspace


# queue orders of plan_varlen_ordered (LB_ORDER_*)
ORDER_LPT = 0
ORDER_DOCUMENTS = 1


def plan_varlen_ordered(cu_seqlens, total_tokens, heads, kv_heads, d, block_weight, pair_weight, order,
                        mask_kind=MASK_CAUSAL_DOC, workspace=None, stream=None):
    """plan_varlen_weighted with a choice of queue order: ORDER_LPT (tiles by the estimate,
    largest first) or ORDER_DOCUMENTS (documents by their largest tile's estimate, largest
    first, each document's tiles together from its last back to its first)."""
    n_seg, workspace = _plan_varlen_args(cu_seqlens, total_tokens, heads, kv_heads, workspace)
    _check(lib().lb_plan_varlen_ordered(_ptr(cu_seqlens), n_seg, total_tokens, heads, kv_heads, d,
                                        int(mask_kind), int(block_weight), int(pair_weight), int(order),
                                        _ptr(workspace), workspace.numel(), ctypes.c_void_p(_stream(stream))),
           "lb_plan_varlen_ordered")
    return workspace


def plan_block(q_pos, q_doc, kv_pos, kv_doc, heads, kv_heads, d, workspace, stream=None, shared_doc=NO_SHARED_DOC):
    """First half of block_attn_fwd: writes the tile plan into ``workspace``."""
    _ws(workspace)
    _meta(q_pos, q_doc, q_pos.numel(), "q", workspace.device)
    _meta(kv_pos, kv_doc, kv_pos.numel(), "kv", workspace.device)
    _gpu(workspace, "workspace")
    _check(lib().lb_plan_block(_ptr(q_pos), _ptr(q_doc), q_pos.numel(), _ptr(kv_pos), _ptr(kv_doc), kv_pos.numel(),
                               heads, kv_heads, d, int(shared_doc), _ptr(workspace), workspace.numel(),
                               ctypes.c_void_p(_stream(stream))), "lb_plan_block")
    return workspace


def plan_block_steps(q_pos, q_doc, kv_pos_list, kv_doc_list, heads, kv_heads, d, workspaces, stream=None,
                     shared_doc=NO_SHARED_DOC):
    """Plans of several block steps of one query shard, one launch: step s plans the shard
    against kv_pos_list[s], kv_doc_list[s] into workspaces[s] exactly as plan_block would."""
    n = len(workspaces)
    if not (len(kv_pos_list) == len(kv_doc_list) == n):
        raise LBError("kv_pos_list, kv_doc_list and workspaces must have one entry per step")
    if n < 1:
        raise LBError("plan_block_steps needs at least one step")
    dev = workspaces[0].device
    _meta(q_pos, q_doc, q_pos.numel(), "q", dev)
    for s_, (kp, kd, w) in enumerate(zip(kv_pos_list, kv_doc_list, workspaces)):
        _meta(kp, kd, kp.numel(), f"step {s_} kv", dev)
        _ws(w, f"workspaces[{s_}]", dev)
    ptrs = lambda ts: (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in ts])
    n_kv = (ctypes.c_int32 * max(n, 1))(*[t.numel() for t in kv_pos_list])
    sizes = (ctypes.c_size_t * max(n, 1))(*[w.numel() for w in workspaces])
    _gpu(q_pos, "q_pos")
    _check(lib().lb_plan_block_steps(_ptr(q_pos), _ptr(q_doc), q_pos.numel(), ptrs(kv_pos_list), ptrs(kv_doc_list),
                                     n_kv, n, heads, kv_heads, d, int(shared_doc), ptrs(workspaces), sizes,
                                     ctypes.c_void_p(_stream(stream))), "lb_plan_block_steps")
    return workspaces


def ring_workspace_bytes(n_steps: int, max_tokens: int, max_segments: int, heads: int, kv_heads: int) -> int:
    n = int(lib().lb_ring_workspace_bytes(n_steps, max_tokens, max_segments, heads, kv_heads))
    if n == 0:
        raise LBError("lb_ring_workspace_bytes: invalid or unsupported arguments")
    return n


def new_ring_workspace(n_steps: int, max_tokens: int, max_segments: int, heads: int, kv_heads: int, device="cuda"):
    """A uint8 device tensor for the merged plan of up to n_steps block steps."""
    return torch.empty(ring_workspace_bytes(n_steps, max_tokens, max_segments, heads, kv_heads), dtype=torch.uint8,
                       device=device)


def plan_ring(workspaces, n_kv, n_q, heads, kv_heads, d, ring_workspace, stream=None, fused=False):
    """Merges the block-step plans in ``workspaces`` (step s made against n_kv[s] key/value
    tokens, all for the same n_q query rows) into one longest-first queue in ring_workspace.
    fused=True (lb_plan_ring_fused): one tile per query tile with the spans of every step,
    run by ring_attn_run_fused."""
    n = len(workspaces)
    if len(n_kv) != n:
        raise LBError("n_kv must have one entry per workspace")
    _ws(ring_workspace, "ring_workspace")
    for i, w in enumerate(workspaces):
        _ws(w, f"workspaces[{i}]", ring_workspace.device)
    ptrs = (ctypes.c_void_p * max(n, 1))(*[w.data_ptr() for w in workspaces])
    sizes = (ctypes.c_size_t * max(n, 1))(*[w.numel() for w in workspaces])
    nkv = (ctypes.c_int32 * max(n, 1))(*[int(x) for x in n_kv])
    _gpu(ring_workspace, "ring_workspace")
    fn, name = (lib().lb_plan_ring_fused, "lb_plan_ring_fused") if fused else (lib().lb_plan_ring, "lb_plan_ring")
    _check(fn(ptrs, sizes, nkv, n, n_q, heads, kv_heads, d, _ptr(ring_workspace), ring_workspace.numel(),
              ctypes.c_void_p(_stream(stream))), name)
    return ring_workspace


def ring_attn_run(q, ks, vs, outs, lses, ring_workspace, stream=None):
    """Runs a ring workspace's items in one launch: step s reads ks[s], vs[s] (bf16
    [n_kv_s,H_kv,d]) and writes its partial into outs[s] (fp32 [n_q,H,d]) and lses[s]
    (fp32 [H,n_q]), as attn_run would for that step's own plan."""
    _dev(q, "q", torch.bfloat16)
    if q.dim() != 3:
        raise LBError("q must be [n_q, H, d]")
    n_q, H, d = q.shape
    dev = q.device
    n = len(ks)
    if n < 1 or not (len(vs) == len(outs) == len(lses) == n):
        raise LBError("ks, vs, outs and lses must have one entry per step (at least one)")
    _ws(ring_workspace, "ring_workspace", dev)
    if ks[0].dim() != 3:
        raise LBError("ks[s] must be [n_kv, H_kv, d]")
    Hkv = ks[0].shape[1]
    for i in range(n):
        _dev(ks[i], f"ks[{i}]", torch.bfloat16, (ks[i].shape[0], Hkv, d), dev)
        _dev(vs[i], f"vs[{i}]", torch.bfloat16, tuple(ks[i].shape), dev)
        _dev(outs[i], f"outs[{i}]", torch.float32, (n_q, H, d), dev)
        _dev(lses[i], f"lses[{i}]", torch.float32, (H, n_q), dev)
    ptrs = lambda ts: (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in ts])
    nkv = (ctypes.c_int32 * max(n, 1))(*[k.shape[0] for k in ks])
    _gpu(q, "q")
    _check(lib().lb_ring_attn_run(_ptr(q), n_q, H, Hkv, d, n, ptrs(ks), ptrs(vs), nkv, ptrs(outs), ptrs(lses),
                                  _ptr(ring_workspace), ring_workspace.numel(), ctypes.c_void_p(_stream(stream))),
           "lb_ring_attn_run")
    return outs, lses


def ring_attn_run_fused(q, ks, vs, out, lse, ring_workspace, stream=None):
    """Runs a fused ring (plan_ring(..., fused=True)) in one launch: every step's keys and
    values (ks[s], vs[s], bf16 [n_kv_s,H_kv,d]) for each query tile, the merged result into
    out (fp32 [n_q,H,d]) and lse (fp32 [H,n_q])."""
    _dev(q, "q", torch.bfloat16)
    if q.dim() != 3:
        raise LBError("q must be [n_q, H, d]")
    n_q, H, d = q.shape
    dev = q.device
    n = len(ks)
    if n < 1 or len(vs) != n:
        raise LBError("ks and vs must have one entry per step (at least one)")
    _ws(ring_workspace, "ring_workspace", dev)
    if ks[0].dim() != 3:
        raise LBError("ks[s] must be [n_kv, H_kv, d]")
    Hkv = ks[0].shape[1]
    for i in range(n):
        _dev(ks[i], f"ks[{i}]", torch.bfloat16, (ks[i].shape[0], Hkv, d), dev)
        _dev(vs[i], f"vs[{i}]", torch.bfloat16, tuple(ks[i].shape), dev)
    _dev(out, "out", torch.float32, (n_q, H, d), dev)
    _dev(lse, "lse", torch.float32, (H, n_q), dev)
    ptrs = lambda ts: (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in ts])
    nkv = (ctypes.c_int32 * max(n, 1))(*[k.shape[0] for k in ks])
    _gpu(q, "q")
    _check(lib().lb_ring_attn_run_fused(_ptr(q), n_q, H, Hkv, d, n, ptrs(ks), ptrs(vs), nkv, _ptr(out), _ptr(lse),
                                        _ptr(ring_workspace), ring_workspace.numel(),
                                        ctypes.c_void_p(_stream(stream))), "lb_ring_attn_run_fused")
    return out, lse


def _run_operands(q, k, v, out, lse, workspace):
    """Checks the operands of a plan's run; returns n_q, H, d, n_kv, H_kv."""
    _dev(q, "q", torch.bfloat16)
    if q.dim() != 3 or k.dim() != 3:
        raise LBError("q must be [n_q, H, d] and k, v [n_kv, H_kv, d]")
    n_q, H, d = q.shape
    n_kv, Hkv = k.shape[0], k.shape[1]
    dev = q.device
    _dev(k, "k", torch.bfloat16, (n_kv, Hkv, d), dev)
    _dev(v, "v", torch.bfloat16, (n_kv, Hkv, d), dev)
    _dev(out, "out", (torch.bfloat16, torch.float32), (n_q, H, d), dev)
    _dev(lse, "lse", torch.float32, (H, n_q), dev)
    _ws(workspace, device=dev)
    return n_q, H, d, n_kv, Hkv


def attn_run(q, k, v, out, lse, workspace, stream=None):
    """Second half of either forward: runs the plan held in ``workspace``.

    q [n_q,H,d], k/v [n_kv,H_kv,d] bf16; out bf16 or fp32 [n_q,H,d]; lse fp32 [H,n_q].
    """
    n_q, H, d, n_kv, Hkv = _run_operands(q, k, v, out, lse, workspace)
    _gpu(q, "q")
    _check(lib().lb_attn_run(_ptr(q), _ptr(k), _ptr(v), n_q, n_kv, H, Hkv, d, int(out.dtype == torch.float32),
                             _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                             ctypes.c_void_p(_stream(stream))), "lb_attn_run")
    return out, lse


def attn_run_lower(q, k, v, out, lse, workspace, stream=None):
    """attn_run for plans with lower-bounded spans (INV-CAUSAL / BI-CAUSAL slices)."""
    n_q, H, d, n_kv, Hkv = _run_operands(q, k, v, out, lse, workspace)
    _gpu(q, "q")
    _check(lib().lb_attn_run_lower(_ptr(q), _ptr(k), _ptr(v), n_q, n_kv, H, Hkv, d, int(out.dtype == torch.float32),
                                   _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                   ctypes.c_void_p(_stream(stream))), "lb_attn_run_lower")
    return out, lse


def lse_merge(out_a, lse_a, out_b, lse_b, stream=None):
    """In place: (out_a, lse_a) <- merge((out_a, lse_a), (out_b, lse_b)).  fp32 [R,H,d] and [H,R]."""
    _dev(out_a, "out_a", torch.float32)
    if out_a.dim() != 3:
        raise LBError("out_a must be [R, H, d]")
    R, H, d = out_a.shape
    dev = out_a.device
    _dev(lse_a, "lse_a", torch.float32, (H, R), dev)
    _dev(out_b, "out_b", torch.float32, (R, H, d), dev)
    _dev(lse_b, "lse_b", torch.float32, (H, R), dev)
    _gpu(out_a, "out_a")
    st = lib().lb_lse_merge(_ptr(out_a), _ptr(lse_a), _ptr(out_b), _ptr(lse_b), R, H, d,
                            ctypes.c_void_p(_stream(stream)))
    _check(st, "lb_lse_merge")
    return out_a, lse_a


def lse_merge_parts(outs, lses, stream=None):
    """In place: (outs[0], lses[0]) <- the merge of every partial, 1, 2, ... in order, in one
    pass; the same bits as lse_merge step after step.  fp32 [R,H,d] and [H,R] each."""
    if len(outs) != len(lses) or not 2 <= len(outs) <= MAX_PLAN_STEPS:
        raise LBError(f"lse_merge_parts takes 2 to {MAX_PLAN_STEPS} partials, as many lse as out")
    _dev(outs[0], "outs[0]", torch.float32)
    if outs[0].dim() != 3:
        raise LBError("outs[0] must be [R, H, d]")
    R, H, d = outs[0].shape
    dev = outs[0].device
    for i, (o, l) in enumerate(zip(outs, lses)):
        _dev(o, f"outs[{i}]", torch.float32, (R, H, d), dev)
        _dev(l, f"lses[{i}]", torch.float32, (H, R), dev)
    _gpu(outs[0], "outs[0]")
    P = ctypes.c_void_p
    st = lib().lb_lse_merge_parts((P * len(outs))(*[_ptr(o) for o in outs]), (P * len(lses))(*[_ptr(l) for l in lses]),
                                  len(outs), R, H, d, ctypes.c_void_p(_stream(stream)))
    _check(st, "lb_lse_merge_parts")
    return outs[0], lses[0]


def read_device_error(workspace, stream=None) -> int:
    _ws(workspace)
    err = ctypes.c_int32(0)
    _gpu(workspace, "workspace")
    _check(lib().lb_read_device_error(_ptr(workspace), workspace.numel(), ctypes.byref(err),
                                      ctypes.c_void_p(_stream(stream))), "lb_read_device_error")
    return err.value


def read_plan(workspace, max_tiles: int = 1 << 16, stream=None, with_step=False):
    """The last call's tiles in queue order, as dicts (q_start, q_len, q_pos0, spans, cost, blocks);
    with_step adds each tile's step (a ring workspace's `reserved` field)."""
    _ws(workspace)
    buf = (PlanTile * max_tiles)()
    n = ctypes.c_int32(0)
    _gpu(workspace, "workspace")
    _check(lib().lb_read_plan(_ptr(workspace), workspace.numel(), buf, max_tiles, ctypes.byref(n),
                              ctypes.c_void_p(_stream(stream))), "lb_read_plan")
    out = []
    for i in range(min(n.value, max_tiles)):
        t = buf[i]
        # (k_start, k_len, k_pos0), with k_lo appended when the span has a lower bound
        spans = [(t.k_start[s], t.k_len[s], t.k_pos0[s]) + (() if t.k_lo[s] == NO_LOWER_BOUND else (t.k_lo[s],))
                 for s in range(t.n_spans)]
        out.append(dict(q_start=t.q_start, q_len=t.q_len, q_pos0=t.q_pos0, spans=spans, cost=t.cost,
                        blocks=t.blocks))
        if with_step:
            out[-1]["step"] = t.reserved
    return out


def read_worker_timing(workspace, max_records: int = 4096, stream=None):
    _ws(workspace)
    buf = (WorkerRecord * max_records)()
    n = ctypes.c_int32(0)
    _gpu(workspace, "workspace")
    _check(lib().lb_read_worker_timing(_ptr(workspace), workspace.numel(), buf, max_records, ctypes.byref(n),
                                       ctypes.c_void_p(_stream(stream))), "lb_read_worker_timing")
    return [dict(hw_id=r.hw_id, xcc_id=r.xcc_id, t_start=r.t_start, t_end=r.t_end, pairs=r.pairs,
                 items=r.items, blocks=r.blocks) for r in buf[:min(n.value, max_records)]]


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------
def bwd_workspace_bytes(max_tokens: int, max_segments: int, heads: int, kv_heads: int) -> int:
    n = int(lib().lb_bwd_workspace_bytes(max_tokens, max_segments, heads, kv_heads))
    if n == 0:
        raise LBError("lb_bwd_workspace_bytes: invalid or unsupported arguments")
    return n


def bwd_key_plan_offset(block_path: bool, n_q: int, n_kv: int, n_seg: int, heads: int, kv_heads: int,
                        workspace_bytes: int) -> int:
    """Where the key-tile plan of a backward workspace starts (the query-tile plan is at 0)."""
    return int(lib().lb_bwd_key_plan_offset(int(block_path), n_q, n_kv, n_seg, heads, kv_heads, workspace_bytes))


def block_attn_bwd_ring(q, kvs, dout, lse, dvec, q_pos, q_doc, kv_pos_list, kv_doc_list, dq, dkvs, workspaces,
                        ring_workspace, stream=None, shared_doc=NO_SHARED_DOC, q_ring_workspace=None):
    """The backward of a rank's ring steps: per step s the query shard against kvs[s] (bf16
    [2,n_kv,H_kv,d]) with kv_pos_list[s], kv_doc_list[s]; dq (fp32 [n_q,H,d]) is added to,
    step after step; dkvs[s] (fp32 [2,n_kv,H_kv,d]) receives step s's partial dk, dv.  One
    dQ launch per step and one dK/dV launch over every step's key tiles."""
    _dev(q, "q", torch.bfloat16)
    if q.dim() != 3:
        raise LBError("q must be [n_q, H, d]")
    n_q, H, d = q.shape
    dev = q.device
    n = len(kvs)
    if n < 1 or not (len(kv_pos_list) == len(kv_doc_list) == len(dkvs) == len(workspaces) == n):
        raise LBError("kvs, kv_pos_list, kv_doc_list, dkvs and workspaces need one entry per step (at least one)")
    _dev(dout, "dout", torch.bfloat16, (n_q, H, d), dev)
    _dev(lse, "lse", torch.float32, (H, n_q), dev)
    _dev(dvec, "dvec", torch.float32, (H, n_q), dev)
    _dev(dq, "dq", torch.float32, (n_q, H, d), dev)
    _meta(q_pos, q_doc, n_q, "q", dev)
    _ws(ring_workspace, "ring_workspace", dev)
    if kvs[0].dim() != 4:
        raise LBError("kvs[s] must be [2, n_kv, H_kv, d]")
    Hkv = kvs[0].shape[2]
    for i in range(n):
        n_kv = kvs[i].shape[1]
        _dev(kvs[i], f"kvs[{i}]", torch.bfloat16, (2, n_kv, Hkv, d), dev)
        _dev(dkvs[i], f"dkvs[{i}]", torch.float32, (2, n_kv, Hkv, d), dev)
        _meta(kv_pos_list[i], kv_doc_list[i], n_kv, f"step {i} kv", dev)
        _ws(workspaces[i], f"workspaces[{i}]", dev)
    ptrs = lambda ts: (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in ts])
    nkv = (ctypes.c_int32 * max(n, 1))(*[k.shape[1] for k in kvs])
    sizes = (ctypes.c_size_t * max(n, 1))(*[w.numel() for w in workspaces])
    _gpu(q, "q")
    if q_ring_workspace is not None:  # lb_block_attn_bwd_ring_fused: the dQ side fused per query tile
        _ws(q_ring_workspace, "q_ring_workspace", dev)
        _check(lib().lb_block_attn_bwd_ring_fused(
            _ptr(q), n_q, _ptr(dout), _ptr(lse), _ptr(dvec), _ptr(q_pos), _ptr(q_doc), H, Hkv, d, int(shared_doc), n,
            ptrs(kvs), nkv, ptrs(kv_pos_list), ptrs(kv_doc_list), _ptr(dq), ptrs(dkvs), ptrs(workspaces), sizes,
            _ptr(ring_workspace), ring_workspace.numel(), _ptr(q_ring_workspace), q_ring_workspace.numel(),
            ctypes.c_void_p(_stream(stream))), "lb_block_attn_bwd_ring_fused")
        return dq, dkvs
    _check(lib().lb_block_attn_bwd_ring(_ptr(q), n_q, _ptr(dout), _ptr(lse), _ptr(dvec), _ptr(q_pos), _ptr(q_doc), H,
                                        Hkv, d, int(shared_doc), n, ptrs(kvs), nkv, ptrs(kv_pos_list),
                                        ptrs(kv_doc_list), _ptr(dq), ptrs(dkvs), ptrs(workspaces), sizes,
                                        _ptr(ring_workspace), ring_workspace.numel(),
                                        ctypes.c_void_p(_stream(stream))), "lb_block_attn_bwd_ring")
    return dq, dkvs


def attn_bwd_rowdot(out, dout, dvec=None, stream=None):
    """D [H,R] fp32 = sum over d of out * dout; out bf16 or fp32 [R,H,d], dout bf16 [R,H,d]."""
    _dev(dout, "dout", torch.bfloat16)
    if dout.dim() != 3:
        raise LBError("dout must be [R, H, d]")
    R, H, d = dout.shape
    _dev(out, "out", (torch.bfloat16, torch.float32), (R, H, d), dout.device)
    if dvec is None:
        dvec = torch.empty((H, R), dtype=torch.float32, device=dout.device)
    _dev(dvec, "dvec", torch.float32, (H, R), dout.device)
    _gpu(dout, "dout")
    _check(lib().lb_attn_bwd_rowdot(_ptr(out), int(out.dtype == torch.float32), _ptr(dout), R, H, d, _ptr(dvec),
                                    ctypes.c_void_p(_stream(stream))), "lb_attn_bwd_rowdot")
    return dvec


def varlen_attn_bwd(q, k, v, out, dout, lse, cu_seqlens, mask_kind=MASK_CAUSAL_DOC, dq=None, dk=None, dv=None,
                    workspace=None, stream=None):
    """dq [T,H,d], dk, dv [T,H_kv,d] (bf16) of varlen_attn_fwd from its out and lse."""
    _dev(q, "q", torch.bfloat16)
    if q.dim() != 3 or k.dim() != 3:
        raise LBError("q must be [T, H, d] and k, v [T, H_kv, d]")
    T, H, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    for t, name in ((k, "k"), (v, "v")):
        _dev(t, name, torch.bfloat16, (T, Hkv, d), dev)
    for t, name in ((out, "out"), (dout, "dout")):
        _dev(t, name, torch.bfloat16, (T, H, d), dev)
    _dev(lse, "lse", torch.float32, (H, T), dev)
    _dev(cu_seqlens, "cu_seqlens", torch.int32, device=dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise LBError("cu_seqlens must be 1-D with at least two entries")
    n_seg = cu_seqlens.numel() - 1
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _dev(dq, "dq", torch.bfloat16, (T, H, d), dev)
    _dev(dk, "dk", torch.bfloat16, (T, Hkv, d), dev)
    _dev(dv, "dv", torch.bfloat16, (T, Hkv, d), dev)
    owned = workspace is None
    if owned:
        workspace = torch.empty(bwd_workspace_bytes(T, max(1, n_seg), H, Hkv), dtype=torch.uint8, device=dev)
    _ws(workspace, device=dev)
    _gpu(q, "q")
    _check(lib().lb_varlen_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(cu_seqlens),
                                    n_seg, T, H, Hkv, d, int(mask_kind), _ptr(dq), _ptr(dk), _ptr(dv),
                                    _ptr(workspace), workspace.numel(), ctypes.c_void_p(_stream(stream))),
           "lb_varlen_attn_bwd")
    if owned:
        _raise_bwd_device_error(workspace, False, T, T, n_seg, H, Hkv, "lb_varlen_attn_bwd", stream)
    return dq, dk, dv


def _raise_bwd_device_error(workspace, block_path, n_q, n_kv, n_seg, H, Hkv, what, stream):
    """Both plans of a backward workspace the wrapper allocated: the query-tile plan at its
    start, the key-tile plan at lb_bwd_key_plan_offset."""
    _raise_device_error(workspace, what + " (query tiles)", stream)
    off = bwd_key_plan_offset(block_path, n_q, n_kv, n_seg, H, Hkv, workspace.numel())
    _raise_device_error(workspace[off:], what + " (key tiles)", stream)


def block_attn_bwd(q_shard, kv_chunk, dout, lse, dvec, q_pos, kv_pos, q_doc, kv_doc, dq, dkv=None, workspace=None,
                   stream=None, shared_doc=NO_SHARED_DOC):
    """One ring step of the backward: adds this step's contribution to dq (fp32 [n_q,H,d]) and
    returns dkv (fp32 [2,n_kv,H_kv,d]: this step's dk, dv) together with dq."""
    _dev(q_shard, "q_shard", torch.bfloat16)
    if q_shard.dim() != 3 or kv_chunk.dim() != 4:
        raise LBError("q_shard must be [n_q, H, d] and kv_chunk [2, n_kv, H_kv, d]")
    n_q, H, d = q_shard.shape
    _, n_kv, Hkv, _ = kv_chunk.shape
    dev = q_shard.device
    _dev(kv_chunk, "kv_chunk", torch.bfloat16, (2, n_kv, Hkv, d), dev)
    _dev(dout, "dout", torch.bfloat16, (n_q, H, d), dev)
    _dev(lse, "lse", torch.float32, (H, n_q), dev)
    _dev(dvec, "dvec", torch.float32, (H, n_q), dev)
    _dev(dq, "dq", torch.float32, (n_q, H, d), dev)
    _meta(q_pos, q_doc, n_q, "q", dev)
    _meta(kv_pos, kv_doc, n_kv, "kv", dev)
    if dkv is None:
        dkv = torch.empty((2, n_kv, Hkv, d), dtype=torch.float32, device=dev)
    _dev(dkv, "dkv", torch.float32, (2, n_kv, Hkv, d), dev)
    owned = workspace is None
    if owned:
        half = workspace_bytes(max(n_q, n_kv), max(n_q, n_kv, 1), H, Hkv)
        workspace = torch.empty(2 * half + 512, dtype=torch.uint8, device=dev)
    _ws(workspace, device=dev)
    _gpu(q_shard, "q_shard")
    _check(lib().lb_block_attn_bwd(_ptr(q_shard), n_q, _ptr(kv_chunk), n_kv, _ptr(dout), _ptr(lse), _ptr(dvec),
                                   _ptr(q_pos), _ptr(kv_pos), _ptr(q_doc), _ptr(kv_doc), H, Hkv, d, int(shared_doc),
                                   _ptr(dq),
                                   _ptr(dkv), _ptr(workspace), workspace.numel(), ctypes.c_void_p(_stream(stream))),
           "lb_block_attn_bwd")
    if owned:
        _raise_bwd_device_error(workspace, True, n_q, n_kv, max(n_q, n_kv, 1), H, Hkv, "lb_block_attn_bwd", stream)
    return dq, dkv


# --------------------------------------------------------------------------
# slice-list masks
# --------------------------------------------------------------------------
def _slice_tensor(slices, device):
    """slices: an int32 tensor [n, 5] (q_start, q_len, k_start, k_len, kind) on the device, or a
    list of such tuples (copied to the device)."""
    if isinstance(slices, torch.Tensor):
        if slices.dtype != torch.int32 or slices.dim() != 2 or slices.shape[1] != 5 or not slices.is_contiguous():
            raise LBError("slices must be a contiguous int32 tensor of shape [n, 5]")
        return slices
    return torch.tensor([list(x) for x in slices], dtype=torch.int32, device=device).reshape(-1, 5)


def plan_slices(slices, n_q, n_kv, heads, kv_heads, d, workspace=None, stream=None):
    """The plan of a slice-list mask into ``workspace`` (run it with attn_run)."""
    sl = _slice_tensor(slices, "cuda" if workspace is None else workspace.device)
    _dev(sl, "slices", torch.int32)
    if workspace is None:
        workspace = new_workspace(n_q, 2 * sl.shape[0] + 1, heads, kv_heads, sl.device)
    _ws(workspace, device=sl.device)
    _gpu(sl, "sl")
    _check(lib().lb_plan_slices(_ptr(sl), sl.shape[0], n_q, n_kv, heads, kv_heads, d, _ptr(workspace),
                                workspace.numel(), ctypes.c_void_p(_stream(stream))), "lb_plan_slices")
    return workspace


def slices_attn_fwd(q, k, v, slices, out=None, lse=None, workspace=None, stream=None):
    """out [n_q,H,d] bf16 and lse [H,n_q] of q against k/v under a slice-list mask."""
    _dev(q, "q", torch.bfloat16)
    if q.dim() != 3 or k.dim() != 3:
        raise LBError("q must be [n_q, H, d] and k, v [n_kv, H_kv, d]")
    n_q, H, d = q.shape
    n_kv, Hkv = k.shape[0], k.shape[1]
    dev = q.device
    _dev(k, "k", torch.bfloat16, (n_kv, Hkv, d), dev)
    _dev(v, "v", torch.bfloat16, (n_kv, Hkv, d), dev)
    sl = _slice_tensor(slices, dev)
    _dev(sl, "slices", torch.int32, device=dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, n_q), dtype=torch.float32, device=dev)
    _dev(out, "out", torch.bfloat16, (n_q, H, d), dev)
    _dev(lse, "lse", torch.float32, (H, n_q), dev)
    owned = workspace is None
    if owned:
        workspace = new_workspace(n_q, 2 * sl.shape[0] + 1, H, Hkv, dev)
    _ws(workspace, device=dev)
    _gpu(q, "q")
    _check(lib().lb_slices_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(sl), sl.shape[0], n_q, n_kv, H, Hkv, d, _ptr(out),
                                    _ptr(lse), _ptr(workspace), workspace.numel(), ctypes.c_void_p(_stream(stream))),
           "lb_slices_attn_fwd")
    if owned:
        _raise_device_error(workspace, "lb_slices_attn_fwd", stream)
    return out, lse
