"""Thin ctypes binding of libdecode_attention.so (include/decode_attention.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the current
stream; nothing here computes on tensor data.  If the shared library has not
been built the first call raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdecode_attention.so")

DA_OK, DA_ERR_INVALID_ARG, DA_ERR_UNSUPPORTED, DA_ERR_WORKSPACE, DA_ERR_HIP = 0, -1, -2, -3, -4
DA_F32, DA_BF16 = 0, 1
DA_MASK_NONE, DA_MASK_CAUSAL = 0, 1
DA_MAX_PARTITIONS = 1024
MLA_DEPTH, MLA_DEPTH_V = 576, 512

EXPORTS = ("decode_attention_status_string", "decode_num_partitions", "decode_workspace_size",
           "decode_workspace_o_offset", "decode_workspace_max_offset",
           "decode_workspace_sum_offset", "decode_attention", "decode_attention_ragged",
           "decode_attention_fp8kv", "decode_attention_fp8kv_partials", "mla_decode_ragged",
           "decode_attention_partials", "mla_decode", "mla_decode_partials", "mla_decode_fp8kv",
           "mla_decode_fp8kv_partials", "mla_decode_sparse",
           "mla_decode_sparse_partials", "mla_sparse_num_partitions", "splitk_reduce",
           "decode_attention_ragged_kv", "mla_decode_ragged_kv", "decode_attention_no_alloc")
DA_NO_ALLOC_SCRATCH_BYTES = 32 << 20

_lock = threading.Lock()
_lib = None


class DecodeAttentionError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} ({status})")
        self.status = status


def _declare(lib):
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.decode_attention_status_string.argtypes = [i32]
    lib.decode_attention_status_string.restype = ctypes.c_char_p
    lib.decode_num_partitions.argtypes = [i32] * 9
    lib.decode_num_partitions.restype = i32
    for name in ("decode_workspace_size", "decode_workspace_o_offset",
                 "decode_workspace_max_offset", "decode_workspace_sum_offset"):
        getattr(lib, name).argtypes = [i32] * 5
        getattr(lib, name).restype = sz
    lib.decode_attention.argtypes = [vp, vp, vp, vp, i32, i32, vp, i32, i32, i32, i32, i32, i32,
                                     f32, i32, vp, i32, i32, vp, vp, vp, sz, vp]
    lib.decode_attention.restype = i32
    lib.decode_attention_partials.argtypes = [vp, vp, vp, vp, i32, i32, vp, i32, i32, i32, i32,
                                              i32, i32, f32, i32, i32, i32, vp, sz, vp]
    lib.decode_attention_partials.restype = i32
    lib.decode_attention_ragged.argtypes = [vp, vp, i32, i32, vp, vp, vp, i32, i32, vp, i32, i32,
                                            i32, i32, i32, f32, i32, vp, i32, i32, vp, vp, vp, sz,
                                            vp]
    lib.decode_attention_ragged.restype = i32
    lib.mla_decode_ragged.argtypes = [vp, vp, i32, i32, vp, vp, i32, i32, vp, i32, i32, i32, f32,
                                      i32, vp, i32, vp, vp, vp, sz, vp]
    lib.mla_decode_ragged.restype = i32
    lib.decode_attention_fp8kv.argtypes = [vp, vp, vp, f32, f32, vp, i32, i32, vp, i32, i32, i32,
                                           i32, i32, i32, f32, i32, vp, i32, vp, vp, vp, sz, vp]
    lib.decode_attention_fp8kv.restype = i32
    lib.decode_attention_fp8kv_partials.argtypes = [vp, vp, vp, f32, f32, vp, i32, i32, vp, i32,
                                                    i32, i32, i32, i32, i32, f32, i32, i32, vp,
                                                    sz, vp]
    lib.decode_attention_fp8kv_partials.restype = i32
    lib.mla_decode.argtypes = [vp, vp, vp, i32, i32, vp, i32, i32, i32, i32, f32, i32, vp, i32,
                               vp, vp, vp, sz, vp]
    lib.mla_decode.restype = i32
    lib.mla_decode_partials.argtypes = [vp, vp, vp, i32, i32, vp, i32, i32, i32, i32, f32, i32,
                                        i32, vp, sz, vp]
    lib.mla_decode_partials.restype = i32
    lib.mla_decode_fp8kv.argtypes = [vp, vp, f32, vp, i32, i32, vp, i32, i32, i32, i32, f32,
                                     i32, vp, i32, vp, vp, vp, sz, vp]
    lib.mla_decode_fp8kv.restype = i32
    lib.mla_decode_fp8kv_partials.argtypes = [vp, vp, f32, vp, i32, i32, vp, i32, i32, i32, i32,
                                              f32, i32, i32, vp, sz, vp]
    lib.mla_decode_fp8kv_partials.restype = i32
    i64 = ctypes.c_longlong
    lib.mla_decode_sparse.argtypes = [vp, vp, i64, vp, i32, vp, i32, i32, i32, f32, i32, vp, vp,
                                      vp, vp, sz, vp]
    lib.mla_decode_sparse.restype = i32
    lib.mla_decode_sparse_partials.argtypes = [vp, vp, i64, vp, i32, vp, i32, i32, i32, f32,
                                               i32, vp, sz, vp]
    lib.mla_decode_sparse_partials.restype = i32
    lib.mla_sparse_num_partitions.argtypes = [i32] * 5
    lib.mla_sparse_num_partitions.restype = i32
    lib.splitk_reduce.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp, i32, vp, vp]
    lib.splitk_reduce.restype = i32
    lib.decode_attention_ragged_kv.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                               f32, i32, vp, i32, i32, vp, vp, vp, sz, vp]
    lib.decode_attention_ragged_kv.restype = i32
    lib.mla_decode_ragged_kv.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp, i32,
                                         vp, vp, vp, sz, vp]
    lib.mla_decode_ragged_kv.restype = i32
    lib.decode_attention_no_alloc.argtypes = [vp, vp, vp, vp, i32, i32, vp, i32, i32, i32, i32,
                                              i32, i32, f32, i32, vp, i32, i32, vp, vp, vp]
    lib.decode_attention_no_alloc.restype = i32
    return lib


def library():
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                                   "(python -m decode_attention_07_amd.build)")
            _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def status_string(status: int) -> str:
    return library().decode_attention_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != DA_OK:
        raise DecodeAttentionError(status, where)


class BoundCall:
    """A checked and marshalled C call.  Calling it enqueues the same call again
    (same buffers, same stream) with a single ctypes call and no Python-side
    argument handling, so that a loop of launches is not bound by the host.  It
    keeps the tensors it points into alive."""

    __slots__ = ("fn", "args", "where", "result", "keep")

    def __init__(self, fn, args, where, result, keep):
        self.fn = fn
        self.args = tuple(t(a) if a is not None else None for t, a in zip(fn.argtypes, args))
        self.where = where
        self.result = result
        self.keep = keep

    def __call__(self):
        rc = self.fn(*self.args)
        if rc != DA_OK:
            raise DecodeAttentionError(rc, self.where)
        return self.result


def _finish(fn, args, where, result, keep, prepare):
    call = BoundCall(fn, args, where, result, keep)
    return call if prepare else call()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DA_BF16
    if t.dtype == torch.float32:
        return DA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _need(t, name, dims=None, dtype=None, shape=None, device=None):
    """Checks an array argument; None passes: dimensions, shape, dtype, contiguity
    and (given `device`) the device it shares with the call's other arrays."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dimensions, got {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype not in dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _need_cuda(t, name):
    """The call's anchor tensor (every other array was checked to share its
    device) must live on a GPU: checked after the shapes."""
    if not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA/HIP tensor")


def _need_outputs(out, lse, out_shape, out_dtype, lse_shape, device):
    """Caller-supplied out / lse: exact shape, the output dtype / float32, contiguous,
    on the inputs' device."""
    _need(out, "out", dtype=(out_dtype,), shape=out_shape, device=device)
    _need(lse, "lse", dtype=(torch.float32,), shape=lse_shape, device=device)


def _need_per_sequence(valid_length, sink_weights, batch, num_q_heads, device):
    _need(valid_length, "valid_length", 1, _U32, shape=(batch,), device=device)
    _need(sink_weights, "sink_weights", 1, (torch.float32,), shape=(num_q_heads,),
          device=device)


_U32 = (torch.int32, torch.uint32)


def num_partitions(batch, q_len, num_q_heads, num_kv_heads, depth, depth_v, max_seq_len,
                   ragged=False, num_cus=0) -> int:
    p = library().decode_num_partitions(batch, q_len, num_q_heads, num_kv_heads, depth, depth_v,
                                        max_seq_len, int(bool(ragged)), num_cus)
    if p < 1:
        raise DecodeAttentionError(p, "decode_num_partitions")
    return p


# the C name, for the same-name rule of the binding
decode_num_partitions = num_partitions


def decode_workspace_size(num_partitions, batch, q_len, num_q_heads, depth_v) -> int:
    return int(library().decode_workspace_size(num_partitions, batch, q_len, num_q_heads,
                                               depth_v))


def workspace_views(workspace: torch.Tensor, num_partitions, batch, q_len, num_q_heads, depth_v):
    """(part_o, part_max, part_sum) float32 views of a workspace (layout of the header)."""
    lib = library()
    rows = batch * q_len * num_q_heads
    oo = lib.decode_workspace_o_offset(num_partitions, batch, q_len, num_q_heads, depth_v)
    mo = lib.decode_workspace_max_offset(num_partitions, batch, q_len, num_q_heads, depth_v)
    so = lib.decode_workspace_sum_offset(num_partitions, batch, q_len, num_q_heads, depth_v)
    n = num_partitions * rows
    po = workspace[oo: oo + n * depth_v * 4].view(torch.float32).view(num_partitions, rows,
                                                                      depth_v)
    pm = workspace[mo: mo + n * 4].view(torch.float32).view(num_partitions, rows)
    ps = workspace[so: so + n * 4].view(torch.float32).view(num_partitions, rows)
    return po, pm, ps


def _cache_geometry(q, k, page_table, max_seq_len, batch=None):
    nb = q.shape[0] if batch is None else batch
    if page_table is not None:
        _need(page_table, "page_table", 2, _U32, device=q.device)
        if page_table.shape[0] < nb:
            raise ValueError(f"page_table has {page_table.shape[0]} rows for {nb} sequences")
        page_size, max_pages = k.shape[1], page_table.shape[1]
        S = page_size * max_pages if max_seq_len is None else int(max_seq_len)
    else:
        page_size, max_pages = 0, 0
        S = k.shape[1]
        if max_seq_len is not None and int(max_seq_len) != S:
            raise ValueError("dense cache: max_seq_len must equal k.shape[1]")
        if k.shape[0] != (q.shape[0] if batch is None else batch):
            raise ValueError("dense cache batch must match q")
    return page_size, max_pages, S


def _resolve_partitions(num_parts, batch, T, H, KVH, D, Dv, S, ragged):
    if num_parts is None or num_parts == 0:
        return num_partitions(batch, T, H, KVH, D, Dv, S, ragged)
    return int(num_parts)


def _workspace(workspace, P, B, T, H, Dv, device, always=False):
    if workspace is not None:
        _need(workspace, "workspace", device=device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    need = decode_workspace_size(P, B, T, H, Dv)
    if P == 1 and not always:
        return workspace, nbytes
    if workspace is None:  # zero-filled: the work-queue word starts at 0
        workspace = torch.zeros(need, dtype=torch.uint8, device=device)
        nbytes = need
    elif nbytes < need:
        raise ValueError(f"workspace has {nbytes} bytes, needs {need}")
    return workspace, nbytes


def _kv_like(k, v):
    """v must match k's shape (the V cache mirrors the K cache's layout)."""
    if v is not None and tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"v has shape {tuple(v.shape)}, k {tuple(k.shape)}")


def _mha_inputs(q, k, v, group, kv_dims=4, kv_dtype=None):
    """q, k, v of a GQA call: shapes, dtypes, one device.  Returns the dtype code."""
    qd = q.dim() if isinstance(q, torch.Tensor) else None
    _need(q, "q", qd if qd in (3, 4) else 4, (torch.bfloat16,) if kv_dtype else None)
    _need(k, "k", kv_dims, kv_dtype, device=q.device)
    _need(v, "v", kv_dims, kv_dtype, device=q.device)
    _kv_like(k, v)
    dt = _dtype_code(q)
    if kv_dtype is None and (k.dtype != q.dtype or v.dtype != q.dtype):
        raise TypeError("q, k, v must share a dtype")
    D, H = q.shape[-1], q.shape[-2]
    if group < 1 or H % group or k.shape[-1] != D or k.shape[-2] * group != H:
        raise ValueError("k/v shape does not match q and group")
    return dt


def _mla_inputs(q, kv, kv_dims=4, kv_dtype=(torch.bfloat16,)):
    qd = q.dim() if isinstance(q, torch.Tensor) else None
    _need(q, "q", qd if qd in (3, 4) else 4, (torch.bfloat16,))
    _need(kv, "kv", kv_dims, kv_dtype, device=q.device)
    if q.shape[-1] != MLA_DEPTH or kv.shape[-1] != MLA_DEPTH or kv.shape[-2] != 1:
        raise ValueError("MLA needs q [..., 576] and kv [..., 1, 576]")


def _mask(causal):
    return DA_MASK_CAUSAL if causal else DA_MASK_NONE


def decode_attention(q, k, v, *, group, scale, page_table=None, valid_length=None,
                     max_seq_len=None, num_partitions=0, sink_weights=None, causal=False,
                     out=None, lse=None, workspace=None, stream=None, want_lse=True,
                     prepare=False):
    """GQA/MHA decode attention.  Returns (out [B,T,H,D], lse [B,T,H] or None);
    with prepare=True, a BoundCall that enqueues this call and returns them."""
    dt = _mha_inputs(q, k, v, group)
    B, T, H, D = q.shape
    _need_per_sequence(valid_length, sink_weights, B, H, q.device)
    _need_outputs(out, lse, (B, T, H, D), q.dtype, (B, T, H), q.device)
    page_size, max_pages, S = _cache_geometry(q, k, page_table, max_seq_len)
    _need_cuda(q, "q")
    P = _resolve_partitions(num_partitions, B, T, H, H // group, D, D, S,
                            valid_length is not None)
    if out is None:
        out = torch.empty((B, T, H, D), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    workspace, wbytes = _workspace(workspace, P, B, T, H, D, q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(page_table), page_size, max_pages,
            _ptr(valid_length), B, T, H, group, D, S, float(scale), P, _ptr(sink_weights),
            _mask(causal), dt, _ptr(out), _ptr(lse), _ptr(workspace), wbytes, _stream(stream))
    return _finish(library().decode_attention, args, "decode_attention", (out, lse),
                   (q, k, v, page_table, valid_length, sink_weights, out, lse, workspace),
                   prepare)


def decode_attention_no_alloc(q, k, v, *, group, scale, out, lse=None, page_table=None,
                              valid_length=None, max_seq_len=None, num_partitions=0,
                              sink_weights=None, causal=False, stream=None, prepare=False):
    """decode_attention() for callers that cannot allocate: the split-K workspace is
    the library's static per-device scratch (calls on one device must not overlap),
    and out (and lse, if wanted) are the caller's -- nothing is allocated here either.
    Returns (out, lse); with prepare=True a BoundCall."""
    dt = _mha_inputs(q, k, v, group)
    B, T, H, D = q.shape
    if out is None:
        raise ValueError("out is required (this entry point allocates nothing)")
    _need_per_sequence(valid_length, sink_weights, B, H, q.device)
    _need_outputs(out, lse, (B, T, H, D), q.dtype, (B, T, H), q.device)
    page_size, max_pages, S = _cache_geometry(q, k, page_table, max_seq_len)
    _need_cuda(q, "q")
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(page_table), page_size, max_pages,
            _ptr(valid_length), B, T, H, group, D, S, float(scale), int(num_partitions),
            _ptr(sink_weights), _mask(causal), dt, _ptr(out), _ptr(lse), _stream(stream))
    return _finish(library().decode_attention_no_alloc, args, "decode_attention_no_alloc",
                   (out, lse), (q, k, v, page_table, valid_length, sink_weights, out, lse),
                   prepare)


def decode_attention_partials(q, k, v, *, group, scale, num_partitions, page_table=None,
                              valid_length=None, max_seq_len=None, causal=False, workspace=None,
                              stream=None, prepare=False):
    """Partition pass only.  Returns the workspace (uint8 tensor, header layout), or
    with prepare=True a BoundCall that enqueues the pass and returns it."""
    dt = _mha_inputs(q, k, v, group)
    B, T, H, D = q.shape
    _need_per_sequence(valid_length, None, B, H, q.device)
    page_size, max_pages, S = _cache_geometry(q, k, page_table, max_seq_len)
    _need_cuda(q, "q")
    P = int(num_partitions)
    workspace, wbytes = _workspace(workspace, P, B, T, H, D, q.device, always=True)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(page_table), page_size, max_pages,
            _ptr(valid_length), B, T, H, group, D, S, float(scale), P, _mask(causal), dt,
            _ptr(workspace), wbytes, _stream(stream))
    return _finish(library().decode_attention_partials, args, "decode_attention_partials",
                   workspace, (q, k, v, page_table, valid_length, workspace), prepare)


def _ragged_q(q, q_offsets, max_q_len):
    _need(q, "q", 3)
    _need(q_offsets, "q_offsets", 1, _U32, device=q.device)
    if q_offsets is None or q_offsets.shape[0] < 1:
        raise ValueError("q_offsets [batch + 1] is required")
    if max_q_len is None or int(max_q_len) < 1:
        raise ValueError("max_q_len (an upper bound of every sequence's tokens) is required")
    return q_offsets.shape[0] - 1, int(max_q_len)


def decode_attention_ragged(q, q_offsets, k, v, *, max_q_len, group, scale, page_table=None,
                            valid_length=None, max_seq_len=None, num_partitions=0,
                            sink_weights=None, causal=False, out=None, lse=None, workspace=None,
                            stream=None, want_lse=True, prepare=False):
    """GQA/MHA decode with a ragged q [total, H, D]: the tokens of sequence b are rows
    q_offsets[b] .. q_offsets[b+1].  Returns (out [total, H, D], lse [total, H])."""
    B, Tm = _ragged_q(q, q_offsets, max_q_len)
    dt = _mha_inputs(q, k, v, group)
    total, H, D = q.shape
    _need_per_sequence(valid_length, sink_weights, B, H, q.device)
    _need_outputs(out, lse, (total, H, D), q.dtype, (total, H), q.device)
    page_size, max_pages, S = _cache_geometry(q, k, page_table, max_seq_len, batch=B)
    _need_cuda(q, "q")
    P = _resolve_partitions(num_partitions, B, Tm, H, H // group, D, D, S,
                            valid_length is not None)
    if out is None:
        out = torch.empty((total, H, D), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((total, H), dtype=torch.float32, device=q.device)
    workspace, wbytes = _workspace(workspace, P, 1, total, H, D, q.device)
    args = (_ptr(q), _ptr(q_offsets), total, Tm, _ptr(k), _ptr(v), _ptr(page_table), page_size,
            max_pages, _ptr(valid_length), B, H, group, D, S, float(scale), P,
            _ptr(sink_weights), _mask(causal), dt, _ptr(out), _ptr(lse), _ptr(workspace),
            wbytes, _stream(stream))
    return _finish(library().decode_attention_ragged, args, "decode_attention_ragged",
                   (out, lse), (q, q_offsets, k, v, page_table, valid_length, sink_weights, out,
                                lse, workspace), prepare)


def mla_decode_ragged(q, q_offsets, kv, *, max_q_len, scale, page_table=None,
                      valid_length=None, max_seq_len=None, num_partitions=0, sink_weights=None,
                      causal=False, out=None, lse=None, workspace=None, stream=None,
                      want_lse=True, prepare=False):
    """MLA decode with a ragged q [total, H, 576].  Returns (out [total, H, 512],
    lse [total, H])."""
    B, Tm = _ragged_q(q, q_offsets, max_q_len)
    _mla_inputs(q, kv)
    total, H, D = q.shape
    _need_per_sequence(valid_length, sink_weights, B, H, q.device)
    _need_outputs(out, lse, (total, H, MLA_DEPTH_V), q.dtype, (total, H), q.device)
    page_size, max_pages, S = _cache_geometry(q, kv, page_table, max_seq_len, batch=B)
    _need_cuda(q, "q")
    P = _resolve_partitions(num_partitions, B, Tm, H, 1, MLA_DEPTH, MLA_DEPTH_V, S,
                            valid_length is not None)
    if out is None:
        out = torch.empty((total, H, MLA_DEPTH_V), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((total, H), dtype=torch.float32, device=q.device)
    workspace, wbytes = _workspace(workspace, P, 1, total, H, MLA_DEPTH_V, q.device)
    args = (_ptr(q), _ptr(q_offsets), total, Tm, _ptr(kv), _ptr(page_table), page_size,
            max_pages, _ptr(valid_length), B, H, S, float(scale), P, _ptr(sink_weights),
            _mask(causal), _ptr(out), _ptr(lse), _ptr(workspace), wbytes, _stream(stream))
    return _finish(library().mla_decode_ragged, args, "mla_decode_ragged", (out, lse),
                   (q, q_offsets, kv, page_table, valid_length, sink_weights, out, lse,
                    workspace), prepare)


def _kv_offsets(kv_row_offsets, batch, device):
    _need(kv_row_offsets, "kv_row_offsets", 1, _U32, shape=(batch,), device=device)
    if kv_row_offsets is None and batch > 0:
        raise ValueError("kv_row_offsets [batch] is required")


def decode_attention_ragged_kv(q, k, v, kv_row_offsets, *, group, scale, max_seq_len,
                               valid_length=None, num_partitions=0, sink_weights=None,
                               causal=False, out=None, lse=None, workspace=None, stream=None,
                               want_lse=True, prepare=False):
    """GQA/MHA decode over a ragged KV layout: k, v are one cache [rows, KVH, D] and key
    j of sequence b is row kv_row_offsets[b] + j.  Returns (out [B,T,H,D], lse [B,T,H])."""
    dt = _mha_inputs(q, k, v, group, kv_dims=3)
    B, T, H, D = q.shape
    _kv_offsets(kv_row_offsets, B, q.device)
    _need_per_sequence(valid_length, sink_weights, B, H, q.device)
    _need_outputs(out, lse, (B, T, H, D), q.dtype, (B, T, H), q.device)
    _need_cuda(q, "q")
    S = int(max_seq_len)
    P = _resolve_partitions(num_partitions, B, T, H, H // group, D, D, S,
                            valid_length is not None)
    if out is None:
        out = torch.empty((B, T, H, D), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    workspace, wbytes = _workspace(workspace, P, B, T, H, D, q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(kv_row_offsets), _ptr(valid_length), B, T, H, group,
            D, S, float(scale), P, _ptr(sink_weights), _mask(causal), dt, _ptr(out), _ptr(lse),
            _ptr(workspace), wbytes, _stream(stream))
    return _finish(library().decode_attention_ragged_kv, args, "decode_attention_ragged_kv",
                   (out, lse), (q, k, v, kv_row_offsets, valid_length, sink_weights, out, lse,
                                workspace), prepare)


def mla_decode_ragged_kv(q, kv, kv_row_offsets, *, scale, max_seq_len, valid_length=None,
                         num_partitions=0, sink_weights=None, causal=False, out=None, lse=None,
                         workspace=None, stream=None, want_lse=True, prepare=False):
    """MLA decode over a ragged KV layout: kv is one cache [rows, 1, 576] and key j of
    sequence b is row kv_row_offsets[b] + j.  Returns (out [B,T,H,512], lse [B,T,H])."""
    _mla_inputs(q, kv, kv_dims=3)
    B, T, H, D = q.shape
    _kv_offsets(kv_row_offsets, B, q.device)
    _need_per_sequence(valid_length, sink_weights, B, H, q.device)
    _need_outputs(out, lse, (B, T, H, MLA_DEPTH_V), q.dtype, (B, T, H), q.device)
    _need_cuda(q, "q")
    S = int(max_seq_len)
    P = _resolve_partitions(num_partitions, B, T, H, 1, MLA_DEPTH, MLA_DEPTH_V, S,
                            valid_length is not None)
    if out is None:
        out = torch.empty((B, T, H, MLA_DEPTH_V), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    workspace, wbytes = _workspace(workspace, P, B, T, H, MLA_DEPTH_V, q.device)
    args = (_ptr(q), _ptr(kv), _ptr(kv_row_offsets), _ptr(valid_length), B, T, H, S,
            float(scale), P, _ptr(sink_weights), _mask(causal), _ptr(out), _ptr(lse),
            _ptr(workspace), wbytes, _stream(stream))
    return _finish(library().mla_decode_ragged_kv, args, "mla_decode_ragged_kv", (out, lse),
                   (q, kv, kv_row_offsets, valid_length, sink_weights, out, lse, workspace),
                   prepare)


_FP8 = (torch.uint8, torch.float8_e4m3fn)


def decode_attention_fp8kv(q, k, v, *, k_scale, v_scale, group, scale, page_table=None,
                           valid_length=None, max_seq_len=None, num_partitions=0,
                           sink_weights=None, causal=False, out=None, lse=None, workspace=None,
                           stream=None, want_lse=True, prepare=False):
    """GQA/MHA decode attention over an 8-bit e4m3 KV cache (k, v: uint8 bits or
    float8_e4m3fn; real key = k_scale * k, real value = v_scale * v); q and out
    bf16.  Returns (out, lse), or with prepare=True a BoundCall."""
    _mha_inputs(q, k, v, group, kv_dtype=_FP8)
    B, T, H, D = q.shape
    _need_per_sequence(valid_length, sink_weights, B, H, q.device)
    _need_outputs(out, lse, (B, T, H, D), q.dtype, (B, T, H), q.device)
    page_size, max_pages, S = _cache_geometry(q, k, page_table, max_seq_len)
    _need_cuda(q, "q")
    P = _resolve_partitions(num_partitions, B, T, H, H // group, D, D, S,
                            valid_length is not None)
    if out is None:
        out = torch.empty((B, T, H, D), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    workspace, wbytes = _workspace(workspace, P, B, T, H, D, q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), float(k_scale), float(v_scale), _ptr(page_table),
            page_size, max_pages, _ptr(valid_length), B, T, H, group, D, S, float(scale), P,
            _ptr(sink_weights), _mask(causal), _ptr(out), _ptr(lse), _ptr(workspace), wbytes,
            _stream(stream))
    return _finish(library().decode_attention_fp8kv, args, "decode_attention_fp8kv", (out, lse),
                   (q, k, v, page_table, valid_length, sink_weights, out, lse, workspace),
                   prepare)


def decode_attention_fp8kv_partials(q, k, v, *, k_scale, v_scale, group, scale, num_partitions,
                                    page_table=None, valid_length=None, max_seq_len=None,
                                    causal=False, workspace=None, stream=None, prepare=False):
    """Partition pass of decode_attention_fp8kv() only.  Returns the workspace, or
    with prepare=True a BoundCall."""
    _mha_inputs(q, k, v, group, kv_dtype=_FP8)
    B, T, H, D = q.shape
    _need_per_sequence(valid_length, None, B, H, q.device)
    page_size, max_pages, S = _cache_geometry(q, k, page_table, max_seq_len)
    _need_cuda(q, "q")
    P = int(num_partitions)
    workspace, wbytes = _workspace(workspace, P, B, T, H, D, q.device, always=True)
    args = (_ptr(q), _ptr(k), _ptr(v), float(k_scale), float(v_scale), _ptr(page_table),
            page_size, max_pages, _ptr(valid_length), B, T, H, group, D, S, float(scale), P,
            _mask(causal), _ptr(workspace), wbytes, _stream(stream))
    return _finish(library().decode_attention_fp8kv_partials, args,
                   "decode_attention_fp8kv_partials", workspace,
                   (q, k, v, page_table, valid_length, workspace), prepare)


def mla_decode(q, kv, *, scale, page_table=None, valid_length=None, max_seq_len=None,
               num_partitions=0, sink_weights=None, causal=False, out=None, lse=None,
               workspace=None, stream=None, want_lse=True, prepare=False):
    """MLA decode (one KV head, depth 576, V = K[..., :512]).  Returns (out, lse), or
    with prepare=True a BoundCall that enqueues the call and returns them."""
    _mla_inputs(q, kv)
    B, T, H, D = q.shape
    _need_per_sequence(valid_length, sink_weights, B, H, q.device)
    _need_outputs(out, lse, (B, T, H, MLA_DEPTH_V), q.dtype, (B, T, H), q.device)
    page_size, max_pages, S = _cache_geometry(q, kv, page_table, max_seq_len)
    _need_cuda(q, "q")
    P = _resolve_partitions(num_partitions, B, T, H, 1, MLA_DEPTH, MLA_DEPTH_V, S,
                            valid_length is not None)
    if out is None:
        out = torch.empty((B, T, H, MLA_DEPTH_V), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    workspace, wbytes = _workspace(workspace, P, B, T, H, MLA_DEPTH_V, q.device)
    args = (_ptr(q), _ptr(kv), _ptr(page_table), page_size, max_pages, _ptr(valid_length), B, T,
            H, S, float(scale), P, _ptr(sink_weights), _mask(causal), _ptr(out), _ptr(lse),
            _ptr(workspace), wbytes, _stream(stream))
    return _finish(library().mla_decode, args, "mla_decode", (out, lse),
                   (q, kv, page_table, valid_length, sink_weights, out, lse, workspace), prepare)


def mla_decode_partials(q, kv, *, scale, num_partitions, page_table=None, valid_length=None,
                        max_seq_len=None, causal=False, workspace=None, stream=None,
                        prepare=False):
    """MLA partition pass only.  Returns the workspace, or with prepare=True a BoundCall."""
    _mla_inputs(q, kv)
    B, T, H, D = q.shape
    _need_per_sequence(valid_length, None, B, H, q.device)
    page_size, max_pages, S = _cache_geometry(q, kv, page_table, max_seq_len)
    _need_cuda(q, "q")
    P = int(num_partitions)
    workspace, wbytes = _workspace(workspace, P, B, T, H, MLA_DEPTH_V, q.device, always=True)
    args = (_ptr(q), _ptr(kv), _ptr(page_table), page_size, max_pages, _ptr(valid_length), B, T,
            H, S, float(scale), P, _mask(causal), _ptr(workspace), wbytes, _stream(stream))
    return _finish(library().mla_decode_partials, args, "mla_decode_partials", workspace,
                   (q, kv, page_table, valid_length, workspace), prepare)


def mla_decode_fp8kv(q, kv, *, k_scale, scale, page_table=None, valid_length=None,
                     max_seq_len=None, num_partitions=0, sink_weights=None, causal=False,
                     out=None, lse=None, workspace=None, stream=None, want_lse=True,
                     prepare=False):
    """MLA over an 8-bit e4m3 cache (uint8 / float8_e4m3fn [..., 1, 576]; real element =
    k_scale x stored) with bf16 q.  Returns (out, lse), or with prepare=True a BoundCall."""
    _mla_inputs(q, kv, kv_dtype=_FP8)
    B, T, H, D = q.shape
    _need_per_sequence(valid_length, sink_weights, B, H, q.device)
    _need_outputs(out, lse, (B, T, H, MLA_DEPTH_V), q.dtype, (B, T, H), q.device)
    page_size, max_pages, S = _cache_geometry(q, kv, page_table, max_seq_len)
    _need_cuda(q, "q")
    P = _resolve_partitions(num_partitions, B, T, H, 1, MLA_DEPTH, MLA_DEPTH_V, S,
                            valid_length is not None)
    if out is None:
        out = torch.empty((B, T, H, MLA_DEPTH_V), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    workspace, wbytes = _workspace(workspace, P, B, T, H, MLA_DEPTH_V, q.device)
    args = (_ptr(q), _ptr(kv), float(k_scale), _ptr(page_table), page_size, max_pages,
            _ptr(valid_length), B, T, H, S, float(scale), P, _ptr(sink_weights), _mask(causal),
            _ptr(out), _ptr(lse), _ptr(workspace), wbytes, _stream(stream))
    return _finish(library().mla_decode_fp8kv, args, "mla_decode_fp8kv", (out, lse),
                   (q, kv, page_table, valid_length, sink_weights, out, lse, workspace), prepare)


def mla_decode_fp8kv_partials(q, kv, *, k_scale, scale, num_partitions, page_table=None,
                              valid_length=None, max_seq_len=None, causal=False, workspace=None,
                              stream=None, prepare=False):
    """Partition pass of mla_decode_fp8kv() alone.  Returns the workspace, or with
    prepare=True a BoundCall."""
    _mla_inputs(q, kv, kv_dtype=_FP8)
    B, T, H, D = q.shape
    _need_per_sequence(valid_length, None, B, H, q.device)
    page_size, max_pages, S = _cache_geometry(q, kv, page_table, max_seq_len)
    _need_cuda(q, "q")
    P = int(num_partitions)
    workspace, wbytes = _workspace(workspace, P, B, T, H, MLA_DEPTH_V, q.device, always=True)
    args = (_ptr(q), _ptr(kv), float(k_scale), _ptr(page_table), page_size, max_pages,
            _ptr(valid_length), B, T, H, S, float(scale), P, _mask(causal), _ptr(workspace),
            wbytes, _stream(stream))
    return _finish(library().mla_decode_fp8kv_partials, args, "mla_decode_fp8kv_partials",
                   workspace, (q, kv, page_table, valid_length, workspace), prepare)


def mla_sparse_num_partitions(batch, q_len, num_q_heads, topk, num_cus=0) -> int:
    p = library().mla_sparse_num_partitions(batch, q_len, num_q_heads, topk, num_cus)
    if p < 1:
        raise DecodeAttentionError(p, "mla_sparse_num_partitions")
    return p


def _sparse_args(q, kv, indices, topk_lengths):
    _need(q, "q", 4, (torch.bfloat16,))
    _need(kv, "kv", 3, (torch.bfloat16,), device=q.device)
    B, T, H, D = q.shape
    if D != MLA_DEPTH or kv.shape[1] != 1 or kv.shape[2] != MLA_DEPTH:
        raise ValueError("sparse MLA needs q [..., 576] and a pool kv [rows, 1, 576]")
    _need(indices, "indices", 2, (torch.int32,), device=q.device)
    _need(topk_lengths, "topk_lengths", 1, (torch.int32,), shape=(B,), device=q.device)
    if indices is None or topk_lengths is None or indices.shape[0] != B:
        raise ValueError("indices [B, stride] and topk_lengths [B] must match q's batch")
    return B, T, H, kv.shape[0], indices.shape[1]


def mla_decode_sparse(q, kv, indices, topk_lengths, *, scale, num_partitions=0,
                      sink_weights=None, out=None, lse=None, workspace=None, stream=None,
                      want_lse=True, prepare=False):
    """Sparse top-k MLA: sequence b attends to pool rows indices[b, :topk_lengths[b]]
    of kv [pool_rows, 1, 576].  Returns (out [B,T,H,512], lse [B,T,H]), or with
    prepare=True a BoundCall."""
    B, T, H, R, stride = _sparse_args(q, kv, indices, topk_lengths)
    _need_per_sequence(None, sink_weights, B, H, q.device)
    _need_outputs(out, lse, (B, T, H, MLA_DEPTH_V), q.dtype, (B, T, H), q.device)
    _need_cuda(q, "q")
    P = int(num_partitions) or (mla_sparse_num_partitions(B, T, H, stride) if B else 1)
    if out is None:
        out = torch.empty((B, T, H, MLA_DEPTH_V), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    workspace, wbytes = _workspace(workspace, P, B, T, H, MLA_DEPTH_V, q.device)
    args = (_ptr(q), _ptr(kv), R, _ptr(indices), stride, _ptr(topk_lengths), B, T, H,
            float(scale), P, _ptr(sink_weights), _ptr(out), _ptr(lse), _ptr(workspace), wbytes,
            _stream(stream))
    return _finish(library().mla_decode_sparse, args, "mla_decode_sparse", (out, lse),
                   (q, kv, indices, topk_lengths, sink_weights, out, lse, workspace), prepare)


def mla_decode_sparse_partials(q, kv, indices, topk_lengths, *, scale, num_partitions,
                               workspace=None, stream=None, prepare=False):
    """Partition pass of mla_decode_sparse() alone.  Returns the workspace, or with
    prepare=True a BoundCall."""
    B, T, H, R, stride = _sparse_args(q, kv, indices, topk_lengths)
    _need_cuda(q, "q")
    P = int(num_partitions)
    workspace, wbytes = _workspace(workspace, P, B, T, H, MLA_DEPTH_V, q.device, always=True)
    args = (_ptr(q), _ptr(kv), R, _ptr(indices), stride, _ptr(topk_lengths), B, T, H,
            float(scale), P, _ptr(workspace), wbytes, _stream(stream))
    return _finish(library().mla_decode_sparse_partials, args, "mla_decode_sparse_partials",
                   workspace, (q, kv, indices, topk_lengths, workspace), prepare)


def splitk_reduce(part_o, part_max, part_sum, *, num_q_heads, sink_weights=None,
                  out_dtype=torch.bfloat16, out=None, lse=None, stream=None, want_lse=True,
                  prepare=False):
    """LSE merge of partials [P, rows, Dv] / [P, rows] -> (out [rows, Dv], lse [rows]);
    with prepare=True a BoundCall that enqueues the merge and returns them."""
    _need(part_o, "part_o", 3, (torch.float32,))
    P, rows, Dv = part_o.shape
    dev = part_o.device
    _need(part_max, "part_max", 2, (torch.float32,), shape=(P, rows), device=dev)
    _need(part_sum, "part_sum", 2, (torch.float32,), shape=(P, rows), device=dev)
    _need(sink_weights, "sink_weights", 1, (torch.float32,), shape=(num_q_heads,), device=dev)
    if out is not None:
        out_dtype = out.dtype
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"out dtype {out_dtype}: use bfloat16 or float32")
    _need_outputs(out, lse, (rows, Dv), out_dtype, (rows,), dev)
    _need_cuda(part_o, "part_o")
    if out is None:
        out = torch.empty((rows, Dv), dtype=out_dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((rows,), dtype=torch.float32, device=dev)
    args = (_ptr(part_o), _ptr(part_max), _ptr(part_sum), P, rows, num_q_heads, Dv,
            _ptr(sink_weights), _ptr(out), _dtype_code(out), _ptr(lse), _stream(stream))
    return _finish(library().splitk_reduce, args, "splitk_reduce", (out, lse),
                   (part_o, part_max, part_sum, sink_weights, out, lse), prepare)


# ---- host <-> device marshalling of the seeded numpy inputs ------------------------

def to_device(a: np.ndarray | None, device="cuda"):
    """numpy -> device tensor; uint16 arrays are bfloat16 bit patterns."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).to(device)
    return torch.from_numpy(a).to(device)


def to_numpy_f64(t: torch.Tensor) -> np.ndarray:
    """Device result -> float64 numpy (exact widening)."""
    return t.detach().float().cpu().numpy().astype(np.float64)
