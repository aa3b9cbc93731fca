"""ctypes wrapper around decode_oracle.c, the plain fp64 CPU reference.

TEST INFRASTRUCTURE ONLY.  The product path never imports this module; only the
test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
use it.  It shares nothing with the HIP library except the seeded input arrays it
is handed.

Array conventions (numpy, C-contiguous):
  * float32 arrays are fp32 data; uint16 arrays are bfloat16 bit patterns.
  * q: [B, T, H, D]; k: contiguous [B, S, KVH, D] or page pool
    [num_pages, page_size, KVH, D]; v: same layout with Dv, or None meaning
    V = K[..., :Dv] (the MLA case, "flare_mla_decoding_dispatch", Args ``k``).
  * page_table: uint32 [B, max_pages]; valid_length: uint32 [B]; sink: float32 [H].
  * sparse top-k: k (and v) is a pool [pool_rows, KVH, D]; indices int32 [B, stride]
    lists the pool rows of each sequence's keys, topk_lengths int32 [B] how many
    of them count ("flare_mla_decoding_dispatch", Args ``d_indices``,
    ``indices_stride``, ``topk_lengths``).
  * ragged KV layout: k (and v) is one cache [rows, KVH, D] holding every
    sequence's keys; key j of sequence b is row kv_offsets[b] + j (uint32 [B];
    "mha_sm100_dispatch", Args ``kv_input_row_offsets``); max_seq_len bounds
    every N_b.

Every routine returns float64 results.  The meaning of each argument and the
readings taken where the pages are silent are stated in decode_oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "decode_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False, src: str = _SRC, out: str = _LIB_PATH, extra_flags=()) -> str:
    """Compile decode_oracle.c with gcc (OpenMP) into a shared library."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", "-Wall", "-Werror",
               *extra_flags, src, "-o", out + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)
    return out


def _bind(lib):
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    lib.oracle_decode_attention.argtypes = [vp, vp, vp, i32, f32, f32, vp, i32, i32, vp, i32, i32,
                                            i32, i32, i32, i32, i32, f32, vp, i32, vp, vp, i32, vp,
                                            i64, vp, vp, i64, vp, vp, i32]
    lib.oracle_decode_attention.restype = i32
    lib.oracle_decode_partials.argtypes = [vp, vp, vp, i32, f32, f32, vp, i32, i32, vp, i32, i32,
                                           i32, i32, i32, i32, i32, f32, i32, vp, vp, i32, vp, i64,
                                           vp, i32, i32, vp, vp, vp, i32]
    lib.oracle_decode_partials.restype = i32
    lib.oracle_splitk_merge.argtypes = [vp, vp, vp, i32, i64, i32, i32, vp, vp, vp]
    lib.oracle_splitk_merge.restype = i32
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i32
    return lib


def load_library(path: str | None = None):
    """Load (building first if needed) the oracle library; ``path`` loads another build."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            _lib = _bind(ctypes.CDLL(build()))
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(q, k, v):
    """0: all float32; 1: all bf16 (uint16 bits); 2: q bf16 with k / v in 8-bit
    e4m3 (uint8 bits, dequantised with k_scale / v_scale)."""
    kinds = {a.dtype for a in (q, k, v) if a is not None}
    if kinds == {np.dtype(np.float32)}:
        return 0
    if kinds == {np.dtype(np.uint16)}:
        return 1
    kv = {a.dtype for a in (k, v) if a is not None}
    if q.dtype == np.uint16 and kv == {np.dtype(np.uint8)}:
        return 2
    raise TypeError(f"q/k/v must all be float32, all uint16 (bf16 bits), or bf16 q with uint8 "
                    f"(e4m3 bits) k/v; got {kinds}")


def _contig(a, dtype=None):
    if a is None:
        return None
    a = np.asarray(a) if dtype is None else np.asarray(a, dtype=dtype)
    return np.ascontiguousarray(a)


def _common(q, k, v, page_table, valid_length, sink, depth_v, max_seq_len):
    q, k, v = _contig(q), _contig(k), _contig(v)
    page_table = _contig(page_table, np.uint32)
    valid_length = _contig(valid_length, np.uint32)
    sink = _contig(sink, np.float32)
    code = _dtype_code(q, k, v)
    B, T, H, D = q.shape
    KVH = k.shape[2]
    if k.shape[3] != D:
        raise ValueError("k depth must match q depth")
    Dv = v.shape[3] if v is not None else (depth_v if depth_v is not None else D)
    if page_table is not None:
        page_size, max_pages = k.shape[1], page_table.shape[1]
        S = max_seq_len if max_seq_len is not None else page_size * max_pages
    else:
        page_size, max_pages = 0, 0
        S = k.shape[1]
        if max_seq_len is not None and max_seq_len != S:
            raise ValueError("contiguous cache: max_seq_len must equal k.shape[1]")
    if sink is not None and sink.shape != (H,):
        raise ValueError("sink must have shape [H]")
    return q, k, v, page_table, valid_length, sink, code, (B, T, H, KVH, D, Dv, S, page_size,
                                                           max_pages)


def _ragged(q, q_offsets):
    """Ragged q [total, H, D] with offsets [B+1] -> (q as [1, total, H, D] for the shape
    checks, offsets, B, T = most tokens of a sequence)."""
    if q_offsets is None:
        return q, None, None, None
    qo = np.ascontiguousarray(q_offsets, dtype=np.uint32)
    q = np.asarray(q)
    if q.ndim != 3 or qo.ndim != 1 or qo.shape[0] < 1 or int(qo[-1]) != q.shape[0]:
        raise ValueError("ragged q must be [total, H, D] with offsets [B+1] ending at total")
    B = qo.shape[0] - 1
    T = max(1, int(np.max(np.diff(qo.astype(np.int64)))) if B else 1)
    return q.reshape(1, *q.shape), qo, B, T


def _sparse(k, v, indices, topk_lengths, batch):
    """Sparse top-k: the pool [rows, KVH, D] as [rows, 1, KVH, D] for the shape checks,
    the index list [B, stride], the counts [B], stride and pool rows."""
    if indices is None:
        if topk_lengths is not None:
            raise ValueError("topk_lengths needs indices")
        return k, v, None, None, 0, 0
    k = np.asarray(k)
    if k.ndim != 3 or (v is not None and np.asarray(v).ndim != 3):
        raise ValueError("sparse: k (and v) must be pools [rows, KVH, D]")
    idx = np.ascontiguousarray(indices, dtype=np.int32)
    tl = np.ascontiguousarray(topk_lengths, dtype=np.int32)
    if idx.ndim != 2 or idx.shape[0] != batch or tl.shape != (batch,):
        raise ValueError("sparse: indices must be [B, stride] and topk_lengths [B]")
    k4 = k.reshape(k.shape[0], 1, *k.shape[1:])
    v4 = None if v is None else np.asarray(v).reshape(np.asarray(v).shape[0], 1,
                                                      *np.asarray(v).shape[1:])
    return k4, v4, idx, tl, idx.shape[1], k.shape[0]


def _ragged_kv(k, v, kv_offsets, max_seq_len, batch):
    """Ragged KV layout: the cache [rows, KVH, D] as [rows, 1, KVH, D] for the shape
    checks, the offsets [B], the row count and the key bound S."""
    if kv_offsets is None:
        return k, v, None, 0, max_seq_len
    k = np.asarray(k)
    if k.ndim != 3 or (v is not None and np.asarray(v).ndim != 3):
        raise ValueError("ragged KV layout: k (and v) must be caches [rows, KVH, D]")
    off = np.ascontiguousarray(kv_offsets, dtype=np.uint32)
    if off.shape != (batch,) or max_seq_len is None:
        raise ValueError("ragged KV layout: kv_offsets [B] and max_seq_len are required")
    k4 = k.reshape(k.shape[0], 1, *k.shape[1:])
    v4 = None if v is None else np.asarray(v).reshape(np.asarray(v).shape[0], 1,
                                                      *np.asarray(v).shape[1:])
    return k4, v4, off, k.shape[0], int(max_seq_len)


def attention(q, k, v=None, *, scale, page_table=None, valid_length=None, sink=None,
              causal=False, depth_v=None, max_seq_len=None, rows=None, threads=0, lib=None,
              k_scale=1.0, v_scale=1.0, q_offsets=None, indices=None, topk_lengths=None,
              kv_offsets=None):
    """Reference attention.  Returns (out, lse) as float64.

    q_offsets: ragged q -- q is [total, H, D] and the tokens of sequence b are rows
    q_offsets[b] .. q_offsets[b+1]; out is then [total, H, Dv], lse [total, H].

    k_scale / v_scale: the real key (value) is the scale times the stored element
    (meant for e4m3 k / v; the value slice of MLA, v=None, uses k_scale).

    indices / topk_lengths: sparse top-k -- k (and v) is a pool [pool_rows, KVH, D] and
    the keys of sequence b are its rows indices[b, :topk_lengths[b]] (no mask).

    kv_offsets: ragged KV layout -- k (and v) is a cache [rows, KVH, D] and key j of
    sequence b is its row kv_offsets[b] + j (max_seq_len required).

    With rows=None: out [B, T, H, Dv], lse [B, T, H].  With rows (int64 row ids
    (b*T + t)*H + h): out [len(rows), Dv], lse [len(rows)].
    """
    lib = lib or load_library()
    q, qo, rB, rT = _ragged(q, q_offsets)
    nb = rB if qo is not None else np.shape(q)[0]
    k, v, idx, tl, stride, pool_rows = _sparse(k, v, indices, topk_lengths, nb)
    k, v, kvo, kv_rows, S_kv = _ragged_kv(k, v, kv_offsets, max_seq_len, nb)
    q, k, v, page_table, valid_length, sink, code, dims = _common(
        q, k, v, page_table, valid_length, sink, depth_v, None if kvo is not None else max_seq_len)
    B, T, H, KVH, D, Dv, S, page_size, max_pages = dims
    if idx is not None:
        S = stride
    if kvo is not None:
        S, pool_rows = S_kv, kv_rows
    total = q.shape[0] * q.shape[1]
    if qo is not None:
        B, T = rB, rT
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows.shape[0]
    else:
        n = total * H
    out = np.zeros((n, Dv), np.float64)
    lse = np.zeros((n,), np.float64)
    rc = lib.oracle_decode_attention(_ptr(q), _ptr(k), _ptr(v), code, float(k_scale),
                                     float(v_scale), _ptr(page_table), page_size,
                                     max_pages, _ptr(valid_length), B, T, H, KVH, D, Dv, S,
                                     float(scale), _ptr(sink), int(bool(causal)), _ptr(qo),
                                     _ptr(idx), stride, _ptr(tl), pool_rows, _ptr(kvo), _ptr(rows), n,
                                     _ptr(out), _ptr(lse), int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_decode_attention failed ({rc})")
    if rows is None:
        if qo is not None:
            return out.reshape(total, H, Dv), lse.reshape(total, H)
        return out.reshape(B, T, H, Dv), lse.reshape(B, T, H)
    return out, lse


def partials(q, k, v=None, *, scale, num_partitions, keys_per_partition, page_table=None,
             valid_length=None, causal=False, depth_v=None, max_seq_len=None, threads=0,
             lib=None, k_scale=1.0, v_scale=1.0, q_offsets=None, indices=None,
             topk_lengths=None, kv_offsets=None):
    """Split-K partials.  Returns (O_p [P, rows, Dv], m_p [P, rows], l_p [P, rows]) with
    rows = (q tokens) * H.  Sparse: partition p covers list positions [p*C, (p+1)*C)."""
    lib = lib or load_library()
    q, qo, rB, rT = _ragged(q, q_offsets)
    nb = rB if qo is not None else np.shape(q)[0]
    k, v, idx, tl, stride, pool_rows = _sparse(k, v, indices, topk_lengths, nb)
    k, v, kvo, kv_rows, S_kv = _ragged_kv(k, v, kv_offsets, max_seq_len, nb)
    q, k, v, page_table, valid_length, _, code, dims = _common(
        q, k, v, page_table, valid_length, None, depth_v, None if kvo is not None else max_seq_len)
    B, T, H, KVH, D, Dv, S, page_size, max_pages = dims
    if idx is not None:
        S = stride
    if kvo is not None:
        S, pool_rows = S_kv, kv_rows
    if qo is not None:
        B, T = rB, rT
    rows = q.shape[0] * q.shape[1] * H
    po = np.zeros((num_partitions, rows, Dv), np.float64)
    pm = np.zeros((num_partitions, rows), np.float64)
    pl = np.zeros((num_partitions, rows), np.float64)
    rc = lib.oracle_decode_partials(_ptr(q), _ptr(k), _ptr(v), code, float(k_scale),
                                    float(v_scale), _ptr(page_table), page_size,
                                    max_pages, _ptr(valid_length), B, T, H, KVH, D, Dv, S,
                                    float(scale), int(bool(causal)), _ptr(qo), _ptr(idx), stride,
                                    _ptr(tl), pool_rows, _ptr(kvo), int(num_partitions),
                                    int(keys_per_partition), _ptr(po), _ptr(pm), _ptr(pl),
                                    int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_decode_partials failed ({rc})")
    return po, pm, pl


def merge(part_o, part_m, part_l, *, num_heads, sink=None, lib=None):
    """Log-sum-exp merge of partials.  Returns (out [rows, Dv], lse [rows])."""
    lib = lib or load_library()
    po = np.ascontiguousarray(part_o, dtype=np.float64)
    pm = np.ascontiguousarray(part_m, dtype=np.float64)
    pl = np.ascontiguousarray(part_l, dtype=np.float64)
    P, rows, Dv = po.shape
    sink = _contig(sink, np.float32)
    out = np.zeros((rows, Dv), np.float64)
    lse = np.zeros((rows,), np.float64)
    rc = lib.oracle_splitk_merge(_ptr(po), _ptr(pm), _ptr(pl), P, rows, int(num_heads), Dv,
                                 _ptr(sink), _ptr(out), _ptr(lse))
    if rc != 0:
        raise RuntimeError(f"oracle_splitk_merge failed ({rc})")
    return out, lse


def num_threads() -> int:
    return int(load_library().oracle_num_threads())
