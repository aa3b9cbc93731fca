"""Seeded synthetic inputs for single-query (decode) attention.

This module only draws and lays out input data; it holds none of the attention
arithmetic.  Both the fp64 oracle (in the tests) and the HIP library are fed the
same arrays from here, so that they see identical bits.

Recipe (the same for every workload):
  * numpy PCG64 streams from ``SeedSequence(entropy).spawn(6)``: q, k, v, sink,
    lengths, pages.  ``entropy`` is the workload seed (variant 0) or
    ``[seed, variant]`` for the extra input sets the benchmark rotates through.
  * Large tensors are drawn in fixed 4 Mi-element chunks, each from its own child
    of the tensor's stream, so the result does not depend on the thread count.
  * Values are standard normal float32; bf16 tensors are rounded to the nearest
    bf16 (ties to even) and stored as uint16 bit patterns.
  * Paged caches: pages of ``page_size`` tokens, physical pages assigned by a
    seeded permutation of a shared pool that has one extra NaN-filled poison
    page; unused page-table entries point at the poison page; cache rows past
    a sequence's valid length hold NaN.

The workloads mirror the shapes of the pages' problem statement (q [batch,
q_seq_len, num_heads, depth], a KV cache with KV heads and an optional page
table, uint32 valid lengths, fp32 sink logits; MLA with one KV head, depth 576
and V = K[..., :512]).  No public dataset is involved.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

CHUNK = 1 << 22
BF16_NAN = np.uint16(0x7FC0)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint32)
    bias = (u >> 16) & np.uint32(1)
    bias += np.uint32(0x7FFF)
    u += bias
    out = (u >> 16).astype(np.uint16)
    out[np.isnan(x)] = BF16_NAN
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _fill_chunk(seed_seq, dst_flat, start, stop, as_bf16):
    rng = np.random.Generator(np.random.PCG64(seed_seq))
    x = rng.standard_normal(stop - start, dtype=np.float32)
    if as_bf16:
        u = x.view(np.uint32)
        bias = np.right_shift(u, 16)
        np.bitwise_and(bias, 1, out=bias)
        bias += np.uint32(0x7FFF)
        u += bias
        dst_flat[start:stop] = u.view(np.uint16)[1::2]
    else:
        dst_flat[start:stop] = x


def normal_tensor(seed_seq: np.random.SeedSequence, shape, dtype: str) -> np.ndarray:
    """Standard-normal tensor of ``shape``; dtype 'f32' -> float32, 'bf16' -> uint16 bits."""
    n = int(np.prod(shape)) if len(shape) else 1
    as_bf16 = dtype == "bf16"
    out = np.empty(n, np.uint16 if as_bf16 else np.float32)
    n_chunks = max(1, math.ceil(n / CHUNK))
    children = seed_seq.spawn(n_chunks)
    jobs = [(children[i], i * CHUNK, min(n, (i + 1) * CHUNK)) for i in range(n_chunks)]
    if n_chunks == 1:
        _fill_chunk(jobs[0][0], out, jobs[0][1], jobs[0][2], as_bf16)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(lambda j: _fill_chunk(j[0], out, j[1], j[2], as_bf16), jobs))
    return out.reshape(shape)


@dataclass(frozen=True)
class Workload:
    """One decode-attention problem.  Sizes use the pages' names where they exist."""
    name: str
    seed: int
    batch: int
    num_heads: int            # query heads H
    kv_heads: int             # KV heads; group = num_heads // kv_heads
    depth: int                # QK depth D
    max_seq_len: int          # S: cache length bound (contiguous cache length)
    dtype: str = "bf16"       # 'bf16' or 'f32' for q, k, v and the output
    q_len: int = 1            # T: query tokens per sequence (MTP fold when > 1)
    depth_v: int | None = None  # Dv; None -> depth (MHA); MLA sets 512
    mla: bool = False         # V = K[..., :depth_v], one KV head
    causal: bool = False
    page_size: int = 0        # 0 -> contiguous [B, S, KVH, D]
    ragged: tuple | None = None   # (low, high, forced_ones): N_b ~ U{low..high}
    sink: bool = False
    scale: float | None = None
    num_partitions: int = 0   # 0 = library heuristic
    kv_dtype: str | None = None  # None -> dtype; 'e4m3' -> 8-bit K / V bits (q and out bf16)
    k_scale: float = 1.0      # 8-bit cache: real key = k_scale * stored key
    v_scale: float = 1.0      # 8-bit cache: real value = v_scale * stored value
    topk: int = 0             # sparse top-k MLA: list stride (0 -> keys from the cache)
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def kv_type(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def group(self) -> int:
        return self.num_heads // self.kv_heads

    @property
    def dv(self) -> int:
        return self.depth if self.depth_v is None else self.depth_v

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.depth)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five problem configurations (shapes from the problem statement).
TINY_MHA = Workload("tiny_mha_f32_b1_h8_d64_s256", 7001, batch=1, num_heads=8, kv_heads=8,
                    depth=64, max_seq_len=256, dtype="f32")
GQA = Workload("gqa_bf16_b32_h32_kv8_d128_s4096", 7002, batch=32, num_heads=32, kv_heads=8,
               depth=128, max_seq_len=4096)
PAGED = Workload("paged_ragged_bf16_b64_h64_kv8_d128_s32768_p128", 7003, batch=64,
                 num_heads=64, kv_heads=8, depth=128, max_seq_len=32768, page_size=128,
                 ragged=(1, 32768, 4))
MLA = Workload("mla_bf16_b64_h128_d576_dv512_s8192", 7004, batch=64, num_heads=128, kv_heads=1,
               depth=576, depth_v=512, max_seq_len=8192, mla=True, scale=1.0 / math.sqrt(192))
MLA_MTP = MLA.with_(name="mla_mtp2_bf16_b64_h128_d576_dv512_s8192", q_len=2, causal=True)
LONG = Workload("long_sink_bf16_b1_h32_kv8_d128_s131072", 7005, batch=1, num_heads=32,
                kv_heads=8, depth=128, max_seq_len=131072, sink=True)

# The GQA and ragged paged problems with an 8-bit e4m3 KV cache (stored elements
# e4m3(8 N(0,1)); k_scale = v_scale = 1/8, so the real keys and values are N(0,1)-like).
GQA_FP8 = GQA.with_(name="gqa_fp8_b32_h32_kv8_d128_s4096", kv_dtype="e4m3", k_scale=0.125,
                    v_scale=0.125)
PAGED_FP8 = PAGED.with_(name="paged_ragged_fp8_b64_h64_kv8_d128_s32768_p128", kv_dtype="e4m3",
                        k_scale=0.125, v_scale=0.125)

# Speculative-decode shape of the GQA problem: each sequence brings 1..4 new
# tokens (seeded), causal; q is ragged (rows packed per sequence).
GQA_RAGGED_Q = GQA.with_(name="gqa_ragged_q_b32_h32_kv8_d128_s4096_t1to4", q_len=4, causal=True,
                         extra={"q_tokens": (1, 4)})

# The MLA problem over an 8-bit e4m3 cache (bf16 q; one scale for the stored rows,
# whose first 512 columns are V: stored e4m3(8 N(0,1)), k_scale = 1/8).
MLA_FP8 = MLA.with_(name="mla_fp8_b64_h128_d576_dv512_s8192", kv_dtype="e4m3", k_scale=0.125,
                    v_scale=0.125)

# Sparse top-k MLA (a DeepSeek-style selection of 2048 of each sequence's 8192 cached
# rows): the same 64 sequences and heads as the MLA problem, each attending to its
# own list of 2048 pool rows.
MLA_SPARSE = MLA.with_(name="mla_sparse_bf16_b64_h128_d576_dv512_topk2048_s8192", seed=7006,
                       topk=2048)

ALL = {w.name: w for w in (TINY_MHA, GQA, PAGED, MLA, MLA_MTP, LONG, GQA_FP8, PAGED_FP8,
                           GQA_RAGGED_Q, MLA_SPARSE, MLA_FP8)}


def ragged_q_tokens(wl: Workload):
    """Per-sequence token counts of a ragged-q workload (seeded), or None."""
    rq = wl.extra.get("q_tokens")
    if rq is None:
        return None
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, 77])))
    return rng.integers(rq[0], rq[1], size=wl.batch, endpoint=True).astype(np.int64)


def pack_ragged_q(inp: Inputs, tokens):
    """Ragged q [total, H, D] and offsets [B+1]: the first tokens[b] tokens of each
    sequence of the padded q [B, T, H, D]."""
    qo = np.concatenate([[0], np.cumsum(tokens)]).astype(np.uint32)
    q = np.concatenate([inp.q[b, :int(t)] for b, t in enumerate(tokens)], axis=0)
    return np.ascontiguousarray(q), qo


def ragged_kv_layout(k: np.ndarray, v: np.ndarray | None, lens, seed: int, gap: int = 3):
    """A dense cache [B, S, KVH, D] laid out as one concatenated cache [rows, KVH, D]:
    the valid rows of each sequence, in a seeded random sequence order, with `gap`
    poison rows (NaN) between sequences and after the last one.  Returns (k_cat,
    v_cat, offsets) with offsets uint32 [B] the first row of each sequence."""
    B = k.shape[0]
    lens = np.asarray(lens, np.int64)
    total = gap + int(sum(int(n) + gap for n in lens))
    kind = {np.dtype(np.uint16): "bf16", np.dtype(np.uint8): "e4m3",
            np.dtype(np.float32): "f32"}[k.dtype]
    kc = np.empty((total,) + k.shape[2:], k.dtype)
    _poison(kc, kind)
    vc = None
    if v is not None:
        vc = np.empty((total,) + v.shape[2:], v.dtype)
        _poison(vc, kind)
    offs = np.zeros(B, np.uint32)
    pos = gap
    for b in np.random.Generator(np.random.PCG64(seed)).permutation(B):
        n = int(lens[b])
        offs[b] = pos
        kc[pos:pos + n] = k[b, :n]
        if v is not None:
            vc[pos:pos + n] = v[b, :n]
        pos += n + gap
    return kc, vc, offs


@dataclass
class Inputs:
    """Host arrays of one problem instance (numpy; bf16 as uint16 bits)."""
    wl: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray | None
    valid_length: np.ndarray | None
    page_table: np.ndarray | None
    sink: np.ndarray | None
    indices: np.ndarray | None = None       # sparse: int32 [B, topk] pool rows
    topk_lengths: np.ndarray | None = None  # sparse: int32 [B] listed keys

    def lengths(self) -> np.ndarray:
        if self.topk_lengths is not None:
            return self.topk_lengths.astype(np.int64)
        if self.valid_length is not None:
            return self.valid_length.astype(np.int64)
        return np.full(self.wl.batch, self.wl.max_seq_len, np.int64)

    def kv_bytes(self) -> int:
        """Bytes of K (and V unless MLA) over the valid keys, each read once."""
        esize = {"bf16": 2, "f32": 4, "e4m3": 1}[self.wl.kv_type]
        per_key = self.wl.kv_heads * self.wl.depth * esize
        if not self.wl.mla:
            per_key += self.wl.kv_heads * self.wl.dv * esize
        return int(self.lengths().sum()) * per_key


def _streams(wl: Workload, variant: int):
    entropy = wl.seed if variant == 0 else [wl.seed, variant]
    return dict(zip(("q", "k", "v", "sink", "lengths", "pages"),
                    np.random.SeedSequence(entropy).spawn(6)))


E4M3_NAN = np.uint8(0x7F)
E4M3_SPREAD = 8.0  # stored 8-bit elements are e4m3(8 x N(0,1)): well inside +-448


def e4m3_tensor(seed_seq: np.random.SeedSequence, shape) -> np.ndarray:
    """8-bit e4m3 bit patterns (uint8) of E4M3_SPREAD x N(0,1), rounded to nearest
    by torch's float8_e4m3fn conversion."""
    import torch
    x = normal_tensor(seed_seq, shape, "f32") * np.float32(E4M3_SPREAD)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _kv_tensor(seed_seq, shape, kv_type: str) -> np.ndarray:
    return e4m3_tensor(seed_seq, shape) if kv_type == "e4m3" else normal_tensor(seed_seq, shape,
                                                                                kv_type)


def _poison(arr: np.ndarray, dtype: str):
    if dtype == "e4m3":
        arr[...] = E4M3_NAN
    elif dtype == "bf16":
        arr[...] = BF16_NAN
    else:
        arr[...] = np.float32(np.nan)


def _sparse_inputs(wl: Workload, st, q, ctx, sink, poison: bool) -> Inputs:
    """Sparse top-k: a pool of B*S rows (sequence b's context is rows b*S ..
    b*S + N_b - 1) and one NaN row; sequence b lists min(topk, N_b) distinct rows of
    its context, drawn without replacement in random order (a top-k selection
    keeps no position order); list entries past the count name the NaN row, and so
    do context rows past N_b."""
    B, S, D = wl.batch, wl.max_seq_len, wl.depth
    lens = ctx.astype(np.int64) if ctx is not None else np.full(B, S, np.int64)
    k = _kv_tensor(st["k"], (B * S + 1, wl.kv_heads, D), wl.kv_type)
    nan_row = B * S
    rng = np.random.Generator(np.random.PCG64(st["pages"]))
    tl = np.minimum(lens, wl.topk).astype(np.int32)
    idx = np.full((B, wl.topk), nan_row, np.int32)
    for b in range(B):
        idx[b, :tl[b]] = b * S + rng.choice(int(lens[b]), size=int(tl[b]), replace=False)
    if poison:
        _poison(k[nan_row], wl.kv_type)
        for b in range(B):
            _poison(k[b * S + int(lens[b]):(b + 1) * S], wl.kv_type)
    return Inputs(wl, q, k, None, None, None, sink, indices=idx, topk_lengths=tl)


def make_inputs(wl: Workload, variant: int = 0, poison: bool = True) -> Inputs:
    """Draw one seeded instance of ``wl``."""
    st = _streams(wl, variant)
    B, T, H, KVH, D, S = wl.batch, wl.q_len, wl.num_heads, wl.kv_heads, wl.depth, wl.max_seq_len
    q = normal_tensor(st["q"], (B, T, H, D), wl.dtype)

    valid = None
    if wl.ragged is not None:
        lo, hi, ones = wl.ragged
        rng = np.random.Generator(np.random.PCG64(st["lengths"]))
        lens = rng.integers(lo, hi, size=B, endpoint=True)
        if ones:
            lens[rng.choice(B, size=min(ones, B), replace=False)] = 1
        valid = lens.astype(np.uint32)

    sink = None
    if wl.sink:
        rng = np.random.Generator(np.random.PCG64(st["sink"]))
        sink = rng.standard_normal(H, dtype=np.float32)
    if wl.topk:
        return _sparse_inputs(wl, st, q, valid, sink, poison)

    page_table = None
    if wl.page_size:
        ps = wl.page_size
        max_pages = math.ceil(S / ps)
        lens = valid.astype(np.int64) if valid is not None else np.full(B, S, np.int64)
        need = [math.ceil(int(n) / ps) for n in lens]
        total = int(sum(need))
        poison_page = total
        rng = np.random.Generator(np.random.PCG64(st["pages"]))
        perm = rng.permutation(total).astype(np.uint32)
        page_table = np.full((B, max_pages), poison_page, np.uint32)
        pos = 0
        for b in range(B):
            page_table[b, :need[b]] = perm[pos:pos + need[b]]
            pos += need[b]
        pool_shape = (total + 1, ps, KVH, D)
        k = _kv_tensor(st["k"], pool_shape, wl.kv_type)
        v = None if wl.mla else _kv_tensor(st["v"], (total + 1, ps, KVH, wl.dv), wl.kv_type)
        if poison:
            for arr in (k, v):
                if arr is None:
                    continue
                _poison(arr[poison_page], wl.kv_type)
                for b in range(B):
                    n = int(lens[b])
                    if n % ps and need[b]:
                        _poison(arr[page_table[b, need[b] - 1], n % ps:], wl.kv_type)
    else:
        k = _kv_tensor(st["k"], (B, S, KVH, D), wl.kv_type)
        v = None if wl.mla else _kv_tensor(st["v"], (B, S, KVH, wl.dv), wl.kv_type)
        if poison and valid is not None:
            for arr in (k, v):
                if arr is None:
                    continue
                for b in range(B):
                    _poison(arr[b, int(valid[b]):], wl.kv_type)
    return Inputs(wl, q, k, v, valid, page_table, sink)
