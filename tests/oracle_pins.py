"""Pins of the fp64 oracle to facts other than itself.

Each ``pin_*`` function runs the oracle (the library handle ``lib``) on a tiny
seeded case and checks it against one of:
  * a library routine: torch's fp64 ``scaled_dot_product_attention`` and
    ``logsumexp`` (for the cases that reduce to plain softmax attention, with the
    mask, GQA head map, sink column or MLA value slice built here from the
    readings the oracle states);
  * a closed form (one key, identical keys, zero scale, constant values, two
    keys with a known weight split, sink with identical keys, empty rows);
  * an invariant (key order, page assignment, NaN poison past the valid length,
    causal MTP rows as shorter single-token rows, split-K merge = direct result).

They are plain functions so that the mutation test can run the whole set against
deliberately broken builds of the oracle and show that each planted mistake is
caught by at least one of them.
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

import workloads as W
from oracle import oracle as O

TOL = 1e-10


def _rng(seed):
    return np.random.default_rng(seed)


def _randn(rng, shape, dtype="f32"):
    x = rng.standard_normal(shape).astype(np.float32)
    return W.f32_to_bf16_bits(x) if dtype == "bf16" else x


def _f64(a):
    if a.dtype == np.uint16:
        return W.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def _sdpa(q, k, v, scale, allowed=None, bias=None):
    """torch fp64 SDPA + logsumexp.  q [B,T,H,D]; k [B,S,H,D]; v [B,S,H,Dv] (per query head).

    allowed: bool [B,H,T,S] (True = visible); bias: float [B,H,T,S] added to scores.
    Returns out [B,T,H,Dv], lse [B,T,H].
    """
    tq = torch.from_numpy(_f64(q)).permute(0, 2, 1, 3).contiguous()
    tk = torch.from_numpy(_f64(k)).permute(0, 2, 1, 3).contiguous()
    tv = torch.from_numpy(_f64(v)).permute(0, 2, 1, 3).contiguous()
    B, H, T, _ = tq.shape
    S = tk.shape[2]
    add = torch.zeros(B, H, T, S, dtype=torch.float64)
    if bias is not None:
        add = add + torch.from_numpy(bias)
    if allowed is not None:
        add = add.masked_fill(~torch.from_numpy(allowed), float("-inf"))
    out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=add, scale=scale)
    scores = torch.matmul(tq, tk.transpose(-1, -2).contiguous()) * scale + add
    lse = torch.logsumexp(scores, dim=-1)
    return out.permute(0, 2, 1, 3).numpy(), lse.permute(0, 2, 1).numpy()


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    fin_a, fin_b = np.isfinite(a), np.isfinite(b)
    assert np.array_equal(fin_a, fin_b), f"{what}: finiteness differs"
    assert np.array_equal(a[~fin_a], b[~fin_b]), f"{what}: infinities differ"
    if fin_a.any():
        err = np.max(np.abs(a[fin_a] - b[fin_b]))
        assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _expand_heads(k, group):
    """[B,S,KVH,D] -> [B,S,KVH*group,D]: query head h reads KV head h // group."""
    return np.repeat(k, group, axis=2)


# --------------------------------------------------------------------------
# Library-routine pins (torch fp64 SDPA)
# --------------------------------------------------------------------------

def pin_sdpa_mha_f32(lib):
    rng = _rng(1)
    B, T, H, D, S = 2, 1, 4, 16, 37
    q, k, v = _randn(rng, (B, T, H, D)), _randn(rng, (B, S, H, D)), _randn(rng, (B, S, H, D))
    scale = float(np.float32(0.3))
    out, lse = O.attention(q, k, v, scale=scale, lib=lib)
    ro, rl = _sdpa(q, k, v, scale)
    _close(out, ro, what="out")
    _close(lse, rl, what="lse")


def pin_sdpa_gqa_bf16(lib):
    rng = _rng(2)
    B, T, H, KVH, D, S = 2, 1, 8, 2, 32, 50
    q = _randn(rng, (B, T, H, D), "bf16")
    k = _randn(rng, (B, S, KVH, D), "bf16")
    v = _randn(rng, (B, S, KVH, D), "bf16")
    scale = 1 / math.sqrt(D)
    out, lse = O.attention(q, k, v, scale=np.float32(scale), lib=lib)
    g = H // KVH
    ro, rl = _sdpa(q, _expand_heads(k, g), _expand_heads(v, g), float(np.float32(scale)))
    _close(out, ro, what="out")
    _close(lse, rl, what="lse")


def pin_sdpa_multi_token_noncausal(lib):
    rng = _rng(3)
    B, T, H, KVH, D, S = 2, 3, 6, 3, 8, 11
    q, k, v = (_randn(rng, (B, T, H, D)), _randn(rng, (B, S, KVH, D)),
               _randn(rng, (B, S, KVH, D)))
    out, lse = O.attention(q, k, v, scale=0.7, lib=lib)
    ro, rl = _sdpa(q, _expand_heads(k, 2), _expand_heads(v, 2), float(np.float32(0.7)))
    _close(out, ro, what="out")
    _close(lse, rl, what="lse")


def _visible(lens, T, S, causal):
    """bool [B, T, S]: key j visible to token t of sequence b."""
    B = len(lens)
    j = np.arange(S)[None, None, :]
    n = np.asarray(lens)[:, None, None]
    lim = n if not causal else np.minimum(n, n - T + np.arange(T)[None, :, None] + 1)
    return np.broadcast_to(j < lim, (B, T, S))


def pin_sdpa_ragged(lib):
    rng = _rng(4)
    B, T, H, KVH, D, S = 3, 1, 4, 2, 16, 40
    q, k, v = (_randn(rng, (B, T, H, D)), _randn(rng, (B, S, KVH, D)),
               _randn(rng, (B, S, KVH, D)))
    lens = np.array([40, 17, 3], np.uint32)
    out, lse = O.attention(q, k, v, scale=0.25, valid_length=lens, lib=lib)
    vis = _visible(lens, T, S, False)
    allowed = np.broadcast_to(vis[:, None], (B, H, T, S)).copy()
    ro, rl = _sdpa(q, _expand_heads(k, 2), _expand_heads(v, 2), 0.25, allowed=allowed)
    _close(out, ro, what="out")
    _close(lse, rl, what="lse")


def pin_sdpa_causal_mtp(lib):
    rng = _rng(5)
    B, T, H, KVH, D, S = 2, 3, 4, 1, 16, 20
    q, k, v = (_randn(rng, (B, T, H, D)), _randn(rng, (B, S, KVH, D)),
               _randn(rng, (B, S, KVH, D)))
    lens = np.array([20, 9], np.uint32)
    out, lse = O.attention(q, k, v, scale=0.25, valid_length=lens, causal=True, lib=lib)
    vis = _visible(lens, T, S, True)
    allowed = np.broadcast_to(vis[:, None], (B, H, T, S)).copy()
    ro, rl = _sdpa(q, _expand_heads(k, 4), _expand_heads(v, 4), 0.25, allowed=allowed)
    _close(out, ro, what="out")
    _close(lse, rl, what="lse")


def pin_sdpa_sink_virtual_key(lib):
    """Sink = one extra key with score sigma_h (not scaled) and a zero value row."""
    rng = _rng(6)
    B, T, H, KVH, D, S = 2, 1, 4, 2, 16, 12
    q, k, v = (_randn(rng, (B, T, H, D)), _randn(rng, (B, S, KVH, D)),
               _randn(rng, (B, S, KVH, D)))
    sink = (rng.standard_normal(H) + 2.0).astype(np.float32)
    lens = np.array([12, 5], np.uint32)
    out, lse = O.attention(q, k, v, scale=0.5, valid_length=lens, sink=sink, lib=lib)
    kx = np.concatenate([_expand_heads(k, 2), np.zeros((B, 1, H, D), np.float32)], axis=1)
    vx = np.concatenate([_expand_heads(v, 2), np.zeros((B, 1, H, D), np.float32)], axis=1)
    vis = np.concatenate([_visible(lens, T, S, False), np.ones((B, T, 1), bool)], axis=2)
    allowed = np.broadcast_to(vis[:, None], (B, H, T, S + 1)).copy()
    bias = np.zeros((B, H, T, S + 1))
    bias[..., S] = sink.astype(np.float64)[None, :, None]
    ro, rl = _sdpa(q, kx, vx, 0.5, allowed=allowed, bias=bias)
    _close(out, ro, what="out")
    _close(lse, rl, what="lse")


def pin_sdpa_mla_value_slice(lib):
    """MLA: one KV head, V = K[..., :Dv]."""
    rng = _rng(7)
    B, T, H, D, Dv, S = 2, 2, 8, 24, 16, 13
    q, kv = _randn(rng, (B, T, H, D), "bf16"), _randn(rng, (B, S, 1, D), "bf16")
    out, lse = O.attention(q, kv, None, depth_v=Dv, scale=0.2, causal=True, lib=lib)
    lens = np.full(B, S, np.uint32)
    allowed = np.broadcast_to(_visible(lens, T, S, True)[:, None], (B, H, T, S)).copy()
    kk = _expand_heads(kv, H)
    ro, rl = _sdpa(q, kk, kk[..., :Dv].copy(), float(np.float32(0.2)), allowed=allowed)
    _close(out, ro, what="out")
    _close(lse, rl, what="lse")


# --------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------

def pin_closed_single_key(lib):
    rng = _rng(8)
    B, H, D, S = 1, 2, 8, 6
    q, k, v = _randn(rng, (B, 1, H, D)), _randn(rng, (B, S, H, D)), _randn(rng, (B, S, H, D))
    out, lse = O.attention(q, k, v, scale=0.5, valid_length=np.array([1], np.uint32), lib=lib)
    for h in range(H):
        _close(out[0, 0, h], v[0, 0, h], tol=0, what="out == v0")
        s0 = 0.5 * float(np.dot(q[0, 0, h].astype(np.float64), k[0, 0, h].astype(np.float64)))
        _close(lse[0, 0, h], s0, what="lse == s0")


def pin_closed_identical_keys(lib):
    rng = _rng(9)
    B, H, D, S = 1, 3, 8, 7
    q = _randn(rng, (B, 1, H, D))
    k = np.broadcast_to(_randn(rng, (1, 1, H, D)), (B, S, H, D)).copy()
    v = _randn(rng, (B, S, H, D))
    out, lse = O.attention(q, k, v, scale=0.375, lib=lib)
    for h in range(H):
        s = 0.375 * float(np.dot(q[0, 0, h].astype(np.float64), k[0, 0, h].astype(np.float64)))
        _close(out[0, 0, h], v[0, :, h].astype(np.float64).mean(0), what="mean(V)")
        _close(lse[0, 0, h], s + math.log(S), what="s + ln N")


def pin_closed_zero_scale(lib):
    rng = _rng(10)
    B, H, KVH, D, S = 2, 4, 2, 8, 9
    q, k, v = (_randn(rng, (B, 1, H, D)), _randn(rng, (B, S, KVH, D)),
               _randn(rng, (B, S, KVH, D)))
    out, lse = O.attention(q, k, v, scale=0.0, lib=lib)
    for b in range(B):
        for h in range(H):
            _close(out[b, 0, h], v[b, :, h // 2].astype(np.float64).mean(0), what="mean(V)")
            _close(lse[b, 0, h], math.log(S), what="ln N")


def pin_closed_constant_values(lib):
    rng = _rng(11)
    B, H, D, S = 1, 2, 8, 10
    q, k = _randn(rng, (B, 1, H, D)), _randn(rng, (B, S, H, D))
    c = rng.standard_normal(D).astype(np.float32)
    v = np.broadcast_to(c, (B, S, H, D)).copy()
    out, _ = O.attention(q, k, v, scale=1.3, lib=lib)
    for h in range(H):
        _close(out[0, 0, h], c, what="O == c")


def pin_closed_two_keys(lib):
    """Scores 0 and ln 3 give weights 1/4 and 3/4, and LSE = ln 4."""
    D = 2
    q = np.array([[[[1.0, 0.0]]]], np.float32)
    k = np.array([[[[0.0, 0.0]], [[math.log(3.0), 0.0]]]], np.float32)
    v = np.array([[[[1.0, -2.0]], [[5.0, 4.0]]]], np.float32)
    out, lse = O.attention(q, k, v, scale=1.0, lib=lib)
    s1 = float(np.float32(math.log(3.0)))
    w1 = math.exp(s1) / (1.0 + math.exp(s1))
    expect = (1 - w1) * v[0, 0, 0].astype(np.float64) + w1 * v[0, 1, 0].astype(np.float64)
    _close(out[0, 0, 0], expect, what="weights 1/4, 3/4")
    _close(lse[0, 0, 0], math.log(1.0 + math.exp(s1)), what="ln 4")
    assert D == 2


def pin_closed_sink_identical_keys(lib):
    rng = _rng(12)
    B, H, D, S = 1, 2, 8, 5
    q = _randn(rng, (B, 1, H, D))
    k = np.broadcast_to(_randn(rng, (1, 1, H, D)), (B, S, H, D)).copy()
    v = _randn(rng, (B, S, H, D))
    sink = np.array([0.7, -1.2], np.float32)
    out, lse = O.attention(q, k, v, scale=0.9, sink=sink, lib=lib)
    for h in range(H):
        s = float(np.float32(0.9)) * float(np.dot(q[0, 0, h].astype(np.float64),
                                                 k[0, 0, h].astype(np.float64)))
        den = S * math.exp(s) + math.exp(float(sink[h]))
        mean_v = v[0, :, h].astype(np.float64).mean(0)
        _close(out[0, 0, h], mean_v * S * math.exp(s) / den, what="sink-damped mean")
        _close(lse[0, 0, h], math.log(den), what="ln(N e^s + e^sigma)")


def pin_closed_empty_rows(lib):
    rng = _rng(13)
    B, H, D, S = 2, 2, 8, 4
    q, k, v = _randn(rng, (B, 1, H, D)), _randn(rng, (B, S, H, D)), _randn(rng, (B, S, H, D))
    lens = np.array([0, 0], np.uint32)
    out, lse = O.attention(q, k, v, scale=1.0, valid_length=lens, lib=lib)
    assert np.all(out == 0.0) and np.all(lse == -np.inf), "empty row without sink"
    sink = np.array([0.25, -3.0], np.float32)
    out, lse = O.attention(q, k, v, scale=1.0, valid_length=lens, sink=sink, lib=lib)
    assert np.all(out == 0.0), "empty row with sink: out"
    _close(lse[:, 0, :], np.broadcast_to(sink.astype(np.float64), (B, H)), what="lse == sigma")


def pin_sink_minus_infinity_is_no_sink(lib):
    rng = _rng(14)
    B, H, D, S = 1, 4, 8, 9
    q, k, v = _randn(rng, (B, 1, H, D)), _randn(rng, (B, S, 2, D)), _randn(rng, (B, S, 2, D))
    a = O.attention(q, k, v, scale=0.5, lib=lib)
    b = O.attention(q, k, v, scale=0.5, sink=np.full(H, -np.inf, np.float32), lib=lib)
    _close(a[0], b[0], tol=0, what="out")
    _close(a[1], b[1], tol=0, what="lse")


# --------------------------------------------------------------------------
# Invariants
# --------------------------------------------------------------------------

def pin_key_permutation(lib):
    rng = _rng(15)
    B, H, KVH, D, S = 1, 4, 2, 8, 23
    q, k, v = (_randn(rng, (B, 1, H, D)), _randn(rng, (B, S, KVH, D)),
               _randn(rng, (B, S, KVH, D)))
    perm = rng.permutation(S)
    a = O.attention(q, k, v, scale=0.5, lib=lib)
    b = O.attention(q, k[:, perm].copy(), v[:, perm].copy(), scale=0.5, lib=lib)
    _close(a[0], b[0], tol=1e-12, what="out")
    _close(a[1], b[1], tol=1e-12, what="lse")


def _paged_from_contiguous(rng, k, v, lens, page_size, extra_pages=3):
    """Scatter a contiguous cache into a shuffled page pool with a NaN poison page."""
    B, S = k.shape[:2]
    max_pages = -(-S // page_size)
    need = [-(-int(n) // page_size) for n in lens]
    total = sum(need) + extra_pages
    perm = rng.permutation(total)
    poison = total
    shape_k = (total + 1, page_size) + k.shape[2:]
    shape_v = (total + 1, page_size) + v.shape[2:]
    kp = np.full(shape_k, np.nan, np.float32)
    vp = np.full(shape_v, np.nan, np.float32)
    table = np.full((B, max_pages), poison, np.uint32)
    pos = 0
    for b in range(B):
        for i in range(need[b]):
            phys = perm[pos]
            pos += 1
            table[b, i] = phys
            lo, hi = i * page_size, min((i + 1) * page_size, int(lens[b]))
            kp[phys, :hi - lo] = k[b, lo:hi]
            vp[phys, :hi - lo] = v[b, lo:hi]
    return kp, vp, table


def pin_paged_equals_contiguous(lib):
    rng = _rng(16)
    B, H, KVH, D, S, ps = 3, 4, 2, 8, 30, 4
    q, k, v = (_randn(rng, (B, 1, H, D)), _randn(rng, (B, S, KVH, D)),
               _randn(rng, (B, S, KVH, D)))
    lens = np.array([30, 13, 1], np.uint32)
    ref = O.attention(q, k, v, scale=0.5, valid_length=lens, lib=lib)
    kp, vp, table = _paged_from_contiguous(rng, k, v, lens, ps)
    got = O.attention(q, kp, vp, scale=0.5, valid_length=lens, page_table=table,
                      max_seq_len=S, lib=lib)
    _close(got[0], ref[0], tol=1e-12, what="out")
    _close(got[1], ref[1], tol=1e-12, what="lse")
    kp2, vp2, table2 = _paged_from_contiguous(_rng(99), k, v, lens, ps, extra_pages=0)
    got2 = O.attention(q, kp2, vp2, scale=0.5, valid_length=lens, page_table=table2,
                       max_seq_len=S, lib=lib)
    _close(got2[0], ref[0], tol=1e-12, what="out (other page permutation)")


def pin_nan_poison_past_valid_length(lib):
    rng = _rng(17)
    B, H, D, S = 2, 2, 8, 16
    q, k, v = _randn(rng, (B, 1, H, D)), _randn(rng, (B, S, H, D)), _randn(rng, (B, S, H, D))
    lens = np.array([9, 16], np.uint32)
    ref = O.attention(q, k, v, scale=0.5, valid_length=lens, lib=lib)
    kq, vq = k.copy(), v.copy()
    kq[0, 9:] = np.nan
    vq[0, 9:] = np.nan
    got = O.attention(q, kq, vq, scale=0.5, valid_length=lens, lib=lib)
    _close(got[0], ref[0], tol=0, what="out")
    _close(got[1], ref[1], tol=0, what="lse")


def pin_sdpa_valid_length_above_max_seq_len(lib):
    """A length above max_seq_len counts as max_seq_len (the key bound of
    "mha_sm100_dispatch", Args `max_cache_valid_length_arg`, caps Args
    `valid_length`), also a uint32 length of 2^31 or more: torch SDPA over the
    first S keys, dense and paged, causal and not."""
    rng = _rng(40)
    B, T, H, KVH, D, S, ps = 3, 2, 4, 2, 8, 12, 4
    q, k, v = (_randn(rng, (B, T, H, D)), _randn(rng, (B, S, KVH, D)),
               _randn(rng, (B, S, KVH, D)))
    over = np.array([S + 5, 0xFFFFFFFF, 7], np.uint32)
    capped = np.array([S, S, 7], np.uint32)
    kp, vp, table = _paged_from_contiguous(rng, k, v, capped, ps, extra_pages=0)
    for causal in (False, True):
        vis = _visible(capped, T, S, causal)
        allowed = np.broadcast_to(vis[:, None], (B, H, T, S)).copy()
        ro, rl = _sdpa(q, _expand_heads(k, 2), _expand_heads(v, 2), 0.5, allowed=allowed)
        out, lse = O.attention(q, k, v, scale=0.5, valid_length=over, causal=causal, lib=lib)
        _close(out, ro, what=f"dense out causal={causal}")
        _close(lse, rl, what=f"dense lse causal={causal}")
        out, lse = O.attention(q, kp, vp, scale=0.5, valid_length=over, causal=causal,
                               page_table=table, max_seq_len=S, lib=lib)
        _close(out, ro, what=f"paged out causal={causal}")
        _close(lse, rl, what=f"paged lse causal={causal}")


def _concat_cache(rng, k, v, lens, gap=2):
    """The ragged KV layout of a dense cache: the sequences' valid rows in a shuffled
    order in one cache [rows, KVH, D], NaN rows between and after them (enough
    that a misplaced row read stays inside the array)."""
    B, S = k.shape[:2]
    total = gap + sum(int(n) + gap for n in lens) + B * S + 1
    kc = np.full((total,) + k.shape[2:], np.nan, np.float32)
    vc = None if v is None else np.full((total,) + v.shape[2:], np.nan, np.float32)
    offs = np.zeros(B, np.uint32)
    pos = gap
    for b in rng.permutation(B):
        n = int(lens[b])
        offs[b] = pos
        kc[pos:pos + n] = k[b, :n]
        if v is not None:
            vc[pos:pos + n] = v[b, :n]
        pos += n + gap
    return kc, vc, offs


def pin_ragged_kv_layout_equals_dense(lib):
    """Per-sequence row offsets into one concatenated cache ("mha_sm100_dispatch",
    Args `kv_input_row_offsets`) give the dense call over the same rows, bit for bit:
    GQA causal with a sink, its split-K partials, and MLA (V = K[..., :Dv])."""
    rng = _rng(41)
    B, T, H, KVH, D, S = 3, 2, 4, 2, 8, 11
    q, k, v = (_randn(rng, (B, T, H, D)), _randn(rng, (B, S, KVH, D)),
               _randn(rng, (B, S, KVH, D)))
    lens = np.array([11, 4, 1], np.uint32)
    sink = rng.standard_normal(H).astype(np.float32)
    kc, vc, offs = _concat_cache(rng, k, v, lens)
    kw = dict(scale=0.5, valid_length=lens, causal=True, lib=lib)
    ref = O.attention(q, k, v, sink=sink, **kw)
    got = O.attention(q, kc, vc, sink=sink, kv_offsets=offs, max_seq_len=S, **kw)
    _close(got[0], ref[0], tol=0, what="out")
    _close(got[1], ref[1], tol=0, what="lse")
    for P, C in ((2, 6), (3, 4)):
        a = O.partials(q, k, v, num_partitions=P, keys_per_partition=C, **kw)
        b = O.partials(q, kc, vc, num_partitions=P, keys_per_partition=C, kv_offsets=offs,
                       max_seq_len=S, **kw)
        for x, y, name in zip(a, b, ("O_p", "m_p", "l_p")):
            _close(y, x, tol=0, what=f"{name} P={P}")
    q1, kv = _randn(rng, (B, 1, 8, 10)), _randn(rng, (B, S, 1, 10))
    kc1, _, offs1 = _concat_cache(rng, kv, None, lens)
    ref = O.attention(q1, kv, None, depth_v=6, scale=0.4, valid_length=lens, lib=lib)
    got = O.attention(q1, kc1, None, depth_v=6, scale=0.4, valid_length=lens, kv_offsets=offs1,
                      max_seq_len=S, lib=lib)
    _close(got[0], ref[0], tol=0, what="mla out")
    _close(got[1], ref[1], tol=0, what="mla lse")


def pin_causal_rows_are_shorter_rows(lib):
    """Token t of T under the causal mask = a single-token row over N - T + t + 1 keys."""
    rng = _rng(18)
    B, T, H, D, S = 2, 2, 4, 16, 10
    q, kv = _randn(rng, (B, T, H, D), "bf16"), _randn(rng, (B, S, 1, D), "bf16")
    lens = np.array([10, 6], np.uint32)
    out, lse = O.attention(q, kv, None, depth_v=12, scale=0.3, valid_length=lens, causal=True,
                           lib=lib)
    for t in range(T):
        o1, l1 = O.attention(q[:, t:t + 1].copy(), kv, None, depth_v=12, scale=0.3,
                             valid_length=(lens - (T - 1 - t)).astype(np.uint32), lib=lib)
        _close(out[:, t], o1[:, 0], tol=0, what=f"out token {t}")
        _close(lse[:, t], l1[:, 0], tol=0, what=f"lse token {t}")


def pin_mla_value_slice_equals_explicit_v(lib):
    rng = _rng(19)
    B, T, H, D, Dv, S = 2, 1, 4, 20, 12, 9
    q, kv = _randn(rng, (B, T, H, D)), _randn(rng, (B, S, 1, D))
    a = O.attention(q, kv, None, depth_v=Dv, scale=0.5, lib=lib)
    b = O.attention(q, kv, kv[..., :Dv].copy(), scale=0.5, lib=lib)
    _close(a[0], b[0], tol=0, what="out")
    _close(a[1], b[1], tol=0, what="lse")


def pin_rows_subset(lib):
    rng = _rng(20)
    B, T, H, D, S = 2, 2, 3, 8, 7
    q, k, v = _randn(rng, (B, T, H, D)), _randn(rng, (B, S, 3, D)), _randn(rng, (B, S, 3, D))
    full = O.attention(q, k, v, scale=0.5, lib=lib)
    rows = np.array([5, 0, 11, 7], np.int64)
    got = O.attention(q, k, v, scale=0.5, rows=rows, lib=lib)
    _close(got[0], full[0].reshape(-1, D)[rows], tol=0, what="out")
    _close(got[1], full[1].reshape(-1)[rows], tol=0, what="lse")


def pin_splitk_merge_equals_direct(lib):
    rng = _rng(21)
    B, T, H, KVH, D, S = 3, 2, 4, 2, 8, 29
    q, k, v = (_randn(rng, (B, T, H, D)), _randn(rng, (B, S, KVH, D)),
               _randn(rng, (B, S, KVH, D)))
    lens = np.array([29, 7, 1], np.uint32)
    sink = rng.standard_normal(H).astype(np.float32)
    ref = O.attention(q, k, v, scale=0.5, valid_length=lens, sink=sink, causal=True, lib=lib)
    for P in (1, 2, 3, 7, 16, 40):
        C = -(-S // P)
        po, pm, pl = O.partials(q, k, v, scale=0.5, num_partitions=P, keys_per_partition=C,
                                valid_length=lens, causal=True, lib=lib)
        out, lse = O.merge(po, pm, pl, num_heads=H, sink=sink, lib=lib)
        _close(out.reshape(ref[0].shape), ref[0], tol=1e-12, what=f"out P={P}")
        _close(lse.reshape(ref[1].shape), ref[1], tol=1e-12, what=f"lse P={P}")


def pin_splitk_partial_is_restricted_softmax(lib):
    """A partial equals full attention over exactly that key slice (SDPA on the slice)."""
    rng = _rng(22)
    B, H, D, S, C = 1, 2, 8, 20, 6
    q, k, v = _randn(rng, (B, 1, H, D)), _randn(rng, (B, S, H, D)), _randn(rng, (B, S, H, D))
    po, pm, pl = O.partials(q, k, v, scale=0.5, num_partitions=4, keys_per_partition=C, lib=lib)
    for p in range(4):
        lo, hi = p * C, min(S, (p + 1) * C)
        ro, rl = _sdpa(q, k[:, lo:hi].copy(), v[:, lo:hi].copy(), 0.5)
        _close(po[p].reshape(ro.shape), ro, what=f"O_p p={p}")
        _close((pm[p] + np.log(pl[p])).reshape(rl.shape), rl, what=f"m_p + ln l_p p={p}")


def pin_splitk_identical_partitions(lib):
    rng = _rng(23)
    P, rows, Dv, H = 5, 6, 4, 3
    o = rng.standard_normal((1, rows, Dv))
    m = rng.standard_normal((1, rows))
    l = rng.uniform(0.5, 3.0, (1, rows))
    out, lse = O.merge(np.repeat(o, P, 0), np.repeat(m, P, 0), np.repeat(l, P, 0), num_heads=H,
                       lib=lib)
    _close(out, o[0], what="same O")
    _close(lse, m[0] + np.log(l[0]) + math.log(P), what="LSE + ln P")


def pin_splitk_single_nonempty(lib):
    rng = _rng(24)
    P, rows, Dv, H = 4, 5, 3, 5
    po = np.zeros((P, rows, Dv))
    pm = np.full((P, rows), -np.inf)
    pl = np.zeros((P, rows))
    po[2] = rng.standard_normal((rows, Dv))
    pm[2] = rng.standard_normal(rows)
    pl[2] = rng.uniform(0.5, 2.0, rows)
    out, lse = O.merge(po, pm, pl, num_heads=H, lib=lib)
    _close(out, po[2], what="O of the only partition")
    _close(lse, pm[2] + np.log(pl[2]), what="its LSE")


# --------------------------------------------------------------------------
# Ragged q: per-sequence token counts from cumulative offsets
# --------------------------------------------------------------------------

def _ragged_case(rng, dtype="f32"):
    B, H, KVH, D, S = 4, 4, 2, 16, 23
    tokens = np.array([2, 0, 3, 1])
    qo = np.concatenate([[0], np.cumsum(tokens)]).astype(np.uint32)
    q = _randn(rng, (int(qo[-1]), H, D), dtype)
    k = _randn(rng, (B, S, KVH, D), dtype)
    v = _randn(rng, (B, S, KVH, D), dtype)
    lens = np.array([23, 9, 5, 17], np.uint32)
    return q, qo, k, v, lens, tokens


def pin_ragged_q_equals_sequence_by_sequence(lib):
    """Each sequence of a ragged call equals a one-sequence call with T = its own
    token count (causal and not, with a sink)."""
    rng = _rng(50)
    q, qo, k, v, lens, tokens = _ragged_case(rng)
    sink = rng.standard_normal(q.shape[1]).astype(np.float32)
    for causal in (False, True):
        out, lse = O.attention(q, k, v, scale=0.3, valid_length=lens, sink=sink, causal=causal,
                               q_offsets=qo, lib=lib)
        for b, T in enumerate(tokens):
            if T == 0:
                continue
            r = slice(int(qo[b]), int(qo[b + 1]))
            o1, l1 = O.attention(q[r][None], k[b:b + 1], v[b:b + 1], scale=0.3,
                                 valid_length=lens[b:b + 1], sink=sink, causal=causal, lib=lib)
            _close(out[r], o1[0], tol=0, what=f"seq {b} out")
            _close(lse[r], l1[0], tol=0, what=f"seq {b} lse")


def pin_sdpa_ragged_q_causal(lib):
    """Ragged causal q against fp64 SDPA with explicit masks: token t of the T_b
    tokens of sequence b sees keys j <= N_b - T_b + t."""
    rng = _rng(51)
    q, qo, k, v, lens, tokens = _ragged_case(rng, "bf16")
    H, KVH = q.shape[1], k.shape[2]
    scale = float(np.float32(0.35))
    out, lse = O.attention(q, k, v, scale=scale, valid_length=lens, causal=True, q_offsets=qo,
                           lib=lib)
    for b, T in enumerate(tokens):
        if T == 0:
            continue
        r = slice(int(qo[b]), int(qo[b + 1]))
        S = k.shape[1]
        j = np.arange(S)[None, :]
        lim = int(lens[b]) - int(T) + np.arange(T)[:, None] + 1
        allowed = np.broadcast_to((j < np.minimum(lim, int(lens[b])))[None, None],
                                  (1, H, T, S)).copy()
        ro, rl = _sdpa(q[r][None], _expand_heads(k[b:b + 1], H // KVH),
                       _expand_heads(v[b:b + 1], H // KVH), scale, allowed=allowed)
        _close(out[r], ro[0], what=f"seq {b} out")
        _close(lse[r], rl[0], what=f"seq {b} lse")


# --------------------------------------------------------------------------
# 8-bit e4m3 keys / values with per-tensor scales
# --------------------------------------------------------------------------

def _e4m3_torch(codes):
    """torch's own e4m3 (float8_e4m3fn) conversion of uint8 codes, as float64."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def pin_e4m3_all_codes_single_key(lib):
    """One key: out is its value row, so every one of the 256 codes comes back
    as v_scale times torch's e4m3 value of it (NaN for the two NaN codes)."""
    rng = _rng(40)
    q = _randn(rng, (1, 1, 1, 8), "bf16")
    k = rng.integers(0, 0x7f, size=(1, 1, 1, 8), dtype=np.uint8)  # finite key codes
    v = np.arange(256, dtype=np.uint8).reshape(1, 1, 1, 256)
    v_scale = 0.8125
    out, lse = O.attention(q, k, v, scale=0.5, k_scale=1.0, v_scale=v_scale, lib=lib)
    ref = v_scale * _e4m3_torch(v[0, 0, 0])
    got = out[0, 0, 0]
    if not np.array_equal(np.isnan(got), np.isnan(ref)):
        raise AssertionError("NaN codes differ from torch's e4m3")
    fin = ~np.isnan(ref)
    _close(got[fin], ref[fin], tol=0, what="e4m3 values")
    s0 = 0.5 * float(np.dot(_f64(q[0, 0, 0]), _e4m3_torch(k[0, 0, 0])))
    _close(lse[0, 0, 0], s0, what="lse == scale * q.k")


def pin_sdpa_e4m3_scaled_kv(lib):
    """bf16 q against e4m3 k / v with different scales, ragged and grouped:
    equals fp64 SDPA on keys / values dequantised by torch (code * scale)."""
    rng = _rng(41)
    B, T, H, KVH, D, Dv, S = 2, 1, 6, 2, 16, 24, 29
    q = _randn(rng, (B, T, H, D), "bf16")
    codes = np.concatenate([np.arange(0, 0x7f), np.arange(0x80, 0xff)]).astype(np.uint8)
    k = rng.choice(codes, size=(B, S, KVH, D))
    v = rng.choice(codes, size=(B, S, KVH, Dv))
    lens = np.array([29, 11], np.uint32)
    k_scale, v_scale = 0.0625, 1.75  # exact in fp32, as the oracle takes them
    scale = float(np.float32(0.4))
    out, lse = O.attention(q, k, v, scale=scale, valid_length=lens, k_scale=k_scale,
                           v_scale=v_scale, lib=lib)
    kd = k_scale * _e4m3_torch(k)
    vd = v_scale * _e4m3_torch(v)
    g = H // KVH
    allowed = np.broadcast_to(_visible(lens, T, S, False)[:, None], (B, H, T, S)).copy()
    ro, rl = _sdpa(q, _expand_heads(kd, g), _expand_heads(vd, g), scale, allowed=allowed)
    _close(out, ro, what="out")
    _close(lse, rl, what="lse")


def pin_sdpa_e4m3_mla_value_slice(lib):
    """MLA over an e4m3 cache: V is the first Dv columns of the same stored rows, so
    it is dequantised with k_scale (a v_scale passed alongside plays no part), causal
    MTP rows: fp64 SDPA on the rows dequantised by torch."""
    rng = _rng(45)
    B, T, H, D, Dv, S = 2, 2, 4, 24, 16, 21
    q = _randn(rng, (B, T, H, D), "bf16")
    codes = np.concatenate([np.arange(0, 0x7f), np.arange(0x80, 0xff)]).astype(np.uint8)
    kv = rng.choice(codes, size=(B, S, 1, D))
    lens = np.array([21, 6], np.uint32)
    k_scale = 0.09375
    scale = float(np.float32(0.3))
    out, lse = O.attention(q, kv, None, depth_v=Dv, scale=scale, valid_length=lens,
                           causal=True, k_scale=k_scale, v_scale=7.0, lib=lib)
    kd = _expand_heads(k_scale * _e4m3_torch(kv), H)
    allowed = np.broadcast_to(_visible(lens, T, S, True)[:, None], (B, H, T, S)).copy()
    ro, rl = _sdpa(q, kd, kd[..., :Dv].copy(), scale, allowed=allowed)
    _close(out, ro, what="out")
    _close(lse, rl, what="lse")


# --------------------------------------------------------------------------
# Sparse top-k: each sequence's keys are listed pool rows
# --------------------------------------------------------------------------

def _sparse_case(rng, B, T, H, D, R, stride, lens, dtype="f32"):
    q = _randn(rng, (B, T, H, D), dtype)
    pool = _randn(rng, (R, 1, D), dtype)
    idx = rng.integers(0, R, size=(B, stride)).astype(np.int32)
    return q, pool, idx, np.asarray(lens, np.int32)


def pin_sparse_identity_list_equals_dense(lib):
    """Listing rows b*S .. b*S + N_b - 1 of the dense cache (read as a pool) gives the
    dense result with valid_length N_b; list entries past the count name a NaN row
    and are never read."""
    rng = _rng(40)
    B, T, H, D, Dv, S = 3, 2, 4, 24, 16, 19
    q, kv = _randn(rng, (B, T, H, D), "bf16"), _randn(rng, (B, S, 1, D), "bf16")
    lens = np.array([19, 7, 0], np.uint32)
    sink = rng.standard_normal(H).astype(np.float32)
    ref = O.attention(q, kv, None, depth_v=Dv, scale=0.3, valid_length=lens, sink=sink, lib=lib)
    pool = np.concatenate([kv.reshape(B * S, 1, D), np.full((1, 1, D), 0x7FC0, np.uint16)])
    idx = np.full((B, S + 2), B * S, np.int32)
    for b in range(B):
        idx[b, :lens[b]] = b * S + np.arange(lens[b])
    got = O.attention(q, pool, None, depth_v=Dv, scale=0.3, sink=sink,
                      indices=idx, topk_lengths=lens.astype(np.int32), lib=lib)
    _close(got[0], ref[0], tol=1e-12, what="out")
    _close(got[1], ref[1], tol=1e-12, what="lse")


def pin_sdpa_sparse_gather(lib):
    """torch fp64 SDPA over the gathered rows (a repeated index counts twice, a zero
    count leaves only the sink), MLA value slice, sink as a virtual key."""
    rng = _rng(41)
    B, T, H, D, Dv, R, stride = 3, 2, 4, 20, 12, 40, 9
    q, pool, idx, lens = _sparse_case(rng, B, T, H, D, R, stride, [9, 4, 0])
    idx[0, 3] = idx[0, 5]
    vis = np.arange(stride)[None, :] < lens[:, None]
    idx[~vis] = R                                                      # a NaN row, never read
    pool = np.concatenate([pool, np.full((1, 1, D), np.nan, np.float32)])
    sink = rng.standard_normal(H).astype(np.float32)
    out, lse = O.attention(q, pool, None, depth_v=Dv, scale=0.4, sink=sink, indices=idx,
                           topk_lengths=lens, lib=lib)
    kg = pool[np.where(vis, idx, 0)][:, :, 0]                          # [B, stride, D]
    kx = np.concatenate([np.repeat(kg[:, :, None], H, axis=2),
                         np.zeros((B, 1, H, D), np.float32)], axis=1)  # + sink key
    vis = np.concatenate([vis, np.ones((B, 1), bool)], axis=1)
    allowed = np.broadcast_to(vis[:, None, None, :], (B, H, T, stride + 1)).copy()
    bias = np.zeros((B, H, T, stride + 1))
    bias[..., stride] = sink.astype(np.float64)[None, :, None]
    ro, rl = _sdpa(q, kx, kx[..., :Dv].copy(), float(np.float32(0.4)), allowed=allowed,
                   bias=bias)
    _close(out, ro, what="out")
    _close(lse, rl, what="lse")


def pin_sparse_list_order(lib):
    """The keys form a set: reordering a sequence's listed rows changes nothing."""
    rng = _rng(42)
    B, T, H, D, R, stride = 2, 1, 3, 16, 30, 11
    q, pool, idx, lens = _sparse_case(rng, B, T, H, D, R, stride, [11, 6])
    a = O.attention(q, pool, pool, scale=0.5, indices=idx, topk_lengths=lens, lib=lib)
    idx2 = idx.copy()
    for b in range(B):
        idx2[b, :lens[b]] = idx[b, rng.permutation(lens[b])]
    b_ = O.attention(q, pool, pool, scale=0.5, indices=idx2, topk_lengths=lens, lib=lib)
    _close(a[0], b_[0], tol=1e-12, what="out")
    _close(a[1], b_[1], tol=1e-12, what="lse")


def pin_sparse_paged_list(lib):
    """A page table expanded into one row per key (page size 1) gives the paged result;
    the pool's unused pages are NaN, so a wrong row shows."""
    rng = _rng(43)
    B, H, KVH, D, S, ps = 3, 4, 2, 8, 30, 4
    q, k, v = (_randn(rng, (B, 1, H, D)), _randn(rng, (B, S, KVH, D)),
               _randn(rng, (B, S, KVH, D)))
    lens = np.array([30, 13, 1], np.uint32)
    kp, vp, table = _paged_from_contiguous(rng, k, v, lens, ps)
    ref = O.attention(q, kp, vp, scale=0.5, valid_length=lens, page_table=table, max_seq_len=S,
                      lib=lib)
    j = np.arange(S)
    idx = (table[:, j // ps].astype(np.int64) * ps + j % ps).astype(np.int32)
    got = O.attention(q, kp.reshape(-1, KVH, D), vp.reshape(-1, KVH, D), scale=0.5,
                      indices=idx, topk_lengths=lens.astype(np.int32), lib=lib)
    _close(got[0], ref[0], tol=1e-12, what="out")
    _close(got[1], ref[1], tol=1e-12, what="lse")


def pin_sparse_partials(lib):
    """Sparse partitions cover list positions: each partial is SDPA over its slice of the
    list, and the merge gives the full result."""
    rng = _rng(44)
    B, T, H, D, Dv, R, stride, C = 2, 2, 2, 12, 8, 25, 13, 4
    q, pool, idx, lens = _sparse_case(rng, B, T, H, D, R, stride, [13, 6])
    sink = rng.standard_normal(H).astype(np.float32)
    ref = O.attention(q, pool, None, depth_v=Dv, scale=0.6, sink=sink, indices=idx,
                      topk_lengths=lens, lib=lib)
    P = -(-stride // C)
    po, pm, pl = O.partials(q, pool, None, depth_v=Dv, scale=0.6, num_partitions=P,
                            keys_per_partition=C, indices=idx, topk_lengths=lens, lib=lib)
    out, lse = O.merge(po, pm, pl, num_heads=H, sink=sink, lib=lib)
    _close(out.reshape(ref[0].shape), ref[0], tol=1e-12, what="merged out")
    _close(lse.reshape(ref[1].shape), ref[1], tol=1e-12, what="merged lse")
    po = po.reshape(P, B, T, H, Dv)
    ml = (pm + np.log(np.where(pl > 0, pl, 1.0))).reshape(P, B, T, H)
    for p in range(P):
        for b in range(B):
            lo, hi = p * C, min((p + 1) * C, int(lens[b]))
            if hi <= lo:
                assert np.all(pl.reshape(P, B, T, H)[p, b] == 0), "empty partition"
                continue
            kg = pool[idx[b, lo:hi]][:, 0]
            kk = np.repeat(kg[None, :, None], H, axis=2)
            ro, rl = _sdpa(q[b:b + 1], kk, kk[..., :Dv].copy(), float(np.float32(0.6)))
            _close(po[p, b], ro[0], what=f"O_p p={p} b={b}")
            _close(ml[p, b], rl[0], what=f"m_p + ln l_p p={p} b={b}")


ALL_PINS = {name: fn for name, fn in sorted(globals().items()) if name.startswith("pin_")}


def failing_pins(lib) -> list[str]:
    """Names of the pins that fail (or crash) against ``lib``."""
    bad = []
    for name, fn in ALL_PINS.items():
        try:
            with np.errstate(all="ignore"):
                fn(lib)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            bad.append(name)
    return bad
