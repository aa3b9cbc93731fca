"""Helpers shared by the GPU parity tests: run the HIP path and the oracle on the
same seeded inputs and compare them element by element."""
from __future__ import annotations

import sys

import numpy as np
import torch

import workloads as W
from decode_attention_07_amd import binding as DA
from oracle import oracle as O

# Acceptance bounds (max abs error): bf16 outputs 1e-2, fp32 outputs 2e-5, LSE 1e-3.
TOL_OUT = {"bf16": 1e-2, "f32": 2e-5}
TOL_LSE = 1e-3


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def device_inputs(inp: W.Inputs):
    return dict(q=DA.to_device(inp.q), k=DA.to_device(inp.k), v=DA.to_device(inp.v),
                page_table=DA.to_device(inp.page_table),
                valid_length=DA.to_device(inp.valid_length),
                sink=DA.to_device(inp.sink), indices=DA.to_device(inp.indices),
                topk_lengths=DA.to_device(inp.topk_lengths))


def run_gpu(wl: W.Workload, dev: dict, num_partitions=None, **kw):
    P = wl.num_partitions if num_partitions is None else num_partitions
    if wl.topk:
        return DA.mla_decode_sparse(dev["q"], dev["k"], dev["indices"], dev["topk_lengths"],
                                    scale=wl.softmax_scale, num_partitions=P,
                                    sink_weights=dev["sink"], **kw)
    common = dict(scale=wl.softmax_scale, page_table=dev["page_table"],
                  valid_length=dev["valid_length"], max_seq_len=wl.max_seq_len,
                  num_partitions=P, sink_weights=dev["sink"], causal=wl.causal)
    common.update(kw)
    if wl.mla and wl.kv_type == "e4m3":
        return DA.mla_decode_fp8kv(dev["q"], dev["k"], k_scale=wl.k_scale, **common)
    if wl.mla:
        return DA.mla_decode(dev["q"], dev["k"], **common)
    if wl.kv_type == "e4m3":
        return DA.decode_attention_fp8kv(dev["q"], dev["k"], dev["v"], k_scale=wl.k_scale,
                                         v_scale=wl.v_scale, group=wl.group, **common)
    return DA.decode_attention(dev["q"], dev["k"], dev["v"], group=wl.group, **common)


def run_oracle(wl: W.Workload, inp: W.Inputs, rows=None):
    if wl.topk:
        return O.attention(inp.q, inp.k, None, scale=wl.softmax_scale, sink=inp.sink,
                           depth_v=wl.dv, rows=rows, indices=inp.indices,
                           topk_lengths=inp.topk_lengths)
    return O.attention(inp.q, inp.k, inp.v, scale=wl.softmax_scale, page_table=inp.page_table,
                       valid_length=inp.valid_length, sink=inp.sink, causal=wl.causal,
                       depth_v=wl.dv, max_seq_len=wl.max_seq_len, rows=rows,
                       k_scale=wl.k_scale, v_scale=wl.v_scale)


def compare(wl: W.Workload, out, lse, ref_out, ref_lse, rows=None, what="", ulp_rel=False):
    """Element-by-element check of the HIP result against the oracle.

    ulp_rel: add one bf16 ulp of |ref| (2^-8 |ref|) to the absolute bound, for
    inputs built to give outputs far larger than N(0,1) data does (a bf16 output
    of magnitude 8..16 is only resolved to 2^-4).
    """
    torch.cuda.synchronize()
    got = DA.to_numpy_f64(out)
    gl = DA.to_numpy_f64(lse)
    if rows is not None:
        got = got.reshape(-1, wl.dv)[rows]
        gl = gl.reshape(-1)[rows]
        ref_out = ref_out.reshape(got.shape)
        ref_lse = ref_lse.reshape(gl.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    diff = np.abs(got - ref_out)
    if ulp_rel:
        diff = diff - np.abs(ref_out) * 2.0 ** -8
    err = diff.max() if got.size else 0.0
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(gl), fin), f"{what}: LSE finiteness differs"
    assert np.array_equal(gl[~fin], ref_lse[~fin]), f"{what}: LSE infinities differ"
    lerr = np.abs(gl[fin] - ref_lse[fin]).max() if fin.any() else 0.0
    tol = TOL_OUT[wl.dtype]
    say(f"  {what}: max|out-ref|={err:.3e} (tol {tol:.0e})  max|lse-ref|={lerr:.3e} "
        f"(tol {TOL_LSE:.0e})")
    assert err <= tol, f"{what}: output error {err:.3e} > {tol:.0e}"
    assert lerr <= TOL_LSE, f"{what}: LSE error {lerr:.3e} > {TOL_LSE:.0e}"
    return err, lerr


def check(wl: W.Workload, num_partitions=None, inp=None, rows=None, what=None, ulp_rel=False):
    what = what or f"{wl.name} P={num_partitions if num_partitions is not None else 'auto'}"
    say(f"[gpu] {what}: B={wl.batch} T={wl.q_len} H={wl.num_heads} KVH={wl.kv_heads} "
        f"D={wl.depth} S={wl.max_seq_len} page={wl.page_size} dtype={wl.dtype}")
    inp = inp or W.make_inputs(wl)
    dev = device_inputs(inp)
    out, lse = run_gpu(wl, dev, num_partitions)
    ref_out, ref_lse = run_oracle(wl, inp, rows)
    return compare(wl, out, lse, ref_out, ref_lse, rows=rows, what=what, ulp_rel=ulp_rel)
