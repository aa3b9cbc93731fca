"""GPU parity: ragged q (per-sequence token counts from cumulative offsets) through
decode_attention_ragged() / mla_decode_ragged() against the fp64 oracle."""
import numpy as np
import pytest
import torch

import workloads as W
from decode_attention_07_amd import binding as DA
from gpu_util import TOL_LSE, TOL_OUT, device_inputs, say
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _pack(inp: W.Inputs, tokens):
    """Ragged q [total, H, D] and offsets [B+1] from the padded q [B, T, H, D]: the
    first tokens[b] tokens of each sequence."""
    qo = np.concatenate([[0], np.cumsum(tokens)]).astype(np.uint32)
    q = np.concatenate([inp.q[b, :t] for b, t in enumerate(tokens)], axis=0)
    return np.ascontiguousarray(q), qo


def _run(wl: W.Workload, tokens, P, what):
    inp = W.make_inputs(wl)
    q, qo = _pack(inp, tokens)
    dev = device_inputs(inp)
    dq = DA.to_device(q)
    dqo = DA.to_device(qo)
    common = dict(max_q_len=wl.q_len, scale=wl.softmax_scale, page_table=dev["page_table"],
                  valid_length=dev["valid_length"], max_seq_len=wl.max_seq_len,
                  num_partitions=P, sink_weights=dev["sink"], causal=wl.causal)
    if wl.mla:
        out, lse = DA.mla_decode_ragged(dq, dqo, dev["k"], **common)
    else:
        out, lse = DA.decode_attention_ragged(dq, dqo, dev["k"], dev["v"], group=wl.group,
                                              **common)
    ref_out, ref_lse = O.attention(q, inp.k, inp.v, scale=wl.softmax_scale,
                                   page_table=inp.page_table, valid_length=inp.valid_length,
                                   sink=inp.sink, causal=wl.causal, depth_v=wl.dv,
                                   max_seq_len=wl.max_seq_len, q_offsets=qo)
    torch.cuda.synchronize()
    got = DA.to_numpy_f64(out)
    gl = DA.to_numpy_f64(lse)
    assert got.shape == ref_out.shape and gl.shape == ref_lse.shape
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref_out).max() if got.size else 0.0
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(gl), fin), f"{what}: LSE finiteness differs"
    lerr = np.abs(gl[fin] - ref_lse[fin]).max() if fin.any() else 0.0
    say(f"  {what}: max|out-ref|={err:.3e}  max|lse-ref|={lerr:.3e}")
    assert err <= TOL_OUT[wl.dtype], f"{what}: output error {err:.3e}"
    assert lerr <= TOL_LSE, f"{what}: LSE error {lerr:.3e}"


CASES = [
    # (name, workload kwargs, tokens per sequence)
    ("gqa_g8_two_row_blocks", dict(batch=5, num_heads=32, kv_heads=4, depth=128,
                                   max_seq_len=300, q_len=4, causal=True, ragged=(5, 300, 1),
                                   sink=True), [3, 0, 1, 2, 4]),
    ("gqa_g4_paged_queue", dict(batch=4, num_heads=16, kv_heads=4, depth=128, max_seq_len=520,
                                q_len=4, causal=True, page_size=64, ragged=(4, 520, 0)),
     [4, 2, 1, 3]),
    ("gqa_noncausal_dense", dict(batch=3, num_heads=8, kv_heads=8, depth=64, max_seq_len=190,
                                 q_len=3), [1, 3, 2]),
    ("f32_mha", dict(batch=3, num_heads=4, kv_heads=4, depth=64, max_seq_len=77, q_len=3,
                     dtype="f32", causal=True, ragged=(3, 77, 0)), [2, 1, 3]),
    # fp32 blocks without a row: a sequence without tokens, and second row blocks
    # (rows 8 .. 11 of the 12-row fold) past short sequences' rows
    ("f32_empty_blocks", dict(batch=4, num_heads=16, kv_heads=4, depth=128, max_seq_len=600,
                              q_len=3, dtype="f32", causal=True, ragged=(1, 600, 1),
                              sink=True), [3, 0, 1, 2]),
    ("mla_paged", dict(batch=4, num_heads=128, kv_heads=1, depth=576, depth_v=512,
                       max_seq_len=260, q_len=3, mla=True, causal=True, page_size=32,
                       ragged=(3, 260, 0), scale=1.0 / np.sqrt(192.0), sink=True),
     [1, 3, 0, 2]),
    # P = 3: 576-key partitions (partial rows fp32 for partition 0, bf16 after it);
    # 768 rows in blocks of 128 that start at each sequence's first token row
    ("mla_long_split", dict(batch=3, num_heads=128, kv_heads=1, depth=576, depth_v=512,
                              max_seq_len=1700, q_len=3, mla=True, causal=True,
                              ragged=(3, 1700, 0), scale=1.0 / np.sqrt(192.0), sink=True),
     [3, 1, 2]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("P", [1, 3])
def test_ragged_q(case, P):
    name, kw, tokens = case
    wl = W.Workload(f"ragged_q_{name}", 9800 + len(name), **kw)
    _run(wl, tokens, P, f"{name} P={P}")


def test_ragged_q_uniform_equals_padded_call():
    """Every sequence with the same token count: the ragged call gives the padded
    call's bits."""
    wl = W.Workload("ragged_uniform", 9900, batch=3, num_heads=32, kv_heads=8, depth=128,
                    max_seq_len=400, q_len=2, causal=True, ragged=(2, 400, 0), sink=True)
    inp = W.make_inputs(wl)
    dev = device_inputs(inp)
    q, qo = _pack(inp, [2, 2, 2])
    common = dict(scale=wl.softmax_scale, valid_length=dev["valid_length"],
                  max_seq_len=wl.max_seq_len, num_partitions=3, sink_weights=dev["sink"],
                  causal=True)
    out_r, lse_r = DA.decode_attention_ragged(DA.to_device(q), DA.to_device(qo), dev["k"],
                                              dev["v"], max_q_len=2, group=wl.group, **common)
    out_p, lse_p = DA.decode_attention(dev["q"], dev["k"], dev["v"], group=wl.group, **common)
    torch.cuda.synchronize()
    assert torch.equal(out_r.reshape(out_p.shape).view(torch.int16), out_p.view(torch.int16))
    assert torch.equal(lse_r.reshape(lse_p.shape), lse_p)


@pytest.mark.parametrize("tokens", [[2, 0, 1], [2, 2, 2]])
def test_ragged_q_two_head_fold(tokens):
    """A dense ragged-q call (no valid_length, so no work queue) with 2 tokens x
    group 4 = 8 rows per KV head and P large enough for every CU: the streaming
    kernel folds two KV heads into each block."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wl = W.Workload("ragged_q_fold", 9890, batch=3, num_heads=16, kv_heads=4, depth=128,
                    max_seq_len=300, q_len=2, causal=True, sink=True)
    P = min(1024, -(-2 * cus // (wl.batch * wl.kv_heads)))
    _run(wl, tokens, P, f"fold tokens={tokens} P={P}")
