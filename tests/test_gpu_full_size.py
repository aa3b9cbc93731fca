"""GPU parity at full size, every output row: the MLA problem (T = 1 and the MTP
fold), its 8-bit and sparse forms, and the 8-bit and ragged-q GQA problems, each
in the launch configuration the benchmark times.  The oracle runs over a slice of
the sequences per test so that each test stays within a minute or so."""
import functools

import numpy as np
import pytest

import workloads as W
from gpu_util import compare, device_inputs, run_gpu, run_oracle, say
from decode_attention_07_amd import binding as DA
from oracle import oracle as O

pytestmark = pytest.mark.gpu

MLA_MTP_FP8 = W.MLA_FP8.with_(name="mla_fp8_mtp2_b64_h128_d576_dv512_s8192", q_len=2,
                              causal=True)


@functools.lru_cache(maxsize=1)
def _gpu_results(name, partitions):
    """The inputs of a workload and its GPU outputs at each P (one workload cached)."""
    wl = {w.name: w for w in (*W.ALL.values(), MLA_MTP_FP8)}[name]
    inp = W.make_inputs(wl)
    dev = device_inputs(inp)
    outs = {}
    for P in partitions:
        out, lse = run_gpu(wl, dev, P)
        outs[P] = (out.detach().clone(), lse.detach().clone())
    del dev
    return wl, inp, outs


def _chunk_rows(wl, chunk, n_chunks):
    """Row ids of sequences [chunk * B / n, (chunk + 1) * B / n)."""
    per = wl.batch // n_chunks
    rows_per_seq = wl.q_len * wl.num_heads
    return np.arange(chunk * per * rows_per_seq, (chunk + 1) * per * rows_per_seq,
                     dtype=np.int64)


def _check_chunk(name, partitions, chunk, n_chunks):
    wl, inp, outs = _gpu_results(name, partitions)
    rows = _chunk_rows(wl, chunk, n_chunks)
    say(f"[gpu] {name}: rows {rows[0]}..{rows[-1]} of {wl.batch * wl.q_len * wl.num_heads}")
    ref_out, ref_lse = run_oracle(wl, inp, rows)
    for P, (out, lse) in outs.items():
        compare(wl, out, lse, ref_out, ref_lse, rows=rows,
                what=f"{name} P={P or 'auto'} chunk {chunk}/{n_chunks}")


@pytest.mark.parametrize("chunk", range(4))
def test_mla_every_row(chunk):
    _check_chunk(W.MLA.name, (0, 1), chunk, 4)


@pytest.mark.parametrize("chunk", range(8))
def test_mla_mtp_every_row(chunk):
    _check_chunk(W.MLA_MTP.name, (0,), chunk, 8)


@pytest.mark.parametrize("chunk", range(4))
def test_mla_fp8_every_row(chunk):
    _check_chunk(W.MLA_FP8.name, (0,), chunk, 4)


@pytest.mark.parametrize("chunk", range(8))
def test_mla_fp8_mtp_every_row(chunk):
    _check_chunk(MLA_MTP_FP8.name, (0,), chunk, 8)


@pytest.mark.parametrize("chunk", range(2))
def test_mla_sparse_every_row(chunk):
    _check_chunk(W.MLA_SPARSE.name, (0, 1), chunk, 2)


@pytest.mark.parametrize("wl", [W.GQA_FP8, W.PAGED_FP8], ids=lambda w: w.name)
def test_fp8_gqa_full(wl):
    _check_chunk(wl.name, (0,), 0, 1)


def test_gqa_ragged_q_full():
    """1 to 4 new tokens per sequence (seeded), causal, q packed per sequence."""
    wl = W.GQA_RAGGED_Q
    tokens = W.ragged_q_tokens(wl)
    inp = W.make_inputs(wl)
    q, qo = W.pack_ragged_q(inp, tokens)
    dev = device_inputs(inp)
    say(f"[gpu] {wl.name}: {int(tokens.sum())} tokens")
    out, lse = DA.decode_attention_ragged(DA.to_device(q), DA.to_device(qo), dev["k"], dev["v"],
                                          max_q_len=wl.q_len, group=wl.group,
                                          scale=wl.softmax_scale, max_seq_len=wl.max_seq_len,
                                          causal=True)
    ref_out, ref_lse = O.attention(q, inp.k, inp.v, scale=wl.softmax_scale, causal=True,
                                   max_seq_len=wl.max_seq_len, q_offsets=qo)
    compare(wl, out, lse, ref_out, ref_lse, what=f"{wl.name} P=auto")
