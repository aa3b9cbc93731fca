"""GPU parity: short sequences inside the MLA kernels' own long splits.

Such a split hands the merge partition 0's partial rows in fp32 and the others' in
bf16 ("mha_decoding_single_batch_pipelined", Args `output_ptr`: the partition
kernel's partial output in the output type).  A short sequence's keys all fall in
partition 0, so its partial row is the whole result, of a few keys: kept in fp32,
the output is rounded once, as an unsplit call rounds it; a bf16 partial row would
add a rounding as large as the output's own.  Checked against the fp64 oracle with
the usual bounds, and for the short sequences' rows against the unsplit call's
own error: the split may not be less accurate there."""
import numpy as np
import pytest

import workloads as W
from decode_attention_07_amd import binding as DA
from gpu_util import compare, device_inputs, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu

SCALE = 1.0 / np.sqrt(192.0)


def _check_short(wl, inp, P, short, what):
    dev = device_inputs(inp)
    out, lse = run_gpu(wl, dev, P)
    out1, _ = run_gpu(wl, dev, 1)
    ref_out, ref_lse = run_oracle(wl, inp)
    compare(wl, out, lse, ref_out, ref_lse, what=what)
    got = DA.to_numpy_f64(out)
    got1 = DA.to_numpy_f64(out1)
    for b in short:
        e_split = float(np.abs(got[b] - ref_out[b]).max())
        e_one = float(np.abs(got1[b] - ref_out[b]).max())
        say(f"  {what}, sequence {b}: max error split {e_split:.3e}, unsplit {e_one:.3e}")
        assert e_split <= 1.25 * e_one + 1e-4, f"{what}: sequence {b} less accurate when split"


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "e4m3"])
def test_short_sequences_in_a_long_split(fp8):
    kw = dict(kv_dtype="e4m3", k_scale=0.125, v_scale=0.125) if fp8 else {}
    wl = W.Workload(f"mla_short_{'fp8' if fp8 else 'bf16'}", 9790, batch=4, num_heads=128,
                    kv_heads=1, depth=576, depth_v=512, max_seq_len=2100, q_len=2, mla=True,
                    causal=True, page_size=64, scale=SCALE, sink=True, **kw)
    inp = W.make_inputs(wl, poison=False)
    inp.valid_length = np.array([2100, 7, 1500, 2], np.uint32)
    _check_short(wl, inp, 4, (1, 3), f"{wl.name} P=4 (544-key partitions)")


def test_short_lists_in_a_long_sparse_split():
    wl = W.Workload("sparse_short_lists", 9791, batch=3, num_heads=128, kv_heads=1, depth=576,
                    depth_v=512, max_seq_len=2000, mla=True, scale=SCALE, topk=1300, sink=True)
    inp = W.make_inputs(wl)
    inp.topk_lengths = np.array([1300, 3, 1], np.int32).astype(inp.topk_lengths.dtype)
    _check_short(wl, inp, 2, (1, 2), f"{wl.name} P=2 (650 list positions per partition)")
