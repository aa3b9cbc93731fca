"""GPU: decode_attention_no_alloc() (the split-K workspace is the library's static
per-device scratch) gives the results of decode_attention(), call after call."""
import numpy as np
import pytest
import torch

import workloads as W
from decode_attention_07_amd import binding as DA
from gpu_util import compare, device_inputs, run_oracle, say

pytestmark = pytest.mark.gpu


def _both(wl, P):
    """The same seeded problem through decode_attention() (its own workspace) and
    decode_attention_no_alloc() (the scratch), and the oracle."""
    inp = W.make_inputs(wl)
    dev = device_inputs(inp)
    kw = dict(group=wl.group, scale=wl.softmax_scale, page_table=dev["page_table"],
              valid_length=dev["valid_length"], max_seq_len=wl.max_seq_len, num_partitions=P,
              sink_weights=dev["sink"], causal=wl.causal)
    B, T, H, D = wl.batch, wl.q_len, wl.num_heads, wl.depth
    ref_out, ref_lse = DA.decode_attention(dev["q"], dev["k"], dev["v"], **kw)
    out = torch.full((B, T, H, D), float("nan"), dtype=dev["q"].dtype, device="cuda")
    lse = torch.full((B, T, H), float("nan"), dtype=torch.float32, device="cuda")
    DA.decode_attention_no_alloc(dev["q"], dev["k"], dev["v"], out=out, lse=lse, **kw)
    torch.cuda.synchronize()
    return inp, out, lse, ref_out, ref_lse


def _check(wl, P, what):
    say(f"[gpu] no-alloc {what}: B={wl.batch} H={wl.num_heads} KVH={wl.kv_heads} "
        f"S={wl.max_seq_len} P={P}")
    inp, out, lse, ref_out, ref_lse = _both(wl, P)
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), what
    assert torch.equal(lse, ref_lse), what
    compare(wl, out, lse, *run_oracle(wl, inp), what=what)


def test_no_alloc_two_calls_in_a_row():
    """A ragged paged problem on the work queue (its queue word lives in the scratch),
    then a smaller dense one with sinks: both equal decode_attention() bit for bit
    and the oracle within the bounds."""
    big = W.Workload("no_alloc_big", 9951, batch=16, num_heads=64, kv_heads=8, depth=128,
                     max_seq_len=8192, page_size=128, ragged=(1, 8192, 2))
    P = DA.num_partitions(16, 1, 64, 8, 128, 128, 8192, ragged=True)
    assert P > 1 and DA.decode_workspace_size(P, 16, 1, 64, 128) <= DA.DA_NO_ALLOC_SCRATCH_BYTES
    _check(big, 0, "ragged paged (work queue)")
    small = W.Workload("no_alloc_small", 9952, batch=3, num_heads=8, kv_heads=2, depth=64,
                       max_seq_len=700, sink=True)
    _check(small, 3, "smaller dense, sinks")
    _check(big.with_(name="no_alloc_big2", seed=9953, batch=5), 0, "ragged paged again")


def test_no_alloc_fp32_splits_merged_in_the_pass():
    """Small fp32 split calls merge inside their partition pass with count words in
    the scratch's queue section: two in a row (the second smaller) both equal
    decode_attention() bit for bit and the oracle within the bounds."""
    a = W.Workload("no_alloc_f32_a", 9954, batch=2, num_heads=16, kv_heads=4, depth=128,
                   max_seq_len=1500, ragged=(1, 1500, 1), sink=True, dtype="f32")
    _check(a, 6, "fp32, merged in the pass")
    b = W.Workload("no_alloc_f32_b", 9955, batch=1, num_heads=8, kv_heads=8, depth=64,
                   max_seq_len=256, dtype="f32")
    _check(b, 4, "smaller fp32, merged in the pass")


def test_no_alloc_refuses_an_oversized_workspace():
    """A call whose workspace exceeds the scratch is refused before any launch; the
    next call still works."""
    B, H, KVH, D, S = 8, 64, 8, 128, 4096
    P = 1024
    assert DA.decode_workspace_size(P, B, 1, H, D) > DA.DA_NO_ALLOC_SCRATCH_BYTES
    q = torch.zeros((B, 1, H, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, S, KVH, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(DA.DecodeAttentionError) as e:
        DA.decode_attention_no_alloc(q, k, k, group=H // KVH, scale=0.1, out=out,
                                     num_partitions=P)
    assert e.value.status == DA.DA_ERR_WORKSPACE
    small = W.Workload("no_alloc_after", 9954, batch=2, num_heads=16, kv_heads=4, depth=128,
                       max_seq_len=300, ragged=(1, 300, 1))
    _check(small, 2, "after a refused call")
