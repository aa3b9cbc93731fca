"""GPU: small fp32 split calls merge their partitions inside the partition pass (the
last block of each row group merges the group's rows; "mha_decoding_single_batch_
pipelined", description: the mha_splitk_reduce pass), so the call is one launch.

The in-pass merge is the merge pass's row merge: such a call equals, bit for bit,
its two halves called through the boundary (the partials pass, then
splitk_reduce()).  Also: the oracle, the count words back at zero after every call
(they share the workspace's queue section), and calls that take the separate merge
(more row groups than count words, more than 8 partitions)."""
import numpy as np
import pytest
import torch

import workloads as W
from decode_attention_07_amd import binding as DA
from gpu_util import check, device_inputs, run_gpu, say

pytestmark = pytest.mark.gpu


def _halves(wl, dev, P):
    ws = DA.decode_attention_partials(dev["q"], dev["k"], dev["v"], group=wl.group,
                                      scale=wl.softmax_scale, num_partitions=P,
                                      page_table=dev["page_table"],
                                      valid_length=dev["valid_length"],
                                      max_seq_len=wl.max_seq_len, causal=wl.causal)
    po, pm, ps = DA.workspace_views(ws, P, wl.batch, wl.q_len, wl.num_heads, wl.depth)
    return DA.splitk_reduce(po, pm, ps, num_q_heads=wl.num_heads, sink_weights=dev["sink"],
                            out_dtype=torch.float32)


CASES = [
    # (name, workload kwargs, P); row groups = batch x KV heads x row blocks
    ("tiny_c1", dict(batch=1, num_heads=8, kv_heads=8, depth=64, max_seq_len=256), 4),
    ("gqa4_ragged_sinks", dict(batch=3, num_heads=16, kv_heads=4, depth=128, max_seq_len=900,
                               ragged=(1, 900, 1), sink=True), 5),
    ("mtp3_causal_paged", dict(batch=2, num_heads=8, kv_heads=2, depth=64, max_seq_len=700,
                               q_len=3, causal=True, page_size=32, ragged=(1, 700, 0)), 7),
    ("fold8_two_row_blocks", dict(batch=2, num_heads=32, kv_heads=2, depth=128,
                                  max_seq_len=3000, sink=True), 8),
    ("empty_partitions", dict(batch=4, num_heads=4, kv_heads=4, depth=64, max_seq_len=2000,
                              ragged=(0, 2000, 2), sink=True), 6),
    # separate merge: 64 row groups (more than the count words), 16 and 48 partitions
    # (the latter the merge pass's two-waves-per-row form) and 80
    ("sixteen_partitions", dict(batch=2, num_heads=8, kv_heads=2, depth=128,
                                max_seq_len=16 * 64, sink=True), 16),
    ("many_groups", dict(batch=8, num_heads=8, kv_heads=8, depth=64, max_seq_len=300), 3),
    ("pair_merge", dict(batch=1, num_heads=8, kv_heads=2, depth=128, max_seq_len=48 * 64,
                        sink=True), 48),
    ("many_partitions", dict(batch=1, num_heads=4, kv_heads=2, depth=64,
                             max_seq_len=80 * 64), 80),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_in_pass_merge_equals_two_halves(case):
    name, kw, P = case
    wl = W.Workload(f"valu_merge_{name}", 9870 + P, dtype="f32", **kw)
    inp = W.make_inputs(wl)
    dev = device_inputs(inp)
    out, lse = run_gpu(wl, dev, P)
    out2, lse2 = _halves(wl, dev, P)
    torch.cuda.synchronize()
    assert torch.equal(out.view(-1, wl.depth), out2), name
    assert torch.equal(lse.view(-1), lse2), name
    check(wl, num_partitions=P, inp=inp, what=f"{name} P={P}")


def test_counts_back_at_zero_on_a_shared_workspace():
    """One zero-filled workspace serves calls with P = 4, 2, 7 and 4 again on problems
    of different sizes: each equals the same call on a fresh workspace, bit for bit,
    and leaves the queue section (queue word and count words) at zero."""
    wls = [W.Workload("valu_reuse_a", 9890, batch=2, num_heads=16, kv_heads=4, depth=128,
                      max_seq_len=1100, ragged=(1, 1100, 1), sink=True, dtype="f32"),
           W.Workload("valu_reuse_b", 9891, batch=1, num_heads=8, kv_heads=8, depth=64,
                      max_seq_len=256, dtype="f32"),
           W.Workload("valu_reuse_c", 9892, batch=3, num_heads=8, kv_heads=2, depth=64,
                      max_seq_len=900, q_len=2, causal=True, dtype="f32")]
    size = max(DA.decode_workspace_size(7, w.batch, w.q_len, w.num_heads, w.depth) for w in wls)
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    for wl, P in zip(wls + [wls[0]], (4, 2, 7, 4)):
        dev = device_inputs(W.make_inputs(wl))
        need = DA.decode_workspace_size(P, wl.batch, wl.q_len, wl.num_heads, wl.depth)
        out, lse = run_gpu(wl, dev, P, workspace=ws[:need])
        fresh = torch.zeros(need, dtype=torch.uint8, device="cuda")
        out2, lse2 = run_gpu(wl, dev, P, workspace=fresh)
        torch.cuda.synchronize()
        assert torch.equal(out, out2) and torch.equal(lse, lse2), f"{wl.name} P={P}"
        assert int(ws[:256].abs().sum()) == 0, f"{wl.name} P={P}: queue section not zero"
        assert int(fresh[:256].abs().sum()) == 0
        say(f"  {wl.name} P={P}: shared workspace equals a fresh one; section at zero")
