"""GPU parity: decode_attention_fp8kv() (bf16 q, 8-bit e4m3 K/V with per-tensor
scales) through the C ABI against the fp64 oracle on the same seeded bits."""
import numpy as np
import pytest
import torch

import workloads as W
from decode_attention_07_amd import binding as DA
from gpu_util import check, device_inputs, run_gpu

pytestmark = pytest.mark.gpu

SMALL = [
    # (B, T, H, KVH, S, page, causal, ragged)
    (2, 1, 8, 8, 300, 0, False, False),      # MHA: one row per KV head
    (3, 1, 32, 8, 517, 0, False, True),      # GQA group 4, ragged tails
    (2, 1, 64, 8, 700, 128, False, True),    # group 8, paged
    (2, 1, 16, 1, 333, 32, False, True),     # group 16: one full row block
    (2, 2, 32, 2, 190, 64, True, True),      # MTP fold: 2 x 16 = 32 rows, 2 row blocks
    (1, 3, 12, 4, 97, 0, True, False),       # 3 tokens x group 3
    (4, 1, 40, 1, 250, 0, False, True),      # group 40: 3 row blocks, last partly filled
]


def _wl(shape, P, sink, k_scale=0.125, v_scale=0.1):
    B, T, H, KVH, S, page, causal, ragged = shape
    return W.Workload(f"fp8_{'x'.join(map(str, shape))}", 9600 + S + 7 * T + H, batch=B,
                      num_heads=H, kv_heads=KVH, depth=128, max_seq_len=S, q_len=T,
                      causal=causal, page_size=page, ragged=(1, S, 1) if ragged else None,
                      sink=sink, kv_dtype="e4m3", k_scale=k_scale, v_scale=v_scale)


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("P", [1, 3, 8])
def test_fp8_small(shape, P):
    check(_wl(shape, P, sink=(P == 3)), num_partitions=P)


@pytest.mark.parametrize("scales", [(1.0, 0.125), (0.03125, 0.16), (0.37, 0.019)],
                         ids=["unit_k", "small_k", "odd"])
def test_fp8_scales(scales):
    """The two scales enter as stated: k_scale in the scores, v_scale in the output.
    The stored elements are e4m3(8 N(0,1)); the pairs keep the real values about
    N(0,1) in size (v_scale * 8 <= 1.3), k_scale = 1 making the softmax very
    peaked, so the plain output bound applies."""
    k_scale, v_scale = scales
    shape = (3, 1, 32, 8, 411, 64, False, True)
    for P in (1, 5):
        check(_wl(shape, P, sink=True, k_scale=k_scale, v_scale=v_scale), num_partitions=P,
              what=f"fp8 scales {scales} P={P}")


def test_fp8_work_queue_many_items():
    """A ragged batch on the work queue with many items per block."""
    wl = W.Workload("fp8_queue", 9700, batch=48, num_heads=32, kv_heads=8, depth=128,
                    max_seq_len=3000, page_size=32, ragged=(1, 3000, 5), sink=True,
                    kv_dtype="e4m3", k_scale=0.125, v_scale=0.1)
    for P in (8, 29):
        check(wl, num_partitions=P)


def test_fp8_gqa_full_size():
    """The GQA decode problem (batch 32, 32/8 heads, 4096 keys) with an 8-bit cache,
    every row compared, at the heuristic's P and at P = 4."""
    wl = W.GQA.with_(name="gqa_fp8_b32_h32_kv8_d128_s4096", kv_dtype="e4m3", k_scale=0.125,
                     v_scale=0.125)
    for P in (0, 4):
        check(wl, num_partitions=P)


def test_fp8_partials_plus_reduce_equals_full_call():
    wl = _wl((2, 1, 32, 8, 640, 128, False, True), 3, sink=True)
    inp = W.make_inputs(wl)
    dev = device_inputs(inp)
    out, lse = run_gpu(wl, dev, 3)
    ws = DA.decode_attention_fp8kv_partials(
        dev["q"], dev["k"], dev["v"], k_scale=wl.k_scale, v_scale=wl.v_scale, group=wl.group,
        scale=wl.softmax_scale, num_partitions=3, page_table=dev["page_table"],
        valid_length=dev["valid_length"], max_seq_len=wl.max_seq_len)
    po, pm, ps = DA.workspace_views(ws, 3, wl.batch, wl.q_len, wl.num_heads, wl.dv)
    out2, lse2 = DA.splitk_reduce(po, pm, ps, num_q_heads=wl.num_heads,
                                  sink_weights=dev["sink"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(out.view(-1, wl.dv).view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse.view(-1), lse2)


def test_fp8_rejects_other_depths():
    q = torch.zeros((1, 1, 4, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 8, 4, 64), dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError, match="unsupported"):
        DA.decode_attention_fp8kv(q, k, k, k_scale=1.0, v_scale=1.0, group=1, scale=0.1)
