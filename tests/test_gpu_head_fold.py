"""GPU parity of the two-head fold of the streaming GQA kernels (bf16 and 8-bit
caches) against the fp64 oracle.

A split call on the static mapping (no valid_length, so no work queue) whose
fold of query rows per KV head is at most 8 runs two KV heads per block, as
long as the blocks still cover every CU: P * batch * (KV heads / 2) >= CUs.
Each case picks P from the device's CU count so that the fold is taken, and the
small key counts leave many partitions empty."""
import math

import pytest
import torch

import workloads as W
from gpu_util import check

pytestmark = pytest.mark.gpu


def _fold_partitions(batch, kv_heads, extra=1):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return min(1024, extra * math.ceil(2 * cus / (batch * kv_heads)))


FOLD = [
    # (B, T, H, KVH, D, S, page, causal, sink)
    (2, 1, 16, 4, 128, 777, 0, False, False),    # group 4: 2 x 4 rows per block
    (1, 1, 32, 4, 128, 3001, 0, False, True),    # group 8: 2 x 8 rows, sinks
    (2, 2, 8, 2, 128, 500, 0, True, True),       # 2 tokens x group 4, causal
    (2, 1, 16, 4, 128, 1024, 32, False, False),  # paged, no valid_length
    (3, 1, 6, 2, 128, 333, 0, False, False),     # group 3: padded rows in each slot
    (2, 1, 16, 4, 64, 600, 0, False, True),      # depth 64
]


@pytest.mark.parametrize("shape", FOLD, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("more", [1, 3])
def test_bf16_two_head_fold(shape, more):
    B, T, H, KVH, D, S, page, causal, sink = shape
    wl = W.Workload(f"fold_{'x'.join(map(str, shape))}", 9900 + S + 7 * T + H, batch=B,
                    num_heads=H, kv_heads=KVH, depth=D, max_seq_len=S, q_len=T,
                    causal=causal, page_size=page, sink=sink)
    check(wl, num_partitions=_fold_partitions(B, KVH, more))


@pytest.mark.parametrize("shape", [s for s in FOLD if s[4] == 128],
                         ids=lambda s: "x".join(map(str, s)))
def test_fp8_two_head_fold(shape):
    B, T, H, KVH, D, S, page, causal, sink = shape
    wl = W.Workload(f"fold8_{'x'.join(map(str, shape))}", 9950 + S + 7 * T + H, batch=B,
                    num_heads=H, kv_heads=KVH, depth=D, max_seq_len=S, q_len=T,
                    causal=causal, page_size=page, sink=sink, kv_dtype="e4m3",
                    k_scale=0.125, v_scale=0.1)
    check(wl, num_partitions=_fold_partitions(B, KVH))


def test_long_context_fp8_auto():
    """The long-context problem over an 8-bit cache with the automatic P (64 on
    MI355X: two heads per block), sampled rows against the oracle."""
    wl = W.LONG.with_(name="long_fp8", kv_dtype="e4m3", k_scale=0.125, v_scale=0.1)
    check(wl, num_partitions=0)
