"""GPU parity: a valid_length above max_seq_len (including 2^31 and more as uint32)
counts as max_seq_len, in every kernel, dense and paged, P = 1 and split."""
import numpy as np
import pytest

import workloads as W
from gpu_util import check

pytestmark = pytest.mark.gpu

OVER = lambda S: np.array([S + 5, 0xFFFFFFFF, 7, S, 0x80000000, 1], np.uint32)  # noqa: E731

CASES = [
    # (name, workload kwargs)
    ("bf16_dense", dict(num_heads=16, kv_heads=4, depth=128, max_seq_len=300)),
    ("bf16_paged", dict(num_heads=32, kv_heads=4, depth=128, max_seq_len=320, page_size=64)),
    ("f32_dense", dict(num_heads=8, kv_heads=8, depth=64, max_seq_len=130, dtype="f32")),
    ("fp8_paged", dict(num_heads=16, kv_heads=2, depth=128, max_seq_len=256, page_size=32,
                       kv_dtype="e4m3", k_scale=0.125, v_scale=0.125)),
    ("mla_dense_mtp", dict(num_heads=128, kv_heads=1, depth=576, depth_v=512, max_seq_len=200,
                           q_len=2, causal=True, mla=True, scale=1.0 / np.sqrt(192.0))),
    ("mla_fp8_paged", dict(num_heads=128, kv_heads=1, depth=576, depth_v=512, max_seq_len=192,
                           page_size=64, mla=True, scale=1.0 / np.sqrt(192.0), kv_dtype="e4m3",
                           k_scale=0.125)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("P", [1, 3])
def test_valid_length_above_max_seq_len(name, kw, P):
    # drawn with every sequence full (all pages real), then given the lengths
    wl = W.Workload(f"over_{name}", 9900 + len(name), batch=6, sink=(P == 3), **kw)
    inp = W.make_inputs(wl, poison=False)
    inp.valid_length = OVER(wl.max_seq_len)  # the kernel and the oracle both cap these
    check(wl, num_partitions=P, inp=inp, what=f"over-long lengths {name} P={P}")
