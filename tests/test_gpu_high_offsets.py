"""GPU parity with cache rows past 2 GiB of their pool: the kernels pin 64-bit byte
offsets to scalar registers, and a low half with bit 31 set must stay a plain
unsigned offset.  Each case lifts a seeded paged problem to the top of a pool of
more than 2 GiB (the pages below are zeros that no table entry names); the oracle
sees the compact pool."""
import pytest
import torch

import workloads as W
from gpu_util import compare, device_inputs, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu


def _lift(t: torch.Tensor, base: int) -> torch.Tensor:
    big = torch.zeros((base + t.shape[0],) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)
    big[base:] = t
    return big


CASES = [
    # (name, workload, first page index of the lifted pool)
    ("gqa_bf16_p128", W.Workload("high_gqa", 9801, batch=3, num_heads=32, kv_heads=8, depth=128,
                                 max_seq_len=1500, page_size=128, ragged=(1, 1500, 1),
                                 sink=True),
     (1 << 31) // (128 * 8 * 128 * 2) + 3),
    ("gqa_e4m3_p64", W.Workload("high_fp8", 9802, batch=3, num_heads=64, kv_heads=8, depth=128,
                                max_seq_len=900, page_size=64, ragged=(1, 900, 1),
                                kv_dtype="e4m3", k_scale=0.125, v_scale=0.125),
     (1 << 31) // (64 * 8 * 128) + 5),
    ("mla_p64", W.Workload("high_mla", 9803, batch=2, num_heads=128, kv_heads=1, depth=576,
                           depth_v=512, max_seq_len=700, mla=True, page_size=64,
                           ragged=(1, 700, 0), scale=1.0 / 192 ** 0.5),
     (1 << 31) // (64 * 576 * 2) + 2),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_pages_past_2gib(case):
    name, wl, base = case
    inp = W.make_inputs(wl)
    dev = device_inputs(inp)
    row_bytes = inp.k[0].nbytes
    say(f"[gpu] {name}: pool lifted by {base} pages, first used byte offset "
        f"{base * row_bytes} (2^31 = {1 << 31})")
    assert base * row_bytes >= 1 << 31
    dev["k"] = _lift(dev["k"], base)
    if dev["v"] is not None:
        dev["v"] = _lift(dev["v"], base)
    dev["page_table"] = dev["page_table"] + base
    ref_out, ref_lse = run_oracle(wl, inp)
    for P in (1, 3):
        out, lse = run_gpu(wl, dev, P)
        compare(wl, out, lse, ref_out, ref_lse, what=f"{name} P={P}")
    del dev
    torch.cuda.empty_cache()
