"""Write oracle regression fixtures for tiny seeded cases.

The pages print no worked example with numbers, so the only stored expected
values in this folder are the oracle's own outputs on small seeded inputs,
written by this script (which calls nothing but oracle/ and the seeded input
generator).  They let the CPU suite notice any later change to the oracle's
arithmetic.  Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import workloads as W  # noqa: E402
from oracle import oracle as O  # noqa: E402

CASES = {
    # the tiny fp32 MHA problem (batch 1, 8 heads, depth 64, 256 keys)
    "tiny_mha_f32": W.TINY_MHA,
    # a small GQA bf16 problem with ragged lengths, pages and sink logits
    "small_paged_sink_bf16": W.Workload("small_paged_sink_bf16", 9101, batch=3, num_heads=8,
                                        kv_heads=2, depth=64, max_seq_len=80, page_size=16,
                                        ragged=(1, 80, 1), sink=True),
    # a small MLA-shaped problem with two MTP tokens under the causal mask
    "small_mla_mtp_bf16": W.Workload("small_mla_mtp_bf16", 9102, batch=2, num_heads=4,
                                     kv_heads=1, depth=40, depth_v=32, max_seq_len=24, mla=True,
                                     q_len=2, causal=True, ragged=(2, 24, 0)),
}


def compute(wl):
    inp = W.make_inputs(wl)
    out, lse = O.attention(inp.q, inp.k, inp.v, scale=wl.softmax_scale,
                           page_table=inp.page_table, valid_length=inp.valid_length,
                           sink=inp.sink, causal=wl.causal, depth_v=wl.dv,
                           max_seq_len=wl.max_seq_len)
    return out, lse


def main():
    data = {}
    for name, wl in CASES.items():
        out, lse = compute(wl)
        data[name] = {"out": [float(f"{x:.17g}") for x in out.reshape(-1)],
                      "lse": [float(f"{x:.17g}") for x in lse.reshape(-1)],
                      "shape": list(out.shape)}
    with open(os.path.join(HERE, "oracle_regression.json"), "w") as f:
        json.dump(data, f, indent=0)


if __name__ == "__main__":
    main()
