"""GPU parity: the ragged KV layout (per-sequence row offsets into one concatenated
cache) through decode_attention_ragged_kv() / mla_decode_ragged_kv() against the
fp64 oracle, and bit for bit against the same call on the dense layout."""
import numpy as np
import pytest
import torch

import workloads as W
from decode_attention_07_amd import binding as DA
from gpu_util import compare, device_inputs, run_gpu, say
from oracle import oracle as O

pytestmark = pytest.mark.gpu

CASES = [
    # (name, workload kwargs, partitions)
    ("gqa_bf16_static", dict(batch=4, num_heads=16, kv_heads=4, depth=128, max_seq_len=700,
                             ragged=(1, 700, 1), sink=True), 1),
    ("gqa_bf16_queue", dict(batch=5, num_heads=32, kv_heads=8, depth=128, max_seq_len=900,
                            ragged=(1, 900, 1)), 5),          # ragged split: work queue
    ("gqa_bf16_two_heads", dict(batch=8, num_heads=32, kv_heads=8, depth=128,
                                max_seq_len=4096), 0),        # dense split: two-head fold
    ("gqa_bf16_causal_d64", dict(batch=3, num_heads=8, kv_heads=2, depth=64, max_seq_len=333,
                                 q_len=3, causal=True, ragged=(3, 333, 0)), 3),
    ("mha_f32", dict(batch=3, num_heads=8, kv_heads=8, depth=64, max_seq_len=300, dtype="f32",
                     ragged=(1, 300, 1), sink=True), 4),
    ("mla_t1", dict(batch=3, num_heads=128, kv_heads=1, depth=576, depth_v=512,
                    max_seq_len=500, mla=True, ragged=(1, 500, 1), sink=True), 2),
    ("mla_mtp2", dict(batch=3, num_heads=128, kv_heads=1, depth=576, depth_v=512,
                      max_seq_len=400, q_len=2, mla=True, causal=True, ragged=(2, 400, 0)), 1),
]


@pytest.mark.parametrize("name,kw,P", CASES, ids=[c[0] for c in CASES])
def test_ragged_kv_layout(name, kw, P):
    wl = W.Workload(f"ragged_kv_{name}", 9800 + len(name), **kw)
    if wl.mla:
        wl = wl.with_(scale=1.0 / np.sqrt(192.0))
    run_ragged_kv(wl, P, name)


def run_ragged_kv(wl, P, name):
    """One problem in the ragged KV layout against the oracle, and bit for bit
    against the same call on the dense layout."""
    say(f"[gpu] ragged KV layout {name}: B={wl.batch} T={wl.q_len} H={wl.num_heads} "
        f"KVH={wl.kv_heads} D={wl.depth} S={wl.max_seq_len} P={P}")
    inp = W.make_inputs(wl)
    kc, vc, offs = W.ragged_kv_layout(inp.k, inp.v, inp.lengths(), seed=wl.seed)
    dev = device_inputs(inp)
    dk, dv, doffs = DA.to_device(kc), DA.to_device(vc), DA.to_device(offs)
    common = dict(scale=wl.softmax_scale, max_seq_len=wl.max_seq_len,
                  valid_length=dev["valid_length"], num_partitions=P,
                  sink_weights=dev["sink"], causal=wl.causal)
    if wl.mla:
        out, lse = DA.mla_decode_ragged_kv(dev["q"], dk, doffs, **common)
    else:
        out, lse = DA.decode_attention_ragged_kv(dev["q"], dk, dv, doffs, group=wl.group,
                                                 **common)
    ref = O.attention(inp.q, kc, vc, scale=wl.softmax_scale, valid_length=inp.valid_length,
                      sink=inp.sink, causal=wl.causal, depth_v=wl.dv,
                      max_seq_len=wl.max_seq_len, kv_offsets=offs)
    compare(wl, out, lse, *ref, what=f"ragged KV {name}")
    # the same keys in the dense layout: the kernels do the same arithmetic
    dense_out, dense_lse = run_gpu(wl, dev, P)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                       dense_out.view(torch.int16) if out.dtype == torch.bfloat16
                       else dense_out), "ragged KV layout differs from the dense layout"
    assert torch.equal(lse, dense_lse)


def test_ragged_kv_shared_rows_and_no_valid_length():
    """Two sequences may start at the same row (a shared prefix), and without
    valid_length every sequence reads max_seq_len rows from its offset."""
    rng = np.random.default_rng(9850)
    B, H, KVH, D, S = 3, 16, 2, 128, 200
    q = W.f32_to_bf16_bits(rng.standard_normal((B, 1, H, D)).astype(np.float32))
    q[1] = q[0]
    k = W.f32_to_bf16_bits(rng.standard_normal((500, KVH, D)).astype(np.float32))
    v = W.f32_to_bf16_bits(rng.standard_normal((500, KVH, D)).astype(np.float32))
    offs = np.array([17, 17, 300], np.uint32)
    wl = W.Workload("ragged_kv_shared", 9851, batch=B, num_heads=H, kv_heads=KVH, depth=D,
                    max_seq_len=S)
    for P in (1, 3):
        out, lse = DA.decode_attention_ragged_kv(DA.to_device(q), DA.to_device(k),
                                                 DA.to_device(v), DA.to_device(offs), group=8,
                                                 scale=0.09, max_seq_len=S, num_partitions=P)
        ref = O.attention(q, k, v, scale=0.09, max_seq_len=S, kv_offsets=offs)
        compare(wl.with_(scale=0.09), out, lse, *ref, what=f"shared rows P={P}")
        got = out.float().cpu()
        assert torch.equal(got[0], got[1]), "same rows and q: same result"


def test_ragged_kv_requires_offsets():
    q = torch.zeros((2, 1, 8, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((64, 2, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        DA.decode_attention_ragged_kv(q, k, k, None, group=4, scale=0.1, max_seq_len=16)
    with pytest.raises(ValueError):  # a dense-layout cache is not a ragged one
        DA.decode_attention_ragged_kv(q, k.view(2, 32, 2, 128), k.view(2, 32, 2, 128),
                                      torch.zeros(2, dtype=torch.int32, device="cuda"), group=4,
                                      scale=0.1, max_seq_len=16)
