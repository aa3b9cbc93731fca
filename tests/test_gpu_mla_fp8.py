"""GPU parity: mla_decode_fp8kv() (bf16 q over an 8-bit e4m3 MLA cache, one scale for
the stored rows and their value slice) through the C ABI against the fp64 oracle."""
import numpy as np
import pytest
import torch

import workloads as W
from decode_attention_07_amd import binding as DA
from gpu_util import check, device_inputs, run_gpu

pytestmark = pytest.mark.gpu

SCALE = 1.0 / np.sqrt(192.0)


def _wl(name, seed, B, T, H, S, page=0, causal=False, ragged=False, sink=False, k_scale=0.125):
    return W.Workload(f"mla_fp8_{name}", seed, batch=B, num_heads=H, kv_heads=1, depth=576,
                      depth_v=512, max_seq_len=S, q_len=T, mla=True, causal=causal,
                      page_size=page, ragged=(1, S, 1) if ragged else None, scale=SCALE,
                      sink=sink, kv_dtype="e4m3", k_scale=k_scale, v_scale=k_scale)


SMALL = [
    # (B, T, H, S, page, causal, ragged)
    (2, 1, 128, 300, 0, False, False),
    (3, 1, 16, 97, 0, False, True),          # one partly filled row block, tails
    (2, 2, 128, 200, 64, True, True),        # MTP fold: two row blocks of 128, paged
    (2, 3, 64, 150, 32, True, True),         # 3 tokens x 64 heads = 192 rows
    (1, 1, 160, 64, 0, False, False),        # 160 rows: second block 32 rows
    (2, 1, 128, 33, 0, False, False),        # one whole tile and one key
    (2, 1, 128, 1536, 64, False, True),      # P = 3: 512-key partitions, bf16 partial rows
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("P", [1, 3])
def test_mla_fp8_small(shape, P):
    B, T, H, S, page, causal, ragged = shape
    check(_wl("x".join(map(str, shape)), 9610 + S + T, B, T, H, S, page, causal, ragged,
              sink=(P == 3)), num_partitions=P)


@pytest.mark.parametrize("k_scale", [0.05, 0.1, -0.125], ids=["small", "mid", "negative"])
def test_mla_fp8_scales(k_scale):
    """The one scale enters the scores and the value slice; a negative one flips both.
    Stored elements are e4m3(8 N(0,1)), so |k_scale| <= 1/8 keeps the real values
    N(0,1)-sized (and the outputs in the range the plain bf16 bound is for)."""
    for P in (1, 4):
        check(_wl(f"scale{k_scale}", 9650, 2, 2, 128, 400, 64, True, True, sink=True,
                  k_scale=k_scale), num_partitions=P, what=f"mla fp8 k_scale={k_scale} P={P}")


def test_mla_fp8_matches_bf16_call_on_converted_cache():
    """The 8-bit form computes the attention of the real cache values: with k_scale =
    1/8 (a power of two, so e4m3 x 1/8 is exact in bf16) the 8-bit call and
    mla_decode() on the converted cache both match the oracle, element by element."""
    from gpu_util import compare, run_oracle
    wl = _wl("converted", 9660, 3, 2, 128, 520, 64, True, True, sink=True, k_scale=0.125)
    inp = W.make_inputs(wl)
    dev = device_inputs(inp)
    k_bf16 = (dev["k"].view(torch.float8_e4m3fn).to(torch.float32) * 0.125).to(torch.bfloat16)
    ref = run_oracle(wl, inp)
    for P in (1, 3):
        out8, lse8 = run_gpu(wl, dev, P)
        out16, lse16 = DA.mla_decode(dev["q"], k_bf16, scale=SCALE, page_table=dev["page_table"],
                                     valid_length=dev["valid_length"], max_seq_len=wl.max_seq_len,
                                     num_partitions=P, sink_weights=dev["sink"], causal=True)
        compare(wl, out8, lse8, *ref, what=f"8-bit call P={P}")
        compare(wl, out16, lse16, *ref, what=f"bf16 call on the converted cache P={P}")


def test_mla_fp8_score_jump_restart():
    """Keys whose scores exceed the first tile's by far force the fixed-reference kernel
    to restart its partition (and reload its 8-bit staging ring); the result must not
    change."""
    wl = _wl("jump", 9670, 2, 1, 128, 256)
    inp = W.make_inputs(wl, poison=False)
    q = W.bf16_bits_to_f32(inp.q)
    for b, (j1, j2) in enumerate([(70, 200), (40, 250)]):
        sgn = np.sign(q[b, 0, 0]).astype(np.float32)
        for j, real in ((j1, 6.0), (j2, 12.0)):   # stored 48 and 96, exact in e4m3
            codes = torch.from_numpy(sgn * np.float32(real / wl.k_scale)).to(
                torch.float8_e4m3fn).view(torch.uint8).numpy()
            inp.k[b, j, 0] = codes
    for P in (1, 2):
        check(wl, num_partitions=P, inp=inp, what=f"mla fp8 score jump P={P}", ulp_rel=True)


def test_mla_fp8_partials_plus_reduce_equals_full_call():
    wl = _wl("halves", 9680, 3, 2, 128, 700, 0, True, True, sink=True)
    inp = W.make_inputs(wl)
    dev = device_inputs(inp)
    P = 3
    out, lse = run_gpu(wl, dev, P)
    ws = DA.mla_decode_fp8kv_partials(dev["q"], dev["k"], k_scale=wl.k_scale, scale=SCALE,
                                      num_partitions=P, valid_length=dev["valid_length"],
                                      causal=True)
    po, pm, ps = DA.workspace_views(ws, P, wl.batch, wl.q_len, wl.num_heads, wl.dv)
    out2, lse2 = DA.splitk_reduce(po, pm, ps, num_q_heads=wl.num_heads,
                                  sink_weights=dev["sink"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(out.view(-1, wl.dv).view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse.view(-1), lse2)


# The 8-bit MLA problem at full size, every row: tests/test_gpu_full_size.py.


def test_mla_fp8_rejects_bad_scale():
    q = torch.zeros((1, 1, 128, 576), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 64, 1, 576), dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError, match="invalid"):
        DA.mla_decode_fp8kv(q, kv, k_scale=float("nan"), scale=0.1)
