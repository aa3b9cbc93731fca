"""GPU parity: mla_decode() through the C ABI against the fp64 oracle."""
import numpy as np
import pytest

import workloads as W
from gpu_util import check

pytestmark = pytest.mark.gpu


# The MLA problem at full size, every row: tests/test_gpu_full_size.py.


# ---- small MLA shapes: every row compared ----------------------------------------

SMALL = [
    # (B, T, H, S, page, causal, ragged)
    (2, 1, 128, 300, 0, False, False),
    (3, 1, 16, 97, 0, False, True),          # 16 heads: one partly filled row block
    (2, 2, 128, 200, 64, True, True),        # MTP fold: two row blocks of 128
    (2, 3, 64, 150, 32, True, True),         # 3 tokens x 64 heads = 192 rows
    (1, 1, 160, 64, 0, False, False),        # 160 rows: second block 32 rows
    (2, 2, 128, 3000, 64, True, True),       # P = 3: 1024-key partitions, bf16 partial rows
    (2, 1, 128, 1536, 0, False, True),       # P = 3: 512-key partitions, the shortest in bf16
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("P", [1, 3])
def test_mla_small(shape, P):
    B, T, H, S, page, causal, ragged = shape
    wl = W.Workload(f"mla_small_{'x'.join(map(str, shape))}", 9200 + S + T, batch=B,
                    num_heads=H, kv_heads=1, depth=576, depth_v=512, max_seq_len=S, q_len=T,
                    mla=True, causal=causal, page_size=page,
                    ragged=(1, S, 1) if ragged else None, scale=1.0 / np.sqrt(192.0),
                    sink=(P == 3))
    check(wl, num_partitions=P)


@pytest.mark.parametrize("n", [1, 2, 3, 33])
def test_mla_mtp_causal_short(n):
    """Two MTP tokens over a handful of keys: the causal mask moves the result by O(1)."""
    wl = W.Workload(f"mla_mtp_short_{n}", 9300 + n, batch=2, num_heads=128, kv_heads=1,
                    depth=576, depth_v=512, max_seq_len=64, q_len=2, mla=True, causal=True,
                    scale=1.0 / np.sqrt(192.0))
    inp = W.make_inputs(wl, poison=False)
    inp.valid_length = np.array([n, max(1, n - 1)], np.uint32)
    check(wl, num_partitions=1, inp=inp, what=f"mla mtp causal N={n}")


def test_mla_score_jump_restart():
    """Keys whose scores exceed the first tile's by ~900 (log2 units) force the
    fixed-reference kernel to restart its partition; the result must not change."""
    wl = W.Workload("mla_jump", 9400, batch=2, num_heads=128, kv_heads=1, depth=576,
                    depth_v=512, max_seq_len=256, mla=True, scale=1.0 / np.sqrt(192.0))
    inp = W.make_inputs(wl, poison=False)
    q = W.bf16_bits_to_f32(inp.q)
    for b, (j1, j2) in enumerate([(70, 200), (40, 250)]):
        sgn = np.sign(q[b, 0, 0]).astype(np.float32)
        inp.k[b, j1, 0] = W.f32_to_bf16_bits(sgn * 6.0)     # large aligned key
        inp.k[b, j2, 0] = W.f32_to_bf16_bits(sgn * 12.0)    # larger still, later
    # |out| reaches 12 here (V rows of +-6 / +-12), beyond the N(0,1) regime of
    # the 1e-2 absolute bound: allow one bf16 ulp of the reference on top.
    for P in (1, 2):
        check(wl, num_partitions=P, inp=inp, what=f"mla score jump P={P}", ulp_rel=True)


@pytest.mark.parametrize("jump", [58.0, 90.0], ids=["inside_headroom", "restart"])
def test_mla_large_values_near_headroom(jump):
    """Cache values of magnitude 2^15 with weights up to 2^58 (inside the fixed-reference
    headroom of 2^64: no restart) or a jump of 90 (restart): the weight x value sums
    of a partition reach about 2^81 and must stay finite and exact to the bound.  The
    scores come from the rope part of q only (q[..., :512] = 0), so the large values
    do not move them; 200 keys past the first tile score `jump` (log2 units) above it.
    Both MLA kernels: the dense call, and the sparse call over an identity list."""
    import torch
    from decode_attention_07_amd import binding as DA
    from gpu_util import compare, device_inputs
    from oracle import oracle as O
    B, H, S = 2, 128, 700
    wl = W.Workload(f"mla_large_values_{int(jump)}", 9450 + int(jump), batch=B, num_heads=H,
                    kv_heads=1, depth=576, depth_v=512, max_seq_len=S, mla=True,
                    scale=1.0 / np.sqrt(192.0))
    rng = np.random.default_rng(9450 + int(jump))
    qpe = rng.standard_normal(64).astype(np.float32)
    q = np.zeros((B, 1, H, 576), np.float32)
    q[..., 512:] = qpe + 0.02 * rng.standard_normal((B, 1, H, 64)).astype(np.float32)
    k = np.zeros((B, S, 1, 576), np.float32)
    k[..., :512] = 2.0 ** 15 * (1.0 + 0.5 * rng.random((B, S, 1, 512), dtype=np.float32))
    k[..., 512:] = 0.1 * rng.standard_normal((B, S, 1, 64)).astype(np.float32)
    log2_per_dot = wl.softmax_scale * np.log2(np.e)
    c = jump / (np.abs(qpe).sum() * log2_per_dot)  # aligned key: score ~ jump
    hot = rng.choice(np.arange(64, S), size=(B, 200), replace=True)
    for b in range(B):
        k[b, hot[b], 0, 512:] = c * np.sign(qpe)
    q16, k16 = W.f32_to_bf16_bits(q), W.f32_to_bf16_bits(k)
    ref = O.attention(q16, k16, None, depth_v=512, scale=wl.softmax_scale, max_seq_len=S)
    dq, dk = DA.to_device(q16), DA.to_device(k16)
    idx = np.stack([b * S + np.arange(S) for b in range(B)]).astype(np.int32)
    counts = np.full(B, S, np.int32)
    for P in (1, 2):
        out, lse = DA.mla_decode(dq, dk, scale=wl.softmax_scale, num_partitions=P)
        compare(wl, out, lse, *ref, what=f"dense |v|~2^15 jump {jump} P={P}", ulp_rel=True)
        out_s, lse_s = DA.mla_decode_sparse(dq, dk.reshape(B * S, 1, 576), DA.to_device(idx),
                                            DA.to_device(counts), scale=wl.softmax_scale,
                                            num_partitions=P)
        compare(wl, out_s, lse_s, *ref, what=f"sparse |v|~2^15 jump {jump} P={P}",
                ulp_rel=True)
    torch.cuda.synchronize()


def test_mla_partials_plus_reduce_equals_full_call():
    """mla_decode() with P > 1 equals, bit for bit, its two halves called through
    the boundary: the partials pass, then splitk_reduce()."""
    import torch
    from decode_attention_07_amd import binding as DA
    from gpu_util import device_inputs, run_gpu
    wl = W.Workload("mla_halves", 9500, batch=3, num_heads=128, kv_heads=1, depth=576,
                    depth_v=512, max_seq_len=700, q_len=2, mla=True, causal=True,
                    ragged=(2, 700, 0), scale=1.0 / np.sqrt(192.0), sink=True)
    inp = W.make_inputs(wl)
    dev = device_inputs(inp)
    P = 3
    out, lse = run_gpu(wl, dev, P)
    ws = DA.mla_decode_partials(dev["q"], dev["k"], scale=wl.softmax_scale, num_partitions=P,
                                valid_length=dev["valid_length"], causal=True)
    po, pm, ps = DA.workspace_views(ws, P, wl.batch, wl.q_len, wl.num_heads, wl.dv)
    out2, lse2 = DA.splitk_reduce(po, pm, ps, num_q_heads=wl.num_heads,
                                  sink_weights=dev["sink"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(out.view(-1, wl.dv).view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse.view(-1), lse2)


@pytest.mark.parametrize("scale", [0.0, -1.0 / np.sqrt(192.0), -0.05], ids=["zero", "neg", "neg_small"])
@pytest.mark.parametrize("P", [1, 3])
def test_mla_zero_and_negative_scale(scale, P):
    """A zero or negative scale: the kernel folds the sign into Q (exact in bf16)
    and applies the magnitude once per weight, after the row max; masked keys
    (causal MTP, ragged tails) must still drop out when the scale is 0."""
    wl = W.Workload(f"mla_scale_{P}_{int(round(scale * 1000))}", 9400 + P, batch=3,
                    num_heads=128, kv_heads=1, depth=576, depth_v=512, max_seq_len=230, q_len=2,
                    mla=True, causal=True, ragged=(1, 230, 1), scale=scale, sink=(P == 3))
    check(wl, num_partitions=P)
