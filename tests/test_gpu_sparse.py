"""GPU parity: sparse top-k MLA (mla_decode_sparse(): each sequence attends to a list of
pool rows) through the C ABI against the fp64 oracle on the same seeded bits."""
import numpy as np
import pytest
import torch

import workloads as W
from decode_attention_07_amd import binding as DA
from gpu_util import check, compare, device_inputs, run_gpu, say
from oracle import oracle as O

pytestmark = pytest.mark.gpu

SCALE = 1.0 / np.sqrt(192.0)


def _wl(name, seed, B, T, H, S, topk, ragged=None, sink=False):
    return W.Workload(f"sparse_{name}", seed, batch=B, num_heads=H, kv_heads=1, depth=576,
                      depth_v=512, max_seq_len=S, q_len=T, mla=True, scale=SCALE, topk=topk,
                      ragged=ragged, sink=sink)


SMALL = [
    # (name, B, T, H, context S, topk, ragged contexts)
    ("h128_ragged", 3, 1, 128, 300, 100, (1, 300, 1)),
    ("h16_rows_partial", 2, 1, 16, 260, 77, None),
    ("mtp2_h64", 2, 2, 64, 200, 64, (40, 200, 0)),
    ("mtp2_h128_two_row_blocks", 2, 2, 128, 333, 96, None),
    ("h40_three_tokens", 2, 3, 40, 180, 50, (1, 180, 1)),
]


def test_sparse_bf16_partial_rows():
    """Long lists split in two (608 list positions per partition): the call's own
    split hands its merge bf16 partial rows; ragged contexts, one of a single key."""
    check(_wl("bf16_rows", 9961, 3, 1, 128, 2000, 1200, (1, 2000, 1), sink=True),
          num_partitions=2)


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
@pytest.mark.parametrize("P", [1, 2, 5])
def test_sparse_small(case, P):
    name, B, T, H, S, topk, ragged = case
    check(_wl(name, 9900 + S + topk, B, T, H, S, topk, ragged, sink=(P == 2)), num_partitions=P)


def _explicit(q, pool, idx, tl, sink=None, P=1):
    """One call on given host arrays (bf16 bits, int32 lists) against the oracle."""
    dq, dk = DA.to_device(q), DA.to_device(pool)
    di, dt = DA.to_device(idx), DA.to_device(tl)
    ds = DA.to_device(sink)
    out, lse = DA.mla_decode_sparse(dq, dk, di, dt, scale=SCALE, num_partitions=P,
                                    sink_weights=ds)
    return out, lse


def test_sparse_tile_boundaries():
    """Counts at and around the 32-key tile edges, a zero count (sink only), a row
    listed twice; list entries past each count hold values no load may follow."""
    rng = np.random.default_rng(9950)
    B, H, R, stride = 8, 128, 500, 70
    counts = np.array([0, 1, 31, 32, 33, 64, 65, 70], np.int32)
    q = W.f32_to_bf16_bits(rng.standard_normal((B, 1, H, 576)).astype(np.float32))
    pool = W.f32_to_bf16_bits(rng.standard_normal((R, 1, 576)).astype(np.float32))
    idx = rng.integers(0, R, size=(B, stride)).astype(np.int32)
    idx[5, 10] = idx[5, 11]
    for b in range(B):
        idx[b, counts[b]:] = [-1, 2**31 - 1, R, -2**31][b % 4]
    sink = rng.standard_normal(H).astype(np.float32)
    ref = O.attention(q, pool, None, depth_v=512, scale=SCALE, sink=sink, indices=idx,
                      topk_lengths=counts)
    wl = _wl("edges", 0, B, 1, H, stride, stride)
    for P in (1, 2, 3):
        out, lse = _explicit(q, pool, idx, counts, sink, P)
        compare(wl, out, lse, *ref, what=f"tile edges P={P}")


def test_sparse_identity_list_equals_dense_call():
    """Listing rows b*S .. b*S + N_b - 1 of the dense cache is mla_decode() with valid
    length N_b: both calls (the sparse one on the one-wave kernel, the dense one on
    the two-waves-per-SIMD kernel) match the oracle of the dense problem."""
    wl = W.Workload("sparse_identity", 9960, batch=4, num_heads=128, kv_heads=1, depth=576,
                    depth_v=512, max_seq_len=640, mla=True, scale=SCALE, ragged=(1, 640, 1),
                    sink=True)
    inp = W.make_inputs(wl)
    dev = device_inputs(inp)
    B, S = wl.batch, wl.max_seq_len
    lens = inp.valid_length.astype(np.int64)
    idx = np.zeros((B, S), np.int32)
    for b in range(B):
        idx[b] = b * S + np.arange(S)
    pool = dev["k"].reshape(B * S, 1, 576)
    ref = O.attention(inp.q, inp.k, None, depth_v=512, scale=SCALE, sink=inp.sink,
                      valid_length=inp.valid_length, max_seq_len=S)
    for P in (1, 3):
        out_d, lse_d = DA.mla_decode(dev["q"], dev["k"], scale=SCALE,
                                     valid_length=dev["valid_length"], num_partitions=P,
                                     sink_weights=dev["sink"])
        out_s, lse_s = DA.mla_decode_sparse(dev["q"], pool, DA.to_device(idx),
                                            DA.to_device(lens.astype(np.int32)), scale=SCALE,
                                            num_partitions=P, sink_weights=dev["sink"])
        compare(wl, out_d, lse_d, *ref, what=f"dense P={P}")
        compare(wl, out_s, lse_s, *ref, what=f"identity list P={P}")


def test_sparse_partials_plus_reduce_equals_full_call():
    wl = _wl("partials", 9970, 3, 2, 128, 400, 150, (20, 400, 0), sink=True)
    inp = W.make_inputs(wl)
    dev = device_inputs(inp)
    out, lse = run_gpu(wl, dev, 3)
    ws = DA.mla_decode_sparse_partials(dev["q"], dev["k"], dev["indices"], dev["topk_lengths"],
                                       scale=SCALE, num_partitions=3)
    po, pm, ps = DA.workspace_views(ws, 3, wl.batch, wl.q_len, wl.num_heads, 512)
    out2, lse2 = DA.splitk_reduce(po, pm, ps, num_q_heads=wl.num_heads,
                                  sink_weights=dev["sink"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(out.view(-1, 512).view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse.view(-1), lse2)
    # the call's partitions hold ceil(150 / 3) positions rounded up to the 32-key step
    ro, rm, rl = O.partials(inp.q, inp.k, None, depth_v=512, scale=SCALE, num_partitions=3,
                            keys_per_partition=64, indices=inp.indices,
                            topk_lengths=inp.topk_lengths)
    mo, ml = O.merge(ro, rm, rl, num_heads=wl.num_heads, sink=inp.sink)
    compare(wl, out2, lse2, mo, ml, what="partials + reduce vs oracle partials + merge")


def test_sparse_out_of_contract_counts_and_rows_are_clamped():
    """Counts above the stride act as the stride, below zero as zero; a counted row
    outside the pool (negative, or past the end) is read as the pool's last row."""
    rng = np.random.default_rng(9980)
    B, H, R, stride = 4, 128, 300, 48
    q = W.f32_to_bf16_bits(rng.standard_normal((B, 1, H, 576)).astype(np.float32))
    pool = W.f32_to_bf16_bits(rng.standard_normal((R, 1, 576)).astype(np.float32))
    idx = rng.integers(0, R, size=(B, stride)).astype(np.int32)
    counts = np.array([stride + 5, -3, 20, 2**31 - 1], np.int32)
    idx[2, 3] = -1
    idx[2, 7] = R
    idx[3, 0] = 2**31 - 1
    out, lse = _explicit(q, pool, idx, counts, None, 2)
    eff_counts = np.clip(counts, 0, stride).astype(np.int32)
    eff_idx = np.where((idx < 0) | (idx >= R), R - 1, idx).astype(np.int32)
    ref = O.attention(q, pool, None, depth_v=512, scale=SCALE, indices=eff_idx,
                      topk_lengths=eff_counts)
    compare(_wl("clamp", 0, B, 1, H, stride, stride), out, lse, *ref, what="clamped")


def test_sparse_rows_at_the_top_of_a_4gib_pool():
    """Rows near the end of the largest pool (2^32 / 1152 rows): the 32-bit byte
    offsets reach their top.  The oracle sees the listed rows through a compact copy."""
    R = (1 << 32) // 1152
    rng = np.random.default_rng(9990)
    B, H, stride = 2, 128, 40
    listed = np.concatenate([np.arange(R - 50, R), rng.choice(R - 50, 30, replace=False)])
    idx = rng.choice(listed, size=(B, stride)).astype(np.int32)
    counts = np.array([40, 33], np.int32)
    rows = W.f32_to_bf16_bits(rng.standard_normal((len(listed), 1, 576)).astype(np.float32))
    q = W.f32_to_bf16_bits(rng.standard_normal((B, 1, H, 576)).astype(np.float32))
    say(f"[gpu] 4 GiB pool: {R} rows, highest listed {int(idx.max())}")
    pool = torch.zeros((R, 1, 576), dtype=torch.bfloat16, device="cuda")
    pool[torch.from_numpy(listed).cuda()] = DA.to_device(rows)
    out, lse = DA.mla_decode_sparse(DA.to_device(q), pool, DA.to_device(idx),
                                    DA.to_device(counts), scale=SCALE, num_partitions=1)
    compact = {int(r): i for i, r in enumerate(listed)}
    cidx = np.vectorize(lambda r: compact[int(r)])(idx).astype(np.int32)
    ref = O.attention(q, rows, None, depth_v=512, scale=SCALE, indices=cidx,
                      topk_lengths=counts)
    compare(_wl("top", 0, B, 1, H, stride, stride), out, lse, *ref, what="4 GiB pool top")
    del pool
    torch.cuda.empty_cache()


# The sparse MLA problem at full size, every row: tests/test_gpu_full_size.py.


def test_sparse_rejects_bad_shapes():
    q = torch.zeros((1, 1, 128, 576), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((10, 1, 576), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    tl = torch.zeros((1,), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        DA.mla_decode_sparse(q, kv.view(10, 576, 1), idx, tl, scale=0.1)
    with pytest.raises(ValueError):
        DA.mla_decode_sparse(q, kv, idx.view(4, 1), tl, scale=0.1)
    # a pool past 2^32 / 1152 rows is refused before any launch
    big = (1 << 32) // 1152 + 1
    rc = DA.library().mla_decode_sparse(q.data_ptr(), kv.data_ptr(), big, idx.data_ptr(), 4,
                                        tl.data_ptr(), 1, 1, 128, 0.1, 1, None, q.data_ptr(),
                                        None, None, 0, None)
    assert rc == DA.DA_ERR_UNSUPPORTED


def test_sparse_zero_stride_and_zero_counts():
    """A list stride of 0 (nothing listed anywhere) and all-zero counts: every row is
    empty -- out = 0 and lse = -inf, or the sink alone (lse = sigma_h)."""
    rng = np.random.default_rng(9995)
    B, H, R = 3, 128, 40
    q = W.f32_to_bf16_bits(rng.standard_normal((B, 2, H, 576)).astype(np.float32))
    pool = W.f32_to_bf16_bits(rng.standard_normal((R, 1, 576)).astype(np.float32))
    sink = rng.standard_normal(H).astype(np.float32)
    wl = _wl("empty", 0, B, 2, H, 0, 0)
    for stride in (0, 40):
        idx = rng.integers(0, R, size=(B, stride)).astype(np.int32)
        counts = np.zeros(B, np.int32)
        for s, P in ((None, 1), (sink, 1), (sink, 3)):
            ref = O.attention(q, pool, None, depth_v=512, scale=SCALE, sink=s, indices=idx,
                              topk_lengths=counts)
            out, lse = _explicit(q, pool, idx, counts, s, P)
            compare(wl, out, lse, *ref, what=f"empty lists stride={stride} sink={s is not None}")
