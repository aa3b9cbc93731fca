"""GPU parity: decode_attention() through the C ABI against the fp64 oracle."""
import numpy as np
import pytest
import torch

import workloads as W
from decode_attention_07_amd import binding as DA
from gpu_util import check, device_inputs, run_gpu, say

pytestmark = pytest.mark.gpu


# ---- the problem configurations at full size ------------------------------------

@pytest.mark.parametrize("P", [1, 4])
def test_tiny_mha_f32(P):
    check(W.TINY_MHA, num_partitions=P)


def test_gqa_full_auto():
    check(W.GQA, num_partitions=0)


@pytest.mark.parametrize("P", [1, 8, 32, 128, 0])
def test_long_context_sinks(P):
    check(W.LONG, num_partitions=P)


# ---- shapes spanning several tiles, ragged tails, splits --------------------------

SMALL = [
    # (B, H, KVH, D, S, dtype)
    (2, 8, 8, 64, 300, "f32"),
    (3, 8, 2, 128, 517, "bf16"),
    (2, 6, 2, 128, 200, "bf16"),      # group 3 -> padded row bucket
    (2, 10, 2, 64, 129, "bf16"),      # group 5
    (1, 4, 4, 128, 33, "f32"),
    (2, 16, 2, 128, 700, "f32"),      # fp32 with 8 rows per block
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("P", [1, 3, 8])
def test_small_shapes(shape, P):
    B, H, KVH, D, S, dt = shape
    wl = W.Workload(f"small_{'x'.join(map(str, shape))}", 8100 + S, batch=B, num_heads=H,
                    kv_heads=KVH, depth=D, max_seq_len=S, dtype=dt)
    check(wl, num_partitions=P)


@pytest.mark.parametrize("P", [1, 2, 5])
def test_ragged_lengths_with_zero_and_sink(P):
    wl = W.Workload("ragged_sink", 8201, batch=5, num_heads=8, kv_heads=2, depth=128,
                    max_seq_len=400, ragged=(0, 400, 1), sink=True)
    inp = W.make_inputs(wl, poison=False)  # lengths are edited below
    inp.valid_length[2] = 0          # an empty sequence
    inp.valid_length[3] = 400        # a full one
    check(wl, num_partitions=P, inp=inp)


@pytest.mark.parametrize("page_size", [32, 64, 128])
@pytest.mark.parametrize("P", [1, 3])
def test_paged_ragged_small(page_size, P):
    wl = W.Workload(f"paged_small_{page_size}", 8300 + page_size, batch=4, num_heads=16,
                    kv_heads=4, depth=128, max_seq_len=1000, page_size=page_size,
                    ragged=(1, 1000, 1))
    check(wl, num_partitions=P)


@pytest.mark.parametrize("T,P", [(2, 1), (2, 3), (3, 2)])
def test_causal_multi_token(T, P):
    wl = W.Workload(f"causal_T{T}", 8400 + T, batch=3, num_heads=4, kv_heads=2, depth=64,
                    max_seq_len=150, q_len=T, causal=True, ragged=(1, 150, 1), dtype="f32")
    check(wl, num_partitions=P)


def test_sink_dominant_small_n():
    """Sink logits of order +3 over a handful of keys: an O(1) effect on out and LSE."""
    wl = W.Workload("sink_small", 8501, batch=2, num_heads=8, kv_heads=4, depth=64,
                    max_seq_len=16, dtype="f32", sink=True)
    inp = W.make_inputs(wl)
    inp.sink[:] += 3.0
    for P in (1, 2, 4):
        check(wl, num_partitions=P, inp=inp, what=f"sink_small P={P}")


# ---- the split-K pieces on their own ----------------------------------------------

def test_partials_plus_reduce_equals_decode_attention():
    wl = W.GQA.with_(batch=4, max_seq_len=1000, ragged=(1, 1000, 1), sink=True)
    inp = W.make_inputs(wl)
    dev = device_inputs(inp)
    P = 4
    out, lse = run_gpu(wl, dev, P)
    ws = DA.decode_attention_partials(dev["q"], dev["k"], dev["v"], group=wl.group,
                                      scale=wl.softmax_scale, num_partitions=P,
                                      valid_length=dev["valid_length"])
    po, pm, ps = DA.workspace_views(ws, P, wl.batch, 1, wl.num_heads, wl.depth)
    out2, lse2 = DA.splitk_reduce(po, pm, ps, num_q_heads=wl.num_heads,
                                  sink_weights=dev["sink"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(out.view(-1, wl.depth).view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse.view(-1), lse2)


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
def test_queue_partial_rows_match_oracle_partials(kv):
    """The partial rows of a ragged paged call on the work queue, row by row against
    the oracle's partials: the partitions past a short sequence's end are exactly
    empty (O = 0, m = -inf, l = 0), the others agree to the partials' tolerance."""
    from oracle import oracle as O
    base = W.GQA if kv == "bf16" else W.GQA_FP8
    wl = base.with_(name="queue_partials", seed=8640, batch=9, max_seq_len=1000, page_size=64,
                    ragged=(1, 1000, 3))
    inp = W.make_inputs(wl)
    dev = device_inputs(inp)
    P = 4
    C = -(-wl.max_seq_len // P)
    C = -(-C // 16) * 16  # partitions of the kernel: a whole number of 16-key steps
    common = dict(group=wl.group, scale=wl.softmax_scale, num_partitions=P,
                  page_table=dev["page_table"], valid_length=dev["valid_length"],
                  max_seq_len=wl.max_seq_len)
    if kv == "bf16":
        ws = DA.decode_attention_partials(dev["q"], dev["k"], dev["v"], **common)
    else:
        ws = DA.decode_attention_fp8kv_partials(dev["q"], dev["k"], dev["v"], k_scale=wl.k_scale,
                                                v_scale=wl.v_scale, **common)
    po, pm, pl = DA.workspace_views(ws, P, wl.batch, 1, wl.num_heads, wl.depth)
    torch.cuda.synchronize()
    ro, rm, rl = O.partials(inp.q, inp.k, inp.v, scale=wl.softmax_scale, num_partitions=P,
                            keys_per_partition=C, page_table=inp.page_table,
                            valid_length=inp.valid_length, max_seq_len=wl.max_seq_len,
                            k_scale=wl.k_scale, v_scale=wl.v_scale)
    go, gm, gl = (x.double().cpu().numpy() for x in (po, pm, pl))
    empty = rl == 0
    assert empty.sum() >= 3 * (P - 1) * wl.num_heads, "too few empty partitions"
    assert (go[empty] == 0).all() and (gl[empty] == 0).all() and np.isneginf(gm[empty]).all()
    full = ~empty
    oerr = np.abs(go[full] - ro[full]).max()
    merr = np.abs(gm[full] - rm[full]).max()
    lerr = (np.abs(gl[full] - rl[full]) / rl[full]).max()
    say(f"  {kv}: {empty.sum()} empty rows; O err {oerr:.2e}, m err {merr:.2e}, l rel {lerr:.2e}")
    assert oerr < 1e-2 and merr < 1e-3 and lerr < 1e-3


@pytest.mark.parametrize("case", [
    # (P, C, batch, heads, kv heads, depth, S): partitions past a row's keys are empty
    (6, 16, 3, 4, 2, 64, 90),
    (40, 4, 3, 3, 1, 64, 90),     # 33..64 partitions: two waves per row; second half empty
    (64, 2, 3, 4, 2, 128, 90),    # ... the second half partly empty, 128 columns
    (33, 3, 5, 3, 1, 128, 100),   # ... one partition in the second half, odd row count
], ids=lambda c: "P%d_C%d_rows%d_dv%d" % (c[0], c[1], c[2] * c[3], c[5]))
def test_splitk_reduce_on_oracle_partials(case):
    """splitk_reduce fed with partials made by the oracle matches the oracle merge."""
    from oracle import oracle as O
    P, C, B, H, KVH, D, S = case
    wl = W.Workload("reduce_src", 8601 + P, batch=B, num_heads=H, kv_heads=KVH, depth=D,
                    max_seq_len=S, ragged=(0, S, 1), dtype="f32", sink=True)
    inp = W.make_inputs(wl)
    po, pm, pl = O.partials(inp.q, inp.k, inp.v, scale=wl.softmax_scale, num_partitions=P,
                            keys_per_partition=C, valid_length=inp.valid_length)
    ref_out, ref_lse = O.merge(po, pm, pl, num_heads=wl.num_heads, sink=inp.sink)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    out, lse = DA.splitk_reduce(t(po), t(pm), t(pl), num_q_heads=wl.num_heads,
                                sink_weights=t(inp.sink), out_dtype=torch.float32)
    torch.cuda.synchronize()
    err = np.abs(out.cpu().numpy() - ref_out).max()
    fin = np.isfinite(ref_lse)
    lerr = np.abs(lse.cpu().numpy()[fin] - ref_lse[fin]).max()
    say(f"  reduce: out err {err:.2e}, lse err {lerr:.2e}")
    assert err < 2e-5 and lerr < 1e-4


def test_deterministic_and_guard_bands():
    wl = W.GQA.with_(batch=3, max_seq_len=700, ragged=(1, 700, 0))
    inp = W.make_inputs(wl)
    dev = device_inputs(inp)
    n = wl.batch * wl.num_heads * wl.depth
    guard = 4096
    buf = torch.full((n + 2 * guard,), 12345.0, dtype=torch.float32, device="cuda").to(
        torch.bfloat16)
    out = buf[guard:guard + n].view(wl.batch, 1, wl.num_heads, wl.depth)
    lbuf = torch.full((wl.batch * wl.num_heads + 2 * guard,), 777.0, device="cuda")
    lse = lbuf[guard:guard + wl.batch * wl.num_heads].view(wl.batch, 1, wl.num_heads)
    run_gpu(wl, dev, 3, out=out, lse=lse)
    first = out.clone(), lse.clone()
    run_gpu(wl, dev, 3, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(first[0].view(torch.int16), out.view(torch.int16))
    assert torch.equal(first[1], lse)
    g = torch.tensor(12345.0).to(torch.bfloat16).cuda()
    assert bool((buf[:guard] == g).all()) and bool((buf[guard + n:] == g).all())
    assert bool((lbuf[:guard] == 777.0).all()) and bool((lbuf[guard + wl.batch * wl.num_heads:]
                                                          == 777.0).all())


# ---- the bf16 streaming matrix-core path -----------------------------------------

def test_paged_ragged_full():
    check(W.PAGED, num_partitions=0)


MFMA = [
    # (B, T, H, KVH, D, S, page, causal)
    (2, 1, 16, 2, 128, 333, 0, False),     # group 8 (half-filled 16-row tile)
    (2, 1, 32, 2, 128, 500, 0, False),     # group 16 (full tile)
    (2, 1, 64, 2, 64, 257, 0, False),      # group 32 -> two row blocks, depth 64
    (3, 2, 24, 2, 128, 300, 64, True),     # MTP fold: 2 tokens x group 12 = 24 rows
    (2, 3, 8, 1, 64, 100, 32, True),       # 3 tokens x group 8, one KV head
]


@pytest.mark.parametrize("shape", MFMA, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("P", [1, 3])
def test_mfma_shapes(shape, P):
    B, T, H, KVH, D, S, page, causal = shape
    wl = W.Workload(f"mfma_{'x'.join(map(str, shape))}", 8700 + S + T, batch=B, num_heads=H,
                    kv_heads=KVH, depth=D, max_seq_len=S, q_len=T, causal=causal,
                    page_size=page, ragged=(1, S, 1), sink=(P == 3))
    check(wl, num_partitions=P)


STREAM = [
    # (B, T, H, KVH, D, S, page, causal, ragged)
    (3, 1, 8, 8, 128, 1000, 32, False, True),   # MHA (one row per KV head), 32-key pages
    (2, 1, 8, 2, 128, 20, 0, False, False),     # two 16-key tiles: waves 2 and 3 idle
    (2, 1, 8, 2, 64, 5, 0, False, False),       # one partial tile, depth 64
    (2, 1, 32, 16, 128, 777, 0, False, True),   # 16 KV heads: 4 KB between a head's keys
    (2, 4, 16, 4, 128, 260, 64, True, True),    # 4 tokens x group 4 = one full 16-row block
    (1, 1, 40, 2, 64, 2100, 128, False, False),  # group 20: 16 + 4 rows, depth 64 (8 stages)
]


@pytest.mark.parametrize("shape", STREAM, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("P", [1, 7])
def test_stream_shapes(shape, P):
    """Tile counts that do not divide among the 4 waves, partitions of C keys with
    C not a multiple of 64, idle waves, and wide head strides."""
    B, T, H, KVH, D, S, page, causal, ragged = shape
    wl = W.Workload(f"stream_{'x'.join(map(str, shape))}", 8800 + S + T + H, batch=B,
                    num_heads=H, kv_heads=KVH, depth=D, max_seq_len=S, q_len=T, causal=causal,
                    page_size=page, ragged=(1, S, 1) if ragged else None, sink=(P == 7))
    check(wl, num_partitions=P)


def test_prepared_call_matches_direct():
    """The binding's prepared (marshal-once) call enqueues the very same C call."""
    wl = W.Workload("prepared", 8901, batch=3, num_heads=16, kv_heads=4, depth=128,
                    max_seq_len=700, page_size=64, ragged=(1, 700, 1), sink=True)
    inp = W.make_inputs(wl)
    dev = device_inputs(inp)
    ref_out, ref_lse = run_gpu(wl, dev, 3)
    out = torch.empty_like(ref_out)
    lse = torch.empty_like(ref_lse)
    call = run_gpu(wl, dev, 3, out=out, lse=lse, prepare=True)
    for _ in range(2):
        out.zero_()
        got_out, got_lse = call()
        torch.cuda.synchronize()
        assert got_out is out and got_lse is lse
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        assert torch.equal(lse, ref_lse)


def test_workspace_reuse_across_partition_counts():
    """Consecutive decode_attention() calls that share one zero-filled workspace,
    sized for the largest P, with different inputs and partition counts are each
    correct, and each leaves the work-queue word of the ragged calls at zero."""
    from gpu_util import compare, run_oracle
    wl = W.Workload("ws_reuse", 8951, batch=3, num_heads=16, kv_heads=4, depth=128,
                    max_seq_len=900, page_size=64, ragged=(1, 900, 1), sink=True)
    B, H = wl.batch, wl.num_heads
    ws = torch.zeros(DA.decode_workspace_size(7, B, 1, H, wl.depth), dtype=torch.uint8,
                     device="cuda")
    for variant, P in ((0, 7), (1, 3), (2, 7), (3, 1), (4, 5)):
        inp = W.make_inputs(wl, variant=variant)
        dev = device_inputs(inp)
        out, lse = run_gpu(wl, dev, P, workspace=ws)
        ref_out, ref_lse = run_oracle(wl, inp)
        compare(wl, out, lse, ref_out, ref_lse, what=f"workspace reuse P={P}")
        assert int(ws[:8].view(torch.int64).item()) == 0, "work-queue word not back at zero"


def test_work_queue_many_items_per_block():
    """A ragged batch with far more (partition, sequence, KV head) items than
    resident blocks: every block runs many items from the queue, short and
    empty ones among them, and the result matches the oracle at every P."""
    from gpu_util import check
    wl = W.Workload("queue_many", 8960, batch=48, num_heads=32, kv_heads=8, depth=128,
                    max_seq_len=3000, page_size=32, ragged=(1, 3000, 5), sink=True)
    for P in (8, 23, 64):
        check(wl, num_partitions=P)
