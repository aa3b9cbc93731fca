"""GPU parity over seeded random shapes: every decode kernel family (GQA in bf16,
fp32 and over an 8-bit cache; MLA over bf16 and 8-bit caches; sparse top-k MLA)
through the C ABI against the fp64 oracle, on problems drawn from the ranges the
entry points accept (batch, heads and grouping, depth, lengths, pages, causal
multi-token q, sinks, partition count, element type), so that combinations the
hand-picked cases do not name are compared too.  Each case prints its draw before
the GPU call."""
import numpy as np
import pytest

import workloads as W
from gpu_util import check
from test_gpu_ragged_kv import run_ragged_kv
from test_gpu_ragged_q import _run as run_ragged_q

pytestmark = pytest.mark.gpu


def _gqa_case(i):
    rng = np.random.default_rng(20_000 + i)
    kv = ["bf16", "f32", "e4m3"][i % 3]
    kvh = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    while kvh * group > 64:
        group //= 2
    T = int(rng.choice([1, 1, 2, 3, 4]))
    S = int(rng.integers(1, 3001))
    page = int(rng.choice([0, 0, 32, 64, 128]))
    low = int(rng.choice([0, 1, S // 2]))
    kw = dict(batch=int(rng.integers(1, 7)), num_heads=kvh * group, kv_heads=kvh,
              depth=128 if kv == "e4m3" else int(rng.choice([64, 128])), max_seq_len=S,
              q_len=T, causal=bool(T > 1 and rng.random() < 0.7), page_size=page,
              ragged=(low, S, int(rng.integers(0, 2))) if rng.random() < 0.7 else None,
              sink=bool(rng.random() < 0.5))
    if kv == "e4m3":
        kw.update(kv_dtype="e4m3", k_scale=0.125, v_scale=0.125)
    else:
        kw.update(dtype=kv)
    P = int(rng.choice([0, 1, 2, 3, 5, 8, 13]))
    return W.Workload(f"rand_gqa_{i}", 21_000 + i, **kw), P


def _mla_case(i):
    rng = np.random.default_rng(30_000 + i)
    fp8 = i % 2 == 1
    T = int(rng.choice([1, 1, 2, 3]))
    H = int(rng.choice([16, 64, 128, 160]))
    while T * H > 256:
        T -= 1
    S = int(rng.integers(1, 1601))
    page = int(rng.choice([0, 0, 32, 64]))
    kw = dict(batch=int(rng.integers(1, 4)), num_heads=H, kv_heads=1, depth=576, depth_v=512,
              max_seq_len=S, q_len=T, mla=True, causal=bool(T > 1), page_size=page,
              ragged=(int(rng.choice([0, 1])), S, int(rng.integers(0, 2)))
              if rng.random() < 0.7 else None,
              sink=bool(rng.random() < 0.5), scale=1.0 / np.sqrt(192.0))
    if fp8:
        kw.update(kv_dtype="e4m3", k_scale=0.125, v_scale=0.125)
    P = int(rng.choice([0, 1, 2, 3, 4, 6]))
    return W.Workload(f"rand_mla_{i}", 31_000 + i, **kw), P


def _sparse_case(i):
    rng = np.random.default_rng(40_000 + i)
    T = int(rng.choice([1, 1, 2]))
    H = int(rng.choice([16, 64, 128]))
    S = int(rng.integers(2, 3001))
    kw = dict(batch=int(rng.integers(1, 4)), num_heads=H, kv_heads=1, depth=576, depth_v=512,
              max_seq_len=S, q_len=T, mla=True, topk=int(rng.integers(1, min(S, 1400) + 1)),
              ragged=(1, S, int(rng.integers(0, 2))) if rng.random() < 0.6 else None,
              sink=bool(rng.random() < 0.5), scale=1.0 / np.sqrt(192.0))
    P = int(rng.choice([0, 1, 2, 3, 5]))
    return W.Workload(f"rand_sparse_{i}", 41_000 + i, **kw), P


def _describe(wl, P):
    return (f"{wl.name}: {wl.kv_type} B={wl.batch} T={wl.q_len} H={wl.num_heads} "
            f"KVH={wl.kv_heads} D={wl.depth} S={wl.max_seq_len} page={wl.page_size} "
            f"ragged={wl.ragged} causal={wl.causal} sink={wl.sink} topk={wl.topk} P={P}")


@pytest.mark.parametrize("i", range(64))
def test_random_gqa_shapes(i):
    wl, P = _gqa_case(i)
    check(wl, num_partitions=P, what=_describe(wl, P))


@pytest.mark.parametrize("i", range(24))
def test_random_mla_shapes(i):
    wl, P = _mla_case(i)
    check(wl, num_partitions=P, what=_describe(wl, P))


@pytest.mark.parametrize("i", range(12))
def test_random_sparse_shapes(i):
    wl, P = _sparse_case(i)
    check(wl, num_partitions=P, what=_describe(wl, P))


@pytest.mark.parametrize("i", range(16))
def test_random_ragged_kv(i):
    """The dense draws (bf16 and fp32 GQA, bf16 MLA) in the ragged KV layout."""
    if i % 4 == 3:
        wl, P = _mla_case(2 * i)  # an even draw: the bf16 cache
        wl = wl.with_(page_size=0)
    else:
        wl, P = _gqa_case(300 + 3 * i + (i % 2))  # bf16 and fp32 draws (index mod 3)
        wl = wl.with_(page_size=0)
    run_ragged_kv(wl, P, _describe(wl, P))


@pytest.mark.parametrize("i", range(16))
def test_random_ragged_q(i):
    """Multi-token draws with per-sequence token counts (0 .. T) from offsets."""
    rng = np.random.default_rng(50_000 + i)
    if i % 4 == 3:
        wl, P = _mla_case(2 * i)
        wl = wl.with_(q_len=2, causal=True)
    else:
        wl, P = _gqa_case(600 + 3 * i + (i % 2))  # bf16 and fp32 draws (index mod 3)
        wl = wl.with_(q_len=int(rng.integers(2, 5)), causal=bool(rng.random() < 0.7))
    tokens = [int(t) for t in rng.integers(0, wl.q_len + 1, size=wl.batch)]
    run_ragged_q(wl, tokens, P, _describe(wl, P) + f" tokens={tokens}")
