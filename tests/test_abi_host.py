"""The C ABI on the host: exports, status codes, heuristic and workspace layout,
and argument checks that return before anything reaches the GPU (CPU only)."""
import ctypes
import os
import re

import pytest

from decode_attention_07_amd import binding as DA

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "decode_attention.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[a-z_][\w \*]*?\b([a-z_]\w*)\s*\(", text, flags=re.M)))


def test_every_declared_function_is_exported():
    names = header_functions()
    assert len(names) == 23, names
    lib = ctypes.CDLL(DA.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"
    assert sorted(DA.EXPORTS) == names


def test_only_declared_functions_are_exported():
    """The library is built with hidden visibility: its exported functions are exactly
    the header's declarations (no internal C++ symbol leaks into the ABI)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", DA.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(line.split()[-1] for line in out.splitlines()
                      if len(line.split()) == 3 and line.split()[1] == "T")
    assert exported == header_functions()


def test_status_strings():
    for code in (0, -1, -2, -3, -4):
        assert DA.status_string(code) not in ("", "unknown status")
    assert DA.status_string(-99) == "unknown status"


@pytest.mark.parametrize("B,T,H,KVH,D,Dv,S", [
    (32, 1, 32, 8, 128, 128, 4096), (64, 1, 64, 8, 128, 128, 32768), (1, 1, 32, 8, 128, 128, 131072),
    (1, 1, 8, 8, 64, 64, 256), (64, 1, 128, 1, 576, 512, 8192), (64, 2, 128, 1, 576, 512, 8192),
    (1, 1, 1, 1, 64, 64, 0), (7, 3, 12, 4, 64, 64, 17), (512, 1, 64, 8, 128, 128, 128)])
def test_heuristic_bounds_and_determinism(B, T, H, KVH, D, Dv, S):
    for cus in (1, 80, 256, 304):
        for ragged in (False, True):
            p = DA.num_partitions(B, T, H, KVH, D, Dv, S, ragged=ragged, num_cus=cus)
            assert 1 <= p <= DA.DA_MAX_PARTITIONS
            assert p == DA.num_partitions(B, T, H, KVH, D, Dv, S, ragged=ragged, num_cus=cus)
            if ragged:  # a ragged batch never gets fewer partitions than a dense one
                assert p >= DA.num_partitions(B, T, H, KVH, D, Dv, S, num_cus=cus)


def test_heuristic_fills_the_device():
    # 256 (batch, KV head) pairs on 256 compute units: one resident block each
    assert DA.num_partitions(32, 1, 32, 8, 128, 128, 4096, num_cus=256) == 1
    # the same pairs with ragged lengths: smaller partitions, several per unit
    assert DA.num_partitions(32, 1, 32, 8, 128, 128, 4096, ragged=True, num_cus=256) >= 4
    # a single sequence of 131072 keys over 8 KV heads: enough partitions for every unit
    assert DA.num_partitions(1, 1, 32, 8, 128, 128, 131072, num_cus=256) >= 32
    # 64 MLA sequences of 8192 keys: 4 partitions of 2048 keys
    assert DA.num_partitions(64, 1, 128, 1, 576, 512, 8192, num_cus=256) == 4
    # short caches are not split below the minimum partition length
    assert DA.num_partitions(1, 1, 8, 8, 64, 64, 256, num_cus=256) == 1


def test_heuristic_doubles_for_the_two_head_fold():
    # a dense split call at depth 128 whose fold leaves room for two KV heads per
    # block gets twice the partitions (the streaming kernels then fold the heads)
    assert DA.num_partitions(1, 1, 32, 8, 128, 128, 131072, num_cus=256) == 64
    assert DA.num_partitions(2, 2, 16, 4, 128, 128, 65536, num_cus=256) == 64  # fold 2 x 4
    # ... but never past the minimum partition length (10000 keys: at most 40)
    assert DA.num_partitions(1, 1, 32, 8, 128, 128, 10000, num_cus=256) == 40
    # no doubling: depth 64, a fold of 16 rows, an odd KV head count, a ragged
    # batch (work queue), or a call that is not split
    assert DA.num_partitions(1, 1, 32, 8, 64, 64, 131072, num_cus=256) == 32
    assert DA.num_partitions(1, 1, 128, 8, 128, 128, 131072, num_cus=256) == 32
    assert DA.num_partitions(1, 1, 12, 3, 128, 128, 131072, num_cus=256) == 86
    assert DA.num_partitions(1, 1, 32, 8, 128, 128, 131072, ragged=True, num_cus=256) == 512
    assert DA.num_partitions(32, 1, 32, 8, 128, 128, 4096, num_cus=256) == 1


def test_heuristic_rejects_bad_shapes():
    lib = DA.library()
    assert lib.decode_num_partitions(0, 1, 8, 8, 64, 64, 10, 0, 256) == DA.DA_ERR_INVALID_ARG
    assert lib.decode_num_partitions(1, 1, 8, 3, 64, 64, 10, 0, 256) == DA.DA_ERR_INVALID_ARG


def test_workspace_layout():
    lib = DA.library()
    P, B, T, H, Dv = 4, 3, 2, 5, 128
    rows = B * T * H
    o = P * rows * Dv * 4
    oo = lib.decode_workspace_o_offset(P, B, T, H, Dv)
    mo = lib.decode_workspace_max_offset(P, B, T, H, Dv)
    so = lib.decode_workspace_sum_offset(P, B, T, H, Dv)
    size = lib.decode_workspace_size(P, B, T, H, Dv)
    # the 8-byte work-queue word owns the first 256 bytes, whatever P is
    assert oo == 256 and all(lib.decode_workspace_o_offset(q, B, T, H, Dv) == 256
                             for q in (1, 2, 7, 64))
    assert mo >= oo + o and mo % 256 == 0 and mo - oo - o < 256
    assert so >= mo + P * rows * 4 and so % 256 == 0
    assert size >= so + P * rows * 4 and size % 256 == 0
    assert lib.decode_workspace_size(0, B, T, H, Dv) == 0
    assert lib.decode_workspace_size(1, B, T, H, Dv) > 0


def _call_decode(**over):
    args = dict(q=1, k=1, v=1, page_table=None, page_size=0, max_pages=0, valid_length=None,
                batch=1, q_len=1, num_q_heads=8, group=1, depth=64, max_seq_len=256, scale=0.1,
                num_partitions=0, sink=None, mask=0, dtype=0, out=1, lse=None, workspace=None,
                wbytes=0, stream=None)
    args.update(over)
    a = args
    return DA.library().decode_attention(
        a["q"], a["k"], a["v"], a["page_table"], a["page_size"], a["max_pages"],
        a["valid_length"], a["batch"], a["q_len"], a["num_q_heads"], a["group"], a["depth"],
        a["max_seq_len"], a["scale"], a["num_partitions"], a["sink"], a["mask"], a["dtype"],
        a["out"], a["lse"], a["workspace"], a["wbytes"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(q=None), DA.DA_ERR_INVALID_ARG),
    (dict(out=None), DA.DA_ERR_INVALID_ARG),
    (dict(batch=-1), DA.DA_ERR_INVALID_ARG),
    (dict(q_len=0), DA.DA_ERR_INVALID_ARG),
    (dict(group=3), DA.DA_ERR_INVALID_ARG),
    (dict(group=0), DA.DA_ERR_INVALID_ARG),
    (dict(depth=96), DA.DA_ERR_UNSUPPORTED),
    (dict(dtype=7), DA.DA_ERR_UNSUPPORTED),
    (dict(mask=2), DA.DA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), DA.DA_ERR_INVALID_ARG),
    (dict(max_seq_len=-5), DA.DA_ERR_INVALID_ARG),
    (dict(num_partitions=-1), DA.DA_ERR_INVALID_ARG),
    (dict(num_partitions=DA.DA_MAX_PARTITIONS + 1), DA.DA_ERR_INVALID_ARG),
    (dict(page_table=1, page_size=48, max_pages=8), DA.DA_ERR_UNSUPPORTED),
    (dict(page_table=1, page_size=16, max_pages=16), DA.DA_ERR_UNSUPPORTED),
    (dict(page_table=1, page_size=64, max_pages=3), DA.DA_ERR_INVALID_ARG),
    (dict(page_table=1, page_size=0, max_pages=3), DA.DA_ERR_INVALID_ARG),
    (dict(num_partitions=4), DA.DA_ERR_WORKSPACE),
    (dict(num_partitions=4, workspace=1, wbytes=16), DA.DA_ERR_WORKSPACE),
    (dict(batch=0), DA.DA_OK),          # empty batch: a no-op, nothing launched
])
def test_decode_attention_argument_checks(over, code):
    assert _call_decode(**over) == code


def test_mla_and_reduce_argument_checks():
    lib = DA.library()
    # mla_decode(q, kv, table, ps, max_pages, valid, B, T, H, S, scale, P, sink, mask, out, lse,
    #            ws, wbytes, stream)
    assert lib.mla_decode(None, 1, None, 0, 0, None, 1, 1, 128, 64, 0.1, 1, None, 0, 1, None,
                          None, 0, None) == DA.DA_ERR_INVALID_ARG
    assert lib.mla_decode(1, 1, None, 0, 0, None, 1, 1, 128, 64, 0.1, 1, None, 3, 1, None,
                          None, 0, None) == DA.DA_ERR_INVALID_ARG
    assert lib.mla_decode(1, 1, None, 0, 0, None, 0, 1, 128, 64, 0.1, 1, None, 0, 1, None,
                          None, 0, None) == DA.DA_OK
    # splitk_reduce(po, pm, ps, P, rows, H, Dv, sink, out, dtype, lse, stream)
    assert lib.splitk_reduce(1, 1, 1, 2, 4, 2, 96, None, 1, 1, None, None) == \
        DA.DA_ERR_UNSUPPORTED
    assert lib.splitk_reduce(1, 1, 1, 0, 4, 2, 128, None, 1, 1, None, None) == \
        DA.DA_ERR_INVALID_ARG
    assert lib.splitk_reduce(None, 1, 1, 2, 4, 2, 128, None, 1, 1, None, None) == \
        DA.DA_ERR_INVALID_ARG
    assert lib.splitk_reduce(1, 1, 1, 2, 0, 2, 128, None, 1, 1, None, None) == DA.DA_OK


def _call_fp8(**over):
    a = dict(q=1, k=1, v=1, k_scale=1.0, v_scale=1.0, page_table=None, page_size=0, max_pages=0,
             valid_length=None, batch=1, q_len=1, num_q_heads=8, group=1, depth=128,
             max_seq_len=256, scale=0.1, num_partitions=0, sink=None, mask=0, out=1, lse=None,
             workspace=None, wbytes=0, stream=None)
    a.update(over)
    return DA.library().decode_attention_fp8kv(
        a["q"], a["k"], a["v"], a["k_scale"], a["v_scale"], a["page_table"], a["page_size"],
        a["max_pages"], a["valid_length"], a["batch"], a["q_len"], a["num_q_heads"], a["group"],
        a["depth"], a["max_seq_len"], a["scale"], a["num_partitions"], a["sink"], a["mask"],
        a["out"], a["lse"], a["workspace"], a["wbytes"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(k=None), DA.DA_ERR_INVALID_ARG),
    (dict(out=None), DA.DA_ERR_INVALID_ARG),
    (dict(depth=64), DA.DA_ERR_UNSUPPORTED),      # the 8-bit kernel is built for depth 128
    (dict(k_scale=float("inf")), DA.DA_ERR_INVALID_ARG),
    (dict(v_scale=float("nan")), DA.DA_ERR_INVALID_ARG),
    (dict(scale=1e30, k_scale=1e30), DA.DA_ERR_INVALID_ARG),   # scale * k_scale overflows
    (dict(group=3), DA.DA_ERR_INVALID_ARG),
    (dict(num_partitions=4), DA.DA_ERR_WORKSPACE),
    (dict(batch=0), DA.DA_OK),
])
def test_fp8kv_argument_checks(over, code):
    assert _call_fp8(**over) == code


def _call_ragged(**over):
    a = dict(q=1, q_offsets=1, total=3, max_q_len=2, k=1, v=1, page_table=None, page_size=0,
             max_pages=0, valid_length=None, batch=2, num_q_heads=8, group=2, depth=128,
             max_seq_len=256, scale=0.1, num_partitions=0, sink=None, mask=1, dtype=1, out=1,
             lse=None, workspace=None, wbytes=0, stream=None)
    a.update(over)
    return DA.library().decode_attention_ragged(
        a["q"], a["q_offsets"], a["total"], a["max_q_len"], a["k"], a["v"], a["page_table"],
        a["page_size"], a["max_pages"], a["valid_length"], a["batch"], a["num_q_heads"],
        a["group"], a["depth"], a["max_seq_len"], a["scale"], a["num_partitions"], a["sink"],
        a["mask"], a["dtype"], a["out"], a["lse"], a["workspace"], a["wbytes"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(q_offsets=None), DA.DA_ERR_INVALID_ARG),
    (dict(total=-1), DA.DA_ERR_INVALID_ARG),
    (dict(max_q_len=0), DA.DA_ERR_INVALID_ARG),
    (dict(group=3), DA.DA_ERR_INVALID_ARG),
    (dict(depth=96), DA.DA_ERR_UNSUPPORTED),
    # workspace sized for rows = total * H: 3 tokens x 8 heads at P = 4
    (dict(num_partitions=4, workspace=1, wbytes=16), DA.DA_ERR_WORKSPACE),
    (dict(total=0), DA.DA_OK),                     # no tokens: nothing launched
])
def test_ragged_argument_checks(over, code):
    assert _call_ragged(**over) == code


def test_mla_ragged_argument_checks():
    lib = DA.library()
    # mla_decode_ragged(q, q_offsets, total, max_q_len, kv, table, ps, max_pages, valid, B, H,
    #                   S, scale, P, sink, mask, out, lse, ws, wbytes, stream)
    assert lib.mla_decode_ragged(1, None, 4, 2, 1, None, 0, 0, None, 2, 128, 64, 0.1, 1, None,
                                 1, 1, None, None, 0, None) == DA.DA_ERR_INVALID_ARG
    assert lib.mla_decode_ragged(1, 1, 4, 0, 1, None, 0, 0, None, 2, 128, 64, 0.1, 1, None,
                                 1, 1, None, None, 0, None) == DA.DA_ERR_INVALID_ARG
    assert lib.mla_decode_ragged(1, 1, 0, 2, 1, None, 0, 0, None, 2, 128, 64, 0.1, 1, None,
                                 1, 1, None, None, 0, None) == DA.DA_OK


def _call_sparse(**over):
    a = dict(q=1, kv=1, pool_rows=1000, indices=1, stride=64, topk=1, batch=2, q_len=1,
             num_q_heads=128, scale=0.1, num_partitions=1, sink=None, out=1, lse=None,
             workspace=None, wbytes=0, stream=None)
    a.update(over)
    return DA.library().mla_decode_sparse(
        a["q"], a["kv"], a["pool_rows"], a["indices"], a["stride"], a["topk"], a["batch"],
        a["q_len"], a["num_q_heads"], a["scale"], a["num_partitions"], a["sink"], a["out"],
        a["lse"], a["workspace"], a["wbytes"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(indices=None), DA.DA_ERR_INVALID_ARG),
    (dict(indices=None, stride=0, batch=0), DA.DA_OK),   # nothing listed: no list needed
    (dict(topk=None), DA.DA_ERR_INVALID_ARG),
    (dict(kv=None), DA.DA_ERR_INVALID_ARG),
    (dict(out=None), DA.DA_ERR_INVALID_ARG),
    (dict(pool_rows=0), DA.DA_ERR_INVALID_ARG),
    (dict(stride=-1), DA.DA_ERR_INVALID_ARG),
    (dict(q_len=0), DA.DA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), DA.DA_ERR_INVALID_ARG),
    (dict(num_partitions=-1), DA.DA_ERR_INVALID_ARG),
    # rows are addressed by 32-bit byte offsets: at most 2^32 / 1152 of them
    (dict(pool_rows=(1 << 32) // 1152 + 1), DA.DA_ERR_UNSUPPORTED),
    (dict(stride=(1 << 28) + 1), DA.DA_ERR_UNSUPPORTED),
    (dict(num_partitions=3), DA.DA_ERR_WORKSPACE),
    (dict(batch=0), DA.DA_OK),
    (dict(batch=0, num_partitions=0), DA.DA_OK),
])
def test_sparse_argument_checks(over, code):
    assert _call_sparse(**over) == code


def test_sparse_partials_and_heuristic_checks():
    lib = DA.library()
    # mla_decode_sparse_partials(q, kv, R, idx, stride, topk, B, T, H, scale, P, ws, wbytes, s)
    assert lib.mla_decode_sparse_partials(1, 1, 10, 1, 8, 1, 2, 1, 128, 0.1, 0, None, 0,
                                          None) == DA.DA_ERR_INVALID_ARG
    assert lib.mla_decode_sparse_partials(1, 1, 10, 1, 8, 1, 2, 1, 128, 0.1, 2, None, 0,
                                          None) == DA.DA_ERR_WORKSPACE
    assert DA.mla_sparse_num_partitions(64, 1, 128, 2048, num_cus=256) == 4
    assert DA.mla_sparse_num_partitions(64, 2, 128, 2048, num_cus=256) == 2
    assert DA.mla_sparse_num_partitions(1, 1, 128, 2048, num_cus=256) == 4
    assert DA.mla_sparse_num_partitions(8, 1, 128, 100, num_cus=256) == 1
    assert lib.mla_sparse_num_partitions(0, 1, 128, 2048, 256) == DA.DA_ERR_INVALID_ARG


def test_mla_fp8kv_argument_checks():
    lib = DA.library()
    # mla_decode_fp8kv(q, kv, k_scale, table, ps, max_pages, valid, B, T, H, S, scale, P, sink,
    #                  mask, out, lse, ws, wbytes, stream)
    ok = [1, 1, 0.125, None, 0, 0, None, 1, 1, 128, 64, 0.1, 1, None, 0, 1, None, None, 0, None]
    for i, v, code in [(0, None, DA.DA_ERR_INVALID_ARG), (1, None, DA.DA_ERR_INVALID_ARG),
                       (2, float("nan"), DA.DA_ERR_INVALID_ARG),
                       (2, 1e30, DA.DA_ERR_INVALID_ARG),        # scale x k_scale overflows
                       (11, float("inf"), DA.DA_ERR_INVALID_ARG), (14, 5, DA.DA_ERR_INVALID_ARG),
                       (15, None, DA.DA_ERR_INVALID_ARG), (12, 3, DA.DA_ERR_WORKSPACE)]:
        a = list(ok)
        a[i] = v
        if i == 2 and v == 1e30:
            a[11] = 1e10
        assert lib.mla_decode_fp8kv(*a) == code, (i, v)
    a = list(ok)
    a[7] = 0
    assert lib.mla_decode_fp8kv(*a) == DA.DA_OK   # empty batch: nothing launched
    # partials: P must be >= 1 and the workspace given
    assert lib.mla_decode_fp8kv_partials(1, 1, 0.125, None, 0, 0, None, 1, 1, 128, 64, 0.1, 0,
                                         0, None, 0, None) == DA.DA_ERR_INVALID_ARG
    assert lib.mla_decode_fp8kv_partials(1, 1, 0.125, None, 0, 0, None, 1, 1, 128, 64, 0.1, 2,
                                         0, None, 0, None) == DA.DA_ERR_WORKSPACE


def test_ragged_kv_argument_checks():
    lib = DA.library()
    # decode_attention_ragged_kv(q, k, v, offs, valid, B, T, H, group, D, S, scale, P, sink,
    #                            mask, dtype, out, lse, ws, wbytes, stream)
    ok = [1, 1, 1, 1, None, 2, 1, 8, 2, 128, 256, 0.1, 1, None, 0, 1, 1, None, None, 0, None]
    for i, v, code in [(3, None, DA.DA_ERR_INVALID_ARG),    # the offsets are required
                       (0, None, DA.DA_ERR_INVALID_ARG), (16, None, DA.DA_ERR_INVALID_ARG),
                       (8, 3, DA.DA_ERR_INVALID_ARG), (9, 96, DA.DA_ERR_UNSUPPORTED),
                       (10, -1, DA.DA_ERR_INVALID_ARG), (14, 2, DA.DA_ERR_INVALID_ARG),
                       (12, 4, DA.DA_ERR_WORKSPACE)]:
        a = list(ok)
        a[i] = v
        assert lib.decode_attention_ragged_kv(*a) == code, (i, v)
    a = list(ok)
    a[5], a[3] = 0, None
    assert lib.decode_attention_ragged_kv(*a) == DA.DA_OK   # empty batch: nothing launched
    # mla_decode_ragged_kv(q, kv, offs, valid, B, T, H, S, scale, P, sink, mask, out, lse, ws,
    #                      wbytes, stream)
    ok = [1, 1, 1, None, 2, 1, 128, 256, 0.1, 1, None, 0, 1, None, None, 0, None]
    for i, v, code in [(2, None, DA.DA_ERR_INVALID_ARG), (1, None, DA.DA_ERR_INVALID_ARG),
                       (12, None, DA.DA_ERR_INVALID_ARG), (11, 5, DA.DA_ERR_INVALID_ARG),
                       (9, 3, DA.DA_ERR_WORKSPACE)]:
        a = list(ok)
        a[i] = v
        assert lib.mla_decode_ragged_kv(*a) == code, (i, v)


# ---- the Python binding checks its arguments before marshalling (host tensors) -------

def _bf16(*shape):
    import torch
    return torch.zeros(shape, dtype=torch.bfloat16)


def test_binding_rejects_misshaped_outputs_and_per_sequence_arrays():
    import torch
    q, k, v = _bf16(2, 1, 8, 128), _bf16(2, 64, 2, 128), _bf16(2, 64, 2, 128)
    bad = [
        dict(out=_bf16(2, 1, 8, 64)),                                     # out shape
        dict(out=torch.zeros((2, 1, 8, 128), dtype=torch.float32)),       # out dtype
        dict(lse=torch.zeros((2, 1, 7), dtype=torch.float32)),            # lse shape
        dict(lse=torch.zeros((2, 1, 8), dtype=torch.float64)),            # lse dtype
        dict(out=_bf16(2, 1, 128, 8).transpose(2, 3)),                    # not contiguous
        dict(valid_length=torch.zeros(3, dtype=torch.int32)),             # one per sequence
        dict(sink_weights=torch.zeros(4, dtype=torch.float32)),           # one per query head
        dict(page_table=torch.zeros((1, 4), dtype=torch.int32)),          # a row per sequence
    ]
    for kw in bad:
        with pytest.raises((ValueError, TypeError)) as e:
            DA.decode_attention(q, k, v, group=4, scale=0.1, **kw)
        assert "CUDA" not in str(e.value), kw   # rejected by the shape check itself
    with pytest.raises(ValueError):  # v must mirror k
        DA.decode_attention(q, k, _bf16(2, 64, 2, 64), group=4, scale=0.1)
    with pytest.raises(ValueError):
        DA.decode_attention_ragged_kv(q, _bf16(100, 2, 128), _bf16(100, 2, 128),
                                      torch.zeros(3, dtype=torch.int32), group=4, scale=0.1,
                                      max_seq_len=64)


def test_binding_rejects_misshaped_reduce_arguments():
    import torch
    po = torch.zeros((4, 6, 128), dtype=torch.float32)
    pm = torch.zeros((4, 6), dtype=torch.float32)
    for kw in (dict(part_max=torch.zeros((4, 5), dtype=torch.float32)),
               dict(part_sum=torch.zeros((3, 6), dtype=torch.float32)),
               dict(out=_bf16(6, 64)),
               dict(lse=torch.zeros(5, dtype=torch.float32)),
               dict(sink_weights=torch.zeros(3, dtype=torch.float32))):
        a = dict(part_max=pm, part_sum=pm, num_q_heads=2)
        a.update(kw)
        with pytest.raises((ValueError, TypeError)) as e:
            DA.splitk_reduce(po, a.pop("part_max"), a.pop("part_sum"), **a)
        assert "CUDA" not in str(e.value), kw


def test_no_alloc_argument_checks():
    """decode_attention_no_alloc() refuses a workspace larger than its scratch, and bad
    arguments, before anything reaches the GPU."""
    lib = DA.library()
    # decode_attention_no_alloc(q, k, v, table, ps, max_pages, valid, B, T, H, group, D, S,
    #                           scale, P, sink, mask, dtype, out, lse, stream)
    ok = [1, 1, 1, None, 0, 0, None, 8, 1, 64, 8, 128, 4096, 0.1, 1, None, 0, 1, 1, None, None]
    assert DA.decode_workspace_size(1024, 8, 1, 64, 128) > DA.DA_NO_ALLOC_SCRATCH_BYTES
    for i, v, code in [(14, 1024, DA.DA_ERR_WORKSPACE), (0, None, DA.DA_ERR_INVALID_ARG),
                       (18, None, DA.DA_ERR_INVALID_ARG), (10, 3, DA.DA_ERR_INVALID_ARG),
                       (11, 96, DA.DA_ERR_UNSUPPORTED), (14, -1, DA.DA_ERR_INVALID_ARG),
                       (7, 0, DA.DA_OK)]:
        a = list(ok)
        a[i] = v
        assert lib.decode_attention_no_alloc(*a) == code, (i, v)
