"""The library's calls are capturable (they allocate nothing, never synchronise and
never read device memory on the host): one HIP graph holding a ragged paged GQA call
on the work queue, a causal MTP MLA call and a sparse MLA call, replayed several
times with new inputs written between the replays, matches eager calls bit for bit,
and leaves the work-queue word at zero."""
import numpy as np
import pytest
import torch

import workloads as W
from decode_attention_07_amd import binding as DA
from gpu_util import device_inputs, say

pytestmark = pytest.mark.gpu

SCALE_MLA = 1.0 / np.sqrt(192.0)


def _setup():
    wl_g = W.Workload("graph_gqa", 9850, batch=6, num_heads=32, kv_heads=8, depth=128,
                      max_seq_len=2000, page_size=64, ragged=(1, 2000, 1), sink=True)
    wl_m = W.Workload("graph_mla", 9851, batch=3, num_heads=128, kv_heads=1, depth=576,
                      depth_v=512, max_seq_len=900, q_len=2, mla=True, causal=True,
                      ragged=(1, 900, 1), scale=SCALE_MLA, sink=True)
    wl_s = W.Workload("graph_sparse", 9852, batch=4, num_heads=128, kv_heads=1, depth=576,
                      depth_v=512, max_seq_len=500, mla=True, topk=200, scale=SCALE_MLA)
    dg, dm, ds = (device_inputs(W.make_inputs(w)) for w in (wl_g, wl_m, wl_s))
    Pg, Pm, Ps = 5, 3, 2

    def alloc(wl, P):
        out = torch.empty((wl.batch, wl.q_len, wl.num_heads, wl.dv), dtype=torch.bfloat16,
                          device="cuda")
        lse = torch.empty((wl.batch, wl.q_len, wl.num_heads), dtype=torch.float32,
                          device="cuda")
        ws = torch.zeros(DA.decode_workspace_size(P, wl.batch, wl.q_len, wl.num_heads, wl.dv),
                         dtype=torch.uint8, device="cuda")  # queue word starts at zero
        return out, lse, ws

    bufs = [alloc(wl_g, Pg), alloc(wl_m, Pm), alloc(wl_s, Ps)]

    def run_all():
        (og, lg, wg), (om, lm, wm), (os_, ls, ws) = bufs
        DA.decode_attention(dg["q"], dg["k"], dg["v"], group=wl_g.group,
                            scale=wl_g.softmax_scale, page_table=dg["page_table"],
                            valid_length=dg["valid_length"], max_seq_len=wl_g.max_seq_len,
                            num_partitions=Pg, sink_weights=dg["sink"], out=og, lse=lg,
                            workspace=wg)
        DA.mla_decode(dm["q"], dm["k"], scale=SCALE_MLA, valid_length=dm["valid_length"],
                      num_partitions=Pm, sink_weights=dm["sink"], causal=True, out=om, lse=lm,
                      workspace=wm)
        DA.mla_decode_sparse(ds["q"], ds["k"], ds["indices"], ds["topk_lengths"],
                             scale=SCALE_MLA, num_partitions=Ps, out=os_, lse=ls, workspace=ws)

    return (dg, dm, ds), bufs, run_all


def _snapshot(bufs):
    return [(o.clone(), l.clone()) for o, l, _ in bufs]


def _queue_words(bufs):
    return [int(ws[:8].view(torch.int64).item()) for _, _, ws in bufs]


def test_graph_replays_match_eager_calls():
    devs, bufs, run_all = _setup()
    # warm-up on a side stream (the pattern torch's capture expects)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_all()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_all()
    torch.cuda.synchronize()

    gen = torch.Generator(device="cuda").manual_seed(5)
    for rep in range(4):
        if rep:  # eager work between the replays: new queries in the captured buffers
            for d in devs:
                d["q"].copy_(torch.randn(d["q"].shape, device="cuda", generator=gen)
                             .to(d["q"].dtype))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(bufs)
        assert _queue_words(bufs) == [0, 0, 0], "work-queue word not back at zero"
        run_all()  # the same calls, eager
        torch.cuda.synchronize()
        ref = _snapshot(bufs)
        for (go, gl), (ro, rl), name in zip(got, ref, ("gqa queue", "mla mtp", "sparse mla")):
            assert torch.equal(go.view(torch.int16), ro.view(torch.int16)), f"{name} rep {rep}"
            assert torch.equal(gl, rl), f"{name} lse rep {rep}"
        say(f"  graph replay {rep}: three calls equal to eager")
