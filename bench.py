#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

A step is one full decode-attention pass (every kernel of the call: the
partition pass and, when the keys are split, the log-sum-exp merge) over one
batch of synthetic inputs already resident in HBM.  The default workload is the
largest configured problem: ragged paged decode (batch 64, 64 query / 8 KV heads,
depth 128, bf16, lengths uniform in [1, 32768] with four set to 1, 128-key pages
placed by a seeded permutation of one pool; 3.69 GB of KV per step).  Prints one
JSON line.

  value      = algorithmic KV bytes per step / time per step  (GB/s)
  roofline   = the partition-pass kernel alone: the same bytes / its average
               HIP-event duration, against the 8 TB/s HBM peak
  cpu_baseline = the fp64 CPU oracle on this host, on a bounded sample
  step_us    = the distribution of single steps (median, p10, p90), each timed
               between its own pair of HIP events in a separate pass

Input sets are rotated so that consecutive steps never find their KV cache in
the 256 MB last-level cache.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "decode-attention μs/step + achieved KV-read HBM GB/s (% of peak), 1 MI355X"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak
ROTATE_BYTES = 2 << 30  # >= 8x the last-level cache

WORKLOADS = {"tiny": W.TINY_MHA, "gqa": W.GQA, "paged": W.PAGED, "mla": W.MLA,
             "mla_mtp": W.MLA_MTP, "long": W.LONG, "gqa_fp8": W.GQA_FP8,
             "paged_fp8": W.PAGED_FP8, "gqa_ragged_q": W.GQA_RAGGED_Q,
             "mla_sparse": W.MLA_SPARSE, "mla_fp8": W.MLA_FP8}

CSRC = os.path.join(ROOT, "decode_attention_07_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 1 << 30  # bytes read (and written) by one calibration copy


def kernel_sources(wl: W.Workload):
    """Source files of the partition-pass kernel a workload runs."""
    if wl.mla and not wl.topk:
        main = ["mla_wave8.hip"]
    elif wl.mla:
        main = ["mla_mfma.hip"]
    elif wl.kv_type == "e4m3":
        main = ["decode_stream_fp8.hip", "da_stream.h"]
    elif wl.dtype == "bf16":
        main = ["decode_stream.hip", "da_stream.h"]
    else:
        main = ["decode_valu.hip", "da_merge.h"]
    return [os.path.join(CSRC, f) for f in (*main, "da_device.h", "da_params.h")]


def kernel_hash(wl: W.Workload) -> str:
    h = hashlib.sha256()
    for f in kernel_sources(wl):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:12]


def recorded_traffic(workload: str, P: int, khash: str):
    """HBM bytes per launch of the partition-pass kernel, as measured by the
    FETCH_SIZE / WRITE_SIZE counter runs recorded in the profiles/ summaries
    (table rows: workload | partitions | kernel | kernel source | FETCH_SIZE |
    WRITE_SIZE | KiB per unit x2 | HBM bytes) for this workload, partition count
    and kernel source; None when no row matches (for instance after the kernel
    changed)."""
    if not os.path.isdir(PROFILES):
        return None
    for name in sorted(os.listdir(PROFILES)):
        if not name.endswith(".md"):
            continue
        with open(os.path.join(PROFILES, name)) as fh:
            for line in fh:
                cols = [c.strip() for c in line.strip().strip("|").split("|")]
                if (len(cols) >= 9 and cols[0] == workload and cols[1] == str(P)
                        and cols[3] == khash and cols[8].isdigit()):
                    return int(cols[8])
    return None


def calibrate_copy():
    """A plain copy kernel of known size for the FETCH_SIZE / WRITE_SIZE scale:
    each launch reads COPY_BYTES and writes COPY_BYTES (fp32 negation)."""
    import torch
    n = COPY_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "fp32 negation", "bytes_read_per_launch": COPY_BYTES,
                      "bytes_written_per_launch": COPY_BYTES, "launches": 5}), flush=True)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def read_ceiling():
    """Context for the roofline: a plain streaming-read kernel's rate on this
    device (torch's int32 row maximum over 4 GiB: reads 4 GiB, writes 4 MiB)."""
    import torch
    n = 1 << 30  # int32 elements = 4 GiB
    x = torch.ones(n, dtype=torch.int32, device="cuda").view(-1, 1024)
    for _ in range(3):
        x.amax(dim=1)
    torch.cuda.synchronize()
    times = []
    for _ in range(10):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        x.amax(dim=1)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = statistics.median(times)
    print(json.dumps({"read_ceiling": "torch int32 row max over 4 GiB", "bytes_read": 4 * n,
                      "ms": round(ms, 4), "GB/s": round(4 * n / ms / 1e6, 1),
                      "frac_of_8TB/s": round(4 * n / ms / 1e6 / HBM_PEAK_GBS, 4)}), flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="paged")
    ap.add_argument("--partitions", type=int, default=0, help="0 = library heuristic")
    ap.add_argument("--rotate", type=int, default=0, help="input sets (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="rough budget of the CPU-oracle sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run the copy kernel that scales the memory counters")
    ap.add_argument("--ceiling", action="store_true",
                    help="only measure a plain streaming-read kernel (context for the roofline)")
    return ap.parse_args()


def algorithmic_flops(inp: W.Inputs, tokens=None) -> int:
    """2 (D + Dv) flops per (query row, visible key): the two products of attention.
    tokens: per-sequence token counts of a ragged q (else q_len each)."""
    wl = inp.wl
    lens = inp.lengths()
    keys = 0
    for b in range(wl.batch):
        n = int(lens[b])
        t_b = wl.q_len if tokens is None else int(tokens[b])
        if wl.causal:
            keys += sum(max(0, min(n, n - t_b + t + 1)) for t in range(t_b))
        else:
            keys += t_b * n
    return 2 * keys * wl.num_heads * (wl.depth + wl.dv)


def sample_inputs(inp: W.Inputs, nb: int) -> W.Inputs:
    """The first nb sequences of an instance (same cache pool when paged or sparse)."""
    wl = inp.wl.with_(batch=nb)
    if inp.indices is not None:
        return W.Inputs(wl, inp.q[:nb], inp.k, None, None, None, inp.sink,
                        indices=inp.indices[:nb], topk_lengths=inp.topk_lengths[:nb])
    k = inp.k if inp.page_table is not None else inp.k[:nb]
    v = None if inp.v is None else (inp.v if inp.page_table is not None else inp.v[:nb])
    return W.Inputs(wl, inp.q[:nb], k, v,
                    None if inp.valid_length is None else inp.valid_length[:nb],
                    None if inp.page_table is None else inp.page_table[:nb], inp.sink)


def cpu_baseline(inp: W.Inputs, budget_s: float):
    """Time the oracle as it stands on a bounded sample of the workload."""
    from oracle import oracle as O
    wl = inp.wl
    threads = O.num_threads()
    tokens = W.ragged_q_tokens(wl)

    def oracle_call(smp):
        if smp.indices is not None:
            return O.attention(smp.q, smp.k, None, scale=wl.softmax_scale, sink=smp.sink,
                               depth_v=wl.dv, indices=smp.indices,
                               topk_lengths=smp.topk_lengths)
        kw = dict(scale=wl.softmax_scale, page_table=smp.page_table,
                  valid_length=smp.valid_length, sink=smp.sink, causal=wl.causal,
                  depth_v=wl.dv, max_seq_len=wl.max_seq_len, k_scale=wl.k_scale,
                  v_scale=wl.v_scale)
        if tokens is None:
            return O.attention(smp.q, smp.k, smp.v, **kw)
        q, qo = W.pack_ragged_q(smp, tokens[:smp.wl.batch])
        return O.attention(q, smp.k, smp.v, q_offsets=qo, **kw)

    # Size the sample from one short probe run on one sequence.
    probe = sample_inputs(inp, 1)
    t0 = time.perf_counter()
    oracle_call(probe)
    per_seq = max(time.perf_counter() - t0, 1e-4)
    nb = int(max(1, min(wl.batch, budget_s / 3 / per_seq)))
    smp = sample_inputs(inp, nb)
    times = []
    t_start = time.perf_counter()
    while len(times) < 3 or (len(times) < 5 and time.perf_counter() - t_start < budget_s / 2):
        t0 = time.perf_counter()
        oracle_call(smp)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    gbs = smp.kv_bytes() / t / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"first {nb} of {wl.batch} sequences (all heads, all keys), median of "
                      f"{len(times)} runs of {t * 1e3:.1f} ms; full-step equivalent "
                      f"{t * inp.kv_bytes() / smp.kv_bytes() * 1e6:.0f} us",
            "us_per_step_equiv": round(t * inp.kv_bytes() / smp.kv_bytes() * 1e6, 1)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.ceiling:
        read_ceiling()
        return
    import torch
    from decode_attention_07_amd import binding as DA

    wl = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    log(f"workload {wl.name}")
    first = W.make_inputs(wl)
    footprint = first.kv_bytes()
    R = args.rotate or max(1, min(4, math.ceil(ROTATE_BYTES / max(footprint, 1))))
    if wl.ragged is not None:
        R = 1  # ragged draws differ per set; keep the one instance whose bytes we report
    host_sets = [first] + [W.make_inputs(wl, variant=r) for r in range(1, R)]
    log(f"{R} input set(s) of {footprint / 2**20:.1f} MiB KV each")
    dev_sets = []
    for inp in host_sets:
        dev_sets.append(dict(q=DA.to_device(inp.q), k=DA.to_device(inp.k),
                             v=DA.to_device(inp.v), table=DA.to_device(inp.page_table),
                             valid=DA.to_device(inp.valid_length), sink=DA.to_device(inp.sink),
                             indices=DA.to_device(inp.indices),
                             topk=DA.to_device(inp.topk_lengths)))
    ragged_q = W.ragged_q_tokens(wl)
    if ragged_q is not None:  # q rows packed per sequence (its first tokens[b] tokens)
        for inp, d in zip(host_sets, dev_sets):
            q, qo = W.pack_ragged_q(inp, ragged_q)
            d["q"], d["q_offsets"] = DA.to_device(q), DA.to_device(qo)
        log(f"ragged q: {int(ragged_q.sum())} tokens, {int(ragged_q.min())}..{int(ragged_q.max())} "
            f"per sequence")
    kv_bytes = footprint
    S = wl.max_seq_len
    B, T, H = wl.batch, wl.q_len, wl.num_heads
    if wl.topk:
        P = args.partitions or DA.mla_sparse_num_partitions(B, T, H, wl.topk)
    else:
        P = args.partitions or DA.num_partitions(B, T, H, wl.kv_heads, wl.depth, wl.dv, S,
                                                 ragged=first.valid_length is not None)
    split = P > 1 and ragged_q is None  # a ragged-q call is timed as one full call
    ws = torch.zeros(DA.decode_workspace_size(P, B, T, H, wl.dv), dtype=torch.uint8,
                     device="cuda")  # zero-filled once: the work-queue word starts at 0
    out = torch.empty((B, T, H, wl.dv), dtype=dev_sets[0]["q"].dtype, device="cuda")
    lse = torch.empty((B, T, H), dtype=torch.float32, device="cuda")
    if ragged_q is not None:
        n_tok = int(ragged_q.sum())
        out = torch.empty((n_tok, H, wl.dv), dtype=dev_sets[0]["q"].dtype, device="cuda")
        lse = torch.empty((n_tok, H), dtype=torch.float32, device="cuda")

    # Each launch is marshalled once (binding BoundCall): a timed step costs the host
    # one ctypes call per kernel, far less than the kernel itself, so the device
    # never waits for the host.
    def partition_call(d):
        if wl.topk:
            return DA.mla_decode_sparse_partials(d["q"], d["k"], d["indices"], d["topk"],
                                                 scale=wl.softmax_scale, num_partitions=P,
                                                 workspace=ws, prepare=True)
        if wl.mla and wl.kv_type == "e4m3":
            return DA.mla_decode_fp8kv_partials(d["q"], d["k"], k_scale=wl.k_scale,
                                                scale=wl.softmax_scale, num_partitions=P,
                                                page_table=d["table"], valid_length=d["valid"],
                                                max_seq_len=S, causal=wl.causal, workspace=ws,
                                                prepare=True)
        if wl.mla:
            return DA.mla_decode_partials(d["q"], d["k"], scale=wl.softmax_scale,
                                          num_partitions=P, page_table=d["table"],
                                          valid_length=d["valid"], max_seq_len=S,
                                          causal=wl.causal, workspace=ws, prepare=True)
        kw = dict(group=wl.group, scale=wl.softmax_scale, num_partitions=P,
                  page_table=d["table"], valid_length=d["valid"], max_seq_len=S,
                  causal=wl.causal, workspace=ws, prepare=True)
        if wl.kv_type == "e4m3":
            return DA.decode_attention_fp8kv_partials(d["q"], d["k"], d["v"], k_scale=wl.k_scale,
                                                      v_scale=wl.v_scale, **kw)
        return DA.decode_attention_partials(d["q"], d["k"], d["v"], **kw)

    def full_call(d):
        if wl.topk:
            return DA.mla_decode_sparse(d["q"], d["k"], d["indices"], d["topk"],
                                        scale=wl.softmax_scale, num_partitions=P,
                                        sink_weights=d["sink"], out=out, lse=lse, workspace=ws,
                                        prepare=True)
        kw = dict(scale=wl.softmax_scale, page_table=d["table"], valid_length=d["valid"],
                  max_seq_len=S, num_partitions=P, sink_weights=d["sink"], causal=wl.causal,
                  out=out, lse=lse, workspace=ws, prepare=True)
        if ragged_q is not None:
            return DA.decode_attention_ragged(d["q"], d["q_offsets"], d["k"], d["v"],
                                              max_q_len=T, group=wl.group, **kw)
        if wl.mla and wl.kv_type == "e4m3":
            return DA.mla_decode_fp8kv(d["q"], d["k"], k_scale=wl.k_scale, **kw)
        if wl.mla:
            return DA.mla_decode(d["q"], d["k"], **kw)
        if wl.kv_type == "e4m3":
            return DA.decode_attention_fp8kv(d["q"], d["k"], d["v"], k_scale=wl.k_scale,
                                             v_scale=wl.v_scale, group=wl.group, **kw)
        return DA.decode_attention(d["q"], d["k"], d["v"], group=wl.group, **kw)

    # A step is the call a user makes (one C call: the partition pass and, when split,
    # the merge).  The dominant kernel is timed on its own through the partials-only
    # entry point; for the MLA kernels that call writes fp32 partial rows where the
    # full call writes bf16 ones for partitions 1 .. P-1 over long partitions, so its
    # time is, if anything, the longer.
    steps = [full_call(d) for d in dev_sets]
    kernels = [partition_call(d) if split else steps[j] for j, d in enumerate(dev_sets)]

    def step(i):
        steps[i % R]()

    log(f"P={P} split={split}; warmup {args.warmup}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: exactly K steps, synchronised on both sides, no per-step
    # events (an event pair between launches costs several microseconds of idle
    # device time per step).
    K = args.steps
    log(f"timing {K} steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for i in range(K):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    ev_ms_per_step = ev0.elapsed_time(ev1) / K

    # The dominant kernel (the partition pass, or the single decode kernel when
    # the keys are not split) alone: K back-to-back launches between two HIP
    # events on the stream it is launched on; the average includes the few
    # hundred nanoseconds between consecutive launches.
    for i in range(min(R, K)):
        kernels[i % R]()
    torch.cuda.synchronize()
    ev0.record()
    for i in range(K):
        kernels[i % R]()
    ev1.record()
    torch.cuda.synchronize()
    kern_avg_ms = ev0.elapsed_time(ev1) / K

    # The step distribution: a separate pass of K steps, each between its own pair of
    # events (the pairs add idle time between steps, which is why the headline above
    # times the steps back to back).
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(K)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(pairs):
        a.record()
        step(i)
        b.record()
    torch.cuda.synchronize()
    step_us = sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)

    def pct(q):
        return round(step_us[min(len(step_us) - 1, int(q * (len(step_us) - 1) + 0.5))], 2)

    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    # The roofline of the dominant kernel is the tighter of its two bounds: the KV
    # bytes at the HBM peak, or (bf16 matrix-core kernels) its flops at the MFMA peak.
    flops = algorithmic_flops(first, ragged_q)
    mfma_bound = (wl.dtype == "bf16" and flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
                  > kv_bytes / (HBM_PEAK_GBS * 1e9))
    if mfma_bound:
        achieved = flops / (kern_avg_ms * 1e-3) / 1e12
        peak, unit = MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        achieved = kv_bytes / (kern_avg_ms * 1e-3) / 1e9
        peak, unit = HBM_PEAK_GBS, "GB/s"
    log(f"{ms_per_step * 1e3:.1f} us/step ({ev_ms_per_step * 1e3:.1f} on events), "
        f"kernel {kern_avg_ms * 1e3:.1f} us")

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "us_per_step_device": round(ev_ms_per_step * 1e3, 2),
        "step_us": {"p10": pct(0.10), "median": pct(0.50), "p90": pct(0.90),
                    "min": round(step_us[0], 2), "max": round(step_us[-1], 2),
                    "method": f"{K} steps, each between its own pair of HIP events"},
        "hbm_peak_frac": round(value / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16 (e4m3 KV)" if wl.kv_type == "e4m3" else "bf16") if wl.dtype == "bf16"
                 else "f32",
        "data": "synthetic: seeded N(0,1) q/k/v with the workload's shapes "
                "(and its seeded lengths, page placement and sinks)",
        "config": {"workload": wl.name, "batch": B, "q_len": T, "num_q_heads": H,
                   "num_kv_heads": wl.kv_heads, "depth": wl.depth, "depth_v": wl.dv,
                   "max_seq_len": S, "page_size": wl.page_size, "partitions": P,
                   **({"topk": wl.topk} if wl.topk else {}),
                   "kv_bytes_per_step": kv_bytes, "input_sets": R},
        "roofline": {"bound": "mfma" if mfma_bound else "hbm", "achieved": round(achieved, 2),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": recorded_traffic(args.workload, P, kernel_hash(wl)),
                     "kernel": "partition pass" if split else "decode (single partition)",
                     "kernel_source": kernel_hash(wl),
                     "kernel_avg_us": round(kern_avg_ms * 1e3, 2),
                     "algorithmic_bytes": kv_bytes, "algorithmic_flops": flops,
                     "kernel_hbm_frac": round(kv_bytes / (kern_avg_ms * 1e-3) / 1e9
                                              / HBM_PEAK_GBS, 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(first, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
