#!/usr/bin/env python3
"""Throughput of the chunkwise TTT layer, forward + backward, on one MI355X.

A step is one ttt_chunk_fwd + ttt_chunk_bwd over one batch of the 1.45B-shaped
workload (B=4, H=16, T=4096, d_k=d_v=128, C=256, bf16 I/O, fp32 state; IP loss,
SiLU, per-token vector decay), inputs resident in HBM.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Timing: HIP events recorded on the stream the library launches on (torch's
current stream), W untimed warm-up steps, then K timed steps.  Per-entry-point
times (forward and backward separately) are measured the same way in their own
loop and give the roofline figures.  The CPU baseline times the fp64 oracle on
a bounded sample (a few (b, h) chains) on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TTT-layer fwd+bwd tokens/sec at H=16,d=128,T=4096 on 1 GPU; MFMA util %"

# MI355X published peaks
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3


def algorithmic_work(cfg):
    """Algorithmic flop and HBM bytes of one fwd+bwd (and of each half).

    Per token-head (d = d_k = d_v, chunk C; causal C x C products counted once):
      forward flop  6 d^2 + 2 C d      (K W, Q W, K^T G, Q K^T, A G)
      backward flop 12 d^2 + 5 C d     (the six d x d products of the reverse
                                        sweep plus the score-side C x C terms)
      forward bytes  q, k, v + beta + [log a] + o + one W checkpoint per chunk (d^2 * 4 / C)
      backward bytes q, k, v + beta + [log a] + d_o + checkpoint read
                     + dq, dk, dv + dbeta + [dlog a]
    """
    d = cfg["dk"]
    C = cfg["C"]
    io = 2 if cfg["dtype"] == "bf16" else 4
    th = cfg["B"] * cfg["H"] * cfg["T"]
    vec = cfg["decay"] == "vector"
    la = 4 * d if vec else 0
    ck = d * d * 4 / C
    f_fwd = 6 * d * d + 2 * C * d
    f_bwd = 12 * d * d + 5 * C * d
    b_fwd = 3 * d * io + 4 + la + d * io + ck
    b_bwd = 3 * d * io + 4 + la + d * io + ck + 3 * d * io + 4 + la
    return dict(token_heads=th, flop_fwd=f_fwd * th, flop_bwd=f_bwd * th, bytes_fwd=b_fwd * th,
                bytes_bwd=b_bwd * th, flop_per_th=(f_fwd, f_bwd), bytes_per_th=(b_fwd, b_bwd))


def cpu_baseline(name, chains, budget_s=25.0):
    """Time the fp64 oracle (as it stands) on a few chains; returns the dict for the JSON line."""
    import numpy as np
    from chunkwise_weight_recurrence_amd import workloads as wl
    from oracle import chunk_backward, chunk_forward
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads") or 0) for p in threadpool_info()) or None
    except Exception:
        pass
    cores = threads or len(os.sched_getaffinity(0))
    inp = wl.make_ttt_inputs(name)
    cfg = inp["cfg"]
    done = 0
    t_total = 0.0
    for ch in chains:
        s = wl.select_chains(inp, [ch])
        kw = wl.oracle_kwargs(s)
        t0 = time.perf_counter()
        chunk_forward(s["q"], s["k"], s["v"], s["beta"], cfg["b"], cfg["C"], **kw)
        if cfg.get("bwd"):
            chunk_backward(s["q"], s["k"], s["v"], s["beta"], cfg["b"], cfg["C"], s["d_o"], **kw)
        t_total += time.perf_counter() - t0
        done += 1
        if t_total > budget_s:
            break
    # one token of the layer needs all H heads: tokens/s = chains * T / (H * seconds)
    value = done * cfg["T"] / (cfg["H"] * t_total)
    return dict(value=value, unit="tokens/s", cores=int(cores), kind="oracle",
                sample=f"{done} of {cfg['B'] * cfg['H']} (b,h) chains of {name}, full T={cfg['T']}, "
                       f"fwd+bwd in fp64 NumPy, {t_total:.1f} s; scaled by 1/H to layer tokens")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="1.45b-fwdbwd")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-chains", type=int, default=2)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the (b, h) chains shard over GPUs without communication; see DESIGN.md).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from chunkwise_weight_recurrence_amd import workloads as wl
    from chunkwise_weight_recurrence_amd.layer import TTTLayerBuffers

    name = args.workload
    inp = wl.make_ttt_inputs(name)
    cfg = inp["cfg"]
    bufs = TTTLayerBuffers(inp, device="cuda", with_bwd=True)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step():
        bufs.forward()
        bufs.backward()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    tokens = cfg["B"] * cfg["T"]
    value = tokens / (ms_per_step / 1e3)

    # per entry point: forward and backward timed on their own
    def time_entry(fn, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    n_each = max(3, args.steps // 2)
    t_fwd = time_entry(bufs.forward, n_each)
    t_bwd = time_entry(bufs.backward, n_each)

    work = algorithmic_work(cfg)
    flop = work["flop_fwd"] + work["flop_bwd"]
    byts = work["bytes_fwd"] + work["bytes_bwd"]
    mfma_util = flop / (ms_per_step / 1e3) / (PEAK_BF16_TFLOPS * 1e12)
    # the dominant entry point, priced against the roofline its intensity puts it on
    dom = "bwd" if t_bwd >= t_fwd else "fwd"
    t_dom = t_bwd if dom == "bwd" else t_fwd
    f_dom = work["flop_" + dom]
    b_dom = work["bytes_" + dom]
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if f_dom / b_dom < ridge:
        roof = dict(bound="hbm", achieved=b_dom / (t_dom / 1e3) / 1e9, peak=PEAK_HBM_GBS, unit="GB/s")
    else:
        roof = dict(bound="mfma", achieved=f_dom / (t_dom / 1e3) / 1e12, peak=PEAK_BF16_TFLOPS,
                    unit="TFLOP/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["kernel"] = f"ttt_chunk_{dom} (entry point, {t_dom:.3f} ms per launch)"

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": f"{name}: B={cfg['B']} H={cfg['H']} T={cfg['T']} d={cfg['dk']} "
                               f"C={cfg['C']} loss={cfg['loss']} act={cfg['act']} decay={cfg['decay']}",
                   "global_batch": cfg["B"], "seq_len": cfg["T"], "parallelism": "single-gpu"},
        "mfma_util": mfma_util,
        "ms_fwd": t_fwd,
        "ms_bwd": t_bwd,
        "algorithmic": {"gflop": flop / 1e9, "gbytes": byts / 1e9,
                        "hbm_frac_whole_step": byts / (ms_per_step / 1e3) / (PEAK_HBM_GBS * 1e9)},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        chains = [(b, h) for b in range(cfg["B"]) for h in range(cfg["H"])][:max(1, args.cpu_chains)]
        out["cpu_baseline"] = cpu_baseline(name, chains)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
