#!/usr/bin/env python3
"""Throughput of the chunkwise TTT layer, forward + backward, on one MI355X.

A step is one ttt_chunk_fwd + ttt_chunk_bwd over one batch of the 1.45B-shaped
workload (B=4, H=16, T=4096, d_k=d_v=128, C=256, bf16 I/O, fp32 state; IP loss,
SiLU, per-token vector decay), inputs resident in HBM.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
  python bench.py --copy-calibration MIB     (plain device copy, for counter scaling)
  python bench.py --workload inplace-wdown   (In-Place TTT W_down apply + update instead)
  python bench.py --workload inplace-wdown-guarded   (the same with update clipping and
                                             document resets)
  python bench.py --workload inplace-wdown-fwdbwd / inplace-wdown-guarded-fwdbwd
                                            (either, then its W_down backward)
  python bench.py --workload 160m-mlp-fwd    (two-layer fast net (TTT-MLP) forward)
  python bench.py --workload 160m-mlp-fwdbwd (the same, forward + outer backward)
  python bench.py --workload 160m-norm-fwdbwd (the Norm primitive as the act, forward + backward)

Timing: W untimed warm-up steps, then K timed steps with the per-kernel timer
off, bracketed by a device synchronisation on both sides and HIP events on the
stream the library launches on (torch's current stream): `value` and
`ms_per_step` come from that mean; one event pair around each step gives the
median and the minimum.  A second run of K steps with the library's per-kernel
timer on (HIP events around every kernel on the same stream) gives each
kernel's mean duration and from it the roofline figures.  For the layer
workloads a third run writes a 512 MiB buffer before every step (past the L2
and the MALL) and reports the cold-cache median and minimum.  The CPU baseline
times the fp64 oracle on a bounded sample (a few (b, h) chains, or a few rows
of W_down) on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TTT-layer fwd+bwd tokens/sec at H=16,d=128,T=4096 on 1 GPU; MFMA util %"

# MI355X published peaks
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3


FLUSH_BYTES = 512 << 20  # larger than the L2s (8 x 4 MiB) and the MALL (256 MiB) together


def run_timed(torch, step, steps, stream, flush=None):
    """Run step() `steps` times.  Returns the mean over the whole run (bracketed by a
    synchronisation on both sides) and the median, minimum and maximum of one HIP event
    pair per step.  With `flush`, flush() runs before every step, outside its events
    (the mean then includes it and is not reported)."""
    import statistics
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for a, b in pairs:
        if flush is not None:
            flush()
        a.record(stream)
        step()
        b.record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in pairs)
    out = dict(steps=steps, median_ms=statistics.median(per), min_ms=per[0], max_ms=per[-1])
    if flush is None:
        out["mean_ms"] = e0.elapsed_time(e1) / steps
    return out


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
    # the inner-product loss without an act needs no train-view product K W
    f_fwd = (4 if linear_path(cfg) else 6) * d * d + 2 * C * d
    f_bwd = 12 * d * d + 5 * C * d
    b_fwd = 3 * d * io + 4 + la + d * io + ck
    b_bwd = 3 * d * io + 4 + la + d * io + ck + 3 * d * io + 4 + la
    return dict(token_heads=th, flop_fwd=f_fwd * th, flop_bwd=f_bwd * th, bytes_fwd=b_fwd * th,
                bytes_bwd=b_bwd * th, flop_per_th=(f_fwd, f_bwd), bytes_per_th=(b_fwd, b_bwd))


def linear_path(cfg):
    """Inner-product loss, no act: the chunk-parallel forward (G = -V needs no state)."""
    return cfg["loss"] == "ip" and cfg["act"] == "none" and cfg["dtype"] == "bf16"


def kernel_work(cfg):
    """Algorithmic flop and bytes per token-head of each matrix-core kernel.

    The path's algorithmic bytes are split by the kernel that must read (first)
    or write (last) them; the flop by the kernel that forms each product:
      fwd        all of the forward (see algorithmic_work)
      bwd_seq    reads q, k, v, beta, [log a], d_o, the checkpoint; writes dv.
                 Products Q~^T dY, K_bar dW', K^T dZ (2 d^2 each) and A^T dY (C d).
      bwd_cross  writes dq, dk, dbeta, [dlog a].
                 Products dY W^T, dZ W^T, G~ dW'^T (2 d^2 each) and the score
                 side dY G~^T, dS K~, dS^T Q~ and the d_eta reduction (C d each).
    The two backward kernels sum to the backward figures of algorithmic_work.
    """
    d = cfg["dk"]
    C = cfg["C"]
    io = 2 if cfg["dtype"] == "bf16" else 4
    la = 4 * d if cfg["decay"] == "vector" else 0
    ck = d * d * 4 / C
    return {
        "fwd": (6 * d * d + 2 * C * d, 3 * d * io + 4 + la + d * io + ck),
        "bwd_seq": (6 * d * d + C * d, 3 * d * io + 4 + la + d * io + ck + d * io),
        "bwd_cross": (6 * d * d + 4 * C * d, 2 * d * io + 4 + la),
        # chunk-parallel forward: lin_state reads k, v, beta, [log a] and forms K^T G~;
        # lin_scan writes the checkpoints; lin_out reads q, writes o, forms Q W and the scores
        "lin_state": (2 * d * d, 2 * d * io + 4 + la),
        "lin_scan": (0, ck),
        "lin_out": (2 * d * d + 2 * C * d, 2 * d * io),
        # the fp32 VALU path and the row path (fp32 matrix cores, one workgroup per chain):
        # one kernel for the forward, one for the backward
        "generic_fwd": (6 * d * d + 2 * C * d, 3 * d * io + 4 + la + d * io + ck),
        "generic_bwd": (12 * d * d + 5 * C * d, 3 * d * io + 4 + la + d * io + ck + 3 * d * io + 4 + la),
        # the row path's forward: the sequential train view and transition (norm_fwd:
        # K W, K^T G; reads k, v, beta, writes the checkpoints), then the query view of
        # every chunk at once (norm_query: Q W and the scores; reads q, writes o)
        "norm_fwd": (4 * d * d, 2 * d * io + 4 + la + ck),
        "norm_query": (2 * d * d + 2 * C * d, 2 * d * io),
        # the row path's backward: the chunk-parallel pre-pass (norm_bwd_pre: dY W^T, Q^T dY and
        # the score side; reads q, k, v, beta, d_o, the checkpoints, writes dq), then the reverse
        # sweep that carries dW (norm_bwd: K dW', G dW'^T, dZ W^T, K^T dZ; writes dk, dv, dbeta)
        "norm_bwd_pre": (4 * d * d + 4 * C * d, 3 * d * io + 4 + d * io + ck + d * io),
        "norm_bwd": (8 * d * d, ck + 2 * d * io + 4),
    }


KERNEL_NAMES = {"fwd": "ttt_fwd_mfma_kernel", "bwd_seq": "ttt_bwd_seq_kernel",
                "bwd_cross": "ttt_bwd_cross_kernel", "lin_state": "lin_state_kernel",
                "lin_scan": "lin_scan_kernel", "lin_out": "lin_out_kernel",
                "generic_fwd": "fwd_generic_kernel", "generic_bwd": "bwd_generic_kernel",
                "norm_fwd": "norm_fwd_kernel", "norm_query": "norm_query_kernel", "norm_bwd_pre": "norm_bwd_pre_kernel",
                "norm_bwd": "norm_bwd_kernel"}
# vector decay runs the tile-relative kernels
KERNEL_NAMES_VECTOR = {"fwd": "ttt_fwd_vec_kernel", "bwd_seq": "ttt_bwd_seq_vec_kernel"}


# The device sources each family of kernels is compiled from: a counter figure
# stays valid while these hash the same (host-side files do not change a kernel).
KERNEL_SOURCES = {
    "ttt": ("mfma_util.h", "ttt_device.h", "ttt_mfma_common.h", "ttt_decay_prep.hip", "ttt_mfma_fwd.hip",
            "ttt_mfma_bwd.hip", "ttt_linear.hip"),
    "inplace": ("ttt_device.h", "inplace.hip"),
    "mlp": ("tile_gemm.h", "ttt_device.h", "ttt_mlp_common.h", "ttt_mlp.hip", "ttt_mlp_bwd.hip"),
    "norm": ("tile_gemm.h", "ttt_device.h", "ttt_norm.hip"),
    "generic": ("ttt_device.h", "ttt_generic.hip"),
}


def kernel_family(kernel):
    if kernel.startswith("inplace"):
        return "inplace"
    if kernel.startswith(("fwd_generic", "bwd_generic")):
        return "generic"
    if kernel.startswith("norm"):
        return "norm"
    return "mlp" if kernel.startswith("mlp") else "ttt"


def kernel_source_digest(family="ttt"):
    """sha256 over the device sources of one kernel family: counter figures taken on
    other sources are stale."""
    src = os.path.join(ROOT, "chunkwise_weight_recurrence_amd", "csrc")
    h = hashlib.sha256()
    for fn in sorted(KERNEL_SOURCES[family]):
        h.update(fn.encode())
        path = os.path.join(src, fn)
        if os.path.exists(path):
            with open(path, "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter summary,
    or None when there is none or it was taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    if not os.path.exists(path):
        return None
    digest = kernel_source_digest(kernel_family(kernel))
    for line in open(path):
        m = re.match(r"\s*traffic-record:\s*(\{.*\})\s*$", line)
        if not m:
            continue
        rec = json.loads(m.group(1))
        if rec.get("kernel") == kernel and rec.get("workload") == workload and rec.get("sources") == digest:
            return rec["bytes_per_launch"]
    return None


def copy_calibration(mib):
    """Plain device-to-device copies of a known size, to scale FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = mib * 1024 * 1024 // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4, "copies": 3}), flush=True)


def bench_inplace(args):
    """One step = one inplace_ttt_fwd over the whole In-Place workload (apply then
    update for each of the T / C chunks), and with ``bwd`` in the workload one
    inplace_ttt_bwd after it; w_down reset outside the timed region."""
    import numpy as np
    import torch
    from chunkwise_weight_recurrence_amd import binding as B
    from chunkwise_weight_recurrence_amd import workloads as wl
    from chunkwise_weight_recurrence_amd.layer import InplaceBuffers

    def mm(a, b):  # input synthesis only (outside every timed region)
        return (torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda() @
                torch.from_numpy(np.ascontiguousarray(b, dtype=np.float32)).cuda()).cpu().numpy()

    inp = wl.make_inplace_inputs(args.workload, matmul=mm)
    cfg = inp["cfg"]
    bufs = InplaceBuffers(inp)
    with_bwd = bool(cfg.get("bwd"))
    if with_bwd:
        from chunkwise_weight_recurrence_amd.layer import to_device
        g = wl.make_inplace_grads(cfg, seed=cfg.get("seed", 0) + 1)
        d_o, d_wf = to_device(g["d_o_dev"]), to_device(g["d_wfinal_dev"])
    stream = torch.cuda.current_stream()

    def step():
        bufs.forward()
        if with_bwd:
            bufs.backward(d_o, d_wf)

    for _ in range(args.warmup):
        bufs.reset()
        step()
    torch.cuda.synchronize()
    times = []
    B.ttt_timing_enable(True)
    for _ in range(args.steps):
        bufs.reset()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    B.ttt_timing_enable(False)
    ms = sum(times) / len(times)
    # the same steps with the per-kernel timer off (W_down reset between steps, outside the events)
    t_off = []
    for _ in range(args.steps):
        bufs.reset()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        t_off.append(e0.elapsed_time(e1))
    import statistics
    t_off.sort()
    timing = dict(steps=args.steps, kernel_timer="off", mean_ms=sum(t_off) / len(t_off),
                  median_ms=statistics.median(t_off), min_ms=t_off[0], max_ms=t_off[-1],
                  mean_ms_kernel_timer_on=ms)
    ms = timing["mean_ms"]
    kernels = {}
    for kid in (B.Kernel.INPLACE_APPLY, B.Kernel.INPLACE_NORM, B.Kernel.INPLACE_UPDATE, B.Kernel.INPLACE_BWD_W,
                B.Kernel.INPLACE_BWD_DZ, B.Kernel.INPLACE_BWD_DV, B.Kernel.INPLACE_BWD_DW):
        total, n = B.ttt_timing_read(kid)
        if n:
            kernels[kid.name.lower()] = {"ms_per_launch": total / n, "launches": n, "ms_per_step": total / args.steps}
    T, dm, dff, C = cfg["T"] * cfg["B"], cfg["d_model"], cfg["d_ff"], cfg["C"]
    # algorithmic work: apply O = Z W^T (2 T dm dff) and update W += eta Vhat^T Z (2 T dm dff);
    # with clipping, the update's norm is one more product of the update's size
    flop_apply = 2.0 * T * dm * dff
    nchunk = cfg["B"] * sum((n + C - 1) // C for n in (cfg.get("doc_lens") or (cfg["T"],)))
    clip_bwd = with_bwd and bool(cfg.get("clip_tau"))
    # the clipped backward's correction: the chunk's Gram matrices Z Z^T, V_hat V_hat^T
    # and their products with V_hat and Z, 2 c^2 (d_model + d_ff) for each of dV_hat and dZ
    flop_gram = 2.0 * C * T * (dm + dff) if clip_bwd else 0.0
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    # per launch (one chunk, the mean length): 2 T d_model d_ff / chunks for every step but dZ,
    # which forms two products, and the clip correction's share of dZ and dV_hat
    f_dom = flop_apply / nchunk * (2 if dom == "inplace_bwd_dz" else 1)
    if dom in ("inplace_bwd_dz", "inplace_bwd_dv"):
        f_dom += flop_gram / nchunk
    roof = dict(bound="mfma", achieved=f_dom / (kernels[dom]["ms_per_launch"] / 1e3) / 1e12,
                peak=PEAK_BF16_TFLOPS, unit="TFLOP/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = counter_traffic(dom, args.workload)
    roof["kernel"] = {"inplace_apply": "apply_kernel (split-K 256x128 tiles) + split_reduce_kernel",
                      "inplace_norm": "update_kernel<true> (the update's products, per-tile sums of squares) + "
                                      "clip_scale_kernel",
                      "inplace_update": "update_kernel (persistent 256x128 tiles, fp32 read-modify-write + bf16 copy)",
                      "inplace_bwd_w": "update_kernel (state rewind, persistent 256x128 tiles)",
                      "inplace_bwd_dz": "apply_kernel<true> (dZ, two terms as two splits) + split_reduce_kernel" +
                                        (" + Gram V_hat V_hat^T, its product with Z, dz_combine_kernel"
                                         if clip_bwd else ""),
                      "inplace_bwd_dv": "apply_kernel (dV_hat, split-K) + split_reduce_kernel" +
                                        (" + Gram Z Z^T, its product with V_hat, pdot/kappa/dv_combine kernels"
                                         if clip_bwd else ""),
                      "inplace_bwd_dw": "update_kernel (dW chain, persistent 256x128 tiles)"}[dom]
    roof["ms_per_launch"] = kernels[dom]["ms_per_launch"]
    out = {
        "metric": ("In-Place TTT W_down apply+clip+update, forward + backward, document resets, tokens/sec (1 GPU)"
                   if with_bwd and bufs.guarded else
                   "In-Place TTT W_down apply+update, forward + backward, tokens/sec (1 GPU)" if with_bwd else
                   "In-Place TTT W_down apply+update tokens/sec (1 GPU)" if not bufs.guarded else
                   "In-Place TTT W_down apply+clip+update tokens/sec, document resets (1 GPU)"),
        "value": T / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: B={cfg['B']} T={cfg['T']} d_model={dm} d_ff={dff} C={C}" +
                   (f" clip_tau={cfg['clip_tau']:g} docs={list(cfg['doc_lens'])}" if bufs.guarded else ""),
                   "global_batch": cfg["B"], "seq_len": cfg["T"], "parallelism": "single-gpu"},
        # algorithmic products: apply and update, [the norm], [dZ (two), dV_hat, dW, the clip correction];
        # the rewind, the backward's norms and the replays of earlier documents are recomputation
        "mfma_util": ((2 + bool(cfg.get("clip_tau")) + 4 * with_bwd) * flop_apply + 2 * flop_gram) / (ms / 1e3) /
                     (PEAK_BF16_TFLOPS * 1e12),
        "kernels": kernels,
        "timing": timing,
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not with_bwd and not bufs.guarded:
        # algorithmic HBM bytes of the pass with W_down kept on chip (its floor): Z and V_hat read
        # once, O written once, W_down (fp32) read and written once
        b_floor = cfg["B"] * (T // cfg["B"] * (dff + 2 * dm) * 2 + 2 * dm * dff * 4)
        # with W_down streamed per chunk: the apply reads its bf16 copy (2 B a weight), the update
        # reads and writes it in fp32 and writes the bf16 copy (10 B)
        b_stream = cfg["B"] * (T // cfg["B"] * (dff + 2 * dm) * 2 + 12 * nchunk * dm * dff)
        out["hbm"] = {"algorithmic_gbytes_w_stationary": b_floor / 1e9,
                      "algorithmic_gbytes_w_streamed": b_stream / 1e9,
                      "achieved_gbs_w_stationary": b_floor / (ms / 1e3) / 1e9,
                      "achieved_gbs_w_streamed": b_stream / (ms / 1e3) / 1e9,
                      "counter_gbytes_per_pass": counter_pass_bytes(args.workload)}
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline_inplace(inp, mm)
    print(json.dumps(out), flush=True)


def counter_pass_bytes(workload):
    """Counter HBM bytes of one In-Place pass (the apply and update kernels of every chunk)
    from the committed counter summary, or None."""
    per = [counter_traffic(k, workload) for k in ("inplace_apply", "inplace_update")]
    if any(p is None for p in per):
        return None
    cfg_chunks = None
    from chunkwise_weight_recurrence_amd import workloads as wl
    c = wl.INPLACE_WORKLOADS[workload]
    cfg_chunks = math.ceil(c["T"] / c["C"]) * c["B"]
    return sum(per) * cfg_chunks / 1e9


def cpu_baseline_inplace(inp, mm, rows_n=64, budget_s=25.0):
    """The fp64 oracle of the In-Place pass on a sample of W_down's rows (each row evolves on
    its own), over the whole sequence, scaled to the full d_model rows."""
    import numpy as np
    from chunkwise_weight_recurrence_amd import workloads as wl
    from oracle import inplace_rows
    cfg = inp["cfg"]
    dm = cfg["d_model"]
    z = wl.inplace_values(inp, "z_dev")
    vh = wl.inplace_values(inp, "vhat_dev")
    done, t_total, n = 0, 0.0, 0
    step = max(1, dm // rows_n)
    while t_total < min(5.0, budget_s):
        rows = list(range(n % step, dm, step))[:rows_n]
        w0 = inp["w0_dev"][:, rows].astype(np.float64)
        t0 = time.perf_counter()
        inplace_rows(z, vh, w0, rows, cfg["C"], cfg["eta"])
        t_total += time.perf_counter() - t0
        done += len(rows)
        n += 1
    tokens = cfg["B"] * cfg["T"]
    return dict(value=tokens / (t_total * dm / done), unit="tokens/s", cores=_oracle_cores(), kind="oracle",
                sample=f"{done} of {dm} rows of W_down ({n} runs of {rows_n} rows), the whole sequence "
                       f"(T={cfg['T']}, C={cfg['C']}), apply + update in fp64 NumPy, {t_total:.1f} s; "
                       f"scaled by rows to the full layer")


def norm_work(cfg):
    """Algorithmic flop of the Linear -> Norm forward's two kernels and of the backward (the
    backward without its recomputed forward).  Forward per token-head: the sequential
    kernel's K W and K^T G (4 d_k d_v), the query kernel's Q W (2 d_k d_v) and, per
    lower-triangle entry of each chunk, Q K^T and S G (2 (d_k + d_v)).  Backward per
    token-head: the pre-pass's dY W^T and Q^T dY (4 d_k d_v) and, per entry, dS, S^T dY,
    dS K, dS^T Q (2 (2 d_v + 2 d_k)); the sweep's K dW', G dW'^T, dZ W^T and K^T dZ
    (8 d_k d_v).  The per-token normalisations are O(d_v) and not counted."""
    dk, dv, C, T = cfg["dk"], cfg["dv"], cfg["C"], cfg["T"]
    tri = sum(c * (c + 1) // 2 for c in (min(C, T - s) for s in range(0, T, C)))
    chains = cfg["B"] * cfg["H"]
    fwd = chains * 4 * dk * dv * T
    query = chains * (2 * dk * dv * T + tri * 2 * (dk + dv))
    bwd_pre = chains * (4 * dk * dv * T + tri * 2 * (2 * dv + 2 * dk))
    bwd = chains * 8 * dk * dv * T
    return fwd, query, bwd_pre, bwd


def mlp_work(cfg):
    """Algorithmic flop of one two-layer forward.  Per token-head: train view K W1
    (2 d_k d_h), [A W2 (2 d_h d_v), MSE only], G2 W2^T (2 d_v d_h); query view Q W1, A_q W2
    (2 d_k d_h + 2 d_h d_v); state steps K^T G1, A^T G2 (2 d_k d_h + 2 d_h d_v).  Per chunk
    of c tokens, over the lower triangle (diagonal included, c (c + 1) / 2 entries):
    Tril(Q K^T), Tril(A_q A^T) and their products with eta G1, eta G2, 2 (d_k + 2 d_h + d_v)
    flop per entry.  HBM bytes: q, k, v, o and beta per token-head, and the two weights
    read and written once per chain."""
    dk, dh, dv, C, T = cfg["dk"], cfg["dh"], cfg["dv"], cfg["C"], cfg["T"]
    mse = cfg["loss"] == "mse"
    f_th = 6 * dk * dh + (6 + 2 * mse) * dh * dv
    tri = sum(c * (c + 1) // 2 for c in (min(C, T - s) for s in range(0, T, C)))
    io = 2 if cfg["dtype"] == "bf16" else 4
    chains = cfg["B"] * cfg["H"]
    th = chains * T
    flop = f_th * th + chains * tri * 2 * (dk + 2 * dh + dv)
    byts = th * (io * (2 * dk + 2 * dv) + 4) + chains * 2 * 4 * (dk * dh + dh * dv)
    return flop, byts


def mlp_fwd_split(cfg):
    """mlp_work's flop by kernel: the sequential train view and state steps (mlp_fwd: K W1,
    [A W2], G2 W2^T, K^T G1, A^T G2) and the query view of every chunk (mlp_query: Q W1,
    A_q W2 and the two causal score matrices with their products)."""
    dk, dh, dv, C, T = cfg["dk"], cfg["dh"], cfg["dv"], cfg["C"], cfg["T"]
    mse = cfg["loss"] == "mse"
    tri = sum(c * (c + 1) // 2 for c in (min(C, T - s) for s in range(0, T, C)))
    th = cfg["B"] * cfg["H"] * T
    seq = (4 * dk * dh + (4 + 2 * mse) * dh * dv) * th
    query = (2 * dk * dh + 2 * dh * dv) * th + cfg["B"] * cfg["H"] * tri * 2 * (dk + 2 * dh + dv)
    return {"mlp_fwd": seq, "mlp_query": query}


def mlp_bwd_work(cfg):
    """Algorithmic flop of one two-layer outer backward, without the forward it recomputes
    per chunk.  Per token-head: 12 d_k d_h (dQ, d(eta G1), dK's two products, dW1's two) and
    (12 + 4 [MSE]) d_h d_v (d(eta G2), dA_q, dA, dG2, dW2's two; MSE adds dV_hat W2^T and
    A^T dV_hat).  Per lower-triangle entry of each chunk: 2 (2 d_v + 4 d_h + 2 d_k) flop
    (dS2 and its two uses, dS1 and its three uses, S2^T dO, S1^T dX1)."""
    dk, dh, dv, C, T = cfg["dk"], cfg["dh"], cfg["dv"], cfg["C"], cfg["T"]
    mse = cfg["loss"] == "mse"
    f_th = 12 * dk * dh + (12 + 4 * mse) * dh * dv
    tri = sum(c * (c + 1) // 2 for c in (min(C, T - s) for s in range(0, T, C)))
    chains = cfg["B"] * cfg["H"]
    return f_th * chains * T + chains * tri * 2 * (2 * dv + 4 * dh + 2 * dk)


def mlp_bwd_split(cfg):
    """mlp_bwd_work's flop by kernel: the pre-pass (mlp_bwd_pre: dQ's two products, Q^T dX1,
    A_q^T dO, dO W2^T and the score side) and the reverse sweep (mlp_bwd: the products with
    the carried dW1, dW2 and what follows from them: A dW2', (eta G2) dW2'^T, K dW1',
    (eta G1) dW1'^T, dP W2, dZ1 W1^T, K^T dZ1, dP^T G2 and, for MSE, dV_hat W2^T, A^T dV_hat)."""
    dk, dh, dv, T = cfg["dk"], cfg["dh"], cfg["dv"], cfg["T"]
    mse = cfg["loss"] == "mse"
    th = cfg["B"] * cfg["H"] * T
    sweep = (8 * dk * dh + (8 + 4 * mse) * dh * dv) * th
    return {"mlp_bwd_pre": mlp_bwd_work(cfg) - sweep, "mlp_bwd": sweep}


def bench_mlp(args):
    """One step = one ttt_mlp_chunk_fwd over the whole two-layer workload."""
    import torch
    from chunkwise_weight_recurrence_amd import binding as B
    from chunkwise_weight_recurrence_amd import workloads as wl
    from chunkwise_weight_recurrence_amd.layer import MlpBuffers

    from chunkwise_weight_recurrence_amd.layer import to_device
    inp = wl.make_mlp_inputs(args.workload)
    cfg = inp["cfg"]
    with_bwd = bool(cfg.get("bwd"))
    bufs = MlpBuffers(inp, with_bwd=with_bwd)
    d_o = to_device(wl.make_mlp_grads(cfg, cfg["seed"] + 1)["d_o_dev"]) if with_bwd else None
    stream = torch.cuda.current_stream()

    def step():
        bufs.forward()
        if with_bwd:
            bufs.backward(d_o)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    B.ttt_timing_enable(True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    B.ttt_timing_enable(False)
    ms = ev0.elapsed_time(ev1) / args.steps
    kernels = {}
    for kid in (B.Kernel.MLP_FWD, B.Kernel.MLP_QUERY, B.Kernel.MLP_BWD_PRE, B.Kernel.MLP_BWD):
        total, n = B.ttt_timing_read(kid)
        if n:
            kernels[kid.name.lower()] = {"ms_per_launch": total / n, "launches": n}
    flop, byts = mlp_work(cfg)
    flop_b = mlp_bwd_work(cfg) if with_bwd else 0
    per_kernel = dict(mlp_fwd_split(cfg), **(mlp_bwd_split(cfg) if with_bwd else {}))
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_launch"])
    t_dom = kernels[dom]["ms_per_launch"]
    f_dom = per_kernel[dom]
    roof = dict(bound="mfma", achieved=f_dom / (t_dom / 1e3) / 1e12, peak=PEAK_FP32_TFLOPS, unit="TFLOP/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = counter_traffic(dom, args.workload)
    roof["kernel"] = {"mlp_fwd": "mlp_fwd_kernel (train view and state steps, one workgroup per chain, fp32 "
                                 "32x32x2 matrix-core tiles)",
                      "mlp_query": "mlp_query_kernel (query view, one workgroup per chunk of every chain, fp32 "
                                   "32x32x2 matrix-core tiles)",
                      "mlp_bwd_pre": "mlp_bwd_pre_kernel (one workgroup per chunk of every chain: the chunk's "
                                     "forward, saved or recomputed, and the backward's terms free of the carried dW)",
                      "mlp_bwd": "mlp_bwd_kernel (one workgroup per chain, reverse chunk sweep carrying dW1, dW2, "
                                 "fp32 32x32x2 matrix-core tiles)"}[dom]
    roof["ms_per_launch"] = t_dom
    roof["algorithmic_per_launch"] = {"flop": f_dom}
    tokens = cfg["B"] * cfg["T"]
    out = {
        "metric": ("TTT-MLP layer forward + backward tokens/sec (1 GPU)" if with_bwd else
                   "TTT-MLP layer forward tokens/sec (1 GPU)"),
        "value": tokens / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{args.workload}: B={cfg['B']} H={cfg['H']} T={cfg['T']} d_k={cfg['dk']} "
                               f"d_h={cfg['dh']} d_v={cfg['dv']} C={cfg['C']} loss={cfg['loss']} "
                               f"act={cfg['act']} decay={cfg['decay']}, {cfg['dtype']} I/O",
                   "global_batch": cfg["B"], "seq_len": cfg["T"], "parallelism": "single-gpu"},
        "kernels": kernels,
        "algorithmic": {"gflop": (flop + flop_b) / 1e9, "gbytes_forward": byts / 1e9},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        # the whole workload takes the oracle a few seconds: time every chain (within the budget)
        out["cpu_baseline"] = cpu_baseline_mlp(args.workload, cfg["B"] * cfg["H"])
    print(json.dumps(out), flush=True)


def cpu_baseline_mlp(name, n_chains, budget_s=25.0):
    """The fp64 oracle of the two-layer forward on a few chains (the same role as cpu_baseline)."""
    from chunkwise_weight_recurrence_amd import workloads as wl
    from oracle import mlp_chunk_backward, mlp_chunk_forward
    inp = wl.make_mlp_inputs(name)
    cfg = inp["cfg"]
    with_bwd = bool(cfg.get("bwd"))
    d_o = wl.make_mlp_grads(cfg, cfg["seed"] + 1)["d_o"] if with_bwd else None
    chains = [(b, h) for b in range(cfg["B"]) for h in range(cfg["H"])][:n_chains]
    done, t_total = 0, 0.0
    for ch in chains:
        s = wl.select_mlp_chains(inp, [ch])
        t0 = time.perf_counter()
        mlp_chunk_forward(s["q"], s["k"], s["v"], s["beta"], cfg["b"], cfg["C"], cfg["loss"], cfg["act"],
                          cfg["decay"], s["gamma"], s["w1_0"], s["w2_0"])
        if with_bwd:
            mlp_chunk_backward(s["q"], s["k"], s["v"], s["beta"], cfg["b"], cfg["C"], d_o[ch[0], ch[1]][None, None],
                               cfg["loss"], cfg["act"], cfg["decay"], s["gamma"], s["w1_0"], s["w2_0"])
        t_total += time.perf_counter() - t0
        done += 1
        if t_total > budget_s:
            break
    return dict(value=done * cfg["T"] / (cfg["H"] * t_total), unit="tokens/s", cores=_oracle_cores(),
                kind="oracle", sample=f"{done} of {cfg['B'] * cfg['H']} (b,h) chains of {name}, full T={cfg['T']}, "
                                      f"{'forward + backward' if with_bwd else 'forward'} in fp64 NumPy, {t_total:.2f} s; "
                                      f"scaled by 1/H to layer tokens")


def _oracle_cores():
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads") or 0) for p in threadpool_info()) or None
    except Exception:
        threads = None
    return int(threads or len(os.sched_getaffinity(0)))


def cpu_baseline(name, chains, budget_s=25.0, token_loop=False):
    """Time the fp64 oracle (as it stands) on a few chains; returns the dict for the JSON line.
    A problem the oracle finishes quickly is repeated until about 5 s of work, and with
    ``token_loop`` the token-by-token form is timed beside it."""
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
    what = "fwd+bwd" if cfg.get("bwd") else "forward"
    done = 0
    t_total = 0.0
    while True:  # every listed chain once; a quick problem again until about 5 s
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
        if t_total > min(5.0, budget_s):
            break
    # one token of the layer needs all H heads: tokens/s = chains * T / (H * seconds)
    value = done * cfg["T"] / (cfg["H"] * t_total)
    out = dict(value=value, unit="tokens/s", cores=int(cores), kind="oracle",
               sample=f"{done} chain runs ({len(chains)} of {cfg['B'] * cfg['H']} (b,h) chains) of {name}, "
                      f"full T={cfg['T']}, {what} in fp64 NumPy (chunk form), {t_total:.1f} s; "
                      f"scaled by 1/H to layer tokens")
    if token_loop:
        from oracle import token_loop_forward
        n, t_loop = 0, 0.0
        while t_loop < 5.0:
            s = wl.select_chains(inp, [chains[n % len(chains)]])
            kw = wl.oracle_kwargs(s)
            t0 = time.perf_counter()
            token_loop_forward(s["q"], s["k"], s["v"], s["beta"], cfg["b"], cfg["C"], **kw)
            t_loop += time.perf_counter() - t0
            n += 1
        out["token_loop"] = dict(value=n * cfg["T"] / (cfg["H"] * t_loop), unit="tokens/s",
                                 sample=f"{n} chain runs of the token-by-token forward, {t_loop:.1f} s")
    return out


def norm_bench_line(args, name, cfg, kernels, ms_per_step, value, with_bwd):
    """The JSON line of a Linear -> Norm workload: its two kernels against the fp32 matrix peak."""
    f_fwd, f_query, f_bwd_pre, f_bwd = norm_work(cfg)
    flops = {"norm_fwd": f_fwd, "norm_query": f_query, "norm_bwd_pre": f_bwd_pre, "norm_bwd": f_bwd}
    timed = {k: v for k, v in kernels.items() if k in flops}
    dom = max(timed, key=lambda k: timed[k]["ms_per_launch"])
    t_dom = timed[dom]["ms_per_launch"]
    roof = dict(bound="mfma", achieved=flops[dom] / (t_dom / 1e3) / 1e12, peak=PEAK_FP32_TFLOPS, unit="TFLOP/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = counter_traffic(dom, name)
    roof["kernel"] = {"norm_fwd": "norm_fwd_kernel (train view and transition, one workgroup per chain, fp32 "
                                  "32x32x2 matrix-core tiles)",
                      "norm_query": "norm_query_kernel (query view, one workgroup per chunk of every chain, fp32 "
                                    "32x32x2 matrix-core tiles)",
                      "norm_bwd_pre": "norm_bwd_pre_kernel (one workgroup per chunk of every chain: the chunk's "
                                      "forward again and the backward's terms free of the carried dW)",
                      "norm_bwd": "norm_bwd_kernel (one workgroup per chain, reverse chunk sweep carrying dW)"}[dom]
    roof["ms_per_launch"] = t_dom
    roof["algorithmic_per_launch"] = {"flop": flops[dom]}
    return {
        "metric": "TTT layer with the Norm primitive, " + ("forward + backward" if with_bwd else "forward") +
                  " tokens/sec (1 GPU)",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{name}: B={cfg['B']} H={cfg['H']} T={cfg['T']} d={cfg['dk']} C={cfg['C']} "
                               f"loss={cfg['loss']} act=norm decay={cfg['decay']}, {cfg['dtype']} I/O",
                   "global_batch": cfg["B"], "seq_len": cfg["T"], "parallelism": "single-gpu"},
        "kernels": kernels,
        "algorithmic": {"gflop": (f_fwd + (f_bwd if with_bwd else 0)) / 1e9},
        "roofline": roof,
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_norm(name),
    }


def cpu_baseline_norm(name, budget_s=25.0):
    """The fp64 oracle of the Linear -> Norm forward + backward over whole chains."""
    from chunkwise_weight_recurrence_amd import workloads as wl
    from oracle import norm_chunk_backward, norm_chunk_forward
    inp = wl.make_ttt_inputs(name)
    cfg = inp["cfg"]
    done, t_total = 0, 0.0
    for ch in [(b, h) for b in range(cfg["B"]) for h in range(cfg["H"])]:
        s = wl.select_chains(inp, [ch])
        t0 = time.perf_counter()
        norm_chunk_forward(s["q"], s["k"], s["v"], s["beta"], cfg["b"], cfg["C"], cfg["loss"], cfg["decay"],
                           s["gamma"], s["w0"])
        if cfg.get("bwd"):
            norm_chunk_backward(s["q"], s["k"], s["v"], s["beta"], cfg["b"], cfg["C"], s["d_o"], cfg["loss"],
                                cfg["decay"], s["gamma"], s["w0"])
        t_total += time.perf_counter() - t0
        done += 1
        if t_total > budget_s:
            break
    return dict(value=done * cfg["T"] / (cfg["H"] * t_total), unit="tokens/s", cores=_oracle_cores(), kind="oracle",
                sample=f"{done} of {cfg['B'] * cfg['H']} (b,h) chains of {name}, full T={cfg['T']}, "
                       f"{'forward + backward' if cfg.get('bwd') else 'forward'} in fp64 NumPy, {t_total:.2f} s; "
                       f"scaled by 1/H to layer tokens")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="1.45b-fwdbwd")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-L2/MALL run")
    ap.add_argument("--cpu-chains", type=int, default=8)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the (b, h) chains shard over GPUs without communication; see DESIGN.md).",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.workload.startswith("inplace"):
        bench_inplace(args)
        return
    from chunkwise_weight_recurrence_amd import workloads as wl0
    if args.workload in wl0.MLP_WORKLOADS:
        bench_mlp(args)
        return

    import torch
    from chunkwise_weight_recurrence_amd import binding as B
    from chunkwise_weight_recurrence_amd import workloads as wl
    from chunkwise_weight_recurrence_amd.layer import TTTLayerBuffers

    name = args.workload
    inp = wl.make_ttt_inputs(name)
    cfg = inp["cfg"]
    with_bwd = bool(cfg.get("bwd", True))
    bufs = TTTLayerBuffers(inp, device="cuda", with_bwd=with_bwd)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step():
        bufs.forward()
        if with_bwd:
            bufs.backward()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # (1) the headline: K steps, per-kernel timer off
    timing = run_timed(torch, step, args.steps, stream)
    timing["kernel_timer"] = "off"
    ms_per_step = timing["mean_ms"]
    tokens = cfg["B"] * cfg["T"]
    value = tokens / (ms_per_step / 1e3)
    # (2) per-kernel device time: K more steps with the library's timer on
    B.ttt_timing_enable(True)
    run_timed(torch, step, args.steps, stream)
    B.ttt_timing_enable(False)
    kernels = {}
    for kid in B.Kernel:
        total, n = B.ttt_timing_read(kid)
        if n:
            kernels[kid.name.lower()] = {"ms_per_launch": total / n, "launches": n}
    # (3) cold L2 / MALL: a 512 MiB write before every step
    cold = None
    if not args.no_cold:
        flush_buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        cold = run_timed(torch, step, min(args.steps, 20), stream, flush=flush_buf.zero_)
        cold["flush_bytes"] = FLUSH_BYTES
        del flush_buf
    # (4) the same step with the backward recomputing each chunk's forward
    # intermediates instead of reading the forward's saved context
    recompute = None
    if with_bwd and bufs.saved is not None:
        rb = TTTLayerBuffers(inp, device="cuda", with_bwd=True, saved=False)

        def step_rc():
            rb.forward()
            rb.backward()

        for _ in range(args.warmup):
            step_rc()
        recompute = run_timed(torch, step_rc, min(args.steps, 20), stream)
        recompute["kernel_timer"] = "off"
        recompute["saved_context_bytes"] = int(bufs.saved.numel())
        del rb
    if cfg["act"] == "norm":
        out = norm_bench_line(args, name, cfg, kernels, ms_per_step, value, with_bwd)
        out["timing"] = timing
        out["cold_l2"] = cold
        print(json.dumps(out), flush=True)
        return
    work = algorithmic_work(cfg)
    flop = work["flop_fwd"] + (work["flop_bwd"] if with_bwd else 0)
    byts = work["bytes_fwd"] + (work["bytes_bwd"] if with_bwd else 0)
    mfma_util = flop / (ms_per_step / 1e3) / (PEAK_BF16_TFLOPS * 1e12)
    # the dominant kernel (largest device time per step), priced against the
    # roofline its algorithmic intensity puts it on
    per_kernel = kernel_work(cfg)
    timed = {k: v for k, v in kernels.items() if k in per_kernel}
    if not timed:
        raise RuntimeError("none of the layer's kernels ran")
    dom = max(timed, key=lambda k: timed[k]["ms_per_launch"] * timed[k]["launches"])
    t_dom = timed[dom]["ms_per_launch"]
    f_th, b_th = per_kernel[dom]
    f_dom = f_th * work["token_heads"]
    b_dom = b_th * work["token_heads"]
    kname = (KERNEL_NAMES_VECTOR if cfg["decay"] == "vector" else {}).get(dom, KERNEL_NAMES[dom])
    generic = dom.startswith(("generic", "norm"))
    if generic:
        # fp32 on the VALU (generic) or the fp32 matrix cores (the row path): the
        # ridge is the fp32 peak (the same 157.3 TFLOP/s for both) over the HBM peak
        ridge = PEAK_FP32_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
        compute = dict(bound="alu" if dom.startswith("generic") else "mfma", peak=PEAK_FP32_TFLOPS)
    else:
        ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
        compute = dict(bound="mfma", peak=PEAK_BF16_TFLOPS)
    hbm_gbs = b_dom / (t_dom / 1e3) / 1e9
    if f_dom / b_dom < ridge:
        roof = dict(bound="hbm", achieved=hbm_gbs, peak=PEAK_HBM_GBS, unit="GB/s")
    else:
        roof = dict(bound=compute["bound"], achieved=f_dom / (t_dom / 1e3) / 1e12, peak=compute["peak"],
                    unit="TFLOP/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = counter_traffic(kname, name)
    roof["kernel"] = kname
    roof["ms_per_launch"] = t_dom
    roof["algorithmic_per_launch"] = {"bytes": b_dom, "flop": f_dom}
    roof["hbm_achieved_gbs"] = hbm_gbs
    if generic:
        chains = cfg["B"] * cfg["H"]
        wgs = chains * max(1, cfg['dv'] // 32) if dom.startswith("generic") else chains
        roof["limit"] = (f"latency: {chains} chain(s) of {math.ceil(cfg['T'] / cfg['C'])} chunks run one chunk "
                         f"after another on {wgs} workgroup(s) of the 256 CUs; "
                         f"{b_dom / 1e6:.2f} MB at 8 TB/s would take {b_dom / 8e12 * 1e6:.2f} us and "
                         f"{f_dom / 1e6:.1f} MFLOP at the fp32 peak {f_dom / 157.3e12 * 1e6:.2f} us")

    out = {
        "metric": METRIC if with_bwd else "TTT-layer fwd tokens/sec (1 GPU); MFMA util %",
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
        "kernels": kernels,
        "algorithmic": {"gflop": flop / 1e9, "gbytes": byts / 1e9,
                        "hbm_frac_whole_step": byts / (ms_per_step / 1e3) / (PEAK_HBM_GBS * 1e9)},
        "timing": timing,
        "cold_l2": cold,
        "recompute": recompute,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        chains = [(b, h) for b in range(cfg["B"]) for h in range(cfg["H"])][:max(1, args.cpu_chains)]
        out["cpu_baseline"] = cpu_baseline(name, chains, token_loop=(cfg["B"] * cfg["H"] * cfg["T"] <= 4096))
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
