"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle, compare."""
import numpy as np

from chunkwise_weight_recurrence_amd import workloads as wl

# max |gpu - oracle| / max |oracle|, per output tensor
TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if not np.all(np.isfinite(got)):
        return float("inf")
    scale = float(np.abs(ref).max())
    if scale == 0.0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max()) / scale


def gpu_run(inp, bwd=None, d_wfinal=None, saved=True):
    """Run ttt_chunk_fwd (and ttt_chunk_bwd) on cuda:0; return float64 numpy outputs.

    saved=True passes the library's saved context from the forward to the
    backward (when the problem has one); saved=False makes the backward
    recompute the forward's chunk intermediates."""
    import torch
    from chunkwise_weight_recurrence_amd.layer import TTTLayerBuffers, to_f64, to_device
    bufs = TTTLayerBuffers(inp, device="cuda", with_bwd=bwd, saved=saved)
    bufs.forward()
    out = dict(O=bufs.o, W_T=bufs.w_final, ckpt=bufs.w_ckpt)
    if bufs.has_bwd:
        dwf = to_device(np.ascontiguousarray(d_wfinal, dtype=np.float32)) if d_wfinal is not None else None
        bufs.backward(d_wfinal=dwf)
        out.update(dq=bufs.dq, dk=bufs.dk, dv=bufs.dv, dbeta=bufs.dbeta, dw0=bufs.dw0)
        if bufs.dgamma is not None:
            out["dgamma"] = bufs.dgamma
        if bufs.dlog_a is not None:
            out["dlog_a"] = bufs.dlog_a
    torch.cuda.synchronize()
    return {k: to_f64(v) for k, v in out.items()}


def oracle_run(inp, bwd=None, d_wfinal=None):
    from oracle import chunk_backward, chunk_forward
    cfg = inp["cfg"]
    kw = wl.oracle_kwargs(inp)
    O, WT, ck = chunk_forward(inp["q"], inp["k"], inp["v"], inp["beta"], cfg["b"], cfg["C"],
                              return_ckpt=True, **kw)
    out = dict(O=O, W_T=WT, ckpt=ck)
    if bwd if bwd is not None else cfg.get("bwd", False):
        g = chunk_backward(inp["q"], inp["k"], inp["v"], inp["beta"], cfg["b"], cfg["C"], inp["d_o"],
                           d_wT=d_wfinal, **kw)
        out.update(dq=g["dq"], dk=g["dk"], dv=g["dv"], dbeta=g["dbeta"], dw0=g["dw0"])
        if g["dgamma"] is not None:
            out["dgamma"] = g["dgamma"]
        if g["dlog_a"] is not None:
            out["dlog_a"] = g["dlog_a"]
    return out


def compare(got, ref, dtype, keys=None, tol=None):
    tol = TOL[dtype] if tol is None else tol
    errs = {}
    for k in (keys or ref.keys()):
        errs[k] = rel_err(got[k], ref[k])
    bad = {k: e for k, e in errs.items() if not e <= tol}
    return errs, bad


def small_cfg(dtype, loss, act, decay, B=2, H=2, T=300, dk=64, dv=64, C=64, bwd=True, b=-2.0,
              w0="normal"):
    return dict(B=B, H=H, T=T, dk=dk, dv=dv, C=C, dtype=dtype, loss=loss, act=act, decay=decay,
                b=b, gamma="sigmoid_u36", w0=w0, bwd=bwd, seed=4242)
