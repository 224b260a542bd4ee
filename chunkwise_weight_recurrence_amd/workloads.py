"""Seeded synthetic workloads for the chunkwise TTT layer and the In-Place update.

This module only draws random inputs and casts them to the I/O precision.  It
holds none of the layer's arithmetic, so that the fp64 oracle and the HIP
path see the same input values without sharing any computation.

Shapes and distributions follow the workloads the Modular TTT and In-Place
TTT summary pages describe (160M / 410M / 1.45B-shaped layers, chunk 256;
In-Place d_model 2560, d_ff 9728, chunk 1024).  Everything is synthetic.

bf16 values are produced by round-to-nearest-even of the fp32 value; both
sides receive the identical bits (``*_bits`` as uint16) and the oracle gets
them widened exactly to float64.
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# The workload table
# --------------------------------------------------------------------------

WORKLOADS = {
    # Tiny forward that the oracle finishes in well under a second.
    "tiny-fwd-f32": dict(B=1, H=1, T=1024, dk=64, dv=64, C=256, dtype="f32", loss="mse",
                         act="none", decay="scalar", b=-4.0, gamma="const", w0="zeros",
                         bwd=False, seed=1000),
    # 410M-shaped layer, forward: MSE, linear, per-head scalar decay.
    "410m-fwd": dict(B=8, H=8, T=2048, dk=128, dv=128, C=256, dtype="bf16", loss="mse",
                     act="none", decay="scalar", b=-4.0, gamma="sigmoid_u36", w0="normal",
                     bwd=False, seed=1001),
    # 410M-shaped single-nonlinearity variant, forward + outer backward.
    "410m-silu-fwdbwd": dict(B=8, H=8, T=2048, dk=128, dv=128, C=256, dtype="bf16",
                             loss="mse", act="silu", decay="scalar", b=-4.0,
                             gamma="sigmoid_u36", w0="normal", bwd=True, seed=1002),
    # 1.45B-shaped layer, forward + backward: IP loss, SiLU, per-token vector decay.
    "1.45b-fwdbwd": dict(B=4, H=16, T=4096, dk=128, dv=128, C=256, dtype="bf16", loss="ip",
                         act="silu", decay="vector", b=-4.0, gamma=None, w0="normal",
                         bwd=True, seed=1003),
    # The inner-product linear variant of the 1.45B layer (no act), one long
    # sequence, forward + backward: the chunk-parallel path's case (B * H = 16 chains).
    "1.45b-iplin-32k": dict(B=1, H=16, T=32768, dk=128, dv=128, C=256, dtype="bf16", loss="ip",
                            act="none", decay="vector", b=-4.0, gamma=None, w0="normal",
                            bwd=True, seed=1005),
    # The Norm primitive as the fast net's act (Linear -> per-token normalisation) on the
    # 160M layer shape of the two-layer workloads: 12 heads of 64, chunk 256, forward + backward.
    "160m-norm-fwdbwd": dict(B=8, H=12, T=2048, dk=64, dv=64, C=256, dtype="bf16", loss="mse",
                             act="norm", decay="scalar", b=-4.0, gamma="const", gamma_value=0.99,
                             w0="normal", bwd=True, seed=1007),
}

# Two-layer fast net (TTT-MLP), forward: the 160M model's layer shape read as
# 12 heads of width 64 (d_model 768), hidden width 4 x 64 = 256, chunk 256,
# scalar decay 0.99, Gaussian fast-weight init std 0.02 (both layers).
MLP_WORKLOADS = {
    "160m-mlp-fwd": dict(B=8, H=12, T=2048, dk=64, dh=256, dv=64, C=256, dtype="bf16", loss="mse",
                         act="silu", decay="scalar", b=-4.0, gamma_value=0.99, w0="normal", seed=1006),
    # The same layer, forward then the outer backward (dO ~ N(0, 1) bf16, drawn with seed + 1).
    "160m-mlp-fwdbwd": dict(B=8, H=12, T=2048, dk=64, dh=256, dv=64, C=256, dtype="bf16", loss="mse",
                            act="silu", decay="scalar", b=-4.0, gamma_value=0.99, w0="normal", seed=1006, bwd=True),
}

INPLACE_WORKLOADS = {
    "inplace-wdown": dict(B=1, T=32768, d_model=2560, d_ff=9728, C=1024, eta=1e-3, seed=1004),
    # The same inputs, forward then the W_down backward (dO ~ N(0, 1), dW_T ~ N(0, 1)).
    "inplace-wdown-fwdbwd": dict(B=1, T=32768, d_model=2560, d_ff=9728, C=1024, eta=1e-3, seed=1004, bwd=True),
    # The same inputs with the long-context safeguards: update clipping at the
    # page's tau = 1e-5 and four packed documents of mixed lengths (none a
    # multiple of C, so every document ends on a short chunk).
    "inplace-wdown-guarded": dict(B=1, T=32768, d_model=2560, d_ff=9728, C=1024, eta=1e-3, seed=1004,
                                  clip_tau=1e-5, doc_lens=(9000, 7000, 12000, 4768)),
    # The guarded inputs, forward then the guarded backward (the clip factor differentiated).
    "inplace-wdown-guarded-fwdbwd": dict(B=1, T=32768, d_model=2560, d_ff=9728, C=1024, eta=1e-3, seed=1004,
                                         clip_tau=1e-5, doc_lens=(9000, 7000, 12000, 4768), bwd=True),
}


def inplace_doc_starts(cfg):
    """(per-sequence start lists, flat positions b * T + t) of the documents of
    ``cfg["doc_lens"]`` (the same packing in every sequence; none: no starts)."""
    lens = cfg.get("doc_lens")
    T, B = cfg["T"], cfg["B"]
    if not lens:
        return [[] for _ in range(B)], []
    assert sum(lens) == T, "document lengths must fill the sequence"
    starts = list(np.cumsum(lens)[:-1].astype(int))
    per_seq = [list(map(int, starts)) for _ in range(B)]
    flat = [b * T + t for b in range(B) for t in per_seq[b]]
    return per_seq, flat


# --------------------------------------------------------------------------
# Precision casts
# --------------------------------------------------------------------------

def bf16_bits(x):
    """Round float values to bfloat16 (nearest-even); returns the uint16 bit patterns."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f64(bits):
    """Widen bfloat16 bit patterns exactly to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def _cast(x, dtype):
    """Return (values as float64, device payload as numpy array) for the I/O dtype."""
    if dtype == "bf16":
        bits = bf16_bits(x)
        return bf16_to_f64(bits), bits
    f = np.asarray(x, dtype=np.float32)
    return f.astype(np.float64), f


def _l2_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _push_from_zero(x, margin):
    """x moved away from zero by `margin` (x + margin sign(x)); margin 0 leaves it as drawn.
    Test inputs for the L1 loss use it so that no target sits near a prediction."""
    return x + margin * np.sign(x) if margin else x


def _log_sigmoid(z):
    # log(sigmoid(z)) = -log(1 + exp(-z)), evaluated stably for both signs
    return np.minimum(z, 0.0) - np.log1p(np.exp(-np.abs(z)))


# --------------------------------------------------------------------------
# TTT layer inputs
# --------------------------------------------------------------------------

def make_ttt_inputs(name_or_cfg, seed=None, **overrides):
    """Draw one seeded input set.

    Draw order (fixed): Q, K, V, beta, decay, W0, dO.  Q and K rows are
    L2-normalised before the cast.  Returns a dict with the config and, per
    tensor, float64 values (``q`` ...) plus the device payload (``q_dev`` ...:
    uint16 bf16 bits or float32).
    """
    cfg = dict(WORKLOADS[name_or_cfg]) if isinstance(name_or_cfg, str) else dict(name_or_cfg)
    cfg.update(overrides)
    if seed is None:
        seed = cfg.get("seed", 0)
    rng = np.random.Generator(np.random.PCG64(seed))
    B, H, T, dk, dv = cfg["B"], cfg["H"], cfg["T"], cfg["dk"], cfg["dv"]
    dt = cfg["dtype"]
    out = dict(cfg=cfg)
    q = _l2_rows(rng.standard_normal((B, H, T, dk)))
    k = _l2_rows(rng.standard_normal((B, H, T, dk)))
    v = _push_from_zero(rng.standard_normal((B, H, T, dv)), cfg.get("v_margin", 0.0))
    beta = rng.standard_normal((B, H, T))
    for nm, arr in (("q", q), ("k", k), ("v", v)):
        out[nm], out[nm + "_dev"] = _cast(arr, dt)
    out["beta"], out["beta_dev"] = _cast(beta, "f32")
    out["gamma"] = out["gamma_dev"] = None
    out["log_a"] = out["log_a_dev"] = None
    if cfg["decay"] == "scalar":
        if cfg.get("gamma") == "sigmoid_u36":
            u = rng.uniform(3.0, 6.0, size=H)
            g = 1.0 / (1.0 + np.exp(-u))
        else:
            g = np.full(H, cfg.get("gamma_value", 0.99))
        out["gamma"], out["gamma_dev"] = _cast(g, "f32")
    elif cfg["decay"] == "vector":
        zmean = cfg.get("z_mean", 4.0)
        z = rng.normal(zmean, 1.0, size=(B, H, T, dk))
        out["log_a"], out["log_a_dev"] = _cast(_log_sigmoid(z), "f32")
    if cfg.get("w0", "zeros") == "normal":
        w = np.broadcast_to(rng.normal(0.0, 0.02, size=(1, H, dk, dv)), (B, H, dk, dv))
        out["w0"], out["w0_dev"] = _cast(np.ascontiguousarray(w), "f32")
    else:
        out["w0"] = np.zeros((B, H, dk, dv))
        out["w0_dev"] = None
    if cfg.get("bwd", False):
        out["d_o"], out["d_o_dev"] = _cast(rng.standard_normal((B, H, T, dv)), dt)
    return out


def oracle_kwargs(inp):
    """Keyword arguments for the oracle's chunk_forward / chunk_backward."""
    cfg = inp["cfg"]
    return dict(loss=cfg["loss"], act=cfg["act"], decay=cfg["decay"], gamma=inp["gamma"],
                log_a=inp["log_a"], w0=inp["w0"])


def select_chains(inp, chains):
    """Restrict an input set to a list of (b, h) chains, as a batch of 1 x len(chains)."""
    out = dict(inp)
    cfg = dict(inp["cfg"])
    bs = [c[0] for c in chains]
    hs = [c[1] for c in chains]
    for key in ("q", "k", "v", "beta", "log_a", "w0", "d_o"):
        if inp.get(key) is not None:
            out[key] = inp[key][bs, hs][None]
    if inp.get("gamma") is not None:
        out["gamma"] = inp["gamma"][hs]
    cfg.update(B=1, H=len(chains))
    out["cfg"] = cfg
    return out


# --------------------------------------------------------------------------
# Two-layer fast net (TTT-MLP) inputs
# --------------------------------------------------------------------------

def make_mlp_inputs(name_or_cfg, seed=None, **overrides):
    """Draw one seeded input set of the two-layer fast net.

    Draw order (fixed): Q, K, V, beta, W1_0, W2_0.  Q and K rows are
    L2-normalised before the cast; beta ~ N(0, 1); the initial weights are
    N(0, 0.02^2) per head, shared over the batch (w0 "normal"), or zero.
    gamma is the constant ``gamma_value`` per head (scalar decay).
    """
    cfg = dict(MLP_WORKLOADS[name_or_cfg]) if isinstance(name_or_cfg, str) else dict(name_or_cfg)
    cfg.update(overrides)
    if seed is None:
        seed = cfg.get("seed", 0)
    rng = np.random.Generator(np.random.PCG64(seed))
    B, H, T, dk, dh, dv = cfg["B"], cfg["H"], cfg["T"], cfg["dk"], cfg["dh"], cfg["dv"]
    dt = cfg["dtype"]
    out = dict(cfg=cfg)
    for nm, d in (("q", dk), ("k", dk)):
        out[nm], out[nm + "_dev"] = _cast(_l2_rows(rng.standard_normal((B, H, T, d))), dt)
    out["v"], out["v_dev"] = _cast(_push_from_zero(rng.standard_normal((B, H, T, dv)), cfg.get("v_margin", 0.0)), dt)
    out["beta"], out["beta_dev"] = _cast(rng.standard_normal((B, H, T)), "f32")
    out["gamma"] = out["gamma_dev"] = None
    if cfg["decay"] == "scalar":
        out["gamma"], out["gamma_dev"] = _cast(np.full(H, cfg.get("gamma_value", 0.99)), "f32")
    for nm, shp in (("w1_0", (dk, dh)), ("w2_0", (dh, dv))):
        if cfg.get("w0", "zeros") == "normal":
            w = np.broadcast_to(rng.normal(0.0, 0.02, size=(1, H) + shp), (B, H) + shp)
            out[nm], out[nm + "_dev"] = _cast(np.ascontiguousarray(w), "f32")
        else:
            out[nm] = np.zeros((B, H) + shp)
            out[nm + "_dev"] = None
    return out


def make_mlp_grads(cfg, seed):
    """Seeded upstream gradient of the two-layer forward's output: dO ~ N(0, 1) in the I/O dtype."""
    rng = np.random.Generator(np.random.PCG64(seed))
    d_o = rng.standard_normal((cfg["B"], cfg["H"], cfg["T"], cfg["dv"]))
    vals, dev = _cast(d_o, cfg["dtype"])
    return dict(d_o=vals, d_o_dev=dev)


def select_mlp_chains(inp, chains):
    """Restrict a two-layer input set to a list of (b, h) chains, as a batch of 1 x len(chains)."""
    out = dict(inp)
    cfg = dict(inp["cfg"])
    bs = [c[0] for c in chains]
    hs = [c[1] for c in chains]
    for key in ("q", "k", "v", "beta", "w1_0", "w2_0"):
        out[key] = inp[key][bs, hs][None]
    if inp.get("gamma") is not None:
        out["gamma"] = inp["gamma"][hs]
    cfg.update(B=1, H=len(chains))
    out["cfg"] = cfg
    return out


# --------------------------------------------------------------------------
# In-Place TTT inputs
# --------------------------------------------------------------------------

def make_inplace_inputs(name_or_cfg, seed=None, matmul=None, **overrides):
    """Seeded inputs of the In-Place W_down update.

    Z = SiLU(H W_gate^T) (.) (H W_up^T) with H ~ N(0,1) (bf16), W_up, W_gate ~
    N(0, 0.02^2); V_hat = Conv1D_4(X0) W_target with X0 ~ N(0,1), a depthwise
    causal-in-reverse kernel of 4 taps reading x_t .. x_{t+3} (zero past the
    end), taps ~ N(0, 1/4), W_target ~ N(0, 0.02^2), which gives V_hat about unit
    scale at d_model = 2560; W_down0 ~ N(0, 0.02^2) fp32.  Z and V_hat are cast
    to bf16.

    ``matmul(a, b)`` may be supplied to form the two large products faster
    (for example on a device); it must return float32 numpy arrays.
    """
    cfg = dict(INPLACE_WORKLOADS[name_or_cfg]) if isinstance(name_or_cfg, str) \
        else dict(name_or_cfg)
    cfg.update(overrides)
    if seed is None:
        seed = cfg.get("seed", 0)
    rng = np.random.Generator(np.random.PCG64(seed))
    B, T, dm, dff = cfg["B"], cfg["T"], cfg["d_model"], cfg["d_ff"]
    mm = matmul or (lambda a, b: np.asarray(a, np.float32) @ np.asarray(b, np.float32))
    Hs = bf16_to_f64(bf16_bits(rng.standard_normal((B * T, dm), dtype=np.float32)))
    Hs = Hs.astype(np.float32)
    w_up = (rng.standard_normal((dm, dff), dtype=np.float32) * np.float32(0.02))
    w_gate = (rng.standard_normal((dm, dff), dtype=np.float32) * np.float32(0.02))
    gate = mm(Hs, w_gate)
    up = mm(Hs, w_up)
    del Hs
    z = (gate / (1.0 + np.exp(-gate))) * up
    del gate, up
    x0 = rng.standard_normal((B, T, dm), dtype=np.float32)
    taps = rng.normal(0.0, 0.5, size=(4, dm)).astype(np.float32)
    conv = np.zeros_like(x0)
    for j in range(4):
        conv[:, :T - j] += taps[j] * x0[:, j:]
    w_target = rng.standard_normal((dm, dm), dtype=np.float32) * np.float32(0.02)
    vhat = mm(conv.reshape(B * T, dm), w_target).reshape(B, T, dm)
    w0 = (rng.standard_normal((B, dm, dff), dtype=np.float32) * np.float32(0.02))
    out = dict(cfg=cfg)
    out["z_dev"] = bf16_bits(z.reshape(B, T, dff))
    out["vhat_dev"] = bf16_bits(vhat)
    out["w0_dev"] = w0
    return out


def make_inplace_grads(cfg, seed, with_dwfinal=True):
    """Seeded upstream gradients for the In-Place backward: dO ~ N(0, 1) (bf16 bits,
    [B, T, d_model]) and, optionally, dW_final ~ N(0, 1) ([B, d_model, d_ff] fp32)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B, T, dm, dff = cfg["B"], cfg["T"], cfg["d_model"], cfg["d_ff"]
    out = {"d_o_dev": bf16_bits(rng.standard_normal((B, T, dm), dtype=np.float32))}
    out["d_wfinal_dev"] = rng.standard_normal((B, dm, dff), dtype=np.float32) if with_dwfinal else None
    return out


def inplace_values(inp, key):
    """float64 values of a bf16 payload of :func:`make_inplace_inputs`."""
    return bf16_to_f64(inp[key])
