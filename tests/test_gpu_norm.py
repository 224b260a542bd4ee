"""GPU parity of the Linear -> Norm fast net (TTT_ACT_NORM: forward and analytic
backward through ttt_chunk_fwd / ttt_chunk_bwd) against the fp64 oracle
(``oracle.norm_chunk_forward`` / ``norm_chunk_backward``).

Bar: max |gpu - oracle| / max |oracle| per output, 1e-4 for fp32 I/O and 2e-2 for
bf16 I/O (fp32 arithmetic either way).  The L1 loss's sign decisions get a checked
margin: its targets are drawn at least 5 away from zero, beyond the normalised
predictions.
"""
import itertools

import numpy as np
import pytest

from chunkwise_weight_recurrence_amd import workloads as wl
from tests.parity_utils import compare, gpu_run

pytestmark = pytest.mark.gpu


def _oracle(inp, d_wfinal):
    from oracle import norm_chunk_backward, norm_chunk_forward
    cfg = inp["cfg"]
    args = (inp["q"], inp["k"], inp["v"], inp["beta"], cfg["b"], cfg["C"])
    O, WT, ck = norm_chunk_forward(*args, cfg["loss"], cfg["decay"], inp["gamma"], inp["w0"], return_ckpt=True)
    g = norm_chunk_backward(*args, inp["d_o"], cfg["loss"], cfg["decay"], inp["gamma"], inp["w0"], d_wfinal)
    out = dict(O=O, W_T=WT, ckpt=np.stack(ck, axis=2), dq=g["dq"], dk=g["dk"], dv=g["dv"], dbeta=g["dbeta"],
               dw0=g["dw0"])
    if cfg["decay"] == "scalar":
        out["dgamma"] = g["dgamma"]
    return out


def _margin(inp):
    """Smallest |N(K W_i) - V| over the chunks' train views (oracle weights)."""
    from oracle import norm_chunk_forward
    from oracle.norm_oracle import norm_f
    cfg = inp["cfg"]
    C, T = cfg["C"], cfg["T"]
    _, _, ck = norm_chunk_forward(inp["q"], inp["k"], inp["v"], inp["beta"], cfg["b"], C, cfg["loss"],
                                  cfg["decay"], inp["gamma"], inp["w0"], return_ckpt=True)
    return min(float(np.abs(norm_f(inp["k"][:, :, s0:s0 + C] @ ck[i])[0] - inp["v"][:, :, s0:s0 + C]).min())
               for i, s0 in enumerate(range(0, T, C)))


def _cfg(dtype, loss, decay, **kw):
    base = dict(B=2, H=2, T=300, dk=64, dv=64, C=64, dtype=dtype, loss=loss, act="norm", decay=decay, b=-3.0,
                gamma="sigmoid_u36", w0="normal", bwd=True, seed=77)
    if loss == "l1":
        base["v_margin"] = 5.0
    base.update(kw)
    return base


def _check(name, cfg):
    inp = wl.make_ttt_inputs(cfg)
    if cfg["loss"] == "l1":
        assert _margin(inp) > 0.05
    dwf = np.random.default_rng(9).standard_normal(inp["w0"].shape).astype(np.float32)
    got = gpu_run(inp, d_wfinal=dwf)
    ref = _oracle(inp, dwf.astype(np.float64))
    errs, bad = compare(got, ref, cfg["dtype"])
    print(f"[parity] {name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert not bad, f"{name}: over tolerance {bad}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("loss,decay", list(itertools.product(["mse", "ip", "l1"], ["none", "scalar"])))
def test_norm_fwd_bwd(dtype, loss, decay):
    _check(f"norm {dtype} {loss} {decay}", _cfg(dtype, loss, decay))


@pytest.mark.parametrize("shape", [
    dict(B=1, H=3, T=250, dk=40, dv=24, C=48),     # ragged widths and a short last chunk
    dict(B=1, H=2, T=700, dk=128, dv=96, C=256),   # several row tiles per chunk; a row spans two wave passes
    dict(B=1, H=1, T=130, dk=64, dv=256, C=128),   # the widest rows
    dict(B=1, H=2, T=33, dk=8, dv=8, C=1),         # token-level chunks
    dict(B=1, H=1, T=1, dk=64, dv=64, C=256),      # one token
])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_norm_edge_shapes(shape, dtype):
    _check(f"norm edge {shape} {dtype}", _cfg(dtype, "mse", "scalar", seed=78, **shape))


def test_norm_vector_decay_is_unsupported():
    from chunkwise_weight_recurrence_amd import binding as B
    with pytest.raises(B.TTTError):
        B.ttt_workspace_size(B.make_desc(1, 1, 64, 64, 64, 64, act="norm", decay="vector"), B.ENTRY_FWD)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("act,decay", list(itertools.product(["none", "silu", "gelu", "norm"], ["none", "scalar"])))
def test_rmse_fwd_bwd(dtype, act, decay):
    """The RMSE loss (row-coupled, so on the one-workgroup-per-chain path) with every act."""
    cfg = _cfg(dtype, "rmse", decay, act=act, seed=79)
    if act == "norm":
        _check(f"rmse {dtype} {act} {decay}", cfg)
        return
    inp = wl.make_ttt_inputs(cfg)
    from oracle import chunk_backward, chunk_forward
    kw = wl.oracle_kwargs(inp)
    dwf = np.random.default_rng(9).standard_normal(inp["w0"].shape).astype(np.float32)
    O, WT, ck = chunk_forward(inp["q"], inp["k"], inp["v"], inp["beta"], cfg["b"], cfg["C"], return_ckpt=True, **kw)
    g = chunk_backward(inp["q"], inp["k"], inp["v"], inp["beta"], cfg["b"], cfg["C"], inp["d_o"],
                       d_wT=dwf.astype(np.float64), **kw)
    ref = dict(O=O, W_T=WT, ckpt=ck, dq=g["dq"], dk=g["dk"], dv=g["dv"], dbeta=g["dbeta"], dw0=g["dw0"])
    if decay == "scalar":
        ref["dgamma"] = g["dgamma"]
    got = gpu_run(inp, d_wfinal=dwf)
    errs, bad = compare(got, ref, dtype)
    print(f"[parity] rmse {dtype} {act} {decay}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert not bad, bad


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_norm_many_chunks_query_per_chunk(dtype):
    """256 (chain, chunk) items: the query view runs one workgroup per chunk (fewer
    items split each chunk's rows over workgroups, as every other case here does);
    forward and backward over every chain against the oracle."""
    _check(f"norm {dtype} 256 chunks", _cfg(dtype, "mse", "scalar", B=2, H=16, T=2048, C=256))


@pytest.mark.parametrize("dtype,act,loss", [("f32", "none", "mse"), ("bf16", "norm", "rmse")])
def test_row_forward_without_caller_checkpoints(dtype, act, loss):
    """The row path's query view reads each chunk's start state from the caller's
    checkpoint buffer when one is given and from the workspace otherwise: both give
    the oracle's O and W_T, and the same bits."""
    import torch
    from chunkwise_weight_recurrence_amd import binding as B
    from chunkwise_weight_recurrence_amd.layer import TTTLayerBuffers, to_f64
    from tests.parity_utils import oracle_run
    cfg = dict(B=1, H=3, T=700, dk=64, dv=64, C=256, dtype=dtype, loss=loss, act=act, decay="scalar", b=-3.0,
               gamma="sigmoid_u36", w0="normal", bwd=False, seed=77)
    inp = wl.make_ttt_inputs(cfg)
    with_ck = gpu_run(inp, bwd=False)
    bufs = TTTLayerBuffers(inp, device="cuda", with_bwd=False)
    bufs.o.zero_()
    B.ttt_chunk_fwd(bufs.desc, bufs.q, bufs.k, bufs.v, bufs.beta, bufs.gamma, bufs.log_a, bufs.w0, bufs.o,
                    bufs.w_final, None, None, bufs.ws_fwd)
    torch.cuda.synchronize()
    got = dict(O=to_f64(bufs.o), W_T=to_f64(bufs.w_final))
    if act == "norm" or loss == "rmse":
        from oracle import norm_chunk_forward
        from oracle.ttt_oracle import chunk_forward
        args = (inp["q"], inp["k"], inp["v"], inp["beta"], cfg["b"], cfg["C"])
        if act == "norm":
            O, WT = norm_chunk_forward(*args, loss, "scalar", inp["gamma"], inp["w0"])
        else:
            O, WT = chunk_forward(*args, **wl.oracle_kwargs(inp))
        ref = dict(O=O, W_T=WT)
    else:
        ref = oracle_run(inp, bwd=False)
    errs, bad = compare(got, ref, dtype, keys=["O", "W_T"])
    print(f"row fwd without checkpoints {dtype}/{act}/{loss}:", {k: f"{v:.1e}" for k, v in errs.items()}, flush=True)
    assert not bad, bad
    assert np.array_equal(got["O"], with_ck["O"]) and np.array_equal(got["W_T"], with_ck["W_T"])
