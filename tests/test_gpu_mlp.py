"""GPU parity of the two-layer fast net (TTT-MLP) forward through the C ABI
against the fp64 oracle (``oracle.mlp_chunk_forward``).

Bar: max |gpu - oracle| / max |oracle| <= 1e-4 per output for fp32 I/O and
<= 2e-2 for bf16 I/O (the arithmetic is fp32 either way; bf16 rounds the
inputs, which both sides share, and the output).  Shapes span several 64 x 64
tiles, ragged tiles (d_h, d_k, d_v and C not multiples of 64) and a short last
chunk.
"""
import numpy as np
import pytest

from chunkwise_weight_recurrence_amd import workloads as wl
from tests.parity_utils import compare

pytestmark = pytest.mark.gpu


def _gpu(inp):
    import torch
    from chunkwise_weight_recurrence_amd.layer import MlpBuffers, to_f64
    bufs = MlpBuffers(inp)
    bufs.forward()
    torch.cuda.synchronize()
    return dict(O=to_f64(bufs.o), W1=to_f64(bufs.w1), W2=to_f64(bufs.w2))


def _oracle(inp):
    from oracle import mlp_chunk_forward
    cfg = inp["cfg"]
    O, W1, W2 = mlp_chunk_forward(inp["q"], inp["k"], inp["v"], inp["beta"], cfg["b"], cfg["C"], cfg["loss"],
                                  cfg["act"], cfg["decay"], inp["gamma"], inp["w1_0"], inp["w2_0"])
    return dict(O=O, W1=W1, W2=W2)


def _check(name, inp):
    got, ref = _gpu(inp), _oracle(inp)
    errs, bad = compare(got, ref, inp["cfg"]["dtype"])
    print(f"[parity] {name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert not bad, f"{name}: over tolerance {bad}"


BASE = dict(B=2, H=2, T=300, dk=64, dh=256, dv=64, C=64, b=-3.0, gamma_value=0.97, w0="normal", seed=61)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("loss", ["mse", "ip", "rmse"])
@pytest.mark.parametrize("act", ["none", "silu", "gelu"])
@pytest.mark.parametrize("decay", ["none", "scalar"])
def test_mlp_combos(dtype, loss, act, decay):
    # the linear IP case grows exponentially over the chunks at b = -3 (each layer's write scales with
    # the other layer); b = -4 keeps it bounded
    inp = wl.make_mlp_inputs(dict(BASE, dtype=dtype, loss=loss, act=act, decay=decay, b=-4.0 if loss == "ip" else -3.0))
    _check(f"mlp {dtype} {loss} {act} {decay}", inp)


def _mlp_l1_margin(inp):
    """Smallest |V_hat - V| over every chunk's train view, with the oracle's chunk-start
    weights (the forward run on each prefix)."""
    from oracle import mlp_chunk_forward
    from oracle.mlp_oracle import mlp_train_view
    cfg = inp["cfg"]
    C, T = cfg["C"], cfg["T"]
    m = np.inf
    for s0 in range(0, T, C):
        if s0 == 0:
            W1, W2 = inp["w1_0"], inp["w2_0"]
        else:
            _, W1, W2 = mlp_chunk_forward(inp["q"][:, :, :s0], inp["k"][:, :, :s0], inp["v"][:, :, :s0],
                                          inp["beta"][:, :, :s0], cfg["b"], C, cfg["loss"], cfg["act"], cfg["decay"],
                                          inp["gamma"], inp["w1_0"], inp["w2_0"])
        kc, vc = inp["k"][:, :, s0:s0 + C], inp["v"][:, :, s0:s0 + C]
        _, A, _, G2 = mlp_train_view(kc, vc, W1, W2, "mse", cfg["act"])  # MSE's G2 is V_hat - V
        m = min(m, float(np.abs(G2).min()))
    return m


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("act", ["none", "silu", "gelu"])
@pytest.mark.parametrize("decay", ["none", "scalar"])
def test_mlp_l1(dtype, act, decay):
    """L1 inner loss: targets drawn at least 1 away from zero, so every sign decision has a
    margin (checked first) far above fp32 rounding."""
    inp = wl.make_mlp_inputs(dict(BASE, dtype=dtype, loss="l1", act=act, decay=decay, b=-4.0, v_margin=1.0))
    assert _mlp_l1_margin(inp) > 0.05
    _check(f"mlp l1 {dtype} {act} {decay}", inp)


@pytest.mark.parametrize("shape", [
    dict(B=1, H=3, T=250, dk=40, dh=72, dv=24, C=48),      # every width ragged, short last chunk
    dict(B=1, H=1, T=700, dk=128, dh=300, dv=96, C=256),   # several row tiles per chunk, ragged d_h
    dict(B=2, H=1, T=97, dk=64, dh=1024, dv=64, C=100),    # the widest hidden layer, one short chunk
    dict(B=1, H=2, T=33, dk=8, dh=16, dv=8, C=1),          # token-level chunks
    dict(B=1, H=1, T=1, dk=64, dh=256, dv=64, C=256),      # one token
    dict(B=1, H=2, T=512, dk=256, dh=64, dv=256, C=128),   # wide keys and values, narrow hidden layer
])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mlp_edge_shapes(shape, dtype):
    inp = wl.make_mlp_inputs(dict(BASE, **shape, dtype=dtype, loss="mse", act="gelu", decay="scalar", seed=62))
    _check(f"mlp edge {shape} {dtype}", inp)


def test_mlp_zero_initial_state_f32():
    inp = wl.make_mlp_inputs(dict(BASE, dtype="f32", loss="mse", act="silu", decay="none", w0="zeros"))
    assert inp["w1_0_dev"] is None
    _check("mlp zero W0", inp)


def test_mlp_full_size_all_chains():
    """B 8, H 12, T 2048, d 64, d_h 256, C 256, bf16, MSE, SiLU, scalar decay: every chain."""
    inp = wl.make_mlp_inputs("160m-mlp-fwd")
    _check("mlp 160m-mlp-fwd (all 96 chains)", inp)


def test_mlp_repeat_is_deterministic():
    import torch
    from chunkwise_weight_recurrence_amd.layer import MlpBuffers
    inp = wl.make_mlp_inputs(dict(BASE, dtype="bf16", loss="mse", act="silu", decay="scalar"))
    bufs = MlpBuffers(inp)
    outs = []
    for _ in range(2):
        bufs.forward()
        torch.cuda.synchronize()
        outs.append((bufs.o.clone(), bufs.w1.clone(), bufs.w2.clone()))
    assert all(torch.equal(a, b) for a, b in zip(*outs))


def test_mlp_empty_sequence_passes_state_through():
    import torch
    from chunkwise_weight_recurrence_amd.layer import MlpBuffers, to_f64
    inp = wl.make_mlp_inputs(dict(BASE, T=0, dtype="f32", loss="mse", act="silu", decay="none"))
    bufs = MlpBuffers(inp)
    bufs.forward()
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(bufs.w1), inp["w1_0"]) and np.array_equal(to_f64(bufs.w2), inp["w2_0"])


# ---------------------------------------------------------------------------
# outer backward (ttt_mlp_chunk_bwd) against oracle.mlp_chunk_backward
# ---------------------------------------------------------------------------

def _upstream(inp, seed):
    cfg = inp["cfg"]
    rng = np.random.default_rng(seed)
    B, H, T, dk, dh, dv = (cfg[x] for x in ("B", "H", "T", "dk", "dh", "dv"))
    d_o = rng.standard_normal((B, H, T, dv))
    if cfg["dtype"] == "bf16":
        d_o = wl.bf16_to_f64(wl.bf16_bits(d_o))
    return d_o, rng.standard_normal((B, H, dk, dh)), rng.standard_normal((B, H, dh, dv))


def _gpu_bwd(inp, d_o, d1, d2, saved=True):
    import torch
    from chunkwise_weight_recurrence_amd.layer import MlpBuffers, to_f64
    bufs = MlpBuffers(inp, with_bwd=True, saved=saved)
    assert (bufs.saved is not None) == saved
    bufs.forward()
    dt = bufs.o.dtype
    t = lambda x, dtype: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype).cuda()
    bufs.backward(t(d_o, dt), t(d1, torch.float32), t(d2, torch.float32))
    torch.cuda.synchronize()
    out = dict(O=bufs.o, dq=bufs.dq, dk=bufs.dk, dv=bufs.dv, dbeta=bufs.dbeta, dw1_0=bufs.dw1, dw2_0=bufs.dw2)
    if bufs.dgamma is not None:
        out["dgamma"] = bufs.dgamma
    return {k: to_f64(v) for k, v in out.items()}


def _oracle_bwd(inp, d_o, d1, d2):
    from oracle import mlp_chunk_backward
    cfg = inp["cfg"]
    g = mlp_chunk_backward(inp["q"], inp["k"], inp["v"], inp["beta"], cfg["b"], cfg["C"], d_o, cfg["loss"],
                           cfg["act"], cfg["decay"], inp["gamma"], inp["w1_0"], inp["w2_0"], d1, d2)
    g["O"] = _oracle(inp)["O"]
    if cfg["decay"] != "scalar":
        g.pop("dgamma")
    return g


def _check_bwd(name, inp, seed=7, saved=True):
    d_o, d1, d2 = _upstream(inp, seed)
    got, ref = _gpu_bwd(inp, d_o, d1, d2, saved), _oracle_bwd(inp, d_o, d1, d2)
    if inp["cfg"]["loss"] == "l1":
        assert np.all(ref["dv"] == 0.0)
    errs, bad = compare(got, ref, inp["cfg"]["dtype"])
    print(f"[parity] {name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert not bad, f"{name}: over tolerance {bad}"


@pytest.mark.parametrize("saved", [True, False])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("loss", ["mse", "ip", "l1", "rmse"])
@pytest.mark.parametrize("act", ["none", "silu", "gelu"])
@pytest.mark.parametrize("decay", ["none", "scalar"])
def test_mlp_backward_combos(dtype, loss, act, decay, saved):
    """The backward from the forward's saved context and recomputing each chunk."""
    extra = dict(b=-4.0, v_margin=1.0) if loss == "l1" else dict(b=-4.0 if loss == "ip" else -3.0)
    inp = wl.make_mlp_inputs(dict(BASE, dtype=dtype, loss=loss, act=act, decay=decay, **extra))
    if loss == "l1":
        assert _mlp_l1_margin(inp) > 0.05
    _check_bwd(f"mlp bwd {dtype} {loss} {act} {decay} saved={saved}", inp, saved=saved)


@pytest.mark.parametrize("shape", [
    dict(B=1, H=3, T=250, dk=40, dh=72, dv=24, C=48),      # every width ragged, short last chunk
    dict(B=1, H=1, T=700, dk=128, dh=300, dv=96, C=256),   # several row tiles per chunk, ragged d_h
    dict(B=1, H=2, T=33, dk=8, dh=16, dv=8, C=1),          # token-level chunks
    dict(B=1, H=1, T=1, dk=64, dh=256, dv=64, C=256),      # one token
])
@pytest.mark.parametrize("dtype,saved", [("f32", True), ("bf16", True), ("bf16", False)])
def test_mlp_backward_edge_shapes(shape, dtype, saved):
    inp = wl.make_mlp_inputs(dict(BASE, **shape, dtype=dtype, loss="mse", act="gelu", decay="scalar", seed=63))
    _check_bwd(f"mlp bwd edge {shape} {dtype} saved={saved}", inp, saved=saved)


def test_mlp_backward_full_size_sampled_chains():
    """The 160M workload (B 8, H 12, T 2048, d_h 256, C 256): the whole batch runs on the GPU;
    chains are independent, so three of them are compared with the oracle run on those alone."""
    inp = wl.make_mlp_inputs("160m-mlp-fwd")
    d_o, d1, d2 = _upstream(inp, 11)
    got = _gpu_bwd(inp, d_o, d1, d2)
    chains = [(0, 0), (3, 7), (7, 11)]
    sub = wl.select_mlp_chains(inp, chains)
    bs, hs = [c[0] for c in chains], [c[1] for c in chains]
    ref = _oracle_bwd(sub, d_o[bs, hs][None], d1[bs, hs][None], d2[bs, hs][None])
    got = {k: v[bs, hs][None] for k, v in got.items()}
    errs, bad = compare(got, ref, "bf16")
    print("[parity] mlp bwd full size (3 chains): " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert not bad, bad


def test_mlp_backward_empty_sequence():
    import torch
    from chunkwise_weight_recurrence_amd.layer import MlpBuffers, to_f64
    inp = wl.make_mlp_inputs(dict(BASE, T=0, dtype="f32", loss="mse", act="silu", decay="scalar"))
    bufs = MlpBuffers(inp, with_bwd=True)
    bufs.forward()
    d1 = torch.randn((2, 2, 64, 256), device="cuda")
    d2 = torch.randn((2, 2, 256, 64), device="cuda")
    bufs.backward(torch.empty((2, 2, 0, 64), device="cuda"), d1, d2)
    torch.cuda.synchronize()
    assert torch.equal(bufs.dw1, d1) and torch.equal(bufs.dw2, d2)
    assert np.all(to_f64(bufs.dgamma) == 0.0)


@pytest.mark.parametrize("dv", [128, 48])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("saved", [True, False])
def test_mlp_rmse_row_widths(dv, dtype, saved):
    """The RMSE loss's row passes (the signal after the V_hat product in the forward, its
    Jacobian in the backward) loop lane, lane + 64, ... over d_v: d_v = 128 gives every lane
    two elements, d_v = 48 leaves lanes 48..63 idle.  Forward and backward, from the saved
    context and recomputed."""
    inp = wl.make_mlp_inputs(dict(BASE, dv=dv, dtype=dtype, loss="rmse", act="gelu", decay="scalar", seed=63))
    _check(f"mlp rmse dv={dv} {dtype}", inp)
    _check_bwd(f"mlp bwd rmse dv={dv} {dtype} saved={saved}", inp, saved=saved)
