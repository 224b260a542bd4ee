"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bar: max |gpu - oracle| / max |oracle| <= 1e-4 for fp32 I/O and <= 2e-2 for
bf16 I/O (fp32 accumulation), per output tensor.  Small cases span several
chunks and a ragged tail and are compared element by element; the full-size
workloads are compared on sampled (b, h) chains, which the oracle computes on
their own (chains are independent).
"""
import itertools

import numpy as np
import pytest

from chunkwise_weight_recurrence_amd import workloads as wl
from tests.parity_utils import compare, gpu_run, oracle_run, small_cfg

pytestmark = pytest.mark.gpu

COMBOS = list(itertools.product(["mse", "ip"], ["none", "silu", "gelu"], ["none", "scalar", "vector"]))


def _report(name, errs, bad):
    print(f"[parity] {name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert not bad, f"{name}: over tolerance {bad}"


@pytest.mark.parametrize("dtype,saved", [("f32", True), ("bf16", True), ("bf16", False)])
@pytest.mark.parametrize("loss,act,decay", COMBOS)
def test_small_fwd_bwd(dtype, saved, loss, act, decay):
    """64-wide heads, C = 64, T = 300: four full chunks and a 44-token tail.  bf16 runs
    the backward both from the forward's saved context and recomputing it."""
    inp = wl.make_ttt_inputs(small_cfg(dtype, loss, act, decay))
    rng = np.random.default_rng(5)
    dwf = rng.standard_normal(inp["w0"].shape).astype(np.float32)
    got = gpu_run(inp, d_wfinal=dwf, saved=saved)
    ref = oracle_run(inp, d_wfinal=dwf.astype(np.float64))
    _report(f"small {dtype} {loss}/{act}/{decay} saved={saved}", *compare(got, ref, dtype))


def _l1_margin(inp):
    """Smallest |f(K W_i) - V| over every chunk's train view, with the oracle's W_i: how
    far the L1 signal's sign decisions sit from a tie."""
    from oracle import act_f, chunk_forward
    cfg = inp["cfg"]
    C, T = cfg["C"], cfg["T"]
    _, _, ck = chunk_forward(inp["q"], inp["k"], inp["v"], inp["beta"], cfg["b"], C, return_ckpt=True,
                             **wl.oracle_kwargs(inp))
    return min(float(np.abs(act_f(inp["k"][:, :, s0:s0 + C] @ ck[:, :, i], cfg["act"]) -
                            inp["v"][:, :, s0:s0 + C]).min()) for i, s0 in enumerate(range(0, T, C)))


@pytest.mark.parametrize("dtype,saved", [("f32", True), ("bf16", True), ("bf16", False)])
@pytest.mark.parametrize("act,decay", list(itertools.product(["none", "silu", "gelu"], ["none", "scalar", "vector"])))
def test_l1_fwd_bwd(dtype, saved, act, decay):
    """L1 inner loss.  Its signal is the sign of f(K W_i) - V, decided in fp32 here and in
    fp64 by the oracle, so the targets are drawn at least 1 away from zero (|f(K W_i)| stays
    well below that): every decision has a margin, checked first, far above the rounding."""
    cfg = dict(small_cfg(dtype, "l1", act, decay, b=-4.0), v_margin=1.0)
    inp = wl.make_ttt_inputs(cfg)
    assert _l1_margin(inp) > 0.05
    rng = np.random.default_rng(6)
    dwf = rng.standard_normal(inp["w0"].shape).astype(np.float32)
    got = gpu_run(inp, d_wfinal=dwf, saved=saved)
    ref = oracle_run(inp, d_wfinal=dwf.astype(np.float64))
    assert np.all(ref["dv"] == 0.0)  # no gradient reaches V through the sign
    _report(f"l1 {dtype} {act}/{decay} saved={saved}", *compare(got, ref, dtype))


@pytest.mark.parametrize("act,decay,saved", [("silu", "vector", True), ("silu", "vector", False),
                                             ("none", "scalar", True), ("gelu", "none", False)])
def test_l1_d128_chunk256_bf16(act, decay, saved):
    """L1 at the matrix-core shape: d = 128, C = 256, two chains, 2.5 chunks."""
    cfg = dict(small_cfg("bf16", "l1", act, decay, B=1, H=2, T=640, dk=128, dv=128, C=256, b=-4.0), v_margin=1.0)
    inp = wl.make_ttt_inputs(cfg)
    assert _l1_margin(inp) > 0.05
    got = gpu_run(inp, saved=saved)
    ref = oracle_run(inp)
    _report(f"l1 d128 {act}/{decay} saved={saved}", *compare(got, ref, "bf16"))


@pytest.mark.parametrize("loss,act,decay,saved", [("mse", "none", "scalar", True), ("mse", "silu", "scalar", True),
                                                  ("ip", "silu", "vector", True), ("ip", "silu", "vector", False),
                                                  ("ip", "none", "none", True), ("ip", "gelu", "vector", True),
                                                  ("mse", "gelu", "scalar", False)])
def test_d128_chunk256_bf16(loss, act, decay, saved):
    """The matrix-core shape: d = 128, C = 256, two chains, 2.5 chunks."""
    cfg = small_cfg("bf16", loss, act, decay, B=1, H=2, T=640, dk=128, dv=128, C=256, b=-4.0)
    inp = wl.make_ttt_inputs(cfg)
    got = gpu_run(inp, saved=saved)
    ref = oracle_run(inp)
    _report(f"d128 {loss}/{act}/{decay} saved={saved}", *compare(got, ref, "bf16"))


def _min_chunk_log_decay(inp):
    """The most negative per-feature log-decay over one chunk, L_last = sum of log a."""
    C, T = inp["cfg"]["C"], inp["cfg"]["T"]
    return min(float(inp["log_a"][:, :, s0:s0 + C].sum(axis=2).min()) for s0 in range(0, T, C))


@pytest.mark.parametrize("saved", [True, False])
@pytest.mark.parametrize("loss,act", list(itertools.product(["mse", "ip", "l1"], ["none", "silu", "gelu"])))
def test_vector_decay_strong_small(loss, act, saved):
    """Vector decay far stronger than the workloads' (z ~ N(-2, 1), a = sigmoid(z) ~ 0.13 per
    token): every chunk's decay passes e^{-88}, where e^{-L} from the chunk start leaves the
    fp32 range.  d = 64, C = 64, T = 300 (four chunks and a 44-token tail)."""
    cfg = dict(small_cfg("bf16", loss, act, "vector", b=-4.0), z_mean=-2.0)
    if loss == "l1":
        cfg["v_margin"] = 1.0
    inp = wl.make_ttt_inputs(cfg)
    assert _min_chunk_log_decay(inp) < -88.0
    if loss == "l1":
        assert _l1_margin(inp) > 0.05
    rng = np.random.default_rng(8)
    dwf = rng.standard_normal(inp["w0"].shape).astype(np.float32)
    got = gpu_run(inp, d_wfinal=dwf, saved=saved)
    ref = oracle_run(inp, d_wfinal=dwf.astype(np.float64))
    _report(f"strong decay small {loss}/{act} saved={saved}", *compare(got, ref, "bf16"))


@pytest.mark.parametrize("saved", [True, False])
@pytest.mark.parametrize("z_mean", [0.0, -2.0, -4.0])
@pytest.mark.parametrize("loss,act", [("ip", "silu"), ("mse", "none"), ("mse", "gelu"), ("ip", "none")])
def test_vector_decay_strong_d128_chunk256(loss, act, z_mean, saved):
    """The matrix-core shape (d = 128, C = 256, two chains, 2.5 chunks) with the decay drawn
    at z ~ N(z_mean, 1): per-chunk log-decay down to about -250 (z_mean 0), -600 (-2) and
    -1100 (-4) per feature; at z_mean -4 a 32-token tile alone decays by about e^{-130}.
    The inner-product loss without an act takes the chunk-parallel path."""
    cfg = dict(small_cfg("bf16", loss, act, "vector", B=1, H=2, T=640, dk=128, dv=128, C=256, b=-4.0),
               z_mean=z_mean)
    inp = wl.make_ttt_inputs(cfg)
    assert _min_chunk_log_decay(inp) < -88.0
    rng = np.random.default_rng(9)
    dwf = rng.standard_normal(inp["w0"].shape).astype(np.float32)
    got = gpu_run(inp, d_wfinal=dwf, saved=saved)
    ref = oracle_run(inp, d_wfinal=dwf.astype(np.float64))
    _report(f"strong decay d128 {loss}/{act} z={z_mean} saved={saved}", *compare(got, ref, "bf16"))


@pytest.mark.parametrize("shape", [dict(dk=64, dv=64, T=100, C=32), dict(dk=128, dv=32, T=300, C=128),
                                   dict(dk=64, dv=128, T=257, C=256)])
@pytest.mark.parametrize("saved", [True, False])
def test_vector_decay_strong_chunk_sizes(shape, saved):
    """Strong vector decay (z ~ N(-2, 1)) at the other chunk sizes: one and four 32-token
    tiles per chunk, a 44-token tail, and a one-token last chunk."""
    cfg = dict(small_cfg("bf16", "ip", "silu", "vector", B=1, H=2, b=-4.0, **shape), z_mean=-2.0)
    inp = wl.make_ttt_inputs(cfg)
    got = gpu_run(inp, saved=saved)
    ref = oracle_run(inp)
    _report(f"strong decay {shape} saved={saved}", *compare(got, ref, "bf16"))


@pytest.mark.parametrize("shape,combo", [
    (dict(dk=64, dv=64, T=100, C=32), ("mse", "silu", "vector")),    # C = 32: two k-steps per chunk
    (dict(dk=64, dv=64, T=100, C=32), ("ip", "none", "scalar")),
    (dict(dk=128, dv=128, T=300, C=128), ("ip", "silu", "vector")),  # C = 128, 44-token tail
    (dict(dk=128, dv=32, T=200, C=128), ("mse", "none", "none")),    # one 32-column block
    (dict(dk=64, dv=128, T=257, C=256), ("mse", "silu", "scalar")),  # one-token last chunk
])
def test_matrix_core_chunk_sizes_bf16(shape, combo):
    """The bf16 matrix-core kernels at every chunk size they take (32 ... 256)."""
    cfg = small_cfg("bf16", *combo, B=1, H=2, b=-3.0, **shape)
    inp = wl.make_ttt_inputs(cfg)
    got = gpu_run(inp)
    ref = oracle_run(inp)
    _report(f"bf16 {shape} {'/'.join(combo)}", *compare(got, ref, "bf16"))


@pytest.mark.parametrize("shape,decay", [
    (dict(dk=128, dv=32, T=300, C=128), "vector"),          # one 32-column block, 44-token tail
    (dict(dk=64, dv=128, T=600, C=256), "scalar"),
    (dict(dk=128, dv=64, T=257, C=32), "none"),             # 8 chunks of 32 and a 1-token chunk
    (dict(dk=64, dv=64, T=1000, C=64, B=1, H=3), "vector"),  # 16 chunks, a 40-token tail
])
@pytest.mark.parametrize("saved", [True, False])
def test_linear_path_bf16(shape, decay, saved):
    """Inner-product loss without an act: the chunk-parallel forward (per-chunk K^T G~,
    the state scan, per-chunk query view), and the backward from its checkpoints."""
    shape = dict(shape)
    B, H = shape.pop("B", 2), shape.pop("H", 2)
    cfg = small_cfg("bf16", "ip", "none", decay, B=B, H=H, b=-3.0, **shape)
    inp = wl.make_ttt_inputs(cfg)
    got = gpu_run(inp, saved=saved)
    ref = oracle_run(inp)
    _report(f"linear {shape} {decay} saved={saved}", *compare(got, ref, "bf16"))


@pytest.mark.parametrize("T,C", [(1, 64), (63, 64), (64, 64), (65, 32)])
def test_linear_path_edge_lengths_bf16(T, C):
    """The chunk-parallel path with one token, one short chunk, exactly one chunk,
    and a one-token last chunk."""
    cfg = small_cfg("bf16", "ip", "none", "vector", B=1, H=2, T=T, dk=64, dv=64, C=C, b=-3.0)
    inp = wl.make_ttt_inputs(cfg)
    got = gpu_run(inp)
    ref = oracle_run(inp)
    _report(f"linear edge T={T} C={C}", *compare(got, ref, "bf16"))


def test_ip_linear_many_chains_sequential_bf16():
    """Inner-product loss without an act on enough chains (5 x 14 x 1 column block) that
    the forward stays on the sequential kernel."""
    cfg = small_cfg("bf16", "ip", "none", "vector", B=5, H=14, T=200, dk=64, dv=32, C=64, b=-3.0)
    inp = wl.make_ttt_inputs(cfg)
    got = gpu_run(inp)
    ref = oracle_run(inp)
    _report("ip/none sequential 70 chains", *compare(got, ref, "bf16"))


@pytest.mark.parametrize("shape", [
    dict(T=1, C=64), dict(T=63, C=64), dict(T=64, C=64), dict(T=65, C=64), dict(T=40, C=1),
    dict(dk=1, dv=3, T=50, C=7), dict(dk=40, dv=72, T=130, C=32), dict(dk=256, dv=32, T=70, C=256),
])
def test_edge_shapes_f32(shape):
    cfg = small_cfg("f32", "mse", "silu", "vector", B=1, H=1, **shape)
    inp = wl.make_ttt_inputs(cfg)
    got = gpu_run(inp)
    ref = oracle_run(inp)
    _report(f"edge {shape}", *compare(got, ref, "f32"))


def test_zero_tokens_passes_state_through():
    import torch
    from chunkwise_weight_recurrence_amd.layer import TTTLayerBuffers, to_f64
    inp = wl.make_ttt_inputs(small_cfg("bf16", "mse", "none", "scalar", T=0))
    bufs = TTTLayerBuffers(inp)
    bufs.forward()
    bufs.backward()
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(bufs.w_final), inp["w0"])
    assert np.all(to_f64(bufs.dw0) == 0) and np.all(to_f64(bufs.dgamma) == 0)


def test_deterministic_and_nan_propagation():
    import torch
    from chunkwise_weight_recurrence_amd.layer import TTTLayerBuffers, to_f64
    inp = wl.make_ttt_inputs(small_cfg("bf16", "ip", "silu", "vector", T=256, C=64))
    bufs = TTTLayerBuffers(inp)
    outs = []
    for _ in range(2):
        bufs.forward()
        bufs.backward()
        torch.cuda.synchronize()
        outs.append([to_f64(t) for t in (bufs.o, bufs.w_final, bufs.dq, bufs.dk, bufs.dv, bufs.dbeta,
                                         bufs.dlog_a)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    # a NaN in one token of chain 0 poisons that chain's later outputs, not the other chains
    bufs.q[0, 0, 70, 3] = float("nan")
    bufs.forward()
    torch.cuda.synchronize()
    o = to_f64(bufs.o)
    assert np.isnan(o[0, 0, 70:]).any()
    assert np.all(np.isfinite(o[0, 1])) and np.all(np.isfinite(o[1]))


# ---------------------------------------------------------------------------
# the workloads at full size
# ---------------------------------------------------------------------------

SAMPLED = {
    "tiny-fwd-f32": None,                   # small enough for the whole problem
    "410m-fwd": [(0, 0), (1, 1), (2, 2), (3, 3), (4, 4), (5, 5), (6, 6), (7, 7)],
    "410m-silu-fwdbwd": [(0, 1), (1, 2), (2, 3), (3, 4), (4, 5), (5, 6), (6, 7), (7, 0)],
    # one chain on each of the eight XCDs (the forward and both backward kernels hand
    # chains b * H + h = 8 x .. 8 x + 7 to XCD x), each at a different slot 0..7 within it
    "1.45b-fwdbwd": [(0, 0), (0, 9), (1, 2), (1, 11), (2, 4), (2, 13), (3, 6), (3, 15)],
    "1.45b-iplin-32k": [(0, 11)],           # chunk-parallel forward and dW chain, 128 chunks
}


@pytest.mark.parametrize("name", list(SAMPLED))
def test_workload_full_size(name):
    inp = wl.make_ttt_inputs(name)
    cfg = inp["cfg"]
    print(f"[parity] running {name} on the GPU", flush=True)
    got = gpu_run(inp)
    chains = SAMPLED[name]
    if chains is None:
        ref = oracle_run(inp)
        sub = got
    else:
        ref = oracle_run(wl.select_chains(inp, chains))
        bs = [c[0] for c in chains]
        hs = [c[1] for c in chains]
        sub = {k: v[bs, hs][None] for k, v in got.items()}
    _report(f"{name} {cfg['dtype']}", *compare(sub, ref, cfg["dtype"]))


def test_workload_full_size_recompute():
    """The 1.45B workload with the backward recomputing the forward's intermediates."""
    name = "1.45b-fwdbwd"
    inp = wl.make_ttt_inputs(name)
    got = gpu_run(inp, saved=False)
    chains = SAMPLED[name]
    ref = oracle_run(wl.select_chains(inp, chains))
    bs = [c[0] for c in chains]
    hs = [c[1] for c in chains]
    sub = {k: v[bs, hs][None] for k, v in got.items()}
    _report(f"{name} recompute", *compare(sub, ref, "bf16"))


# ---------------------------------------------------------------------------
# In-Place TTT
# ---------------------------------------------------------------------------

def _inplace_gpu(inp, workspace=True):
    import torch
    from chunkwise_weight_recurrence_amd.layer import InplaceBuffers, to_f64
    bufs = InplaceBuffers(inp, workspace=workspace)
    bufs.forward()
    torch.cuda.synchronize()
    return to_f64(bufs.o), to_f64(bufs.w), bufs.ws_bytes


@pytest.mark.parametrize("workspace", [True, False])
@pytest.mark.parametrize("shape", [
    dict(B=2, T=300, d_model=96, d_ff=200, C=64),    # ragged tail, tiles cut at both edges
    dict(B=1, T=2048, d_model=256, d_ff=512, C=1024),
    dict(B=1, T=1100, d_model=136, d_ff=2056, C=512),  # split d_ff contraction, ragged everywhere
])
def test_inplace_small(shape, workspace):
    from oracle import inplace_forward
    inp = wl.make_inplace_inputs(dict(shape, eta=1e-2, seed=77))
    O, W, ws_bytes = _inplace_gpu(inp, workspace)
    if workspace and shape["d_ff"] > 2048:
        assert ws_bytes > 0  # the split path is the one under test
    Or, Wr = inplace_forward(wl.inplace_values(inp, "z_dev"), wl.inplace_values(inp, "vhat_dev"),
                             inp["w0_dev"].astype(np.float64), shape["C"], 1e-2)
    errs, bad = compare(dict(O=O, W=W), dict(O=Or, W=Wr), "bf16")
    _report(f"inplace {shape} workspace={workspace}", errs, bad)


def test_inplace_full_size_sampled_rows():
    """d_model 2560, d_ff 9728, T 32768, C 1024: compare 8 sampled rows of W_down and O."""
    import torch
    from oracle import inplace_rows

    def mm(a, b):
        return (torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda() @
                torch.from_numpy(np.ascontiguousarray(b, dtype=np.float32)).cuda()).cpu().numpy()

    inp = wl.make_inplace_inputs("inplace-wdown", matmul=mm)
    cfg = inp["cfg"]
    O, W, _ = _inplace_gpu(inp)
    rows = [0, 1, 777, 1280, 2047, 2100, 2558, 2559]
    z = wl.inplace_values(inp, "z_dev")
    vh = wl.inplace_values(inp, "vhat_dev")
    Or, Wr = inplace_rows(z, vh, inp["w0_dev"][:, rows].astype(np.float64), rows, cfg["C"], cfg["eta"])
    errs, bad = compare(dict(O=O[:, :, rows], W=W[:, rows]), dict(O=Or, W=Wr), "bf16")
    _report("inplace full size (8 rows)", errs, bad)


# ---------------------------------------------------------------------------
# In-Place backward
# ---------------------------------------------------------------------------

def _inplace_fwd_bwd(inp, grads):
    import torch
    from chunkwise_weight_recurrence_amd.layer import InplaceBuffers, to_device, to_f64
    bufs = InplaceBuffers(inp)
    bufs.forward()
    d_o = to_device(grads["d_o_dev"])
    dwf = to_device(grads["d_wfinal_dev"]) if grads["d_wfinal_dev"] is not None else None
    dz, dv, dw0 = bufs.backward(d_o, dwf)
    torch.cuda.synchronize()
    return to_f64(dz), to_f64(dv), to_f64(dw0)


@pytest.mark.parametrize("shape,with_dwf", [
    (dict(B=2, T=300, d_model=96, d_ff=200, C=64), True),      # ragged tail, tiles cut at both edges
    (dict(B=2, T=300, d_model=96, d_ff=200, C=64), False),
    (dict(B=1, T=1100, d_model=136, d_ff=2056, C=512), True),  # split dV_hat contraction, ragged everywhere
    (dict(B=1, T=2048, d_model=256, d_ff=512, C=1024), False),
])
def test_inplace_backward_small(shape, with_dwf):
    from oracle import inplace_backward
    inp = wl.make_inplace_inputs(dict(shape, eta=1e-2, seed=95))
    g = wl.make_inplace_grads(inp["cfg"], seed=96, with_dwfinal=with_dwf)
    dz, dv, dw0 = _inplace_fwd_bwd(inp, g)
    rz, rv, rw = inplace_backward(wl.inplace_values(inp, "z_dev"), wl.inplace_values(inp, "vhat_dev"),
                                  inp["w0_dev"].astype(np.float64), shape["C"], 1e-2, wl.bf16_to_f64(g["d_o_dev"]),
                                  None if g["d_wfinal_dev"] is None else g["d_wfinal_dev"].astype(np.float64))
    errs, bad = compare(dict(dz=dz, dvhat=dv, dw0=dw0), dict(dz=rz, dvhat=rv, dw0=rw), "bf16")
    _report(f"inplace backward {shape} dW_T={with_dwf}", errs, bad)


def test_inplace_short_last_chunk_splits_further():
    """T 556 at C 300, d_model 10880, d_ff 2048: the 256-token last chunk has one
    row tile where a full chunk has two, so its apply splits d_ff three ways (85
    column tiles on 256 CUs) while a full chunk does not split; the workspace
    holds those partials.  Forward and backward against the oracle."""
    from oracle import inplace_backward, inplace_forward
    shape = dict(B=1, T=556, d_model=10880, d_ff=2048, C=300)
    inp = wl.make_inplace_inputs(dict(shape, eta=1e-2, seed=161))
    z = wl.inplace_values(inp, "z_dev")
    vh = wl.inplace_values(inp, "vhat_dev")
    w0 = inp["w0_dev"].astype(np.float64)
    O, W, _ = _inplace_gpu(inp)
    Or, Wr = inplace_forward(z, vh, w0, shape["C"], 1e-2)
    errs, bad = compare(dict(O=O, W=W), dict(O=Or, W=Wr), "bf16")
    _report(f"inplace {shape}", errs, bad)
    g = wl.make_inplace_grads(inp["cfg"], seed=162)
    dz, dv, dw0 = _inplace_fwd_bwd(inp, g)
    rz, rv, rw = inplace_backward(z, vh, w0, shape["C"], 1e-2, wl.bf16_to_f64(g["d_o_dev"]),
                                  g["d_wfinal_dev"].astype(np.float64))
    errs, bad = compare(dict(dz=dz, dvhat=dv, dw0=dw0), dict(dz=rz, dvhat=rv, dw0=rw), "bf16")
    _report(f"inplace backward {shape}", errs, bad)


@pytest.mark.parametrize("T,C", [(1, 64), (100, 256), (256, 64)])
def test_inplace_backward_edge_lengths(T, C):
    """One token, one short chunk, and chunks that divide T exactly."""
    from oracle import inplace_backward
    shape = dict(B=1, T=T, d_model=64, d_ff=136, C=C)
    inp = wl.make_inplace_inputs(dict(shape, eta=1e-2, seed=98))
    g = wl.make_inplace_grads(inp["cfg"], seed=99)
    dz, dv, dw0 = _inplace_fwd_bwd(inp, g)
    rz, rv, rw = inplace_backward(wl.inplace_values(inp, "z_dev"), wl.inplace_values(inp, "vhat_dev"),
                                  inp["w0_dev"].astype(np.float64), C, 1e-2, wl.bf16_to_f64(g["d_o_dev"]),
                                  g["d_wfinal_dev"].astype(np.float64))
    errs, bad = compare(dict(dz=dz, dvhat=dv, dw0=dw0), dict(dz=rz, dvhat=rv, dw0=rw), "bf16")
    _report(f"inplace backward T={T} C={C}", errs, bad)


def test_inplace_backward_full_size_sampled():
    """d_model 2560, d_ff 9728, T 32768, C 1024: dz and dw0 on sampled columns of d_ff,
    dvhat on sampled tokens (the oracle forms those one by one)."""
    import torch
    from oracle import inplace_backward_sampled

    def mm(a, b):
        return (torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda() @
                torch.from_numpy(np.ascontiguousarray(b, dtype=np.float32)).cuda()).cpu().numpy()

    inp = wl.make_inplace_inputs("inplace-wdown", matmul=mm)
    cfg = inp["cfg"]
    g = wl.make_inplace_grads(cfg, seed=97)
    dz, dv, dw0 = _inplace_fwd_bwd(inp, g)
    cols = [0, 1, 4000, 9727]
    toks = [0, 1023, 1024, 20000, 31743, 32767]
    dwf = g["d_wfinal_dev"].astype(np.float64)
    rz, rw, rv = inplace_backward_sampled(wl.inplace_values(inp, "z_dev"), wl.inplace_values(inp, "vhat_dev"),
                                          inp["w0_dev"][:, :, cols].astype(np.float64), cols, toks, cfg["C"], cfg["eta"],
                                          wl.bf16_to_f64(g["d_o_dev"]), dwf[:, :, cols], dwf)
    got = dict(dz=dz[:, :, cols], dw0=dw0[:, :, cols], dvhat=dv[:, toks])
    errs, bad = compare(got, dict(dz=rz, dw0=rw, dvhat=rv), "bf16")
    _report("inplace backward full size (4 columns, 6 tokens)", errs, bad)
