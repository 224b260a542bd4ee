"""GPU parity of the guarded In-Place forward (update clipping, document resets)
through the C ABI against the fp64 oracle.

Bar as for the plain In-Place update: max |gpu - oracle| / max |oracle| <= 2e-2
per output (bf16 operands, fp32 accumulation), here also on the accumulated
update W_final - W0, which the clipping scales.  The clip thresholds sit
between two chunks' update norms, so some chunks are clipped and some are not.
"""
import numpy as np
import pytest

from chunkwise_weight_recurrence_amd import workloads as wl
from tests.parity_utils import compare

pytestmark = pytest.mark.gpu


def _report(name, errs, bad):
    print(f"[parity] {name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert not bad, f"{name}: over tolerance {bad}"


def _tau_between(norms, q):
    """A threshold between two neighbouring update norms (no chunk sits on it)."""
    s = np.sort(norms)
    i = min(max(int(q * len(s)), 1), len(s) - 1)
    return float(np.sqrt(s[i - 1] * s[i]))


def _run(inp, workspace=True):
    import torch
    from chunkwise_weight_recurrence_amd.layer import InplaceBuffers, to_f64
    bufs = InplaceBuffers(inp, workspace=workspace, guarded=True)
    bufs.forward()
    torch.cuda.synchronize()
    return to_f64(bufs.o), to_f64(bufs.w), bufs.ws_bytes


@pytest.mark.parametrize("shape,doc_lens,clip_q", [
    (dict(B=2, T=1100, d_model=136, d_ff=264, C=256), (300, 477, 323), 0.5),   # docs + clip, ragged tiles
    (dict(B=1, T=1100, d_model=136, d_ff=2056, C=512), (700, 400), 0.5),       # split apply + both
    (dict(B=2, T=300, d_model=96, d_ff=200, C=64), (100, 150, 50), None),      # documents only
    (dict(B=1, T=2048, d_model=256, d_ff=512, C=256), None, 0.3),              # clipping only
    (dict(B=1, T=200, d_model=96, d_ff=200, C=64), (1, 198, 1), 0.5),          # one-token documents
    (dict(B=2, T=300, d_model=96, d_ff=200, C=128), (128, 128, 44), 0.5),      # documents on chunk boundaries
])
def test_inplace_guarded_small(shape, doc_lens, clip_q):
    from oracle import inplace_forward_guarded, update_norms
    cfg = dict(shape, eta=1e-2, seed=91, doc_lens=doc_lens)
    inp = wl.make_inplace_inputs(cfg)
    per_seq, _ = wl.inplace_doc_starts(cfg)
    z = wl.inplace_values(inp, "z_dev")
    vh = wl.inplace_values(inp, "vhat_dev")
    w0 = inp["w0_dev"].astype(np.float64)
    tau = None
    if clip_q is not None:
        tau = _tau_between(update_norms(z, vh, shape["C"], 1e-2, per_seq), clip_q)
        inp["cfg"]["clip_tau"] = tau
    O, W, _ = _run(inp)
    Or, Wr = inplace_forward_guarded(z, vh, w0, shape["C"], 1e-2, tau, per_seq, w0)
    errs, bad = compare(dict(O=O, W=W, dW=W - w0), dict(O=Or, W=Wr, dW=Wr - w0), "bf16")
    _report(f"inplace guarded {shape} docs={doc_lens} tau={tau}", errs, bad)


def test_inplace_guarded_off_equals_plain():
    """No threshold and no document starts: bit-identical to inplace_ttt_fwd."""
    import torch
    from chunkwise_weight_recurrence_amd.layer import InplaceBuffers
    cfg = dict(B=2, T=700, d_model=136, d_ff=2056, C=256, eta=1e-2, seed=92)
    inp = wl.make_inplace_inputs(cfg)
    plain = InplaceBuffers(inp, guarded=False)
    plain.forward()
    guarded = InplaceBuffers(inp, guarded=True)
    guarded.forward()
    torch.cuda.synchronize()
    assert torch.equal(plain.o, guarded.o)
    assert torch.equal(plain.w, guarded.w)


def test_inplace_guarded_repeat_is_deterministic():
    """The clip scale is summed in a fixed order: two runs give the same bits."""
    import torch
    from chunkwise_weight_recurrence_amd.layer import InplaceBuffers
    cfg = dict(B=1, T=1100, d_model=136, d_ff=2056, C=512, eta=1e-2, seed=93, doc_lens=(600, 500),
               clip_tau=0.05)
    inp = wl.make_inplace_inputs(cfg)
    bufs = InplaceBuffers(inp)
    outs = []
    for _ in range(2):
        bufs.reset()
        bufs.forward()
        torch.cuda.synchronize()
        outs.append((bufs.o.clone(), bufs.w.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.fixture(scope="module")
def full_inputs():
    import torch

    def mm(a, b):
        return (torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda() @
                torch.from_numpy(np.ascontiguousarray(b, dtype=np.float32)).cuda()).cpu().numpy()

    inp = wl.make_inplace_inputs("inplace-wdown-guarded", matmul=mm)
    cfg = inp["cfg"]
    per_seq, _ = wl.inplace_doc_starts(cfg)
    z = wl.inplace_values(inp, "z_dev")
    vh = wl.inplace_values(inp, "vhat_dev")
    from oracle import update_norms
    norms = update_norms(z, vh, cfg["C"], cfg["eta"], per_seq)
    return inp, z, vh, per_seq, norms


@pytest.mark.parametrize("tau_kind", ["page", "between"])
def test_inplace_guarded_full_size_sampled_rows(full_inputs, tau_kind):
    """T 32768 in documents of 9000, 7000, 12000 and 4768 tokens, d_model 2560, d_ff 9728,
    C 1024: 8 sampled rows of W_down and O.  Thresholds: the page's 1e-5 (every update
    clipped), and one between two chunks' norms (about half clipped)."""
    from oracle import inplace_rows_guarded
    inp, z, vh, per_seq, norms = full_inputs
    cfg = inp["cfg"]
    tau = cfg["clip_tau"] if tau_kind == "page" else _tau_between(norms, 0.5)
    inp = dict(inp, cfg=dict(cfg, clip_tau=tau))
    O, W, _ = _run(inp)
    rows = [0, 1, 777, 1280, 2047, 2100, 2558, 2559]
    w0r = inp["w0_dev"][:, rows].astype(np.float64)
    scales = np.minimum(1.0, tau / norms)
    Or, Wr = inplace_rows_guarded(z, vh, w0r, w0r, rows, cfg["C"], cfg["eta"], scales, per_seq)
    got = dict(O=O[:, :, rows], W=W[:, rows])
    ref = dict(O=Or, W=Wr)
    if tau_kind == "between":  # the update is large enough to compare on its own
        got["dW"], ref["dW"] = W[:, rows] - w0r, Wr - w0r
    errs, bad = compare(got, ref, "bf16")
    _report(f"inplace guarded full size (8 rows) tau={tau:.3g}", errs, bad)
