"""GPU parity of the guarded In-Place backward (clip factor differentiated,
document resets) through the C ABI against the fp64 oracle.

Bar as for the plain In-Place backward: max |gpu - oracle| / max |oracle| <= 2e-2
per output (bf16 operands, fp32 accumulation).  With random upstream gradients
the clip's correction term, kappa D with kappa = s <D, A> / ||D||^2, is tiny
(D and a random A are nearly orthogonal), so dL/dW_final here also carries a
component along every update direction D_i of each sequence's last document:
then the correction is a large part of dZ and dV_hat there, and a mistake in
it shows.  Thresholds sit between two chunks' update norms.
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
    s = np.sort(norms)
    i = min(max(int(q * len(s)), 1), len(s) - 1)
    return float(np.sqrt(s[i - 1] * s[i]))


def _aligned_dwfinal(z, vh, eta, C, per_seq, rng, weight=2.0):
    """dW_final = R + weight ||R|| sum_i D_i / ||D_i|| over the chunks of each
    sequence's last document (D_i = eta V_hat_i^T Z_i), R ~ N(0, 1)."""
    B, T, dff = z.shape
    dm = vh.shape[-1]
    out = rng.standard_normal((B, dm, dff))
    for b in range(B):
        a = per_seq[b][-1] if per_seq[b] else 0
        r = np.linalg.norm(out[b])
        for s0 in range(a, T, C):
            s1 = min(s0 + C, T)
            D = eta * vh[b, s0:s1].T @ z[b, s0:s1]
            n = np.linalg.norm(D)
            if n > 0:
                out[b] += weight * r * D / n
    return out.astype(np.float32)


def _gpu(inp, d_o_bits, dwf):
    import torch
    from chunkwise_weight_recurrence_amd.layer import InplaceBuffers, to_device, to_f64
    bufs = InplaceBuffers(inp, guarded=True)
    bufs.forward()
    dz, dv, dw0 = bufs.backward(to_device(d_o_bits), None if dwf is None else to_device(dwf))
    torch.cuda.synchronize()
    return to_f64(dz), to_f64(dv), to_f64(dw0), to_f64(bufs.dw_init)


def _case(shape, doc_lens, clip_q, seed, aligned=True, eta=1e-2):
    from oracle import inplace_backward_guarded, update_norms
    cfg = dict(shape, eta=eta, seed=seed, doc_lens=doc_lens)
    inp = wl.make_inplace_inputs(cfg)
    per_seq, _ = wl.inplace_doc_starts(cfg)
    z = wl.inplace_values(inp, "z_dev")
    vh = wl.inplace_values(inp, "vhat_dev")
    w0 = inp["w0_dev"].astype(np.float64)
    tau = None
    if clip_q is not None:  # clip_q = 0: below every norm
        norms = update_norms(z, vh, shape["C"], eta, per_seq)
        tau = 0.5 * float(norms.min()) if clip_q == 0 else _tau_between(norms, clip_q)
        inp["cfg"]["clip_tau"] = tau
    g = wl.make_inplace_grads(inp["cfg"], seed=seed + 1, with_dwfinal=not aligned)
    rng = np.random.Generator(np.random.PCG64(seed + 2))
    dwf = _aligned_dwfinal(z, vh, eta, shape["C"], per_seq, rng) if aligned else g["d_wfinal_dev"]
    got = _gpu(inp, g["d_o_dev"], dwf)
    ref = inplace_backward_guarded(z, vh, w0, shape["C"], eta, wl.bf16_to_f64(g["d_o_dev"]),
                                   dwf.astype(np.float64), tau, per_seq, w0)
    keys = ("dz", "dvhat", "dw0", "dw_init")
    G, R = dict(zip(keys, got)), dict(zip(keys, ref))
    if not doc_lens:  # no later documents: dL/dw_init is zero on both sides
        assert not np.any(G.pop("dw_init")) and not np.any(R.pop("dw_init"))
    return G, R, tau


@pytest.mark.parametrize("shape,doc_lens,clip_q", [
    (dict(B=2, T=1100, d_model=136, d_ff=264, C=256), (300, 477, 323), 0.5),   # docs + clip, ragged tiles
    (dict(B=1, T=1100, d_model=136, d_ff=2056, C=512), (700, 400), 0.5),       # split products + both
    (dict(B=2, T=300, d_model=96, d_ff=200, C=64), (100, 150, 50), None),      # documents only
    (dict(B=1, T=2048, d_model=256, d_ff=512, C=256), None, 0.3),              # clipping only
    (dict(B=1, T=200, d_model=96, d_ff=200, C=64), (1, 198, 1), 0.5),          # one-token documents
    (dict(B=2, T=300, d_model=96, d_ff=200, C=128), (128, 128, 44), 0.5),      # documents on chunk boundaries
    (dict(B=1, T=333, d_model=64, d_ff=136, C=100), (33, 300), 0.0),           # every update clipped, C % 8 != 0
])
def test_inplace_guarded_backward_small(shape, doc_lens, clip_q):
    G, R, tau = _case(shape, doc_lens, clip_q, seed=131)
    errs, bad = compare(G, R, "bf16")
    _report(f"inplace guarded backward {shape} docs={doc_lens} tau={tau}", errs, bad)


def test_inplace_guarded_backward_random_upstream():
    """Random dW_final and dO: the correction is small and the rest must match."""
    G, R, tau = _case(dict(B=1, T=1100, d_model=136, d_ff=2056, C=512), (700, 400), 0.5, seed=137, aligned=False)
    errs, bad = compare(G, R, "bf16")
    _report(f"inplace guarded backward, random upstream, tau={tau}", errs, bad)


def test_inplace_guarded_backward_off_equals_plain():
    """No threshold and no document starts: bit-identical to inplace_ttt_bwd."""
    import torch
    from chunkwise_weight_recurrence_amd.layer import InplaceBuffers, to_device
    cfg = dict(B=2, T=700, d_model=136, d_ff=2056, C=256, eta=1e-2, seed=139)
    inp = wl.make_inplace_inputs(cfg)
    g = wl.make_inplace_grads(inp["cfg"], seed=140)
    d_o, dwf = to_device(g["d_o_dev"]), to_device(g["d_wfinal_dev"])
    outs = []
    for guarded in (False, True):
        bufs = InplaceBuffers(inp, guarded=guarded)
        bufs.forward()
        outs.append([x.clone() for x in bufs.backward(d_o, dwf)])
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_inplace_guarded_backward_full_width():
    """d_model 2560, d_ff 9728, C 1024 (the full-size layer's widths and chunk) over
    4096 tokens in two documents (2500 + 1596: chunks of 1024, 1024, 452 | 1024,
    572) with the threshold between two update norms; the whole oracle backward."""
    shape = dict(B=1, T=4096, d_model=2560, d_ff=9728, C=1024)
    G, R, tau = _case(shape, (2500, 1596), 0.5, seed=141, eta=1e-3)
    errs, bad = compare(G, R, "bf16")
    _report(f"inplace guarded backward full width tau={tau:.3g}", errs, bad)


def test_inplace_guarded_backward_uneven_documents():
    """Three sequences, document starts in the middle one only, w_init distinct
    from w0 (so the first document's replay must start from w0 and the others'
    from w_init), through the C ABI directly."""
    import torch
    from chunkwise_weight_recurrence_amd import binding as B
    from chunkwise_weight_recurrence_amd.layer import to_device, to_f64
    from oracle import inplace_backward_guarded, update_norms
    Bn, T, dm, dff, C, eta = 3, 400, 96, 200, 64, 1e-2
    inp = wl.make_inplace_inputs(dict(B=Bn, T=T, d_model=dm, d_ff=dff, C=C, eta=eta, seed=151))
    per_seq = [[], [150, 333], []]
    flat = [T + 150, T + 333]
    z = wl.inplace_values(inp, "z_dev")
    vh = wl.inplace_values(inp, "vhat_dev")
    rng = np.random.Generator(np.random.PCG64(152))
    w0 = inp["w0_dev"]
    wi = (0.02 * rng.standard_normal((Bn, dm, dff))).astype(np.float32)
    tau = _tau_between(update_norms(z, vh, C, eta, per_seq), 0.5)
    g = wl.make_inplace_grads(inp["cfg"], seed=153, with_dwfinal=False)
    dwf = _aligned_dwfinal(z, vh, eta, C, per_seq, rng)
    dev = lambda x: to_device(x)
    zd, vd, w0d, wid, dod, dwfd = (dev(x) for x in (inp["z_dev"], inp["vhat_dev"], w0, wi, g["d_o_dev"], dwf))
    w = w0d.clone()
    o = torch.empty((Bn, T, dm), dtype=torch.bfloat16, device="cuda")
    n = B.inplace_ttt_guarded_workspace_size(Bn, T, dm, dff, C)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    B.inplace_ttt_fwd_guarded(Bn, T, dm, dff, C, eta, tau, flat, zd, vd, wid, w, o, ws, n)
    dz = torch.empty((Bn, T, dff), dtype=torch.bfloat16, device="cuda")
    dv = torch.empty((Bn, T, dm), dtype=torch.bfloat16, device="cuda")
    dw0 = torch.empty((Bn, dm, dff), dtype=torch.float32, device="cuda")
    dwi = torch.empty((Bn, dm, dff), dtype=torch.float32, device="cuda")
    nb = B.inplace_ttt_bwd_guarded_workspace_size(Bn, T, dm, dff, C)
    wsb = torch.empty(nb, dtype=torch.uint8, device="cuda")
    B.inplace_ttt_bwd_guarded(Bn, T, dm, dff, C, eta, tau, flat, zd, vd, w0d, wid, w, dod, dwfd, dz, dv, dw0, dwi,
                              wsb, nb)
    torch.cuda.synchronize()
    ref = inplace_backward_guarded(z, vh, w0.astype(np.float64), C, eta, wl.bf16_to_f64(g["d_o_dev"]),
                                   dwf.astype(np.float64), tau, per_seq, wi.astype(np.float64))
    keys = ("dz", "dvhat", "dw0", "dw_init")
    got = dict(zip(keys, (to_f64(x) for x in (dz, dv, dw0, dwi))))
    errs, bad = compare(got, dict(zip(keys, ref)), "bf16")
    assert not np.any(got["dw_init"][[0, 2]]), "sequences without documents have no w_init derivative"
    _report(f"inplace guarded backward, uneven documents tau={tau:.3g}", errs, bad)
