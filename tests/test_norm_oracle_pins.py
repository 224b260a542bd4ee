"""Pins of the Linear -> Norm oracle against facts fixed outside it: a token-by-token
loop, finite differences (the train-view signal and the whole backward), the
normalisation's own invariants, and a planted mistake.

The graph follows "Modular TTT" (summary page, "Method step details": Algorithm 1
composed over the primitives; "Experimental results" / "Technical novelty": the Norm
primitive and its analytic backward).
"""
import itertools

import numpy as np
import pytest

from oracle import norm_oracle as no

COMBOS = list(itertools.product(["mse", "ip", "l1", "rmse"], ["none", "scalar"]))


@pytest.fixture
def rng():
    return np.random.default_rng(1618)


def _inputs(rng, B=1, H=2, T=11, dk=3, dv=5):
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, T, dv))
    beta = rng.standard_normal((B, H, T))
    gamma = rng.uniform(0.85, 1.0, H)
    w0 = 0.5 * rng.standard_normal((B, H, dk, dv))
    return q, k, v, beta, gamma, w0


@pytest.mark.parametrize("loss,decay", COMBOS)
@pytest.mark.parametrize("C", [1, 4, 16])
def test_norm_chunk_form_equals_token_loop(loss, decay, C, rng):
    q, k, v, beta, gamma, w0 = _inputs(rng)
    O, W = no.norm_chunk_forward(q, k, v, beta, -1.0, C, loss, decay, gamma, w0)
    O2, W2 = no.norm_token_loop_forward(q, k, v, beta, -1.0, C, loss, decay, gamma, w0)
    np.testing.assert_allclose(O, O2, atol=1e-11)
    np.testing.assert_allclose(W, W2, atol=1e-11)


@pytest.mark.parametrize("loss", ["mse", "ip", "l1"])
def test_norm_train_view_signal_is_the_gradient(loss, rng):
    """G = d/dZ of sum_t loss(N(Z_t), V_t) (central differences)."""
    Z = rng.standard_normal((6, 5))
    v = rng.standard_normal((6, 5)) + 3.0 * np.sign(rng.standard_normal((6, 5)))   # no ties for L1

    def L(z):
        n = no.norm_f(z)[0]
        if loss == "mse":
            return 0.5 * float(((n - v) ** 2).sum())
        if loss == "l1":
            return float(np.abs(n - v).sum())
        return -float((n * v).sum())

    n, s = no.norm_f(Z)
    from oracle.ttt_oracle import loss_signal
    G = no.norm_vjp(loss_signal(n, v, loss), n, s)
    h = 1e-6
    num = np.zeros_like(Z)
    for idx in np.ndindex(Z.shape):
        zp, zm = Z.copy(), Z.copy()
        zp[idx] += h
        zm[idx] -= h
        num[idx] = (L(zp) - L(zm)) / (2 * h)
    np.testing.assert_allclose(G, num, atol=1e-7)


def test_norm_output_rows_are_normalised(rng):
    q, k, v, beta, gamma, w0 = _inputs(rng, T=20, dv=8)
    O, _ = no.norm_chunk_forward(q, k, v, beta, -1.0, 8, "mse", "scalar", gamma, w0)
    np.testing.assert_allclose(O.mean(axis=-1), 0.0, atol=1e-12)
    var = (O ** 2).mean(axis=-1)
    assert np.all(var <= 1.0) and np.all(var > 0.99)   # var / (var + eps) with var of order 1


def _fd_check(loss, decay, rng, tol=1e-7):
    q, k, v, beta, gamma, w0 = _inputs(rng, T=9, dk=3, dv=4)
    do = rng.standard_normal(v.shape)
    dwT = rng.standard_normal(w0.shape)
    C, b, h = 4, -1.0, 1e-6
    src = dict(q=q, k=k, v=v, beta=beta, gamma=gamma, w0=w0)

    def F(**over):
        a = dict(src, **over)
        O, W = no.norm_chunk_forward(a["q"], a["k"], a["v"], a["beta"], b, C, loss, decay, a["gamma"], a["w0"])
        return float((O * do).sum() + (W * dwT).sum())

    g = no.norm_chunk_backward(q, k, v, beta, b, C, do, loss, decay, gamma, w0, dwT)
    pairs = dict(q="dq", k="dk", v="dv", beta="dbeta", w0="dw0")
    if decay == "scalar":
        pairs["gamma"] = "dgamma"
    for nm, key in pairs.items():
        arr = src[nm]
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            ap, am = arr.copy(), arr.copy()
            ap[idx] += h
            am[idx] -= h
            num[idx] = (F(**{nm: ap}) - F(**{nm: am})) / (2 * h)
        an = g[key].sum(0) if nm == "gamma" else g[key]
        err = np.abs(an - num).max() / max(np.abs(num).max(), 1e-12)
        assert err < tol, (nm, err)


@pytest.mark.parametrize("loss,decay", COMBOS)
def test_norm_backward_matches_finite_differences(loss, decay, rng):
    _fd_check(loss, decay, rng)


def test_planted_norm_vjp_mistake_is_caught(rng, monkeypatch):
    """The normalisation's VJP without its n <x, n> / d term."""
    monkeypatch.setattr(no, "norm_vjp", lambda x, n, s: (x - x.mean(axis=-1, keepdims=True)) / s)
    with pytest.raises(AssertionError):
        test_norm_train_view_signal_is_the_gradient("mse", rng)
