"""Pins of the TTT-MLP oracle (two fast Linears with a nonlinearity between them)
against facts fixed outside it: a token-by-token loop, finite differences of the
train-view loss, the eta -> 0 limit, and a planted mistake.

The graph follows "Modular TTT" (summary page, "Method step details": Algorithm 1
composed over the primitives; "Experimental results": deeper fast nets).
"""
import itertools

import numpy as np
import pytest

from oracle import mlp_oracle as mo

COMBOS = list(itertools.product(["mse", "ip", "l1", "rmse"], ["none", "silu", "gelu"], ["none", "scalar"]))


@pytest.fixture
def rng():
    return np.random.default_rng(2718)


def _inputs(rng, B=1, H=2, T=11, dk=3, dh=5, dv=4):
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)      # rows L2-normalised, as in the workloads:
    k /= np.linalg.norm(k, axis=-1, keepdims=True)      # the inner descent stays stable
    v = rng.standard_normal((B, H, T, dv))
    beta = rng.standard_normal((B, H, T))
    gamma = rng.uniform(0.85, 1.0, H)
    w1 = 0.5 * rng.standard_normal((B, H, dk, dh))
    w2 = 0.5 * rng.standard_normal((B, H, dh, dv))
    return q, k, v, beta, gamma, w1, w2


@pytest.mark.parametrize("loss,act,decay", COMBOS)
@pytest.mark.parametrize("C", [1, 4, 16])
def test_mlp_chunk_form_equals_token_loop(loss, act, decay, C, rng):
    q, k, v, beta, gamma, w1, w2 = _inputs(rng)
    kw = dict(loss=loss, act=act, decay=decay, gamma=gamma, w1_0=w1, w2_0=w2)
    O, W1, W2 = mo.mlp_chunk_forward(q, k, v, beta, -3.0, C, **kw)
    Ot, W1t, W2t = mo.mlp_token_loop_forward(q, k, v, beta, -3.0, C, **kw)
    np.testing.assert_allclose(O, Ot, atol=1e-11)
    np.testing.assert_allclose(W1, W1t, atol=1e-11)
    np.testing.assert_allclose(W2, W2t, atol=1e-11)


@pytest.mark.parametrize("loss,act", list(itertools.product(["mse", "ip", "l1", "rmse"], ["none", "silu", "gelu"])))
def test_mlp_train_view_signals_are_gradients(loss, act, rng):
    """K^T G1 and A^T G2 are the gradients of the chunk's train-view loss with
    respect to W1 and W2 (central differences along random directions)."""
    _, k, v, _, _, w1, w2 = _inputs(rng, T=7)
    kc, vc, W1, W2 = k[0, 0], v[0, 0], w1[0, 0], w2[0, 0]
    _, A, G1, G2 = mo.mlp_train_view(kc, vc, W1, W2, loss, act)
    g1, g2 = kc.T @ G1, A.T @ G2
    for _ in range(3):
        e1, e2 = rng.standard_normal(W1.shape), rng.standard_normal(W2.shape)
        h = 1e-6
        num = (mo.mlp_inner_loss(kc, vc, W1 + h * e1, W2 + h * e2, loss, act) -
               mo.mlp_inner_loss(kc, vc, W1 - h * e1, W2 - h * e2, loss, act)) / (2 * h)
        an = float((g1 * e1).sum() + (g2 * e2).sum())
        assert abs(an - num) <= 1e-6 * max(1.0, abs(num)), (an, num)


@pytest.mark.parametrize("act", ["none", "silu", "gelu"])
def test_mlp_eta_to_zero(act, rng):
    """With eta -> 0 the weights only decay: O_t = f(q_t gamma^i W1) gamma^i W2 in chunk i."""
    q, k, v, beta, gamma, w1, w2 = _inputs(rng, T=12)
    C = 4
    O, _, _ = mo.mlp_chunk_forward(q, k, v, beta, -80.0, C, loss="mse", act=act, decay="scalar", gamma=gamma,
                                   w1_0=w1, w2_0=w2)
    for h in range(2):
        for t in range(12):
            g = gamma[h] ** (t // C)
            ref = mo.act_f(q[0, h, t] @ (g * w1[0, h]), act) @ (g * w2[0, h])
            np.testing.assert_allclose(O[0, h, t], ref, atol=1e-12)


def test_planted_mlp_gradient_mistake_is_caught(rng, monkeypatch):
    """G1 without the act' factor must break the gradient pin."""
    real = mo.mlp_train_view

    def wrong(k, v, W1, W2, loss, act):
        Z1, A, G1, G2 = real(k, v, W1, W2, loss, act)
        return Z1, A, G2 @ np.swapaxes(W2, -1, -2), G2
    monkeypatch.setattr(mo, "mlp_train_view", wrong)
    with pytest.raises(AssertionError):
        test_mlp_train_view_signals_are_gradients("mse", "gelu", rng)


# ---------------------------------------------------------------------------
# backward: central finite differences of the forward
# ---------------------------------------------------------------------------

def _fd_check(loss, act, decay, rng, tol=1e-7):
    q, k, v, beta, gamma, w1, w2 = _inputs(rng, T=9, dk=3, dh=5, dv=4)
    do = rng.standard_normal(v.shape)
    d1, d2 = rng.standard_normal(w1.shape), rng.standard_normal(w2.shape)
    C, b, h = 4, -1.0, 1e-6
    src = dict(q=q, k=k, v=v, beta=beta, gamma=gamma, w1=w1, w2=w2)

    def F(**over):
        a = dict(src, **over)
        O, W1, W2 = mo.mlp_chunk_forward(a["q"], a["k"], a["v"], a["beta"], b, C, loss, act, decay, a["gamma"],
                                         a["w1"], a["w2"])
        return float((O * do).sum() + (W1 * d1).sum() + (W2 * d2).sum())

    g = mo.mlp_chunk_backward(q, k, v, beta, b, C, do, loss, act, decay, gamma, w1, w2, d1, d2)
    pairs = dict(q="dq", k="dk", v="dv", beta="dbeta", w1="dw1_0", w2="dw2_0")
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
        an = g[key].sum(0) if nm == "gamma" else g[key]      # gamma is per head, shared over the batch
        err = np.abs(an - num).max() / max(np.abs(num).max(), 1e-12)
        assert err < tol, (nm, err)


@pytest.mark.parametrize("loss,act,decay", COMBOS)
def test_mlp_backward_matches_finite_differences(loss, act, decay, rng):
    _fd_check(loss, act, decay, rng)


def test_mlp_backward_zero_upstream_is_zero(rng):
    q, k, v, beta, gamma, w1, w2 = _inputs(rng)
    g = mo.mlp_chunk_backward(q, k, v, beta, -1.0, 4, np.zeros_like(v), "mse", "silu", "scalar", gamma, w1, w2)
    assert all(np.all(x == 0.0) for x in g.values())


def test_planted_mlp_backward_mistake_is_caught(rng, monkeypatch):
    """The backward with f'' dropped (the dZ1 term of G1 = P (.) f'(Z1))."""
    monkeypatch.setattr(mo, "act_d2f", lambda z, act: np.zeros_like(z))
    with pytest.raises(AssertionError):
        _fd_check("mse", "silu", "none", rng)
