"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each test ties the oracle to a closed form, a textbook recurrence, a library
routine, an invariant, or finite differences:

* the chunk form equals a token-by-token loop (every loss x act x decay);
* C = 1 with MSE + linear is the delta rule, W <- (gamma I - eta k^T k) W + eta k^T v;
* inner-product loss + linear + no decay is causal linear attention, for any C;
* the same with per-token vector decay is gated linear attention, for any C;
* the same with scalar decay equals a closed-form T x T weight matrix;
* MSE + linear chunk transitions equal the affine map (gamma I - K^T diag(eta) K) W + K^T diag(eta) V;
* eta -> 0 leaves O = f(Q W_i) with the decayed initial state;
* splitting the sequence at a chunk boundary and resuming from W_T changes nothing;
* the analytic outer backward equals central finite differences;
* the In-Place update equals its associative closed form; its guarded form
  (update clipping, document resets) matches hand-worked examples and invariants;
* and planted mistakes (in the oracle, on the CPU) make the pins fail.

The pages define the layer in "Modular TTT" (summary page, sections
"Prerequisites" and "Method step details", Algorithm 1 and its chunked dual
form) and the In-Place update in "In-Place Test-Time Training" (summary page,
"Core method and technical details").
"""
import itertools

import numpy as np
import pytest
from scipy.special import expit

from oracle import ttt_oracle as to
from oracle import inplace_oracle as io

COMBOS = list(itertools.product(["mse", "ip", "l1", "rmse"], ["none", "silu", "gelu"], ["none", "scalar", "vector"]))


def _rand_inputs(rng, B=1, H=2, T=13, dk=3, dv=4):
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv))
    beta = rng.standard_normal((B, H, T))
    gamma = rng.uniform(0.85, 1.0, H)
    la = -rng.uniform(0.01, 0.4, (B, H, T, dk))
    w0 = 0.3 * rng.standard_normal((B, H, dk, dv))
    return q, k, v, beta, gamma, la, w0


def _close(a, b, tol=1e-12):
    """max |a - b| <= tol * max(1, max |b|): fp64 agreement up to summation order."""
    scale = max(1.0, float(np.abs(b).max()))
    err = float(np.abs(np.asarray(a) - np.asarray(b)).max())
    assert err <= tol * scale, (err, scale)


def _kw(decay, gamma, la, w0, loss, act):
    return dict(loss=loss, act=act, decay=decay, gamma=gamma if decay == "scalar" else None,
                log_a=la if decay == "vector" else None, w0=w0)


# ---------------------------------------------------------------------------
# scalar pieces
# ---------------------------------------------------------------------------

def test_lr_gate_special_values():
    # eta = 2 Sigmoid(beta + b): beta = -b gives exactly 1; the range is (0, 2)
    assert to.lr_gate(np.array([4.0]), -4.0)[0] == 1.0
    assert abs(to.lr_gate(np.array([50.0]), 0.0)[0] - 2.0) < 1e-15
    assert to.lr_gate(np.array([-800.0]), 0.0)[0] == 0.0
    x = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(to.lr_gate(x, -4.0), 2 * expit(x - 4.0), rtol=1e-15, atol=0)
    # the small-lr initialisation b = -4 starts at eta_0 = 2 / (1 + e^4)
    assert abs(to.lr_gate(np.array([0.0]), -4.0)[0] - 2.0 / (1.0 + np.exp(4.0))) < 1e-16


def test_silu_and_derivatives():
    z = np.linspace(-12, 12, 241)
    np.testing.assert_allclose(to.act_f(z, "silu"), z * expit(z), rtol=1e-14, atol=1e-300)
    h = 1e-5
    d1 = (to.act_f(z + h, "silu") - to.act_f(z - h, "silu")) / (2 * h)
    d2 = (to.act_df(z + h, "silu") - to.act_df(z - h, "silu")) / (2 * h)
    np.testing.assert_allclose(to.act_df(z, "silu"), d1, atol=1e-9)
    np.testing.assert_allclose(to.act_d2f(z, "silu"), d2, atol=1e-9)
    assert to.act_df(np.array([0.0]), "silu")[0] == 0.5
    assert to.act_d2f(np.array([0.0]), "silu")[0] == 0.5
    assert np.all(to.act_df(z, "none") == 1) and np.all(to.act_d2f(z, "none") == 0)


# ---------------------------------------------------------------------------
# forward pins
# ---------------------------------------------------------------------------

def test_gelu_and_derivatives():
    """GELU(z) = z Phi(z): Phi(1) = 0.841344746068543 and Phi(-1) = 0.158655253931457
    (normal tables), GELU'(0) = 1/2, GELU''(0) = 2 phi(0) = sqrt(2/pi); the
    derivatives agree with central differences."""
    np.testing.assert_allclose(to.act_f(np.array([1.0, -1.0, 0.0]), "gelu"),
                               [0.8413447460685429, -0.15865525393145707, 0.0], atol=1e-14)
    assert abs(to.act_df(np.array([0.0]), "gelu")[0] - 0.5) < 1e-15
    assert abs(to.act_d2f(np.array([0.0]), "gelu")[0] - np.sqrt(2.0 / np.pi)) < 1e-15
    np.testing.assert_allclose(to.act_f(np.array([12.0, -12.0]), "gelu"), [12.0, 0.0], atol=1e-12)
    z = np.linspace(-4, 4, 33)
    h = 1e-5
    d1 = (to.act_f(z + h, "gelu") - to.act_f(z - h, "gelu")) / (2 * h)
    d2 = (to.act_df(z + h, "gelu") - to.act_df(z - h, "gelu")) / (2 * h)
    np.testing.assert_allclose(to.act_df(z, "gelu"), d1, atol=1e-9)
    np.testing.assert_allclose(to.act_d2f(z, "gelu"), d2, atol=1e-9)


@pytest.mark.parametrize("loss,act,decay", COMBOS)
def test_chunk_form_equals_token_loop(loss, act, decay, rng):
    q, k, v, beta, gamma, la, w0 = _rand_inputs(rng)
    kw = _kw(decay, gamma, la, w0, loss, act)
    for C in (1, 4, 5, 13):
        O, WT = to.chunk_forward(q, k, v, beta, -0.5, C, **kw)
        O2, WT2 = to.token_loop_forward(q, k, v, beta, -0.5, C, **kw)
        _close(O, O2)
        _close(WT, WT2)


@pytest.mark.parametrize("decay", ["none", "scalar"])
def test_chunk_one_is_delta_rule(decay, rng):
    q, k, v, beta, gamma, la, w0 = _rand_inputs(rng, H=1, T=17)
    g = gamma[0] if decay == "scalar" else 1.0
    O, WT = to.chunk_forward(q, k, v, beta, 0.3, 1, **_kw(decay, gamma, la, w0, "mse", "none"))
    eta = 2 * expit(beta + 0.3)
    W = w0[0, 0].copy()
    I = np.eye(W.shape[0])
    for t in range(q.shape[2]):
        kt, vt, qt, et = k[0, 0, t], v[0, 0, t], q[0, 0, t], eta[0, 0, t]
        P = np.outer(kt, kt)
        # the query sees its own token's write, before the per-chunk decay
        o = qt @ ((I - et * P) @ W + et * np.outer(kt, vt))
        np.testing.assert_allclose(O[0, 0, t], o, atol=1e-12)
        W = (g * I - et * P) @ W + et * np.outer(kt, vt)
    np.testing.assert_allclose(WT[0, 0], W, atol=1e-12)


@pytest.mark.parametrize("C", [1, 3, 4, 8, 40])
def test_ip_linear_is_causal_linear_attention(C, rng):
    q, k, v, beta, gamma, la, w0 = _rand_inputs(rng, B=2, H=2, T=40, dk=5, dv=6)
    O, WT = to.chunk_forward(q, k, v, beta, 0.1, C, **_kw("none", gamma, la, w0, "ip", "none"))
    eta = 2 * expit(beta + 0.1)
    M = np.tril(np.ones((40, 40)))
    A = (q @ np.swapaxes(k, -1, -2)) * M * eta[:, :, None, :]
    ref = q @ w0 + A @ v
    np.testing.assert_allclose(O, ref, atol=1e-12)
    np.testing.assert_allclose(WT, w0 + np.swapaxes(k * eta[..., None], -1, -2) @ v, atol=1e-12)


@pytest.mark.parametrize("C", [1, 4, 7, 30])
def test_ip_linear_vector_decay_is_gated_linear_attention(C, rng):
    q, k, v, beta, gamma, la, w0 = _rand_inputs(rng, B=1, H=2, T=30, dk=4, dv=3)
    O, WT = to.chunk_forward(q, k, v, beta, 0.0, C, **_kw("vector", gamma, la, w0, "ip", "none"))
    eta = 2 * expit(beta)
    for h in range(2):
        S = w0[0, h].copy()
        for t in range(30):
            S = np.exp(la[0, h, t])[:, None] * S + eta[0, h, t] * np.outer(k[0, h, t], v[0, h, t])
            np.testing.assert_allclose(O[0, h, t], q[0, h, t] @ S, atol=1e-12)
        np.testing.assert_allclose(WT[0, h], S, atol=1e-12)


@pytest.mark.parametrize("C", [1, 4, 6])
def test_ip_linear_scalar_decay_closed_form(C, rng):
    T = 23
    q, k, v, beta, gamma, la, w0 = _rand_inputs(rng, B=1, H=2, T=T, dk=4, dv=3)
    O, WT = to.chunk_forward(q, k, v, beta, 0.0, C, **_kw("scalar", gamma, la, w0, "ip", "none"))
    eta = 2 * expit(beta)
    ch = np.arange(T) // C
    n = (T + C - 1) // C
    for h in range(2):
        g = gamma[h]
        M = np.zeros((T, T))
        for t in range(T):
            for s in range(T):
                if ch[s] < ch[t]:
                    M[t, s] = g ** (ch[t] - ch[s] - 1)
                elif ch[s] == ch[t] and s <= t:
                    M[t, s] = 1.0
        Wq = np.stack([g ** ch[t] * w0[0, h] for t in range(T)])      # [T, dk, dv]
        ref = np.einsum("td,tde->te", q[0, h], Wq) + \
            ((q[0, h] @ k[0, h].T) * M * eta[0, h][None, :]) @ v[0, h]
        np.testing.assert_allclose(O[0, h], ref, atol=1e-12)
        wt = g ** n * w0[0, h] + sum(g ** (n - 1 - ch[s]) * eta[0, h, s] *
                                    np.outer(k[0, h, s], v[0, h, s]) for s in range(T))
        np.testing.assert_allclose(WT[0, h], wt, atol=1e-12)


@pytest.mark.parametrize("decay", ["none", "scalar"])
def test_mse_linear_transition_is_affine(decay, rng):
    q, k, v, beta, gamma, la, w0 = _rand_inputs(rng, B=1, H=2, T=16, dk=3, dv=2)
    C = 4
    O, WT, ck = to.chunk_forward(q, k, v, beta, -0.2, C, return_ckpt=True,
                                 **_kw(decay, gamma, la, w0, "mse", "none"))
    eta = 2 * expit(beta - 0.2)
    for h in range(2):
        g = gamma[h] if decay == "scalar" else 1.0
        for i in range(4):
            K = k[0, h, i * C:(i + 1) * C]
            V = v[0, h, i * C:(i + 1) * C]
            D = np.diag(eta[0, h, i * C:(i + 1) * C])
            nxt = (g * np.eye(3) - K.T @ D @ K) @ ck[0, h, i] + K.T @ D @ V
            ref = ck[0, h, i + 1] if i < 3 else WT[0, h]
            np.testing.assert_allclose(ref, nxt, atol=1e-12)


@pytest.mark.parametrize("act", ["none", "silu", "gelu"])
@pytest.mark.parametrize("decay", ["none", "scalar", "vector"])
def test_eta_to_zero(act, decay, rng):
    q, k, v, beta, gamma, la, w0 = _rand_inputs(rng, B=1, H=2, T=12, dk=3, dv=3)
    C = 4
    O, WT = to.chunk_forward(q, k, v, beta, -80.0, C, **_kw(decay, gamma, la, w0, "mse", act))
    for h in range(2):
        for t in range(12):
            if decay == "scalar":
                W = gamma[h] ** (t // C) * w0[0, h]
            elif decay == "vector":
                W = np.exp(la[0, h, :t + 1].sum(0))[:, None] * w0[0, h]
            else:
                W = w0[0, h]
            np.testing.assert_allclose(O[0, h, t], to.act_f(q[0, h, t] @ W, act), atol=1e-12)


@pytest.mark.parametrize("loss,act,decay", COMBOS)
def test_split_and_resume(loss, act, decay, rng):
    q, k, v, beta, gamma, la, w0 = _rand_inputs(rng, T=24)
    C, cut = 4, 12
    kw = _kw(decay, gamma, la, w0, loss, act)
    O, WT = to.chunk_forward(q, k, v, beta, -1.0, C, **kw)
    kw1 = dict(kw, log_a=None if la is None or decay != "vector" else la[:, :, :cut])
    O1, W1 = to.chunk_forward(q[:, :, :cut], k[:, :, :cut], v[:, :, :cut], beta[:, :, :cut],
                              -1.0, C, **kw1)
    kw2 = dict(kw, w0=W1, log_a=None if decay != "vector" else la[:, :, cut:])
    O2, W2 = to.chunk_forward(q[:, :, cut:], k[:, :, cut:], v[:, :, cut:], beta[:, :, cut:],
                              -1.0, C, **kw2)
    np.testing.assert_allclose(np.concatenate([O1, O2], axis=2), O, atol=1e-13)
    np.testing.assert_allclose(W2, WT, atol=1e-13)


# ---------------------------------------------------------------------------
# backward pins: central finite differences of the forward
# ---------------------------------------------------------------------------

def _fd_grads(q, k, v, beta, gamma, la, w0, do, dwT, b, C, kw, h=1e-6):
    decay = kw["decay"]

    def F(**over):
        args = dict(q=q, k=k, v=v, beta=beta, gamma=gamma, la=la, w0=w0)
        args.update(over)
        kk = dict(kw, w0=args["w0"], gamma=args["gamma"] if decay == "scalar" else None,
                  log_a=args["la"] if decay == "vector" else None)
        O, WT = to.chunk_forward(args["q"], args["k"], args["v"], args["beta"], b, C, **kk)
        return float((O * do).sum() + (WT * dwT).sum())

    names = ["q", "k", "v", "beta", "w0"] + (["gamma"] if decay == "scalar" else []) + \
        (["la"] if decay == "vector" else [])
    src = dict(q=q, k=k, v=v, beta=beta, gamma=gamma, la=la, w0=w0)
    out = {}
    for nm in names:
        arr = src[nm]
        g = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            ap = arr.copy()
            ap[idx] += h
            am = arr.copy()
            am[idx] -= h
            g[idx] = (F(**{nm: ap}) - F(**{nm: am})) / (2 * h)
        out[nm] = g
    return out


@pytest.mark.parametrize("loss,act,decay", COMBOS)
def test_backward_matches_finite_differences(loss, act, decay, rng):
    q, k, v, beta, gamma, la, w0 = _rand_inputs(rng, B=1, H=2, T=10, dk=2, dv=3)
    do = rng.standard_normal(v.shape)
    dwT = rng.standard_normal(w0.shape)
    kw = _kw(decay, gamma, la, w0, loss, act)
    C, b = 4, -0.7
    g = to.chunk_backward(q, k, v, beta, b, C, do, d_wT=dwT, **kw)
    fd = _fd_grads(q, k, v, beta, gamma, la, w0, do, dwT, b, C, kw)
    pairs = dict(q="dq", k="dk", v="dv", beta="dbeta", w0="dw0", gamma="dgamma", la="dlog_a")
    for nm, num in fd.items():
        an = g[pairs[nm]]
        if nm == "gamma":
            an = an.sum(0)                         # gamma is per head, shared over batch
        err = np.abs(an - num).max() / max(np.abs(num).max(), 1e-12)
        assert err < 1e-7, (nm, err)


@pytest.mark.parametrize("loss,act,decay", [("ip", "silu", "vector"), ("mse", "silu", "scalar")])
def test_backward_directional_derivative_medium(loss, act, decay, rng):
    """Random-direction check at a shape with several full chunks and d = 16."""
    q, k, v, beta, gamma, la, w0 = _rand_inputs(rng, B=1, H=1, T=96, dk=16, dv=16)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    do = rng.standard_normal(v.shape)
    kw = _kw(decay, gamma, la, w0, loss, act)
    C, b, h = 32, -2.0, 1e-5
    g = to.chunk_backward(q, k, v, beta, b, C, do, **kw)
    dirs = {nm: rng.standard_normal(x.shape) for nm, x in
            dict(q=q, k=k, v=v, beta=beta, w0=w0).items()}
    if decay == "vector":
        dirs["la"] = rng.standard_normal(la.shape) * 0.1
    if decay == "scalar":
        dirs["gamma"] = rng.standard_normal(gamma.shape) * 0.1

    def F(sign):
        a = dict(q=q, k=k, v=v, beta=beta, w0=w0, la=la, gamma=gamma)
        for nm, d in dirs.items():
            a[nm] = a[nm] + sign * h * d
        kk = dict(kw, w0=a["w0"], gamma=a["gamma"] if decay == "scalar" else None,
                  log_a=a["la"] if decay == "vector" else None)
        return float((to.chunk_forward(a["q"], a["k"], a["v"], a["beta"], b, C, **kk)[0] * do).sum())

    num = (F(1) - F(-1)) / (2 * h)
    an = sum(float((g[key] * dirs[nm]).sum()) for nm, key in
             dict(q="dq", k="dk", v="dv", beta="dbeta", w0="dw0").items())
    if decay == "vector":
        an += float((g["dlog_a"] * dirs["la"]).sum())
    if decay == "scalar":
        an += float((g["dgamma"].sum(0) * dirs["gamma"]).sum())
    assert abs(an - num) <= 1e-6 * max(1.0, abs(num)), (an, num)


# ---------------------------------------------------------------------------
# In-Place TTT
# ---------------------------------------------------------------------------

def test_inplace_associative_closed_form(rng):
    B, T, dff, dm, C, eta = 2, 20, 7, 5, 4, 0.3
    z = rng.standard_normal((B, T, dff))
    vh = rng.standard_normal((B, T, dm))
    w0 = rng.standard_normal((B, dm, dff))
    O, W = io.inplace_forward(z, vh, w0, C, eta)
    for b in range(B):
        for i in range(T // C):
            Zi = z[b, i * C:(i + 1) * C]
            ref = Zi @ w0[b].T
            for j in range(i):
                Zj = z[b, j * C:(j + 1) * C]
                ref = ref + eta * (Zi @ Zj.T) @ vh[b, j * C:(j + 1) * C]
            np.testing.assert_allclose(O[b, i * C:(i + 1) * C], ref, atol=1e-12)
        np.testing.assert_allclose(W[b], w0[b] + eta * vh[b].T @ z[b], atol=1e-12)
    rows = [0, 3]
    Or, Wr = io.inplace_rows(z, vh, w0[:, rows], rows, C, eta)
    np.testing.assert_allclose(Or, O[:, :, rows], atol=1e-12)
    np.testing.assert_allclose(Wr, W[:, rows], atol=1e-12)


def test_inplace_ragged_tail_and_single_chunk(rng):
    z = rng.standard_normal((1, 10, 6))
    vh = rng.standard_normal((1, 10, 3))
    w0 = rng.standard_normal((1, 3, 6))
    O, W = io.inplace_forward(z, vh, w0, 16, 0.1)       # one chunk: O reads W0 only
    np.testing.assert_allclose(O[0], z[0] @ w0[0].T, atol=1e-13)
    O4, W4 = io.inplace_forward(z, vh, w0, 4, 0.1)       # 4 + 4 + 2 tokens
    np.testing.assert_allclose(W4, W, atol=1e-13)


@pytest.mark.parametrize("C", [3, 4, 20])
def test_inplace_backward_matches_finite_differences(C, rng):
    """L = <dO, O> + <dW_T, W_T> along random directions of z, vhat and w0: the
    analytic derivative equals central differences (the forward is a polynomial
    of degree three in the inputs, so the difference is exact up to O(h^2))."""
    B, T, dff, dm, eta = 2, 10, 5, 3, 0.3
    z = rng.standard_normal((B, T, dff))
    vh = rng.standard_normal((B, T, dm))
    w0 = rng.standard_normal((B, dm, dff))
    d_o = rng.standard_normal((B, T, dm))
    dwT = rng.standard_normal((B, dm, dff))

    def loss(z_, v_, w_):
        O, W = io.inplace_forward(z_, v_, w_, C, eta)
        return float((d_o * O).sum() + (dwT * W).sum())

    dz, dv, dw0 = io.inplace_backward(z, vh, w0, C, eta, d_o, dwT)
    for _ in range(3):
        ez, ev, ew = (rng.standard_normal(x.shape) for x in (z, vh, w0))
        h = 1e-4
        num = (loss(z + h * ez, vh + h * ev, w0 + h * ew) - loss(z - h * ez, vh - h * ev, w0 - h * ew)) / (2 * h)
        an = float((dz * ez).sum() + (dv * ev).sum() + (dw0 * ew).sum())
        assert abs(an - num) <= 1e-6 * max(1.0, abs(num)), (an, num)


def test_inplace_backward_single_chunk_closed_form(rng):
    """One chunk: O = Z W0^T and W_T = W0 + eta V^T Z, so dZ = dO W0 + eta V dW_T,
    dV = eta Z dW_T^T, dW0 = dW_T + dO^T Z; without dW_T the update leaves no trace."""
    z = rng.standard_normal((1, 6, 4))
    vh = rng.standard_normal((1, 6, 3))
    w0 = rng.standard_normal((1, 3, 4))
    d_o = rng.standard_normal((1, 6, 3))
    dz, dv, dw0 = io.inplace_backward(z, vh, w0, 8, 0.5, d_o)
    np.testing.assert_allclose(dz[0], d_o[0] @ w0[0], atol=1e-13)
    np.testing.assert_allclose(dv, 0.0, atol=1e-15)
    np.testing.assert_allclose(dw0[0], d_o[0].T @ z[0], atol=1e-13)


def test_inplace_backward_sampled_agrees(rng):
    """The column / token form used at full size gives the same numbers as the
    whole backward (which the finite-difference pin ties down)."""
    B, T, dff, dm, C, eta = 2, 23, 7, 4, 5, 0.2
    z = rng.standard_normal((B, T, dff))
    vh = rng.standard_normal((B, T, dm))
    w0 = rng.standard_normal((B, dm, dff))
    d_o = rng.standard_normal((B, T, dm))
    dwT = rng.standard_normal((B, dm, dff))
    dz, dv, dw0 = io.inplace_backward(z, vh, w0, C, eta, d_o, dwT)
    cols, toks = [0, 3, 6], [0, 4, 5, 17, 22]
    sz, sw, sv = io.inplace_backward_sampled(z, vh, w0[:, :, cols], cols, toks, C, eta, d_o, dwT[:, :, cols], dwT)
    np.testing.assert_allclose(sz, dz[:, :, cols], atol=1e-12)
    np.testing.assert_allclose(sw, dw0[:, :, cols], atol=1e-12)
    np.testing.assert_allclose(sv, dv[:, toks], atol=1e-12)


def test_inplace_guarded_hand_worked_scalar():
    """d_model = d_ff = 1, C = 2, eta = 1, two sequences; the first has a second
    document starting at t = 3 (w_init = 10), the second has none (W0 = 0).

    Sequence 0, z = (1, 2, 3, 1, 2), v = (1, 1, 1, 2, -3), W0 = 1.  Chunks count
    from each document's start: [0,2), [2,3) | [3,5).  Without clipping:
      [0,2): O = (1, 2), dW = 1 + 2 = 3 -> W = 4;  [2,3): O = 12, dW = 3 -> W = 7;
      reset W = 10;  [3,5): O = (10, 20), dW = 2 - 6 = -4 -> W = 6.
    With tau = 2.5 every update is cut to magnitude 2.5 with its sign:
      W: 1 -> 3.5, O2 = 10.5, W -> 6; reset 10: O = (10, 20), W -> 7.5.
    Sequence 1, z = v = 1, W0 = 0, no document start: chunks [0,2), [2,4), [4,5):
      O = (0, 0, 2, 2, 4), W = 5 unclipped; with tau = 2.5 (updates 2, 2, 1
      stay below it) the same.
    """
    z = np.array([[1, 2, 3, 1, 2], [1, 1, 1, 1, 1]], dtype=float).reshape(2, 5, 1)
    v = np.array([[1, 1, 1, 2, -3], [1, 1, 1, 1, 1]], dtype=float).reshape(2, 5, 1)
    w0 = np.array([1.0, 0.0]).reshape(2, 1, 1)
    wi = np.array([10.0, 99.0]).reshape(2, 1, 1)
    starts = [[3], []]
    O, W = io.inplace_forward_guarded(z, v, w0, 2, 1.0, None, starts, wi)
    np.testing.assert_allclose(O[..., 0], [[1, 2, 12, 10, 20], [0, 0, 2, 2, 4]], atol=1e-14)
    np.testing.assert_allclose(W.ravel(), [6, 5], atol=1e-14)
    O, W = io.inplace_forward_guarded(z, v, w0, 2, 1.0, 2.5, starts, wi)
    np.testing.assert_allclose(O[..., 0], [[1, 2, 10.5, 10, 20], [0, 0, 2, 2, 4]], atol=1e-14)
    np.testing.assert_allclose(W.ravel(), [7.5, 5], atol=1e-14)
    np.testing.assert_allclose(io.update_norms(z, v, 2, 1.0, starts), [3, 3, 4, 2, 2, 1], atol=1e-14)


def test_inplace_guarded_hand_worked_matrix_clip():
    """C = 1, eta = 1, tau = 1, W0 = I (2 x 2), O_t = W z_t (rows of W dotted with z).

    t0: z = (3, 4), v = (1, 0): O = (3, 4); dW = v^T z = [[3, 4], [0, 0]], norm 5,
        cut to [[0.6, 0.8], [0, 0]]: W = [[1.6, 0.8], [0, 1]].
    t1: z = (1, 0), v = (0, 2): O = (1.6, 0); dW = [[0, 0], [2, 0]], norm 2, cut to
        [[0, 0], [1, 0]]: W = [[1.6, 0.8], [1, 1]].
    t2: z = (0, 1), v = (0.1, 0): O = (0.8, 1); dW = [[0, 0.1], [0, 0]], norm 0.1,
        kept: W = [[1.6, 0.9], [1, 1]].
    """
    z = np.array([[3, 4], [1, 0], [0, 1]], dtype=float)[None]
    v = np.array([[1, 0], [0, 2], [0.1, 0]], dtype=float)[None]
    O, W = io.inplace_forward_guarded(z, v, np.eye(2)[None], 1, 1.0, 1.0)
    np.testing.assert_allclose(O[0], [[3, 4], [1.6, 0], [0.8, 1]], atol=1e-14)
    np.testing.assert_allclose(W[0], [[1.6, 0.9], [1, 1]], atol=1e-14)


def test_inplace_guarded_documents_are_independent_streams(rng):
    """With resets, each document equals a fresh run of the plain apply-then-update
    over its own tokens (the first from W0, the others from w_init); without
    starts or clipping the guarded form is the plain one."""
    B, T, dff, dm, C, eta = 2, 23, 6, 4, 4, 0.2
    z = rng.standard_normal((B, T, dff))
    vh = rng.standard_normal((B, T, dm))
    w0 = rng.standard_normal((B, dm, dff))
    wi = rng.standard_normal((B, dm, dff))
    starts = [[5, 14], [9]]
    O, W = io.inplace_forward_guarded(z, vh, w0, C, eta, None, starts, wi)
    for b in range(B):
        bounds = [0] + starts[b] + [T]
        for j in range(len(bounds) - 1):
            a, e = bounds[j], bounds[j + 1]
            init = (w0 if j == 0 else wi)[b:b + 1]
            Od, Wd = io.inplace_forward(z[b:b + 1, a:e], vh[b:b + 1, a:e], init, C, eta)
            np.testing.assert_allclose(O[b, a:e], Od[0], atol=1e-12)
        np.testing.assert_allclose(W[b], Wd[0], atol=1e-12)
    Op, Wp = io.inplace_forward(z, vh, w0, C, eta)
    Og, Wg = io.inplace_forward_guarded(z, vh, w0, C, eta)
    np.testing.assert_allclose(Og, Op, atol=1e-13)
    np.testing.assert_allclose(Wg, Wp, atol=1e-13)


def test_inplace_guarded_clip_invariants(rng):
    """Every applied update has Frobenius norm min(||dW_i||, tau) and points the
    way of the unclipped one (states read off prefix runs, which end on chunk
    boundaries); the sampled-rows form agrees given the per-chunk scales."""
    B, T, dff, dm, C, eta = 1, 16, 5, 3, 4, 0.5
    z = rng.standard_normal((B, T, dff))
    vh = rng.standard_normal((B, T, dm))
    w0 = rng.standard_normal((B, dm, dff))
    norms = io.update_norms(z, vh, C, eta)
    tau = float(np.median(norms))           # some chunks clip, some do not
    assert (norms > tau).any() and (norms <= tau).any()
    prev = w0[0]
    for i in range(T // C):
        _, Wc = io.inplace_forward_guarded(z[:, :(i + 1) * C], vh[:, :(i + 1) * C], w0, C, eta, tau)
        _, Wu = io.inplace_forward_guarded(z[:, i * C:(i + 1) * C], vh[:, i * C:(i + 1) * C], prev[None], C, eta)
        d_clip, d_free = Wc[0] - prev, Wu[0] - prev
        assert abs(np.linalg.norm(d_clip) - min(np.linalg.norm(d_free), tau)) < 1e-12
        cos = (d_clip * d_free).sum() / (np.linalg.norm(d_clip) * np.linalg.norm(d_free))
        assert abs(cos - 1.0) < 1e-12
        prev = Wc[0]
    starts = [[6]]
    wi = rng.standard_normal((B, dm, dff))
    n2 = io.update_norms(z, vh, C, eta, starts)
    O, W = io.inplace_forward_guarded(z, vh, w0, C, eta, tau, starts, wi)
    rows = [0, 2]
    Or, Wr = io.inplace_rows_guarded(z, vh, w0[:, rows], wi[:, rows], rows, C, eta,
                                     np.minimum(1.0, tau / n2), starts)
    np.testing.assert_allclose(Or, O[:, :, rows], atol=1e-12)
    np.testing.assert_allclose(Wr, W[:, rows], atol=1e-12)


def _tau_between(norms):
    """A clip threshold halfway between two neighbouring update norms (some
    chunks clip, some do not) and its distance to the nearest norm."""
    ns = np.sort(norms)
    k = int(np.argmax(np.diff(ns)))
    tau = 0.5 * (ns[k] + ns[k + 1])
    return tau, float(np.min(np.abs(norms - tau)))


def test_inplace_guarded_backward_matches_finite_differences(rng):
    """L = <dO, O> + <dW_T, W_T> of the guarded forward (clipping on some chunks
    and off on others, a document start in each sequence, short chunks at the
    document ends) along random directions of z, vhat, w0 and w_init: the
    analytic derivative equals central differences.  tau sits between two
    update norms, so no norm crosses it within the step."""
    B, T, dff, dm, C, eta = 2, 13, 5, 3, 3, 0.4
    z = rng.standard_normal((B, T, dff))
    vh = rng.standard_normal((B, T, dm))
    w0 = rng.standard_normal((B, dm, dff))
    wi = rng.standard_normal((B, dm, dff))
    d_o = rng.standard_normal((B, T, dm))
    dwT = rng.standard_normal((B, dm, dff))
    starts = [[5], [8]]
    norms = io.update_norms(z, vh, C, eta, starts)
    tau, margin = _tau_between(norms)
    assert (norms > tau).sum() >= 2 and (norms < tau).sum() >= 2 and margin > 1e-2

    def loss(z_, v_, w_, i_):
        O, W = io.inplace_forward_guarded(z_, v_, w_, C, eta, tau, starts, i_)
        return float((d_o * O).sum() + (dwT * W).sum())

    dz, dv, dw0, dwi = io.inplace_backward_guarded(z, vh, w0, C, eta, d_o, dwT, tau, starts, wi)
    for _ in range(4):
        ez, ev, ew, ei = (rng.standard_normal(x.shape) for x in (z, vh, w0, wi))
        h = 1e-5
        num = (loss(z + h * ez, vh + h * ev, w0 + h * ew, wi + h * ei) -
               loss(z - h * ez, vh - h * ev, w0 - h * ew, wi - h * ei)) / (2 * h)
        an = float((dz * ez).sum() + (dv * ev).sum() + (dw0 * ew).sum() + (dwi * ei).sum())
        assert abs(an - num) <= 1e-6 * max(1.0, abs(num)), (an, num)


def test_inplace_guarded_backward_without_safeguards_is_the_plain_one(rng):
    """No threshold and no document start: the plain backward, and no w_init term."""
    B, T, dff, dm, C, eta = 2, 11, 4, 3, 4, 0.3
    z = rng.standard_normal((B, T, dff))
    vh = rng.standard_normal((B, T, dm))
    w0 = rng.standard_normal((B, dm, dff))
    d_o = rng.standard_normal((B, T, dm))
    dwT = rng.standard_normal((B, dm, dff))
    ref = io.inplace_backward(z, vh, w0, C, eta, d_o, dwT)
    got = io.inplace_backward_guarded(z, vh, w0, C, eta, d_o, dwT)
    for r, g in zip(ref, got):
        np.testing.assert_allclose(g, r, atol=1e-12)
    np.testing.assert_array_equal(got[3], 0.0)


def test_inplace_guarded_backward_clip_is_scale_free(rng):
    """One clipped chunk, dO = 0: W_T = W0 + tau D / ||D|| does not move when D is
    rescaled, so along dW_T = D / ||D|| (where L = <dW_T, W_T> is stationary in D)
    z and vhat get no gradient; along a dW_T orthogonal to D the clip acts as the
    fixed factor s = tau / ||D||: the unclipped gradients times s."""
    T, dff, dm, eta = 6, 4, 3, 0.5
    z = rng.standard_normal((1, T, dff))
    vh = rng.standard_normal((1, T, dm))
    w0 = rng.standard_normal((1, dm, dff))
    d_o = np.zeros((1, T, dm))
    D = eta * vh[0].T @ z[0]
    n = np.linalg.norm(D)
    tau = 0.25 * n
    dz, dv, dw0, _ = io.inplace_backward_guarded(z, vh, w0, T, eta, d_o, (D / n)[None], tau)
    np.testing.assert_allclose(dz, 0.0, atol=1e-13)
    np.testing.assert_allclose(dv, 0.0, atol=1e-13)
    np.testing.assert_allclose(dw0[0], D / n, atol=1e-15)
    R = rng.standard_normal((dm, dff))
    P = R - (R * D).sum() / n ** 2 * D                                  # orthogonal to D
    dz, dv, _, _ = io.inplace_backward_guarded(z, vh, w0, T, eta, d_o, P[None], tau)
    dzu, dvu, _ = io.inplace_backward(z, vh, w0, T, eta, d_o, P[None])
    np.testing.assert_allclose(dz, 0.25 * dzu, atol=1e-13)
    np.testing.assert_allclose(dv, 0.25 * dvu, atol=1e-13)


def test_inplace_guarded_backward_documents_are_independent(rng):
    """With resets each document's derivatives are those of a separate stream:
    the last document sees dW_T, the others a zero final adjoint (their last
    state is discarded); dL/dw0 is the first document's, dL/dw_init the sum of
    the others'."""
    B, T, dff, dm, C, eta = 2, 17, 4, 3, 3, 0.3
    z = rng.standard_normal((B, T, dff))
    vh = rng.standard_normal((B, T, dm))
    w0 = rng.standard_normal((B, dm, dff))
    wi = rng.standard_normal((B, dm, dff))
    d_o = rng.standard_normal((B, T, dm))
    dwT = rng.standard_normal((B, dm, dff))
    starts = [[4, 11], [7]]
    tau = float(np.median(io.update_norms(z, vh, C, eta, starts)))
    dz, dv, dw0, dwi = io.inplace_backward_guarded(z, vh, w0, C, eta, d_o, dwT, tau, starts, wi)
    for b in range(B):
        bounds = [0] + starts[b] + [T]
        acc = np.zeros((dm, dff))
        for j in range(len(bounds) - 1):
            a, e = bounds[j], bounds[j + 1]
            init = (w0 if j == 0 else wi)[b:b + 1]
            fin = dwT[b:b + 1] if j == len(bounds) - 2 else None
            rz, rv, r0, _ = io.inplace_backward_guarded(z[b:b + 1, a:e], vh[b:b + 1, a:e], init, C, eta,
                                                        d_o[b:b + 1, a:e], fin, tau)
            np.testing.assert_allclose(dz[b, a:e], rz[0], atol=1e-12)
            np.testing.assert_allclose(dv[b, a:e], rv[0], atol=1e-12)
            if j == 0:
                np.testing.assert_allclose(dw0[b], r0[0], atol=1e-12)
            else:
                acc += r0[0]
        np.testing.assert_allclose(dwi[b], acc, atol=1e-12)


def test_l1_first_chunk_is_linear_attention_on_signs(rng):
    """From W0 = 0 without an act, the L1 train view's signal is sign(0 - V) = -sign(V):
    the first chunk's output is causal linear attention on sign(V) (diagonal included)
    and its state is K^T diag(eta) sign(V)."""
    q, k, v, beta, gamma, la, w0 = _rand_inputs(rng, B=1, H=2, T=6, dk=3, dv=4)
    O, WT = to.chunk_forward(q, k, v, beta, 0.2, 6, **_kw("none", gamma, la, np.zeros_like(w0), "l1", "none"))
    eta = 2 * expit(beta + 0.2)
    sv = np.where(v > 0, 1.0, np.where(v < 0, -1.0, 0.0))
    kT = np.swapaxes(k, -1, -2)
    A = (q @ kT) * np.tril(np.ones((6, 6))) * eta[:, :, None, :]
    np.testing.assert_allclose(O, A @ sv, atol=1e-12)
    np.testing.assert_allclose(WT, kT @ (eta[..., None] * sv), atol=1e-12)


def test_l1_signal_is_the_derivative_of_the_absolute_error(rng):
    x = rng.standard_normal(50)
    v = rng.standard_normal(50)
    h = 1e-7
    num = (np.abs(x + h - v) - np.abs(x - h - v)) / (2 * h)
    np.testing.assert_allclose(to.loss_signal(x, v, "l1"), num, atol=1e-6)
    assert to.loss_signal(np.array([1.5]), np.array([1.5]), "l1")[0] == 0.0  # a tie


# ---------------------------------------------------------------------------
# planted mistakes: each must break at least one pin
# ---------------------------------------------------------------------------

def _linear_attention_error(rng):
    q, k, v, beta, gamma, la, w0 = _rand_inputs(rng, B=1, H=1, T=16, dk=3, dv=3)
    O, _ = to.chunk_forward(q, k, v, beta, 0.0, 4, **_kw("none", gamma, la, w0, "ip", "none"))
    eta = 2 * expit(beta)
    A = (q @ np.swapaxes(k, -1, -2)) * np.tril(np.ones((16, 16))) * eta[:, :, None, :]
    return np.abs(O - (q @ w0 + A @ v)).max()


def test_planted_strict_mask_is_caught(rng, monkeypatch):
    assert _linear_attention_error(rng) < 1e-12
    monkeypatch.setattr(to, "_tril", lambda c: np.tril(np.ones((c, c)), -1))
    assert _linear_attention_error(rng) > 1e-3


def test_planted_gate_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(to, "lr_gate", lambda beta, b: to.sigmoid(np.asarray(beta) + b))
    with pytest.raises(AssertionError):
        test_lr_gate_special_values()


def test_planted_backward_mistake_is_caught(rng, monkeypatch):
    monkeypatch.setattr(to, "act_d2f", lambda z, act: np.zeros_like(z))
    with pytest.raises(AssertionError):
        test_backward_matches_finite_differences("ip", "silu", "none", rng)


def test_planted_decay_sign_is_caught(rng, monkeypatch):
    real = to._decay_pieces

    def flipped(q, k, la, decay, gamma_bh):
        return real(q, k, None if la is None else -la, decay, gamma_bh)

    monkeypatch.setattr(to, "_decay_pieces", flipped)
    with pytest.raises(AssertionError):
        test_ip_linear_vector_decay_is_gated_linear_attention(4, rng)


def test_planted_gelu_mistake_is_caught(monkeypatch):
    """GELU's derivative with the density term dropped (Phi(z) alone)."""
    monkeypatch.setattr(to, "normal_pdf", lambda z: np.zeros_like(np.asarray(z, dtype=np.float64)))
    with pytest.raises(AssertionError):
        test_gelu_and_derivatives()


def test_planted_inplace_backward_mistake_is_caught(rng, monkeypatch):
    """The update's V_hat term dropped from the backward must break the
    finite-difference pin."""
    orig_back = io.inplace_backward

    def wrong(z, vhat, w0, C, eta, d_o, d_wfinal=None):
        dz, dv, dw = orig_back(z, vhat, w0, C, eta, d_o, d_wfinal)
        return dz, dv * 0.0, dw   # the update's V_hat term dropped
    monkeypatch.setattr(io, "inplace_backward", wrong)
    with pytest.raises(AssertionError):
        test_inplace_backward_matches_finite_differences(4, rng)


def test_planted_global_chunk_grid_is_caught(monkeypatch):
    """Chunks counted from the sequence start instead of each document's start."""
    def global_grid(a, e, C):
        cuts = sorted({a, e} | {m for m in range(0, e, C) if a < m})
        return list(zip(cuts[:-1], cuts[1:]))
    monkeypatch.setattr(io, "_chunk_spans", global_grid)
    with pytest.raises(AssertionError):
        test_inplace_guarded_hand_worked_scalar()


def test_planted_missing_reset_is_caught(monkeypatch):
    """Documents after the first continuing from the running state."""
    monkeypatch.setattr(io, "_segments", lambda T, starts: [(0, T)])
    with pytest.raises(AssertionError):
        test_inplace_guarded_hand_worked_scalar()


# ---------------------------------------------------------------------------
# a hand-worked example and the regression fixture
# ---------------------------------------------------------------------------

def test_hand_worked_example():
    """d_k = d_v = 1, two tokens in one chunk, MSE + linear, gamma = 0.9.

    W0 = 0.5; k = (1, 2); v = (3, -1); q = (2, 1); eta = (1, 0.5) (beta = 0 and
    ln(1/3) with b = 0).  By hand: g = kW0 - v = (-2.5, 2);
    o1 = q1 W0 - q1 eta1 k1 g1 = 1 + 5 = 6;
    o2 = q2 W0 - q2 (eta1 k1 g1 + eta2 k2 g2) = 0.5 - (-2.5 + 2) = 1;
    W_T = 0.9 * 0.5 - (-2.5 + 2) = 0.95.
    """
    q = np.array([2.0, 1.0]).reshape(1, 1, 2, 1)
    k = np.array([1.0, 2.0]).reshape(1, 1, 2, 1)
    v = np.array([3.0, -1.0]).reshape(1, 1, 2, 1)
    beta = np.array([0.0, np.log(1.0 / 3.0)]).reshape(1, 1, 2)
    w0 = np.full((1, 1, 1, 1), 0.5)
    O, WT = to.chunk_forward(q, k, v, beta, 0.0, 2, loss="mse", act="none", decay="scalar",
                             gamma=np.array([0.9]), w0=w0)
    np.testing.assert_allclose(O.ravel(), [6.0, 1.0], atol=1e-14)
    np.testing.assert_allclose(WT.ravel(), [0.95], atol=1e-14)


def test_golden_regression_fixture():
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_small.json")
    with open(path) as f:
        data = json.load(f)
    for c in data["cases"]:
        arr = {k: np.array(c[k]) for k in ("q", "k", "v", "beta", "gamma", "log_a", "w0", "d_o")}
        kw = dict(loss=c["loss"], act=c["act"], decay=c["decay"],
                  gamma=arr["gamma"] if c["decay"] == "scalar" else None,
                  log_a=arr["log_a"] if c["decay"] == "vector" else None, w0=arr["w0"])
        O, WT = to.chunk_forward(arr["q"], arr["k"], arr["v"], arr["beta"], c["b"], c["C"], **kw)
        g = to.chunk_backward(arr["q"], arr["k"], arr["v"], arr["beta"], c["b"], c["C"],
                              arr["d_o"], **kw)
        _close(O, np.array(c["O"]), 1e-13)
        _close(WT, np.array(c["W_T"]), 1e-13)
        for key in ("dq", "dk", "dv", "dbeta", "dw0"):
            _close(g[key], np.array(c[key]), 1e-13)


def test_planted_l1_sign_is_caught(rng, monkeypatch):
    """The L1 signal with its sign flipped (sign(V - V_hat))."""
    real = to.loss_signal
    monkeypatch.setattr(to, "loss_signal", lambda vh, v, loss: -real(vh, v, loss) if loss == "l1" else real(vh, v, loss))
    with pytest.raises(AssertionError):
        test_l1_first_chunk_is_linear_attention_on_signs(rng)


def test_rmse_signal_is_the_gradient_of_the_root_mean_square(rng):
    """The RMSE signal e / (sqrt(d) ||e||) and its VJP against central differences of
    ||f - v|| / sqrt(d) per row (and of the signal itself)."""
    x = rng.standard_normal((4, 6))
    v = rng.standard_normal((4, 6))
    h = 1e-6
    f = lambda y: float(np.sqrt(((y - v) ** 2).sum(axis=-1) / y.shape[-1]).sum())
    num = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        num[idx] = (f(xp) - f(xm)) / (2 * h)
    np.testing.assert_allclose(to.loss_signal(x, v, "rmse"), num, atol=1e-8)
    w = rng.standard_normal(x.shape)
    g = lambda y: float((to.loss_signal(y, v, "rmse") * w).sum())
    num2 = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        num2[idx] = (g(xp) - g(xm)) / (2 * h)
    np.testing.assert_allclose(to.loss_signal_vjp(x, v, w, "rmse"), num2, atol=1e-7)
    assert np.all(to.loss_signal(v, v, "rmse") == 0.0)   # e = 0: no signal
