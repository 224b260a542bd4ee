"""Plain fp64 CPU oracle for the fast net Linear -> Norm (the Norm primitive).

TEST INFRASTRUCTURE ONLY (see ``oracle/ttt_oracle.py`` for the rules).

Source: "Modular TTT: Rethinking Test-Time Training as Composable Modules",
summary page on paper.rainbus.top:

* section "Method step details", Algorithm 1: the per-primitive rules composed
  over the graph (train-view forward, train-view backward to the Linear's
  signal, query view with the Linear's chunked dual form);
* sections "Experimental results" and "Technical novelty": Norm as a primitive
  of the fast net (found unstable in the ablation) with a hand-written analytic
  backward.

Graph: Z = K W (W: d_k x d_v), V_hat = N(Z) with the per-token normalisation
N(z) = (z - mean(z)) / sqrt(var(z) + eps) over the d_v features.  Per chunk,
with W at the chunk start and eta_t = 2 sigmoid(beta_t + b):

  Pass 1:  Z = K W,  V_hat = N(Z)
  Pass 2:  E = dl/dV_hat (MSE: V_hat - V; IP: -V; L1: sign(V_hat - V)),
           G = J_N(Z)^T E = (E - mean(E) - N(Z) <E, N(Z)> / d) / s(Z)
  Pass 3:  Y = Q W - Tril(Q K^T) diag(eta) G,  O = N(Y)
  update:  W <- g W - K^T diag(eta) G     (g = gamma_h with scalar decay, else 1)

Readings (the pages give no formulas for the primitive): eps = 1e-5, no affine
scale or shift, the query view normalises like the train view (as the single
act does), decay none or scalar.
"""
from __future__ import annotations

import numpy as np

from .ttt_oracle import loss_signal, loss_signal_vjp, lr_gate

LOSSES = ("mse", "ip", "l1", "rmse")
DECAYS = ("none", "scalar")
EPS = 1e-5


def norm_f(z, eps=EPS):
    """(N(z), s(z)) per row of the last axis."""
    z = np.asarray(z, dtype=np.float64)
    mu = z.mean(axis=-1, keepdims=True)
    s = np.sqrt(((z - mu) ** 2).mean(axis=-1, keepdims=True) + eps)
    return (z - mu) / s, s


def norm_vjp(x, n, s):
    """J_N^T x = (x - mean(x) - n <x, n> / d) / s (J_N is symmetric)."""
    d = n.shape[-1]
    return (x - x.mean(axis=-1, keepdims=True) - n * (x * n).sum(axis=-1, keepdims=True) / d) / s


def _tril(c):
    return np.tril(np.ones((c, c), dtype=np.float64))


def _chunks(T, C):
    return [(s, min(s + C, T)) for s in range(0, T, C)]


def norm_train_view(k, v, W, loss, eps=EPS):
    """Passes 1 and 2 for one chunk: returns (Z, n, s, E, G)."""
    Z = k @ W
    n, s = norm_f(Z, eps)
    E = loss_signal(n, v, loss)
    return Z, n, s, E, norm_vjp(E, n, s)


def norm_chunk_forward(q, k, v, beta, b, C, loss="mse", decay="none", gamma=None, w0=None, eps=EPS,
                       return_ckpt=False):
    """Chunked forward of Linear -> Norm; returns (O, W_T) [, the chunk-start states]."""
    if loss not in LOSSES or decay not in DECAYS:
        raise ValueError((loss, decay))
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    W = np.zeros((B, H, dk, dv)) if w0 is None else np.array(w0, dtype=np.float64)
    eta = lr_gate(beta, b)
    O = np.zeros((B, H, T, dv))
    tT = lambda x: np.swapaxes(x, -1, -2)
    ck = []
    for s0, s1 in _chunks(T, C):
        ck.append(W)
        qc, kc, vc = q[:, :, s0:s1], k[:, :, s0:s1], v[:, :, s0:s1]
        e = eta[:, :, s0:s1, None]
        _, _, _, _, G = norm_train_view(kc, vc, W, loss, eps)
        Y = qc @ W - ((qc @ tT(kc)) * _tril(s1 - s0)) @ (e * G)
        O[:, :, s0:s1] = norm_f(Y, eps)[0]
        g = gamma[None, :, None, None] if decay == "scalar" else 1.0
        W = g * W - tT(kc) @ (e * G)
    return (O, W, ck) if return_ckpt else (O, W)


def norm_token_loop_forward(q, k, v, beta, b, C, loss="mse", decay="none", gamma=None, w0=None, eps=EPS):
    """Per-token form, one chain at a time: inside a chunk every token's gradient is
    taken at the chunk-start state; token t's query reads the state after the writes
    of tokens <= t of the chunk."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    eta = lr_gate(beta, b)
    O = np.zeros((B, H, T, dv))
    WT = np.zeros((B, H, dk, dv))
    for bi in range(B):
        for hi in range(H):
            W = np.zeros((dk, dv)) if w0 is None else np.array(w0[bi, hi], dtype=np.float64)
            for s0, s1 in _chunks(T, C):
                St = W.copy()
                for t in range(s0, s1):
                    z = k[bi, hi, t] @ W
                    n, s = norm_f(z, eps)
                    g = norm_vjp(loss_signal(n, v[bi, hi, t], loss), n, s)
                    St = St - eta[bi, hi, t] * np.outer(k[bi, hi, t], g)
                    O[bi, hi, t] = norm_f(q[bi, hi, t] @ St, eps)[0]
                W = gamma[hi] * W + (St - W) if decay == "scalar" else St
            WT[bi, hi] = W
    return O, WT


def norm_chunk_backward(q, k, v, beta, b, C, d_o, loss="mse", decay="none", gamma=None, w0=None, d_wT=None,
                        eps=EPS):
    """Reverse-mode derivative of norm_chunk_forward for <d_o, O> + <d_wT, W_T>.

    Per chunk in reverse, with G = J_N(Z)^T E, n = N(Z), s = s(Z), M = the
    projection x -> x - mean(x) - n <x, n> / d:
      dY = J_N(Y)^T dO;  dW += Q^T dY + g dW';  dS = -Tril(dY (eta G)^T);  dQ = dY W^T + dS K
      d(eta G) = -S^T dY - K dW';  dG = eta d(eta G);  d eta = <d(eta G), G>
      dZ = ( J_N(Z) u - n <dG, G> / d ) / s,   u = R^T M dG - (<E, n> / d) dG - (<dG, n> / d) E
           (R = dE/dn: I for MSE, the RMSE signal's Jacobian, 0 for IP and L1)
      dV = -J_N(Z) dG (IP), -R^T M dG / s (MSE, RMSE) or 0 (L1)
      dK = dS^T Q - (eta G) dW'^T + dZ W^T;  dW += K^T dZ;  d gamma += <dW', W>
    """
    q, k, v, d_o = (np.asarray(x, dtype=np.float64) for x in (q, k, v, d_o))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    _, WT, ck = norm_chunk_forward(q, k, v, beta, b, C, loss, decay, gamma, w0, eps, return_ckpt=True)
    eta = lr_gate(beta, b)
    tT = lambda x: np.swapaxes(x, -1, -2)
    dWn = np.zeros_like(WT) if d_wT is None else np.array(d_wT, dtype=np.float64)
    dq, dkk, dvv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    deta = np.zeros((B, H, T))
    dg = np.zeros((B, H))
    g = gamma[None, :, None, None] if decay == "scalar" else 1.0
    chunks = _chunks(T, C)
    for i in range(len(chunks) - 1, -1, -1):
        s0, s1 = chunks[i]
        W = ck[i]
        qc, kc, vc, doc = q[:, :, s0:s1], k[:, :, s0:s1], v[:, :, s0:s1], d_o[:, :, s0:s1]
        e = eta[:, :, s0:s1, None]
        m = _tril(s1 - s0)
        Z, n, s, E, G = norm_train_view(kc, vc, W, loss, eps)
        Gh = e * G
        S = (qc @ tT(kc)) * m
        Y = qc @ W - S @ Gh
        ny, sy = norm_f(Y, eps)
        dY = norm_vjp(doc, ny, sy)
        dS = -(dY @ tT(Gh)) * m
        dq[:, :, s0:s1] = dY @ tT(W) + dS @ kc
        dGh = -tT(S) @ dY - kc @ dWn
        dK = tT(dS) @ qc - Gh @ tT(dWn)
        dG = e * dGh
        deta[:, :, s0:s1] = np.sum(dGh * G, axis=-1)
        d = n.shape[-1]
        proj = lambda x: x - x.mean(axis=-1, keepdims=True) - n * (x * n).sum(axis=-1, keepdims=True) / d
        jm = loss_signal_vjp(n, vc, proj(dG), loss)   # (dE/dn)^T M dG
        u = jm - ((E * n).sum(axis=-1, keepdims=True) / d) * dG - ((dG * n).sum(axis=-1, keepdims=True) / d) * E
        dZ = (proj(u) / s - n * (dG * G).sum(axis=-1, keepdims=True) / d) / s
        dvv[:, :, s0:s1] = -proj(dG) / s if loss == "ip" else -jm / s
        dkk[:, :, s0:s1] = dK + dZ @ tT(W)
        dW = g * dWn + tT(qc) @ dY + tT(kc) @ dZ
        if decay == "scalar":
            dg += np.sum(dWn * W, axis=(-1, -2))
        dWn = dW
    dbeta = deta * eta * (1.0 - eta / 2.0)
    return dict(dq=dq, dk=dkk, dv=dvv, dbeta=dbeta, dgamma=dg, dw0=dWn)
