"""Plain fp64 CPU oracle for the two-layer fast net (TTT-MLP) forward.

TEST INFRASTRUCTURE ONLY (see ``oracle/ttt_oracle.py`` for the rules).

Source: "Modular TTT: Rethinking Test-Time Training as Composable Modules",
summary page on paper.rainbus.top:

* section "Method step details", Algorithm 1: the three passes composed over a
  graph of primitives -- Pass 1 runs the train view forward in topological
  order, Pass 2 takes the loss and walks the graph backwards to the signal at
  every fast Linear, Pass 3 runs the query view with each Linear's chunked
  dual form (O = Q W_start - Tril(Q K_hat^T) dV_hat, W_end = W_start - K_hat^T
  dV_hat, K_hat = eta (.) K) fed by the query-view activations;
* section "Experimental results": deeper fast nets (two Linears with a
  nonlinearity between them) as the second throughput workload.

Graph here: Linear(W1: d_k -> d_h) -> act -> Linear(W2: d_h -> d_v), no
biases.  Per chunk, with W1, W2 at the chunk start and eta_t = 2 sigmoid(beta_t + b):

  Pass 1:  Z1 = K W1,  A = f(Z1),  V_hat = A W2
  Pass 2:  G2 = dl/dV_hat (MSE: V_hat - V; IP: -V; L1: sign(V_hat - V);
           RMSE: (V_hat - V) / (sqrt(d_v) ||V_hat - V||) per token),
           G1 = (G2 W2^T) (.) f'(Z1)
  Pass 3:  X1 = Q W1 - Tril(Q K^T) diag(eta) G1,  A_q = f(X1),
           O  = A_q W2 - Tril(A_q A^T) diag(eta) G2
  update:  W1 <- g W1 - K^T diag(eta) G1,  W2 <- g W2 - A^T diag(eta) G2
           (g = gamma_h with scalar decay, else 1; applied once per chunk).

Backward (mlp_chunk_backward): the outer loss <d_o, O> + <d_W1T, W1_T> + <d_W2T, W2_T>
is differentiated chunk by chunk in reverse, each of the steps above in reverse order;
pinned by central finite differences of mlp_chunk_forward.

Readings (the pages give no formulas for this graph): no biases; the hidden
width d_h is a parameter; vector decay is not defined for two layers and is
not offered; the output has no act after the second Linear.
"""
from __future__ import annotations

import numpy as np

from .ttt_oracle import act_d2f, act_df, act_f, loss_signal, loss_signal_vjp, lr_gate

LOSSES = ("mse", "ip", "l1", "rmse")
ACTS = ("none", "silu", "gelu")
DECAYS = ("none", "scalar")


def _tril(c):
    return np.tril(np.ones((c, c), dtype=np.float64))


def _chunks(T, C):
    return [(s, min(s + C, T)) for s in range(0, T, C)]


def mlp_train_view(k, v, W1, W2, loss, act):
    """Passes 1 and 2 for one chunk: returns (Z1, A, G1, G2)."""
    Z1 = k @ W1
    A = act_f(Z1, act)
    Vhat = A @ W2
    G2 = loss_signal(Vhat, v, loss)
    G1 = (G2 @ np.swapaxes(W2, -1, -2)) * act_df(Z1, act)
    return Z1, A, G1, G2


def mlp_chunk_forward(q, k, v, beta, b, C, loss="mse", act="gelu", decay="none", gamma=None, w1_0=None,
                      w2_0=None, d_h=None, return_ckpt=False):
    """Chunked forward of TTT-MLP; returns (O, W1_T, W2_T) and, with return_ckpt,
    the chunk-start weights as two lists (W1_i, W2_i) after them.

    q, k [B,H,T,d_k], v [B,H,T,d_v], beta [B,H,T], gamma [H] (scalar decay),
    w1_0 [B,H,d_k,d_h], w2_0 [B,H,d_h,d_v] (None: zeros, then d_h is required).
    """
    if loss not in LOSSES or act not in ACTS or decay not in DECAYS:
        raise ValueError((loss, act, decay))
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dh = d_h if w1_0 is None else w1_0.shape[-1]
    W1 = np.zeros((B, H, dk, dh)) if w1_0 is None else np.array(w1_0, dtype=np.float64)
    W2 = np.zeros((B, H, dh, dv)) if w2_0 is None else np.array(w2_0, dtype=np.float64)
    eta = lr_gate(beta, b)
    O = np.zeros((B, H, T, dv))
    tT = lambda x: np.swapaxes(x, -1, -2)
    ck1, ck2 = [], []
    for s0, s1 in _chunks(T, C):
        ck1.append(W1)
        ck2.append(W2)
        qc, kc, vc = q[:, :, s0:s1], k[:, :, s0:s1], v[:, :, s0:s1]
        e = eta[:, :, s0:s1, None]
        _, A, G1, G2 = mlp_train_view(kc, vc, W1, W2, loss, act)
        m = _tril(s1 - s0)
        X1 = qc @ W1 - ((qc @ tT(kc)) * m) @ (e * G1)
        Aq = act_f(X1, act)
        O[:, :, s0:s1] = Aq @ W2 - ((Aq @ tT(A)) * m) @ (e * G2)
        g = gamma[None, :, None, None] if decay == "scalar" else 1.0
        W1 = g * W1 - tT(kc) @ (e * G1)
        W2 = g * W2 - tT(A) @ (e * G2)
    if return_ckpt:
        return O, W1, W2, ck1, ck2
    return O, W1, W2


def mlp_chunk_backward(q, k, v, beta, b, C, d_o, loss="mse", act="gelu", decay="none", gamma=None, w1_0=None,
                       w2_0=None, d_w1T=None, d_w2T=None):
    """Reverse-mode derivative of mlp_chunk_forward for the outer loss
    <d_o, O> + <d_w1T, W1_T> + <d_w2T, W2_T>: the chunks in reverse, each chunk's
    forward steps differentiated in reverse order (chain rule, written out below).
    Returns dq, dk, dv, dbeta, dgamma ([B, H], per chain), dw1_0, dw2_0.
    """
    q, k, v, d_o = (np.asarray(x, dtype=np.float64) for x in (q, k, v, d_o))
    B, H, T, dk = q.shape
    _, W1T, W2T, ck1, ck2 = mlp_chunk_forward(q, k, v, beta, b, C, loss, act, decay, gamma, w1_0, w2_0,
                                              return_ckpt=True)
    eta = lr_gate(beta, b)
    tT = lambda x: np.swapaxes(x, -1, -2)
    dW1n = np.zeros_like(W1T) if d_w1T is None else np.array(d_w1T, dtype=np.float64)
    dW2n = np.zeros_like(W2T) if d_w2T is None else np.array(d_w2T, dtype=np.float64)
    dq, dkk, dvv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    deta = np.zeros((B, H, T))
    dg = np.zeros((B, H))
    g = gamma[None, :, None, None] if decay == "scalar" else 1.0
    chunks = _chunks(T, C)
    for i in range(len(chunks) - 1, -1, -1):
        s0, s1 = chunks[i]
        W1, W2 = ck1[i], ck2[i]
        qc, kc, vc, doc = q[:, :, s0:s1], k[:, :, s0:s1], v[:, :, s0:s1], d_o[:, :, s0:s1]
        e = eta[:, :, s0:s1, None]
        m = _tril(s1 - s0)
        # the chunk's forward again
        Z1 = kc @ W1
        A = act_f(Z1, act)
        Vhat = A @ W2
        G2 = loss_signal(Vhat, vc, loss)
        P = G2 @ tT(W2)
        G1 = P * act_df(Z1, act)
        Gh1, Gh2 = e * G1, e * G2
        S1 = (qc @ tT(kc)) * m
        X1 = qc @ W1 - S1 @ Gh1
        Aq = act_f(X1, act)
        S2 = (Aq @ tT(A)) * m
        # O = Aq W2 - S2 Gh2
        dS2 = -(doc @ tT(Gh2)) * m
        dAq = doc @ tT(W2) + dS2 @ A
        dGh2 = -tT(S2) @ doc - A @ dW2n                  # and W2' = g W2 - A^T Gh2
        dA = tT(dS2) @ Aq - Gh2 @ tT(dW2n)
        # Aq = f(X1);  X1 = Q W1 - S1 Gh1
        dX1 = dAq * act_df(X1, act)
        dS1 = -(dX1 @ tT(Gh1)) * m
        dq[:, :, s0:s1] = dX1 @ tT(W1) + dS1 @ kc
        dGh1 = -tT(S1) @ dX1 - kc @ dW1n                 # and W1' = g W1 - K^T Gh1
        dK = tT(dS1) @ qc - Gh1 @ tT(dW1n)
        # Gh = diag(eta) G
        dG1, dG2 = e * dGh1, e * dGh2
        deta[:, :, s0:s1] = np.sum(dGh1 * G1, axis=-1) + np.sum(dGh2 * G2, axis=-1)
        # G1 = P (.) f'(Z1);  P = G2 W2^T
        dP = dG1 * act_df(Z1, act)
        dZ1 = dG1 * P * act_d2f(Z1, act)
        dG2 = dG2 + dP @ W2
        # G2 = signal(V_hat, V)
        dVhat = loss_signal_vjp(Vhat, vc, dG2, loss)     # MSE: dG2; RMSE: its Jacobian; IP, L1: 0
        dvv[:, :, s0:s1] = -dG2 if loss == "ip" else -dVhat
        # V_hat = A W2;  A = f(Z1);  Z1 = K W1
        dA = dA + dVhat @ tT(W2)
        dZ1 = dZ1 + dA * act_df(Z1, act)
        dkk[:, :, s0:s1] = dK + dZ1 @ tT(W1)
        dW1 = g * dW1n + tT(qc) @ dX1 + tT(kc) @ dZ1
        dW2 = g * dW2n + tT(Aq) @ doc + tT(dP) @ G2 + tT(A) @ dVhat
        if decay == "scalar":
            dg += np.sum(dW1n * W1, axis=(-1, -2)) + np.sum(dW2n * W2, axis=(-1, -2))
        dW1n, dW2n = dW1, dW2
    # eta = 2 sigmoid(beta + b):  d eta / d beta = eta (1 - eta / 2)
    dbeta = deta * eta * (1.0 - eta / 2.0)
    return dict(dq=dq, dk=dkk, dv=dvv, dbeta=dbeta, dgamma=dg, dw1_0=dW1n, dw2_0=dW2n)


def mlp_token_loop_forward(q, k, v, beta, b, C, loss="mse", act="gelu", decay="none", gamma=None, w1_0=None,
                           w2_0=None, d_h=None):
    """Per-token form, one chain at a time: inside chunk i every token's gradient
    is taken at the chunk-start weights; the query of token t reads both layers
    after the writes of tokens <= t of the chunk."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dh = d_h if w1_0 is None else w1_0.shape[-1]
    eta = lr_gate(beta, b)
    O = np.zeros((B, H, T, dv))
    W1T = np.zeros((B, H, dk, dh))
    W2T = np.zeros((B, H, dh, dv))
    for bi in range(B):
        for hi in range(H):
            W1 = np.zeros((dk, dh)) if w1_0 is None else np.array(w1_0[bi, hi], dtype=np.float64)
            W2 = np.zeros((dh, dv)) if w2_0 is None else np.array(w2_0[bi, hi], dtype=np.float64)
            for s0, s1 in _chunks(T, C):
                S1, S2 = W1.copy(), W2.copy()
                for t in range(s0, s1):
                    z1 = k[bi, hi, t] @ W1
                    a = act_f(z1, act)
                    vhat = a @ W2
                    g2 = loss_signal(vhat, v[bi, hi, t], loss)
                    g1 = (W2 @ g2) * act_df(z1, act)
                    S1 = S1 - eta[bi, hi, t] * np.outer(k[bi, hi, t], g1)
                    S2 = S2 - eta[bi, hi, t] * np.outer(a, g2)
                    O[bi, hi, t] = act_f(q[bi, hi, t] @ S1, act) @ S2
                if decay == "scalar":
                    W1 = gamma[hi] * W1 + (S1 - W1)
                    W2 = gamma[hi] * W2 + (S2 - W2)
                else:
                    W1, W2 = S1, S2
            W1T[bi, hi], W2T[bi, hi] = W1, W2
    return O, W1T, W2T


def mlp_inner_loss(k, v, W1, W2, loss, act):
    """The train-view loss of one chunk, summed over tokens and features."""
    Vhat = act_f(k @ W1, act) @ W2
    if loss == "mse":
        return 0.5 * float(((Vhat - v) ** 2).sum())
    if loss == "l1":
        return float(np.abs(Vhat - v).sum())
    if loss == "rmse":
        return float(np.sqrt(((Vhat - v) ** 2).sum(axis=-1) / v.shape[-1]).sum())
    return -float((Vhat * v).sum())
