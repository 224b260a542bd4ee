"""Plain fp64 CPU oracle for the chunkwise TTT fast-weight layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the HIP library.

Sources (cited by page title and section; no other reference exists):

* [MTTT-prereq]  "Modular TTT: Rethinking Test-Time Training as Composable
  Modules", summary page on paper.rainbus.top, section "Prerequisites":
  fast weights, train view / query view, chunkwise recurrence, the learning
  rate parametrisation eta_t = 2*Sigmoid(beta_t + b), scalar and vector decay.
* [MTTT-alg1]  same page, section "Method step details": Algorithm 1
  (Pass 1 train-view forward, Pass 2 loss and reverse-topological backward,
  Pass 3 query view) and the chunked dual form of one Linear primitive,
  O = Q W_start - Tril(Q K_hat^T) dV_hat,  W_end = W_start - K_hat^T dV_hat,
  K_hat = eta (.) K, chunk size 256.
* [MTTT-core]  same page, section "Core method": the state transition
  W = W - dW composed from the primitives.
* [MTTT-results]  same page, section "Experimental results": MSE and
  inner-product losses (and the weaker L1 of the loss ablation), single
  nonlinearity after the Linear (SiLU or GELU).

Conventions (row vectors, per batch b and head h):

* ``W`` has shape [d_k, d_v]; the fast net reads ``v_hat = f(k W)``.
* Chunk i covers tokens [i*C, (i+1)*C); the last chunk may be short.
* Losses are summed over tokens and features: MSE is 1/2 ||f(KW) - V||^2,
  the inner-product loss is -<f(KW), V>, L1 is sum |f(KW) - V| (its
  derivative sign(f(KW) - V), taken as 0 at a tie), RMSE is, per token,
  ||f(kW) - v|| / sqrt(d_v) (its derivative e / (sqrt(d_v) ||e||), e = f(kW) - v,
  taken as 0 where e = 0).
* Scalar decay: W_{i+1} = gamma_h W_i - K^T diag(eta) G  (gamma once per chunk;
  the train and query views inside chunk i read the undecayed W_i).
* Vector decay: token recurrence S_t = diag(a_t) S_{t-1} - eta_t k_t^T g_t with
  S_{start-1} = W_i; the query of token t reads S_t; the train view still uses
  W_i; W_{i+1} = S_{last}.  In chunk form (L = inclusive in-chunk cumsum of
  log a over tokens, per feature):
  S_ts = sum_d q_td k_sd exp(L_td - L_sd)  for s <= t, evaluated pairwise here.

Every array is float64.  Inputs are [B, H, T, d] (row-major), beta is
[B, H, T], gamma is [H] (scalar decay), log_a is [B, H, T, d_k] (vector
decay), w0 is [B, H, d_k, d_v] or None for zeros.
"""
from __future__ import annotations

import numpy as np

LOSSES = ("mse", "ip", "l1", "rmse")
ACTS = ("none", "silu", "gelu")
DECAYS = ("none", "scalar", "vector")


# ----------------------------------------------------------------------------
# Scalar pieces
# ----------------------------------------------------------------------------

def sigmoid(x):
    """Logistic function, written out: 1 / (1 + exp(-x))."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def lr_gate(beta, b):
    """eta_t = 2 * Sigmoid(beta_t + b)  [MTTT-prereq, learning-rate parametrisation]."""
    return 2.0 * sigmoid(np.asarray(beta, dtype=np.float64) + b)


def normal_cdf(z):
    """Phi(z) = (1 + erf(z / sqrt 2)) / 2, the standard normal distribution function."""
    from scipy.special import erf
    return 0.5 * (1.0 + erf(np.asarray(z, dtype=np.float64) / np.sqrt(2.0)))


def normal_pdf(z):
    """phi(z) = exp(-z^2 / 2) / sqrt(2 pi)."""
    z = np.asarray(z, dtype=np.float64)
    return np.exp(-0.5 * z * z) / np.sqrt(2.0 * np.pi)


def act_f(z, act):
    """The single nonlinearity after the Linear node [MTTT-results: SiLU or GELU];
    SiLU(z) = z sigmoid(z), GELU(z) = z Phi(z) (the exact form, with the normal
    distribution function)."""
    if act == "none":
        return z
    if act == "silu":
        return z * sigmoid(z)
    if act == "gelu":
        return z * normal_cdf(z)
    raise ValueError(act)


def act_df(z, act):
    """First derivative of the nonlinearity; GELU'(z) = Phi(z) + z phi(z)."""
    if act == "none":
        return np.ones_like(z)
    if act == "silu":
        s = sigmoid(z)
        return s * (1.0 + z * (1.0 - s))
    if act == "gelu":
        return normal_cdf(z) + z * normal_pdf(z)
    raise ValueError(act)


def act_d2f(z, act):
    """Second derivative of the nonlinearity (needed by the outer backward);
    GELU''(z) = phi(z) (2 - z^2)."""
    if act == "none":
        return np.zeros_like(z)
    if act == "silu":
        s = sigmoid(z)
        return s * (1.0 - s) * (2.0 + z * (1.0 - 2.0 * s))
    if act == "gelu":
        return normal_pdf(z) * (2.0 - z * z)
    raise ValueError(act)


def _check(loss, act, decay):
    if loss not in LOSSES or act not in ACTS or decay not in DECAYS:
        raise ValueError((loss, act, decay))


def _chunks(T, C):
    return [(s, min(s + C, T)) for s in range(0, T, C)]


def _tril(c):
    return np.tril(np.ones((c, c), dtype=np.float64))


# ----------------------------------------------------------------------------
# One chunk, per batch of chains: the three passes of Algorithm 1
# ----------------------------------------------------------------------------

def loss_signal(vhat, v, loss):
    """dl/dV_hat of the per-token loss (rows of the last axis)."""
    if loss == "mse":
        return vhat - v
    if loss == "l1":
        return np.sign(vhat - v)
    if loss == "rmse":
        e = np.asarray(vhat - v, dtype=np.float64)
        nrm = np.sqrt((e * e).sum(axis=-1, keepdims=True))
        return np.where(nrm > 0, e / (np.sqrt(e.shape[-1]) * np.where(nrm > 0, nrm, 1.0)), 0.0)
    return -np.asarray(v, dtype=np.float64)


def loss_signal_vjp(vhat, v, x, loss):
    """(d signal / d V_hat)^T x: x for MSE, J x for RMSE with the symmetric
    J = (I - e_hat e_hat^T) / (sqrt(d) ||e||), 0 for IP and L1 (away from ties).
    The signal's derivative in V is the negative of this for MSE and RMSE, -I for IP."""
    if loss == "mse":
        return x
    if loss == "rmse":
        e = np.asarray(vhat - v, dtype=np.float64)
        nrm = np.sqrt((e * e).sum(axis=-1, keepdims=True))
        safe = np.where(nrm > 0, nrm, 1.0)
        eh = e / safe
        out = (x - eh * (eh * x).sum(axis=-1, keepdims=True)) / (np.sqrt(e.shape[-1]) * safe)
        return np.where(nrm > 0, out, 0.0)
    return np.zeros_like(np.asarray(x, dtype=np.float64))


def _train_view(k, v, W, loss, act):
    """Pass 1 and Pass 2 of Algorithm 1 for the graph Linear -> Act.

    Pass 1: Z = K W, V_hat = f(Z).  Pass 2: l = L(V_hat, V); the adjoint
    dl/dV_hat is pulled back through the act to the Linear node, giving
    G = dl/dZ = E (.) f'(Z) with E = V_hat - V (MSE), -V (IP) or
    sign(V_hat - V) (L1).
    """
    Z = k @ W
    Vhat = act_f(Z, act)
    E = loss_signal(Vhat, v, loss)
    G = E * act_df(Z, act)
    return Z, E, G


def _decay_pieces(q, k, la, decay, gamma_bh):
    """Per-chunk decay quantities.

    Returns (S, q_tilde, k_bar, lam, extra):
      S        causal scores, S_ts for s <= t (0 above the diagonal)
      q_tilde  the query as it multiplies W_i in the query view
      k_bar    the key as it enters the state transition
      lam      the row scale applied to W_i in the transition, shape [..., d_k]
    """
    c = q.shape[-2]
    if decay == "vector":
        L = np.cumsum(la, axis=-2)                      # inclusive, per feature
        Lc = L[..., -1:, :]                             # [..., 1, dk]
        # pairwise, not factorised: E_tsd = exp(L_td - L_sd) for s <= t
        diff = L[..., :, None, :] - L[..., None, :, :]  # [..., c, c, dk]
        mask = _tril(c)[..., None]
        Et = np.exp(np.where(mask > 0, diff, 0.0)) * mask
        S = np.einsum("...td,...sd,...tsd->...ts", q, k, Et)
        q_tilde = q * np.exp(L)
        k_bar = k * np.exp(Lc - L)
        lam = np.exp(Lc[..., 0, :])
        return S, q_tilde, k_bar, lam, (L, Et)
    S = (q @ np.swapaxes(k, -1, -2)) * _tril(c)      # Tril(Q K^T), diagonal included
    dk = q.shape[-1]
    if decay == "scalar":
        lam = np.broadcast_to(gamma_bh[..., None], gamma_bh.shape + (dk,)).copy()
    else:
        lam = np.ones(q.shape[:-2] + (dk,))
    return S, q, k, lam, None


def chunk_forward(q, k, v, beta, b, C, loss="mse", act="none", decay="none",
                  gamma=None, log_a=None, w0=None, return_ckpt=False):
    """Chunkwise TTT layer forward [MTTT-alg1, MTTT-core, MTTT-prereq].

    For each chunk: Pass 1/2 (train view at the chunk-start state W_i), Pass 3
    (query view O = f(Q~ W_i - Tril(S) diag(eta) G)), then the state
    transition W_{i+1} = diag(lam) W_i - K_bar^T diag(eta) G.
    Returns (O, W_T) or (O, W_T, ckpt) with ckpt[..., i, :, :] = W_i.
    """
    _check(loss, act, decay)
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    eta = lr_gate(beta, b)
    gamma_bh = None
    if decay == "scalar":
        gamma_bh = np.broadcast_to(np.asarray(gamma, dtype=np.float64).reshape(1, H), (B, H))
    W = np.zeros((B, H, dk, dv)) if w0 is None else np.array(w0, dtype=np.float64)
    O = np.zeros((B, H, T, dv))
    spans = _chunks(T, C)
    ckpt = np.zeros((B, H, len(spans), dk, dv))
    for i, (s0, s1) in enumerate(spans):
        qc, kc, vc, ec = q[:, :, s0:s1], k[:, :, s0:s1], v[:, :, s0:s1], eta[:, :, s0:s1]
        la = None if log_a is None else np.asarray(log_a[:, :, s0:s1], dtype=np.float64)
        ckpt[:, :, i] = W
        _, _, G = _train_view(kc, vc, W, loss, act)
        S, q_t, k_bar, lam, _ = _decay_pieces(qc, kc, la, decay, gamma_bh)
        Gh = ec[..., None] * G                       # diag(eta) G = dV_hat scaled by eta
        Y = q_t @ W - S @ Gh                          # Pass 3: dual form
        O[:, :, s0:s1] = act_f(Y, act)
        W = lam[..., None] * W - np.swapaxes(k_bar, -1, -2) @ Gh
    if return_ckpt:
        return O, W, ckpt
    return O, W


def chunk_backward(q, k, v, beta, b, C, d_o, loss="mse", act="none", decay="none",
                   gamma=None, log_a=None, w0=None, d_wT=None):
    """Analytic outer backward of :func:`chunk_forward` (reverse-mode chain rule).

    The outer loss is F = <d_o, O> + <d_wT, W_T>.  Returns a dict with dq, dk,
    dv, dbeta, dgamma ([B, H]; None unless scalar decay), dlog_a (None unless
    vector decay) and dw0.  Every step differentiates the corresponding
    forward step of one chunk, sweeping the chunks in reverse order and
    carrying dW_{i+1}.
    """
    _check(loss, act, decay)
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    d_o = np.asarray(d_o, dtype=np.float64)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    eta = lr_gate(beta, b)
    gamma_bh = None
    if decay == "scalar":
        gamma_bh = np.broadcast_to(np.asarray(gamma, dtype=np.float64).reshape(1, H), (B, H))
    _, _, ckpt = chunk_forward(q, k, v, beta, b, C, loss, act, decay, gamma, log_a, w0,
                               return_ckpt=True)
    dq = np.zeros_like(q)
    dkk = np.zeros_like(k)
    dvv = np.zeros_like(v)
    deta = np.zeros((B, H, T))
    dgamma = np.zeros((B, H)) if decay == "scalar" else None
    dlog_a = np.zeros((B, H, T, dk)) if decay == "vector" else None
    dWn = np.zeros((B, H, dk, dv)) if d_wT is None else np.array(d_wT, dtype=np.float64)
    spans = _chunks(T, C)
    tT = lambda x: np.swapaxes(x, -1, -2)  # noqa: E731
    for i in reversed(range(len(spans))):
        s0, s1 = spans[i]
        c = s1 - s0
        qc, kc, vc, ec = q[:, :, s0:s1], k[:, :, s0:s1], v[:, :, s0:s1], eta[:, :, s0:s1]
        la = None if log_a is None else np.asarray(log_a[:, :, s0:s1], dtype=np.float64)
        W = ckpt[:, :, i]
        # recompute the forward of this chunk
        Z, E, G = _train_view(kc, vc, W, loss, act)
        S, q_t, k_bar, lam, extra = _decay_pieces(qc, kc, la, decay, gamma_bh)
        Gh = ec[..., None] * G
        Y = q_t @ W - S @ Gh
        dY = d_o[:, :, s0:s1] * act_df(Y, act)
        # Y = q_t W - S Gh
        dq_t = dY @ tT(W)
        dW = tT(q_t) @ dY
        dS = -(dY @ tT(Gh)) * _tril(c)
        dGh = -tT(S) @ dY
        # W' = diag(lam) W - k_bar^T Gh
        dW = dW + lam[..., None] * dWn
        dlam = np.sum(dWn * W, axis=-1)                 # [B, H, dk]
        dk_bar = -Gh @ tT(dWn)
        dGh = dGh - k_bar @ dWn
        # Gh = diag(eta) G
        dG = ec[..., None] * dGh
        deta[:, :, s0:s1] = np.sum(dGh * G, axis=-1)
        # G = E (.) f'(Z);  E = f(Z) - V (MSE), -V (IP), sign(f(Z) - V) (L1, whose
        # derivative in Z and V is zero away from ties) or the RMSE signal
        f1 = act_df(Z, act)
        dE = dG * f1
        dZ = dG * E * act_d2f(Z, act)
        jd = loss_signal_vjp(act_f(Z, act), vc, dE, loss)
        dZ = dZ + jd * f1
        dvv[:, :, s0:s1] = -dE if loss == "ip" else -jd
        # Z = K W
        dk_c = dZ @ tT(W)
        dW = dW + tT(kc) @ dZ
        if decay == "vector":
            L, Et = extra
            eL = np.exp(L)
            Lc = L[..., -1:, :]
            # S_ts = sum_d q_td k_sd Et_tsd (Et already masked)
            dq_s = np.einsum("...ts,...sd,...tsd->...td", dS, kc, Et)
            dk_s = np.einsum("...ts,...td,...tsd->...sd", dS, qc, Et)
            dL = qc * dq_s - kc * dk_s
            dq[:, :, s0:s1] = dq_t * eL + dq_s
            dL = dL + dq_t * q_t
            dk_c = dk_c + dk_bar * np.exp(Lc - L) + dk_s
            dL = dL - dk_bar * k_bar
            dLc = np.sum(dk_bar * k_bar, axis=-2) + dlam * lam
            dL[..., -1, :] += dLc
            # L = inclusive cumsum of log a  =>  dlog a_r = sum_{t >= r} dL_t
            dlog_a[:, :, s0:s1] = np.flip(np.cumsum(np.flip(dL, axis=-2), axis=-2), axis=-2)
        else:
            dq[:, :, s0:s1] = dq_t + dS @ kc
            dk_c = dk_c + dk_bar + tT(dS) @ qc
            if decay == "scalar":
                dgamma += np.sum(dlam, axis=-1)          # lam = gamma on every row
        dkk[:, :, s0:s1] = dk_c
        dWn = dW
    dbeta = deta * eta * (1.0 - eta / 2.0)            # d eta / d beta = eta (1 - eta/2)
    return dict(dq=dq, dk=dkk, dv=dvv, dbeta=dbeta, dgamma=dgamma, dlog_a=dlog_a, dw0=dWn)


# ----------------------------------------------------------------------------
# Token-by-token reference (an independent second implementation)
# ----------------------------------------------------------------------------

def token_loop_forward(q, k, v, beta, b, C, loss="mse", act="none", decay="none",
                       gamma=None, log_a=None, w0=None):
    """Per-token form of the same layer, one (b, h) chain at a time.

    Within chunk i every token's gradient g_t is taken at W_i; the query of
    token t reads the state after the writes of tokens <= t of the chunk:
    S_t = W_i - sum_{s<=t} eta_s k_s^T g_s (none / scalar decay) or
    S_t = diag(a_t) S_{t-1} - eta_t k_t^T g_t (vector decay).
    """
    _check(loss, act, decay)
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    eta = lr_gate(beta, b)
    O = np.zeros((B, H, T, dv))
    WT = np.zeros((B, H, dk, dv))
    for bi in range(B):
        for hi in range(H):
            W = np.zeros((dk, dv)) if w0 is None else np.array(w0[bi, hi], dtype=np.float64)
            for (s0, s1) in _chunks(T, C):
                St = W.copy()
                for t in range(s0, s1):
                    z = k[bi, hi, t] @ W
                    fz = act_f(z, act)
                    e = loss_signal(fz, v[bi, hi, t], loss)
                    g = e * act_df(z, act)
                    if decay == "vector":
                        St = np.exp(log_a[bi, hi, t])[:, None] * St
                    St = St - eta[bi, hi, t] * np.outer(k[bi, hi, t], g)
                    O[bi, hi, t] = act_f(q[bi, hi, t] @ St, act)
                if decay == "vector":
                    W = St
                elif decay == "scalar":
                    W = gamma[hi] * W + (St - W)
                else:
                    W = St
            WT[bi, hi] = W
    return O, WT
