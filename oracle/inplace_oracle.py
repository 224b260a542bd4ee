"""Plain fp64 CPU oracle for the In-Place TTT W_down chunk update.

TEST INFRASTRUCTURE ONLY (see ``oracle/ttt_oracle.py`` for the rules).

Source: "In-Place Test-Time Training" summary page (shdxiang...pages.dev),
section "Core method and technical details":

* the gated MLP output is O = (phi(H W_gate^T) (.) (H W_up^T)) W_down^T, only
  W_down is a fast weight; Z = phi(H W_gate^T) (.) (H W_up^T) is an input here;
* chunk-wise apply-then-update: chunk i first produces O_[i] = Z_[i] W_down^(i)T,
  then updates W_down^(i+1) = W_down^(i) + eta * V_hat_[i]^T Z_[i] (the closed
  form of one gradient step on the inner-product loss).

Shapes: z [B, T, d_ff], vhat [B, T, d_model], w0 [B, d_model, d_ff].

Long-context safeguards (same page, section "Practical advice", the item on
stability): the Frobenius norm of each fast-weight update is clipped at a
threshold tau (the page uses 1e-5), and the fast weight is reset where a new
document begins.  Readings taken here (the page gives no formulas):

* the update of chunk i is dW_i = eta * V_hat_[i]^T Z_[i]; clipping rescales it
  to dW_i * min(1, tau / ||dW_i||_F) (clip-by-norm; a zero update stays zero);
* a document is an independent stream: at its first token the state returns to
  the pretrained W_down (``w_init``), and chunks of C tokens are counted from
  the document's first token (the last chunk of a document may be short).
* the backward of the guarded form (``inplace_backward_guarded``) differentiates
  the clip factor too (it is a function of the update), and a reset cuts the
  state's gradient: the state a document ends in is discarded, and the
  derivative at its starting state goes to ``w0`` or ``w_init``.
"""
from __future__ import annotations

import numpy as np


def inplace_forward(z, vhat, w0, C, eta):
    """Apply-then-update over chunks of C tokens; returns (O, W_final)."""
    z = np.asarray(z, dtype=np.float64)
    vhat = np.asarray(vhat, dtype=np.float64)
    W = np.array(w0, dtype=np.float64)
    B, T, dff = z.shape
    dm = vhat.shape[-1]
    O = np.zeros((B, T, dm))
    for s0 in range(0, T, C):
        s1 = min(s0 + C, T)
        Zi = z[:, s0:s1]
        O[:, s0:s1] = Zi @ np.swapaxes(W, -1, -2)                    # apply
        W = W + eta * np.swapaxes(vhat[:, s0:s1], -1, -2) @ Zi       # update
    return O, W


def inplace_rows(z, vhat, w0_rows, rows, C, eta, chunks=None):
    """O[:, :, rows] and W_final[:, rows] for a few output rows of W_down.

    Each row m of W_down evolves on its own: W[m] += eta * sum_t vhat[t, m] z[t].
    Used to check full-size runs on sampled rows.  ``w0_rows`` is [B, len(rows), d_ff].
    ``chunks`` optionally limits O to the listed chunk indices (others left 0).
    """
    z = np.asarray(z, dtype=np.float64)
    B, T, dff = z.shape
    Wr = np.array(w0_rows, dtype=np.float64)
    vr = np.asarray(vhat[:, :, rows], dtype=np.float64)              # [B, T, R]
    O = np.zeros((B, T, len(rows)))
    for ci, s0 in enumerate(range(0, T, C)):
        s1 = min(s0 + C, T)
        Zi = z[:, s0:s1]
        if chunks is None or ci in chunks:
            O[:, s0:s1] = Zi @ np.swapaxes(Wr, -1, -2)
        Wr = Wr + eta * np.swapaxes(vr[:, s0:s1], -1, -2) @ Zi
    return O, Wr


def inplace_backward(z, vhat, w0, C, eta, d_o, d_wfinal=None):
    """Reverse-mode derivative of ``inplace_forward`` for training the layer
    around it: given dL/dO (and optionally dL/dW_final), returns
    (dL/dz, dL/dvhat, dL/dw0).

    Chunk i reads W_i in the apply (O_i = Z_i W_i^T) and passes it on with the
    update (W_{i+1} = W_i + eta V_hat_i^T Z_i).  Walking the chunks backwards
    with dW = dL/dW_{i+1}:
      dZ_i     = dO_i W_i + eta V_hat_i dW       (apply, and the update's Z)
      dV_hat_i = eta Z_i dW^T                    (the update's V_hat)
      dW      <- dW + dO_i^T Z_i                 (W_i reaches W_{i+1} unchanged)
    and dL/dw0 is dW after the first chunk.  The states W_i are recomputed
    forward first.
    """
    z = np.asarray(z, dtype=np.float64)
    vhat = np.asarray(vhat, dtype=np.float64)
    d_o = np.asarray(d_o, dtype=np.float64)
    B, T, dff = z.shape
    dm = vhat.shape[-1]
    spans = [(s0, min(s0 + C, T)) for s0 in range(0, T, C)]
    Ws = []
    W = np.array(w0, dtype=np.float64)
    for s0, s1 in spans:
        Ws.append(W)
        W = W + eta * np.swapaxes(vhat[:, s0:s1], -1, -2) @ z[:, s0:s1]
    dW = np.zeros((B, dm, dff)) if d_wfinal is None else np.array(d_wfinal, dtype=np.float64)
    dz = np.zeros_like(z)
    dv = np.zeros_like(vhat)
    for (s0, s1), Wi in zip(reversed(spans), reversed(Ws)):
        Zi, Vi, dOi = z[:, s0:s1], vhat[:, s0:s1], d_o[:, s0:s1]
        dz[:, s0:s1] = dOi @ Wi + eta * Vi @ dW
        dv[:, s0:s1] = eta * Zi @ np.swapaxes(dW, -1, -2)
        dW = dW + np.swapaxes(dOi, -1, -2) @ Zi
    return dz, dv, dW


def inplace_backward_sampled(z, vhat, w0_cols, cols, tokens, C, eta, d_o, d_wfinal_cols=None, d_wfinal=None):
    """Parts of ``inplace_backward`` that can be formed one by one at full size.

    * dz[:, :, cols] and dw0[:, :, cols]: column f of W_i and of dL/dW_{i+1}
      involves column f of Z only (W_{i+1}[:, f] = W_i[:, f] + eta V_hat_i^T Z_i[:, f],
      dW_i[:, f] = dW_{i+1}[:, f] + dO_i^T Z_i[:, f]), so the chunk walk of
      ``inplace_backward`` runs on those columns alone.  ``w0_cols`` is
      w0[:, :, cols]; ``d_wfinal_cols`` likewise (or None).
    * dvhat[:, t] for the listed tokens: with dW_{i+1} = dW_T + sum_{j > i} dO_j^T Z_j,
      eta Z_i dW_{i+1}^T at row t is eta (z_t dW_T^T + sum over tokens s of later
      chunks of (z_t . z_s) dO_s); ``d_wfinal`` is the full dW_T (or None).
    Returns (dz_cols [B,T,len(cols)], dw0_cols [B,d_model,len(cols)], dv_rows [B,len(tokens),d_model]).
    """
    z = np.asarray(z, dtype=np.float64)
    vhat = np.asarray(vhat, dtype=np.float64)
    d_o = np.asarray(d_o, dtype=np.float64)
    B, T, _ = z.shape
    dm = vhat.shape[-1]
    spans = [(s0, min(s0 + C, T)) for s0 in range(0, T, C)]
    zc = z[:, :, cols]
    Ws = []
    W = np.array(w0_cols, dtype=np.float64)
    for s0, s1 in spans:
        Ws.append(W)
        W = W + eta * np.swapaxes(vhat[:, s0:s1], -1, -2) @ zc[:, s0:s1]
    dW = np.zeros((B, dm, len(cols))) if d_wfinal_cols is None else np.array(d_wfinal_cols, dtype=np.float64)
    dz = np.zeros((B, T, len(cols)))
    for (s0, s1), Wi in zip(reversed(spans), reversed(Ws)):
        dz[:, s0:s1] = d_o[:, s0:s1] @ Wi + eta * vhat[:, s0:s1] @ dW
        dW = dW + np.swapaxes(d_o[:, s0:s1], -1, -2) @ zc[:, s0:s1]
    dv = np.zeros((B, len(tokens), dm))
    for k, t in enumerate(tokens):
        nxt = (t // C + 1) * C  # first token of the next chunk
        zt = z[:, t]                                                   # [B, d_ff]
        acc = np.zeros((B, dm))
        if d_wfinal is not None:
            acc += np.einsum("bf,bmf->bm", zt, np.asarray(d_wfinal, dtype=np.float64))
        if nxt < T:
            w = np.einsum("bf,bsf->bs", zt, z[:, nxt:])                  # z_t . z_s
            acc += np.einsum("bs,bsm->bm", w, d_o[:, nxt:])
        dv[:, k] = eta * acc
    return dz, dW, dv


def _segments(T, starts):
    """[(a, e), ...] document spans of one sequence; ``starts`` are the positions
    0 < t < T where a new document begins (strictly increasing)."""
    bounds = [0] + [int(t) for t in starts] + [T]
    return list(zip(bounds[:-1], bounds[1:]))


def _chunk_spans(a, e, C):
    """Chunks of C tokens counted from a document's first token a; the last may be short."""
    return [(s0, min(s0 + C, e)) for s0 in range(a, e, C)]


def inplace_forward_guarded(z, vhat, w0, C, eta, clip_tau=None, doc_starts=None, w_init=None):
    """Apply-then-update with update clipping and document resets; returns (O, W_final).

    ``doc_starts``: None, or a list with one list of document start positions per
    sequence (0 < t < T, increasing).  ``w_init`` [B, d_model, d_ff]: the state a
    document other than the first starts from.  ``clip_tau``: None for no clipping.
    """
    z = np.asarray(z, dtype=np.float64)
    vhat = np.asarray(vhat, dtype=np.float64)
    B, T, dff = z.shape
    dm = vhat.shape[-1]
    O = np.zeros((B, T, dm))
    Wf = np.zeros((B, dm, dff))
    for b in range(B):
        starts = [] if doc_starts is None else doc_starts[b]
        W = np.array(w0[b], dtype=np.float64)
        for j, (a, e) in enumerate(_segments(T, starts)):
            if j > 0:
                W = np.array(w_init[b], dtype=np.float64)             # reset at the document start
            for s0, s1 in _chunk_spans(a, e, C):
                Zi = z[b, s0:s1]
                O[b, s0:s1] = Zi @ W.T                                   # apply
                dW = eta * vhat[b, s0:s1].T @ Zi                         # update
                if clip_tau is not None:
                    n = np.linalg.norm(dW)
                    if n > clip_tau:
                        dW = dW * (clip_tau / n)
                W = W + dW
        Wf[b] = W
    return O, Wf


def update_norms(z, vhat, C, eta, doc_starts=None):
    """||eta * V_hat_[i]^T Z_[i]||_F of every chunk, in the order the chunks run
    (per sequence, per document, per chunk); the clipping decisions of
    ``inplace_forward_guarded`` follow from these."""
    z = np.asarray(z, dtype=np.float64)
    vhat = np.asarray(vhat, dtype=np.float64)
    B, T, _ = z.shape
    out = []
    for b in range(B):
        starts = [] if doc_starts is None else doc_starts[b]
        for a, e in _segments(T, starts):
            for s0, s1 in _chunk_spans(a, e, C):
                out.append(eta * np.linalg.norm(vhat[b, s0:s1].T @ z[b, s0:s1]))
    return np.array(out)


def inplace_rows_guarded(z, vhat, w0_rows, w_init_rows, rows, C, eta, scales, doc_starts=None):
    """O[:, :, rows] and W_final[:, rows] of the guarded forward for a few rows of
    W_down, given each chunk's clip scale min(1, tau / ||dW_i||_F) in ``scales``
    (from ``update_norms``; the norm couples the rows, the rest is row by row)."""
    z = np.asarray(z, dtype=np.float64)
    B, T, _ = z.shape
    vr = np.asarray(vhat[:, :, rows], dtype=np.float64)
    O = np.zeros((B, T, len(rows)))
    Wf = np.zeros((B, len(rows), z.shape[-1]))
    i = 0
    for b in range(B):
        starts = [] if doc_starts is None else doc_starts[b]
        Wr = np.array(w0_rows[b], dtype=np.float64)
        for j, (a, e) in enumerate(_segments(T, starts)):
            if j > 0:
                Wr = np.array(w_init_rows[b], dtype=np.float64)
            for s0, s1 in _chunk_spans(a, e, C):
                Zi = z[b, s0:s1]
                O[b, s0:s1] = Zi @ Wr.T
                Wr = Wr + scales[i] * eta * vr[b, s0:s1].T @ Zi
                i += 1
        Wf[b] = Wr
    return O, Wf


def inplace_backward_guarded(z, vhat, w0, C, eta, d_o, d_wfinal=None, clip_tau=None, doc_starts=None, w_init=None):
    """Reverse-mode derivative of ``inplace_forward_guarded``: given dL/dO (and
    optionally dL/dW_final), returns (dL/dz, dL/dvhat, dL/dw0, dL/dw_init).

    Each document is its own stream: its states are recomputed forward from its
    starting state (w0 for a sequence's first document, w_init for the others),
    then its chunks are walked backwards with A = dL/dW_{i+1}.  Chunk i applies
    s D_i with D_i = eta V_hat_i^T Z_i, n = ||D_i||_F and s = min(1, tau / n).
    Where n <= tau the factor is locally constant (s = 1); past it s = tau / n,
    whose derivative with respect to D_i is -tau D_i / n^3, so the adjoint of D_i is
        G = s A - (s <D_i, A> / n^2) D_i      (G = A where the update is not clipped)
    and then
        dZ_i     = dO_i W_i + eta V_hat_i G
        dV_hat_i = eta Z_i G^T
        A       <- A + dO_i^T Z_i
    A document's final state is replaced at the next document's first token, so
    A starts from zero for every document but the sequence's last, which starts
    from dL/dW_final.  A at a document's first token is the derivative with
    respect to its starting state: dL/dw0 for the first document, summed into
    dL/dw_init over the others.
    """
    z = np.asarray(z, dtype=np.float64)
    vhat = np.asarray(vhat, dtype=np.float64)
    d_o = np.asarray(d_o, dtype=np.float64)
    B, T, dff = z.shape
    dm = vhat.shape[-1]
    dz = np.zeros_like(z)
    dv = np.zeros_like(vhat)
    dw0 = np.zeros((B, dm, dff))
    dwi = np.zeros((B, dm, dff))
    for b in range(B):
        starts = [] if doc_starts is None else doc_starts[b]
        segs = _segments(T, starts)
        for j in reversed(range(len(segs))):
            a, e = segs[j]
            spans = _chunk_spans(a, e, C)
            W = np.array(w0[b] if j == 0 else w_init[b], dtype=np.float64)
            Ws, Ds, scales, norms = [], [], [], []
            for s0, s1 in spans:                                         # the document's states
                D = eta * vhat[b, s0:s1].T @ z[b, s0:s1]
                n = np.linalg.norm(D)
                s = clip_tau / n if clip_tau is not None and n > clip_tau else 1.0
                Ws.append(W)
                Ds.append(D)
                scales.append(s)
                norms.append(n)
                W = W + s * D
            last = j == len(segs) - 1
            A = np.array(d_wfinal[b], dtype=np.float64) if last and d_wfinal is not None else np.zeros((dm, dff))
            for (s0, s1), Wi, D, s, n in zip(*(reversed(x) for x in (spans, Ws, Ds, scales, norms))):
                Zi, Vi, dOi = z[b, s0:s1], vhat[b, s0:s1], d_o[b, s0:s1]
                G = s * A
                if s < 1.0:
                    G = G - (s * np.sum(D * A) / n ** 2) * D
                dz[b, s0:s1] = dOi @ Wi + eta * Vi @ G
                dv[b, s0:s1] = eta * Zi @ G.T
                A = A + dOi.T @ Zi
            if j == 0:
                dw0[b] = A
            else:
                dwi[b] += A
    return dz, dv, dw0, dwi
