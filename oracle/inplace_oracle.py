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
