"""Writes tests/golden/oracle_small.json: small oracle outputs kept as a regression guard.

Calls only ``oracle/``.  Inputs are drawn here from a fixed seed and stored
with the outputs, so the fixture stands on its own.  Run from the repo root:
``python tests/golden/make_golden.py``.
"""
import itertools
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from oracle import chunk_forward, chunk_backward  # noqa: E402


def main():
    rng = np.random.default_rng(7)
    B, H, T, dk, dv, C, b = 1, 1, 6, 2, 2, 4, -1.0
    cases = []
    for loss, act, decay in itertools.product(["mse", "ip"], ["none", "silu"],
                                              ["none", "scalar", "vector"]):
        q = np.round(rng.standard_normal((B, H, T, dk)), 3)
        k = np.round(rng.standard_normal((B, H, T, dk)), 3)
        v = np.round(rng.standard_normal((B, H, T, dv)), 3)
        beta = np.round(rng.standard_normal((B, H, T)), 3)
        gamma = np.round(rng.uniform(0.9, 1.0, H), 3)
        la = np.round(-rng.uniform(0.01, 0.3, (B, H, T, dk)), 3)
        w0 = np.round(0.5 * rng.standard_normal((B, H, dk, dv)), 3)
        do = np.round(rng.standard_normal((B, H, T, dv)), 3)
        kw = dict(loss=loss, act=act, decay=decay, gamma=gamma if decay == "scalar" else None,
                  log_a=la if decay == "vector" else None, w0=w0)
        O, WT = chunk_forward(q, k, v, beta, b, C, **kw)
        g = chunk_backward(q, k, v, beta, b, C, do, **kw)
        cases.append(dict(loss=loss, act=act, decay=decay, b=b, C=C,
                          q=q.tolist(), k=k.tolist(), v=v.tolist(), beta=beta.tolist(),
                          gamma=gamma.tolist(), log_a=la.tolist(), w0=w0.tolist(),
                          d_o=do.tolist(), O=O.tolist(), W_T=WT.tolist(),
                          dq=g["dq"].tolist(), dk=g["dk"].tolist(), dv=g["dv"].tolist(),
                          dbeta=g["dbeta"].tolist(), dw0=g["dw0"].tolist()))
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small.json")
    with open(path, "w") as f:
        json.dump(dict(note="regression fixture written by tests/golden/make_golden.py "
                            "from the fp64 oracle only", cases=cases), f, indent=None)
    print("wrote", path)


if __name__ == "__main__":
    main()
