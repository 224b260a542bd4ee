"""Host-side checks of bench.py's accounting (no GPU)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from chunkwise_weight_recurrence_amd import workloads as wl  # noqa: E402


def _cfg(name):
    return dict(wl.WORKLOADS[name])


def test_headline_per_token_head_figures():
    c3 = _cfg("1.45b-fwdbwd")
    w = bench.algorithmic_work(c3)
    assert w["flop_per_th"] == (163840, 360448)       # 6d^2 + 2Cd, 12d^2 + 5Cd at d=128, C=256
    assert w["bytes_per_th"] == (1796, 3080)
    assert w["token_heads"] == 4 * 16 * 4096


@pytest.mark.parametrize("name", ["410m-silu-fwdbwd", "1.45b-fwdbwd"])
def test_kernel_split_sums_to_the_path(name):
    cfg = _cfg(name)
    w = bench.algorithmic_work(cfg)
    k = bench.kernel_work(cfg)
    assert k["fwd"] == w["flop_per_th"][:1] + w["bytes_per_th"][:1]
    assert k["bwd_seq"][0] + k["bwd_cross"][0] == w["flop_per_th"][1]
    assert k["bwd_seq"][1] + k["bwd_cross"][1] == w["bytes_per_th"][1]


def test_linear_path_split_sums_to_the_forward():
    cfg = _cfg("1.45b-iplin-32k")
    assert bench.linear_path(cfg)
    w = bench.algorithmic_work(cfg)
    k = bench.kernel_work(cfg)
    assert w["flop_per_th"][0] == 4 * 128 * 128 + 2 * 256 * 128       # no train-view K W
    assert k["lin_state"][0] + k["lin_scan"][0] + k["lin_out"][0] == w["flop_per_th"][0]
    assert k["lin_state"][1] + k["lin_scan"][1] + k["lin_out"][1] == w["bytes_per_th"][0]


def test_headline_kernels_are_hbm_bound():
    # with vector decay every kernel sits below the bf16 ridge (2.5 PFLOP/s over 8 TB/s)
    for f, b in bench.kernel_work(_cfg("1.45b-fwdbwd")).values():
        assert f / b < 2500.0 / 8.0


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_stale_counter_traffic_is_ignored(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    (tmp_path / "chunkwise_weight_recurrence_amd" / "csrc").mkdir(parents=True)
    csrc = tmp_path / "chunkwise_weight_recurrence_amd" / "csrc"
    (csrc / "ttt_mfma_bwd.hip").write_text("a")
    (csrc / "inplace.hip").write_text("a")
    digest = bench.kernel_source_digest("ttt")
    rec = ('traffic-record: {"kernel": "ttt_bwd_seq_kernel", "workload": "w", "sources": "%s", '
           '"bytes_per_launch": 123}\n')
    (tmp_path / "profiles" / "hbm_traffic.md").write_text(rec % digest)
    assert bench.counter_traffic("ttt_bwd_seq_kernel", "w") == 123
    (csrc / "inplace.hip").write_text("b")          # another family's source: still valid
    assert bench.counter_traffic("ttt_bwd_seq_kernel", "w") == 123
    (csrc / "ttt_mfma_bwd.hip").write_text("b")     # its own source: stale
    assert bench.counter_traffic("ttt_bwd_seq_kernel", "w") is None


@pytest.mark.parametrize("loss", ["mse", "ip"])
def test_mlp_flop_count_matches_the_chunk_products(loss):
    """mlp_work against the chunk's products listed one by one, with each causal
    c x c product counted over its lower triangle (diagonal included) and the
    per-chunk sums taken over every chunk of the sequence."""
    cfg = dict(wl.MLP_WORKLOADS["160m-mlp-fwd"], loss=loss, T=700, C=256)
    dk, dh, dv, C, T = cfg["dk"], cfg["dh"], cfg["dv"], cfg["C"], cfg["T"]
    total = 0
    for s0 in range(0, T, C):
        c = min(C, T - s0)
        tri = c * (c + 1) // 2
        dense = [(c, dk, dh), (c, dv, dh), (c, dk, dh), (c, dh, dv), (dk, c, dh), (dh, c, dv)]
        if loss == "mse":
            dense.append((c, dh, dv))
        total += sum(2 * m * k * n for m, k, n in dense)
        total += 2 * tri * (dk + dh) + 2 * tri * (dh + dv)  # scores and their products with eta G
    flop, _ = bench.mlp_work(cfg)
    assert flop == total * cfg["B"] * cfg["H"]
    assert sum(bench.mlp_fwd_split(cfg).values()) == flop
    assert bench.kernel_family("mlp_fwd") == "mlp"
    assert bench.kernel_family("mlp_query_kernel") == "mlp"


@pytest.mark.parametrize("loss", ["mse", "ip"])
def test_mlp_backward_flop_count_matches_the_adjoint_products(loss):
    """mlp_bwd_work against the backward's products listed one by one (without the
    forward recomputed per chunk); causal products over the lower triangle."""
    cfg = dict(wl.MLP_WORKLOADS["160m-mlp-fwdbwd"], loss=loss, T=700, C=256)
    dk, dh, dv, C, T = cfg["dk"], cfg["dh"], cfg["dv"], cfg["C"], cfg["T"]
    total = 0
    for s0 in range(0, T, C):
        c = min(C, T - s0)
        tri = c * (c + 1) // 2
        dense = [(c, dh, dk), (c, dk, dh), (c, dh, dk), (c, dh, dk),   # dQ, K D1, Gh1 D1^T, dZ1 W1^T
                 (dk, c, dh), (dk, c, dh),                             # Q^T dX1, K^T dZ1
                 (c, dh, dv), (c, dv, dh), (c, dv, dh), (c, dh, dv),   # A D2, dO W2^T, Gh2 D2^T, dP W2
                 (dh, c, dv), (dh, c, dv)]                             # Aq^T dO, dP^T G2
        if loss == "mse":
            dense += [(c, dv, dh), (dh, c, dv)]                        # dG2 W2^T, A^T dG2
        total += sum(2 * m * k * n for m, k, n in dense)
        # dS2, S2^T dO (d_v); dS2 A, dS2^T Aq, dS1, S1^T dX1 (d_h); dS1 K, dS1^T Q (d_k)
        total += 2 * tri * (2 * dv + 4 * dh + 2 * dk)
    assert bench.mlp_bwd_work(cfg) == total * cfg["B"] * cfg["H"]
    # the reverse sweep's products: A dW2', G2e dW2'^T, K dW1', G1e dW1'^T, dP W2, dZ1 W1^T,
    # K^T dZ1, dP^T G2 (+ dV_hat W2^T, A^T dV_hat for MSE)
    n_sweep = 0
    for s0 in range(0, T, C):
        c = min(C, T - s0)
        sweep = [(c, dh, dv), (c, dv, dh), (c, dk, dh), (c, dh, dk), (c, dh, dv), (c, dh, dk), (dk, c, dh),
                 (dh, c, dv)] + ([(c, dv, dh), (dh, c, dv)] if loss == "mse" else [])
        n_sweep += sum(2 * m * k * n for m, k, n in sweep)
    split = bench.mlp_bwd_split(cfg)
    assert split["mlp_bwd"] == n_sweep * cfg["B"] * cfg["H"]
    assert sum(split.values()) == bench.mlp_bwd_work(cfg)


def test_norm_flop_count_matches_the_products():
    cfg = dict(wl.WORKLOADS["160m-norm-fwdbwd"], T=700)
    dk, dv, C, T = cfg["dk"], cfg["dv"], cfg["C"], cfg["T"]
    fwd = query = pre = bwd = 0
    for s0 in range(0, T, C):
        c = min(C, T - s0)
        tri = c * (c + 1) // 2
        fwd += sum(2 * m * k * n for m, k, n in [(c, dk, dv), (dk, c, dv)])      # K W, K^T G
        query += 2 * c * dk * dv + 2 * tri * (dk + dv)                           # Q W, Q K^T, S G
        # dY W^T, Q^T dY; dS, S^T dY, dS K, dS^T Q
        pre += sum(2 * m * k * n for m, k, n in [(c, dv, dk), (dk, c, dv)]) + 2 * tri * (2 * dv + 2 * dk)
        # K dW', G dW'^T, dZ W^T, K^T dZ
        bwd += sum(2 * m * k * n for m, k, n in [(c, dk, dv), (c, dv, dk), (c, dv, dk), (dk, c, dv)])
    f, q, p, b = bench.norm_work(cfg)
    bh = cfg["B"] * cfg["H"]
    assert (f, q, p, b) == (fwd * bh, query * bh, pre * bh, bwd * bh)
    assert bench.kernel_family("norm_bwd") == "norm"
    assert bench.kernel_family("norm_query_kernel") == "norm"
