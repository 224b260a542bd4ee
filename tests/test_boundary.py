"""Host-side tests of the C ABI: no GPU needed.

The library must load, export every function ``include/ttt.h`` declares, and
reject bad arguments on the host (before any HIP call) with the documented
status and a message.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import chunkwise_weight_recurrence_amd as ttt
from chunkwise_weight_recurrence_amd import binding as B
from chunkwise_weight_recurrence_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "ttt.h")).read()
    return sorted(set(re.findall(r"^TTT_API\s+[\w\s*]*?\b(\w+)\s*\(", src, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from chunkwise_weight_recurrence_amd import build
        build.build()
    return B.lib()


def test_exports_match_header(L):
    declared = _header_functions()
    assert declared == sorted(B.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name
    assert ttt.ttt_version().startswith("libttt")


def test_header_enums_match_binding():
    src = open(os.path.join(ROOT, "include", "ttt.h")).read()
    for cls, prefix in ((B.Status, "TTT_"), (B.DType, "TTT_"), (B.Loss, "TTT_LOSS_"),
                        (B.Act, "TTT_ACT_"), (B.Decay, "TTT_DECAY_")):
        for m in cls:
            name = {"Status": {"OK": "TTT_OK"}}.get(cls.__name__, {}).get(m.name)
            if name is None:
                name = (prefix + ("ERR_" if cls is B.Status else "") + m.name)
            mm = re.search(rf"\b{name}\s*=\s*(-?\d+)", src)
            assert mm is not None, name
            assert int(mm.group(1)) == int(m), name
    # struct layout: 10 int32 then one float
    assert ctypes.sizeof(B.TTTDesc) == 44


def _desc(**kw):
    base = dict(B=2, H=3, T=100, dk=64, dv=64, C=32, dtype="bf16", loss="mse", act="none",
                decay="none", lr_bias=-4.0)
    base.update(kw)
    return B.make_desc(**base)


FAKE = 0x1000   # never dereferenced: every case below fails validation first


def _fwd(desc, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, gamma=None, log_decay=None, w0=None, o=FAKE,
             w_final=None, w_ckpt=None, saved=None, ws=None, ws_bytes=0)
    p.update(ptrs)
    return B.lib().ttt_chunk_fwd(ctypes.byref(desc) if desc is not None else None, p["q"], p["k"],
                                 p["v"], p["beta"], p["gamma"], p["log_decay"], p["w0"], p["o"],
                                 p["w_final"], p["w_ckpt"], p["saved"], p["ws"], p["ws_bytes"], None)


def _bwd(desc, **ptrs):
    names = ["q", "k", "v", "beta", "gamma", "log_decay", "w0", "w_ckpt", "saved", "d_o", "d_wfinal", "dq",
             "dk", "dv", "dbeta", "dgamma", "dlog_decay", "dw0"]
    p = {n: FAKE for n in names}
    p.update(gamma=None, log_decay=None, d_wfinal=None, dgamma=None, dlog_decay=None, w0=None, saved=None)
    p.update(ptrs)
    return B.lib().ttt_chunk_bwd(ctypes.byref(desc), *[p[n] for n in names], p.get("ws"),
                                 p.get("ws_bytes", 0), None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(B=-1), -1, "B, H, T"),
    (dict(T=-5), -1, "B, H, T"),
    (dict(dk=0), -1, "dk, dv"),
    (dict(C=0), -1, "chunk length"),
    (dict(dtype=7), -1, "dtype"),
    (dict(loss=5), -1, "loss"),
    (dict(act=9), -1, "act"),
    (dict(decay=3), -1, "decay"),
    (dict(lr_bias=float("nan")), -1, "lr_bias"),
    (dict(dk=300), -2, "<= 256"),
    (dict(C=512), -2, "<= 256"),
])
def test_desc_validation(L, kw, code, msg):
    assert _fwd(_desc(**kw)) == code
    assert msg in ttt.ttt_last_error()
    n = ctypes.c_size_t(0)
    assert L.ttt_workspace_size(ctypes.byref(_desc(**kw)), 0, ctypes.byref(n)) == code


def test_null_desc_and_pointers(L):
    assert _fwd(None) == -1 and "desc is NULL" in ttt.ttt_last_error()
    assert _fwd(_desc(), q=None) == -1 and "required" in ttt.ttt_last_error()
    assert _fwd(_desc(), o=None) == -1
    assert _fwd(_desc(decay="scalar")) == -1 and "gamma" in ttt.ttt_last_error()
    assert _fwd(_desc(decay="vector")) == -1 and "log_decay" in ttt.ttt_last_error()
    assert _bwd(_desc(), w_ckpt=None) == -1 and "w_ckpt" in ttt.ttt_last_error()
    assert _bwd(_desc(decay="scalar"), gamma=FAKE) == -1 and "dgamma" in ttt.ttt_last_error()
    assert _bwd(_desc(decay="vector"), log_decay=FAKE) == -1 and "dlog_decay" in ttt.ttt_last_error()


def test_workspace_checks(L):
    d = _desc(decay="vector", dtype="f32")
    need = ttt.ttt_workspace_size(d, ttt.ENTRY_FWD)
    assert need >= 2 * 3 * 100 * 64 * 4
    assert _fwd(d, log_decay=FAKE) == -3 and "workspace" in ttt.ttt_last_error()
    assert _fwd(d, log_decay=FAKE, ws=FAKE, ws_bytes=need - 1) == -3
    needb = ttt.ttt_workspace_size(d, ttt.ENTRY_BWD)
    assert needb > 0
    assert _bwd(d, log_decay=FAKE, dlog_decay=FAKE, ws=FAKE, ws_bytes=needb - 1) == -3
    n = ctypes.c_size_t(0)
    assert L.ttt_workspace_size(ctypes.byref(d), 2, ctypes.byref(n)) == -1
    with pytest.raises(ttt.TTTError):
        ttt.ttt_workspace_size(_desc(C=0), 0)


def test_empty_problems_need_no_device(L):
    # B*H == 0, and T == 0 without outputs to fill, return OK without touching HIP
    assert _fwd(_desc(B=0), q=None, k=None, v=None, beta=None, o=None) == 0
    assert _fwd(_desc(T=0), q=None, k=None, v=None, beta=None, o=None) == 0
    assert ttt.ttt_last_error() == ""
    assert _bwd(_desc(B=0)) == 0


def test_inplace_validation(L):
    f = L.inplace_ttt_fwd
    assert f(1, 16, 30, 64, 8, 1e-3, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -2   # d_model % 8
    assert "multiples of 8" in ttt.ttt_last_error()
    assert f(1, 16, 32, 64, 0, 1e-3, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -1
    assert f(1, 16, 32, 64, 8, float("inf"), FAKE, FAKE, FAKE, FAKE, None, 0, None) == -1
    assert f(1, 16, 32, 64, 8, 1e-3, None, FAKE, FAKE, FAKE, None, 0, None) == -1
    assert f(-1, 16, 32, 64, 8, 1e-3, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -1
    assert f(0, 16, 32, 64, 8, 1e-3, None, None, None, None, None, 0, None) == 0
    assert f(1, 16, 32, 64, 8, 1e-3, FAKE, FAKE, FAKE, FAKE, FAKE + 4, 64, None) == -1  # misaligned ws
    assert "ws must be 16-byte aligned" in ttt.ttt_last_error()


def test_inplace_workspace_size(L):
    # the workspace holds bf16(W_down), the apply's operand (256-byte aligned),
    # then fp32 partials when the apply splits its d_ff contraction (too few
    # output tiles for the chip)
    n = B.inplace_ttt_workspace_size(1, 32768, 2560, 9728, 1024)
    wb = 2560 * 9728 * 2
    assert wb % 256 == 0 and n > wb
    part = n - wb
    assert part % (1024 * 2560 * 4) == 0 and 2 <= part // (1024 * 2560 * 4) <= 8
    assert B.inplace_ttt_workspace_size(0, 16, 32, 64, 8) == 0
    assert B.inplace_ttt_workspace_size(1, 16, 32, 64, 8) == 32 * 64 * 2   # d_ff too short to split
    with pytest.raises(ttt.TTTError):
        B.inplace_ttt_workspace_size(1, 16, 30, 64, 8)


def test_inplace_guarded_validation(L):
    import ctypes
    f = L.inplace_ttt_fwd_guarded
    big = 1 << 20

    def starts(*p):
        return (ctypes.c_int64 * len(p))(*p), len(p)

    def call(tau=1e-5, docs=(None, 0), w_init=FAKE, ws=FAKE, ws_bytes=big, T=16, B_=2):
        return f(B_, T, 32, 64, 8, 1e-3, tau, docs[0], docs[1], FAKE, FAKE, w_init, FAKE, FAKE, ws, ws_bytes, None)

    assert call(tau=-1.0) == -1 and "clip_tau" in ttt.ttt_last_error()
    assert call(tau=float("nan")) == -1
    assert call(docs=starts(0)) == -1 and "doc_starts[0]" in ttt.ttt_last_error()     # t = 0
    assert call(docs=starts(16)) == -1                                                # b T + 0
    assert call(docs=starts(32)) == -1                                                # past B T
    assert call(docs=starts(9, 5)) == -1 and "increasing" in ttt.ttt_last_error()
    assert call(docs=starts(5, 5)) == -1
    assert call(docs=(None, 2)) == -1 and "NULL" in ttt.ttt_last_error()
    assert call(docs=starts(5), w_init=None) == -1 and "w_init" in ttt.ttt_last_error()
    assert call(ws=None, ws_bytes=0) == -3 and "workspace" in ttt.ttt_last_error()   # clipping needs it
    assert call(ws_bytes=16) == -3
    assert call(docs=starts(5), w_init=FAKE + 4) == -1 and "w_init must be 16-byte aligned" in ttt.ttt_last_error()
    assert call(B_=0, docs=(None, 0)) == 0                                            # nothing to do
    assert f(1, 16, 32, 64, 8, 1e-3, 0.0, None, -1, FAKE, FAKE, None, FAKE, FAKE, None, 0, None) == -1


def test_inplace_guarded_workspace_size(L):
    plain = B.inplace_ttt_workspace_size(1, 32768, 2560, 9728, 1024)
    n = B.inplace_ttt_guarded_workspace_size(1, 32768, 2560, 9728, 1024)
    tiles = 20 * 76                                  # 128 x 128 tiles of the 2560 x 9728 update
    assert n - plain >= tiles * 4 + 4 and n - plain <= tiles * 4 + 512
    assert B.inplace_ttt_guarded_workspace_size(0, 16, 32, 64, 8) == 0


def test_inplace_doc_starts_recipe():
    per_seq, flat = wl.inplace_doc_starts(wl.INPLACE_WORKLOADS["inplace-wdown-guarded"])
    assert per_seq == [[9000, 16000, 28000]] and flat == [9000, 16000, 28000]
    per_seq, flat = wl.inplace_doc_starts(dict(B=2, T=10, doc_lens=(3, 7)))
    assert per_seq == [[3], [3]] and flat == [3, 13]
    assert wl.inplace_doc_starts(dict(B=2, T=10)) == ([[], []], [])


def test_inplace_backward_validation(L):
    f = L.inplace_ttt_bwd
    big = 1 << 30
    args = lambda **kw: [kw.get("B", 1), 16, 32, 64, 8, kw.get("eta", 1e-3), FAKE, FAKE, kw.get("wf", FAKE), FAKE,
                         kw.get("dwf", None), FAKE, FAKE, kw.get("dw0", FAKE), kw.get("ws", FAKE), kw.get("wsb", big), None]
    assert f(*args(ws=None, wsb=0)) == -3 and "workspace" in ttt.ttt_last_error()
    assert f(*args(wsb=16)) == -3
    assert f(*args(wf=None)) == -1 and "required" in ttt.ttt_last_error()
    assert f(*args(dw0=None)) == -1
    assert f(*args(eta=float("nan"))) == -1
    assert f(*args(dwf=FAKE + 4)) == -1 and "d_wfinal must be 16-byte aligned" in ttt.ttt_last_error()
    assert f(*args(B=0)) == 0
    n = B.inplace_ttt_bwd_workspace_size(1, 32768, 2560, 9728, 1024)
    assert n >= 2560 * 9728 * 4 + 2 * 1024 * 9728 * 4


def test_inplace_workspace_covers_a_short_last_chunk(L):
    """A short last chunk has fewer row tiles and can split its apply further
    than a full chunk: T 556 at C 300 ends on a 256-token chunk, which splits
    its d_ff contraction three ways (85 column tiles, 256 compute units) where a
    300-token chunk does not split at all; the workspace must hold those
    partials (256 x 10880 fp32 each)."""
    wb = 10880 * 2048 * 2
    part = 3 * 256 * 10880 * 4
    assert B.inplace_ttt_workspace_size(1, 556, 10880, 2048, 300) >= wb + part
    assert B.inplace_ttt_bwd_workspace_size(1, 556, 10880, 2048, 300) >= wb * 4 + part


def test_inplace_backward_guarded_validation(L):
    import ctypes
    f = L.inplace_ttt_bwd_guarded
    big = 1 << 30

    def starts(*p):
        return (ctypes.c_int64 * len(p))(*p), len(p)

    def call(tau=1e-5, docs=(None, 0), w0=FAKE, wi=FAKE, wf=FAKE, dw0=FAKE, dwi=None, ws=FAKE, wsb=big, B_=2,
             C=8, eta=1e-3):
        return f(B_, 16, 32, 64, C, eta, tau, docs[0], docs[1], FAKE, FAKE, w0, wi, wf, FAKE, None, FAKE, FAKE, dw0,
                 dwi, ws, wsb, None)

    assert call(tau=-1.0) == -1 and "clip_tau" in ttt.ttt_last_error()
    assert call(eta=float("inf")) == -1
    assert call(docs=starts(16)) == -1 and "doc_starts[0]" in ttt.ttt_last_error()
    assert call(docs=starts(9, 5)) == -1 and "increasing" in ttt.ttt_last_error()
    assert call(docs=starts(5), w0=None) == -1 and "w0 and w_init" in ttt.ttt_last_error()
    assert call(docs=starts(5), wi=None) == -1
    assert call(wf=None) == -1 and "required" in ttt.ttt_last_error()
    assert call(dw0=None) == -1
    assert call(ws=None, wsb=0) == -3 and "workspace" in ttt.ttt_last_error()
    assert call(wsb=16) == -3
    assert call(dwi=FAKE + 4) == -1 and "dw_init must be 16-byte aligned" in ttt.ttt_last_error()
    assert call(B_=0) == 0
    assert f(1, 20000, 64, 128, 10000, 1e-3, 1e-5, None, 0, FAKE, FAKE, None, None, FAKE, FAKE, None, FAKE, FAKE,
             FAKE, None, FAKE, big, None) == -2 and "8192" in ttt.ttt_last_error()
    n = B.inplace_ttt_bwd_guarded_workspace_size(1, 32768, 2560, 9728, 1024)
    plain = B.inplace_ttt_bwd_workspace_size(1, 32768, 2560, 9728, 1024)
    assert n >= plain + 1024 * 9728 * 4 + 1024 * 2560 * 4 + 1024 * 1024 * 2   # third dZ product, R, Gram
    with pytest.raises(ttt.TTTError) as ei:
        B.inplace_ttt_bwd_guarded_workspace_size(1, 20000, 64, 128, 10000)      # min(T, C) > 8192
    assert ei.value.status == ttt.Status.UNSUPPORTED


def test_binding_raises_with_message(L):
    with pytest.raises(ttt.TTTError) as ei:
        ttt.ttt_chunk_fwd(_desc(dk=0), FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, None, None, None, None, 0)
    assert ei.value.status == ttt.Status.INVALID_ARG
    assert "dk, dv" in str(ei.value)


def test_last_error_is_thread_local(L):
    import threading
    _fwd(_desc(dk=0))
    seen = {}

    def other():
        seen["msg"] = ttt.ttt_last_error()

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["msg"] == ""
    assert "dk, dv" in ttt.ttt_last_error()


def test_kernel_ids_match_header():
    src = open(os.path.join(ROOT, "include", "ttt.h")).read()
    for m in B.Kernel:
        mm = re.search(rf"\bTTT_KERNEL_{m.name}\s*=\s*(\d+)", src)
        assert mm is not None, m.name
        assert int(mm.group(1)) == int(m), m.name
    assert int(re.search(r"\bTTT_KERNEL_COUNT\s*=\s*(\d+)", src).group(1)) == len(B.Kernel)


def test_timing_records_nothing_for_rejected_calls(L):
    # Enabling, a rejected call and reading back make no HIP call: the record stays empty.
    B.ttt_timing_enable(True)
    try:
        assert _fwd(_desc(dk=0)) == -1
        for k in B.Kernel:
            assert B.ttt_timing_read(k) == (0.0, 0)
    finally:
        B.ttt_timing_enable(False)
    assert L.ttt_timing_read(len(B.Kernel), None, None) == int(B.Status.INVALID_ARG)
    assert L.ttt_timing_read(-1, None, None) == int(B.Status.INVALID_ARG)


def test_misaligned_pointers_are_rejected(L):
    assert _fwd(_desc(), q=FAKE + 8) == -1 and "q must be 16-byte aligned" in ttt.ttt_last_error()
    assert _fwd(_desc(), saved=FAKE + 2) == -1 and "saved" in ttt.ttt_last_error()
    assert _bwd(_desc(), dk=FAKE + 4) == -1 and "dk must be 16-byte aligned" in ttt.ttt_last_error()
    # beta, gamma, dbeta, dgamma are read and written element by element: any alignment
    assert _fwd(_desc(B=0), beta=FAKE + 4) == 0


def test_saved_context_size(L):
    tv = 2 * 3 * 100 * 64 * 2                      # one [B,H,T,dv] bf16 tensor
    none_ip = B.ttt_saved_size(_desc(loss="ip"))   # identity act: only eta (.) G
    assert none_ip == tv
    silu = B.ttt_saved_size(_desc(act="silu"))     # + f'(Y) and Z
    assert silu == 3 * tv
    vec = B.ttt_saved_size(_desc(decay="vector"))  # + Q~, K~, lambda, tile prefixes of L
    nc = (100 + 31) // 32
    assert vec >= tv + 2 * (2 * 3 * 100 * 64 * 2) + 2 * 3 * nc * 64 * 4
    # problems the matrix-core backward does not run keep no context
    assert B.ttt_saved_size(_desc(dtype="f32")) == 0
    assert B.ttt_saved_size(_desc(dk=96, dv=96)) == 0
    assert B.ttt_saved_size(_desc(dv=96)) == 0
    with pytest.raises(ttt.TTTError):
        B.ttt_saved_size(_desc(C=0))


def _mdesc(**kw):
    base = dict(B=2, H=3, T=100, dk=64, dh=256, dv=64, C=32, dtype="bf16", loss="mse", act="silu",
                decay="none", lr_bias=-4.0)
    base.update(kw)
    return B.make_mlp_desc(**base)


def _mfwd(desc, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, gamma=None, w1_0=None, w2_0=None, o=FAKE, w1_final=None,
             w2_final=None, w1_ckpt=None, w2_ckpt=None, saved=None, ws=None, ws_bytes=0)
    p.update(ptrs)
    return B.lib().ttt_mlp_chunk_fwd(ctypes.byref(desc) if desc is not None else None, p["q"], p["k"], p["v"],
                                     p["beta"], p["gamma"], p["w1_0"], p["w2_0"], p["o"], p["w1_final"],
                                     p["w2_final"], p["w1_ckpt"], p["w2_ckpt"], p["saved"], p["ws"], p["ws_bytes"],
                                     None)


def _mbwd(desc, **ptrs):
    names = ["q", "k", "v", "beta", "gamma", "w1_ckpt", "w2_ckpt", "saved", "d_o", "d_w1final", "d_w2final", "dq",
             "dk", "dv", "dbeta", "dgamma", "dw1_0", "dw2_0"]
    p = {n: FAKE for n in names}
    p.update(gamma=None, saved=None, d_w1final=None, d_w2final=None, dgamma=None, dw1_0=None, dw2_0=None, ws=None, ws_bytes=0)
    p.update(ptrs)
    return B.lib().ttt_mlp_chunk_bwd(ctypes.byref(desc), *[p[n] for n in names], p["ws"], p["ws_bytes"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(B=-1), -1, "B, H, T"),
    (dict(dh=0), -1, "dk, dh, dv"),
    (dict(dv=0), -1, "dk, dh, dv"),
    (dict(C=0), -1, "chunk length"),
    (dict(dtype=7), -1, "dtype"),
    (dict(loss=5), -1, "loss"),
    (dict(act=9), -1, "act"),
    (dict(decay="vector"), -2, "vector decay"),
    (dict(decay=5), -1, "decay"),
    (dict(lr_bias=float("inf")), -1, "lr_bias"),
    (dict(dk=257), -2, "dh <= 1024"),
    (dict(dh=1025), -2, "dh <= 1024"),
    (dict(C=257), -2, "<= 256"),
])
def test_mlp_desc_validation(L, kw, code, msg):
    assert _mfwd(_mdesc(**kw)) == code
    assert msg in ttt.ttt_last_error()
    n = ctypes.c_size_t(0)
    assert L.ttt_mlp_workspace_size(ctypes.byref(_mdesc(**kw)), ctypes.byref(n)) == code


def test_mlp_pointer_and_workspace_checks(L):
    assert ctypes.sizeof(B.TTTMlpDesc) == 48
    assert _mfwd(None) == -1 and "desc is NULL" in ttt.ttt_last_error()
    assert _mfwd(_mdesc(), v=None) == -1 and "required" in ttt.ttt_last_error()
    assert _mfwd(_mdesc(decay="scalar")) == -1 and "gamma" in ttt.ttt_last_error()
    d = _mdesc()
    need = ttt.ttt_mlp_workspace_size(d)
    # per chain: two copies of W1 and W2, the chunk's Q, K, V, five [C, d_h] / [C, d_v] buffers and
    # the C x C scores, each region rounded up to 64 floats
    r = lambda n: -(-n // 64) * 64
    per_chain = 2 * r(64 * 256) + 2 * r(256 * 64) + 2 * r(32 * 64) + r(32 * 64) + 3 * r(32 * 256) + \
        2 * r(32 * 64) + r(32 * 32)
    assert need >= 6 * per_chain * 4
    assert _mfwd(d) == -3 and "workspace" in ttt.ttt_last_error()
    assert _mfwd(d, ws=FAKE, ws_bytes=need - 1) == -3
    assert _mfwd(d, o=FAKE + 4, ws=FAKE, ws_bytes=need) == -1 and "aligned" in ttt.ttt_last_error()
    # empty problems touch no device memory
    assert _mfwd(_mdesc(B=0), q=None, k=None, v=None, beta=None, o=None) == 0
    assert _mfwd(_mdesc(T=0), q=None, k=None, v=None, beta=None, o=None) == 0


def test_mlp_workload_recipe():
    inp = wl.make_mlp_inputs("160m-mlp-fwd", T=8, B=2)
    cfg = inp["cfg"]
    assert inp["q_dev"].shape == (2, 12, 8, 64) and inp["v_dev"].shape == (2, 12, 8, 64)
    assert inp["w1_0_dev"].shape == (2, 12, 64, 256) and inp["w2_0_dev"].shape == (2, 12, 256, 64)
    assert np.allclose(np.linalg.norm(inp["q"], axis=-1), 1.0, atol=1e-2)
    assert np.array_equal(inp["w1_0_dev"][0], inp["w1_0_dev"][1])  # shared over the batch
    assert cfg["decay"] == "scalar" and np.all(inp["gamma_dev"] == np.float32(0.99))
    sub = wl.select_mlp_chains(inp, [(1, 3)])
    assert np.array_equal(sub["k"][0, 0], inp["k"][1, 3]) and sub["cfg"]["H"] == 1


def test_mlp_backward_validation(L):
    d = _mdesc(decay="scalar")
    need = ttt.ttt_mlp_bwd_workspace_size(d)
    assert need > ttt.ttt_mlp_workspace_size(d)
    assert _mbwd(_mdesc(), w1_ckpt=None) == -1 and "w1_ckpt" in ttt.ttt_last_error()
    assert _mbwd(_mdesc(), d_o=None) == -1 and "required" in ttt.ttt_last_error()
    assert _mbwd(d, gamma=FAKE) == -1 and "dgamma" in ttt.ttt_last_error()
    assert _mbwd(_mdesc()) == -3 and "workspace" in ttt.ttt_last_error()
    assert _mbwd(_mdesc(), ws=FAKE, ws_bytes=ttt.ttt_mlp_bwd_workspace_size(_mdesc()) - 1) == -3
    assert _mbwd(_mdesc(), dq=FAKE + 2) == -1 and "aligned" in ttt.ttt_last_error()
    assert _mbwd(_mdesc(decay="vector")) == -2
    assert _mbwd(_mdesc(B=0)) == 0
    n = ctypes.c_size_t(0)
    assert L.ttt_mlp_bwd_workspace_size(ctypes.byref(_mdesc(dh=0)), ctypes.byref(n)) == -1


def test_mlp_saved_size(L):
    d = _mdesc(T=100, C=32)   # 4 chunks
    r = lambda n: -(-n // 64) * 64
    per_chunk = 6 * r(32 * 256) + 2 * r(32 * 64) + 2 * r(32 * 32) + r(32)   # ..., the RMSE row scales
    assert ttt.ttt_mlp_saved_size(d) == -(-(4 * 2 * 3 * 4 * per_chunk) // 256) * 256
    assert _mfwd(_mdesc(), saved=FAKE + 8, ws=FAKE, ws_bytes=10 ** 9) == -1 and "saved" in ttt.ttt_last_error()
