"""Device plumbing around the C ABI: move seeded inputs to HBM, allocate
outputs and workspace with torch, and call libttt.  No arithmetic of the layer
happens here -- torch only provides device memory and the stream.
"""
from __future__ import annotations

import math

import numpy as np

from . import binding as B


def _torch():
    import torch
    return torch


def to_device(arr, device="cuda"):
    """numpy payload -> torch tensor on the device (uint16 arrays are bf16 bit patterns)."""
    torch = _torch()
    if arr is None:
        return None
    if arr.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(device)


def to_f64(t):
    """torch tensor (bf16 or f32) -> numpy float64."""
    torch = _torch()
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def desc_from_cfg(cfg):
    return B.make_desc(cfg["B"], cfg["H"], cfg["T"], cfg["dk"], cfg["dv"], cfg["C"],
                       dtype=cfg["dtype"], loss=cfg["loss"], act=cfg["act"], decay=cfg["decay"],
                       lr_bias=cfg["b"])


class TTTLayerBuffers:
    """Device copies of one input set plus every output and workspace buffer.

    With ``saved=True`` (the default) the forward keeps the library's saved
    context for the backward when the problem has one; ``saved=False`` makes
    the backward recompute the forward's chunk intermediates.
    """

    def __init__(self, inp, device="cuda", with_bwd=None, saved=True):
        torch = _torch()
        cfg = inp["cfg"]
        self.cfg = cfg
        self.desc = desc_from_cfg(cfg)
        Bn, H, T, dk, dv, C = cfg["B"], cfg["H"], cfg["T"], cfg["dk"], cfg["dv"], cfg["C"]
        self.nc = math.ceil(T / C) if T > 0 else 0
        io_dt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
        f32 = torch.float32
        d = device
        self.q = to_device(inp["q_dev"], d)
        self.k = to_device(inp["k_dev"], d)
        self.v = to_device(inp["v_dev"], d)
        self.beta = to_device(inp["beta_dev"], d)
        self.gamma = to_device(inp.get("gamma_dev"), d)
        self.log_a = to_device(inp.get("log_a_dev"), d)
        self.w0 = to_device(inp.get("w0_dev"), d)
        self.o = torch.empty((Bn, H, T, dv), dtype=io_dt, device=d)
        self.w_final = torch.empty((Bn, H, dk, dv), dtype=f32, device=d)
        self.w_ckpt = torch.empty((Bn, H, self.nc, dk, dv), dtype=f32, device=d)
        ws_f = B.ttt_workspace_size(self.desc, B.ENTRY_FWD)
        self.ws_fwd = torch.empty(max(ws_f, 1), dtype=torch.uint8, device=d)
        self.has_bwd = cfg.get("bwd", False) if with_bwd is None else with_bwd
        if self.has_bwd:
            self.d_o = to_device(inp["d_o_dev"], d)
            self.dq = torch.empty((Bn, H, T, dk), dtype=io_dt, device=d)
            self.dk = torch.empty((Bn, H, T, dk), dtype=io_dt, device=d)
            self.dv = torch.empty((Bn, H, T, dv), dtype=io_dt, device=d)
            self.dbeta = torch.empty((Bn, H, T), dtype=f32, device=d)
            self.dgamma = torch.empty((Bn, H), dtype=f32, device=d) if cfg["decay"] == "scalar" else None
            self.dlog_a = torch.empty((Bn, H, T, dk), dtype=f32, device=d) \
                if cfg["decay"] == "vector" else None
            self.dw0 = torch.empty((Bn, H, dk, dv), dtype=f32, device=d)
            ws_b = B.ttt_workspace_size(self.desc, B.ENTRY_BWD)
            self.ws_bwd = torch.empty(max(ws_b, 1), dtype=torch.uint8, device=d)
        n_saved = B.ttt_saved_size(self.desc) if (saved and self.has_bwd) else 0
        self.saved = torch.empty(n_saved, dtype=torch.uint8, device=d) if n_saved else None

    def forward(self, stream=None):
        B.ttt_chunk_fwd(self.desc, self.q, self.k, self.v, self.beta, self.gamma, self.log_a, self.w0,
                        self.o, self.w_final, self.w_ckpt, self.saved, self.ws_fwd, stream=stream)

    def backward(self, stream=None, d_wfinal=None):
        B.ttt_chunk_bwd(self.desc, self.q, self.k, self.v, self.beta, self.gamma, self.log_a, self.w0,
                        self.w_ckpt, self.saved, self.d_o, d_wfinal, self.dq, self.dk, self.dv, self.dbeta,
                        self.dgamma, self.dlog_a, self.dw0, self.ws_bwd, stream=stream)


class MlpBuffers:
    """Device copies of one two-layer (TTT-MLP) input set, its outputs and workspace."""

    def __init__(self, inp, device="cuda", with_bwd=False, saved=True):
        torch = _torch()
        cfg = inp["cfg"]
        self.cfg = cfg
        self.desc = B.make_mlp_desc(cfg["B"], cfg["H"], cfg["T"], cfg["dk"], cfg["dh"], cfg["dv"], cfg["C"],
                                    dtype=cfg["dtype"], loss=cfg["loss"], act=cfg["act"], decay=cfg["decay"],
                                    lr_bias=cfg["b"])
        Bn, H, T, dk, dh, dv = cfg["B"], cfg["H"], cfg["T"], cfg["dk"], cfg["dh"], cfg["dv"]
        io_dt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
        d = device
        self.q = to_device(inp["q_dev"], d)
        self.k = to_device(inp["k_dev"], d)
        self.v = to_device(inp["v_dev"], d)
        self.beta = to_device(inp["beta_dev"], d)
        self.gamma = to_device(inp.get("gamma_dev"), d)
        self.w1_0 = to_device(inp.get("w1_0_dev"), d)
        self.w2_0 = to_device(inp.get("w2_0_dev"), d)
        self.o = torch.empty((Bn, H, T, dv), dtype=io_dt, device=d)
        self.w1 = torch.empty((Bn, H, dk, dh), dtype=torch.float32, device=d)
        self.w2 = torch.empty((Bn, H, dh, dv), dtype=torch.float32, device=d)
        self.ws_bytes = B.ttt_mlp_workspace_size(self.desc)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=d)
        self.has_bwd = with_bwd
        self.w1_ckpt = self.w2_ckpt = None
        if with_bwd:
            nc = -(-T // cfg["C"]) if T > 0 else 0
            f32 = torch.float32
            self.w1_ckpt = torch.empty((Bn, H, nc, dk, dh), dtype=f32, device=d)
            self.w2_ckpt = torch.empty((Bn, H, nc, dh, dv), dtype=f32, device=d)
            self.dq = torch.empty((Bn, H, T, dk), dtype=io_dt, device=d)
            self.dk = torch.empty((Bn, H, T, dk), dtype=io_dt, device=d)
            self.dv = torch.empty((Bn, H, T, dv), dtype=io_dt, device=d)
            self.dbeta = torch.empty((Bn, H, T), dtype=f32, device=d)
            self.dgamma = torch.empty((Bn, H), dtype=f32, device=d) if cfg["decay"] == "scalar" else None
            self.dw1 = torch.empty((Bn, H, dk, dh), dtype=f32, device=d)
            self.dw2 = torch.empty((Bn, H, dh, dv), dtype=f32, device=d)
            self.ws_bwd_bytes = B.ttt_mlp_bwd_workspace_size(self.desc)
            self.ws_bwd = torch.empty(max(self.ws_bwd_bytes, 1), dtype=torch.uint8, device=d)
        n_saved = B.ttt_mlp_saved_size(self.desc) if (with_bwd and saved) else 0
        self.saved = torch.empty(n_saved, dtype=torch.uint8, device=d) if n_saved else None

    def forward(self, stream=None):
        B.ttt_mlp_chunk_fwd(self.desc, self.q, self.k, self.v, self.beta, self.gamma, self.w1_0, self.w2_0,
                            self.o, self.w1, self.w2, self.w1_ckpt, self.w2_ckpt, self.saved, self.ws,
                            self.ws_bytes, stream=stream)

    def backward(self, d_o, d_w1final=None, d_w2final=None, stream=None):
        """The outer backward from the forward's checkpoints; fills dq, dk, dv, dbeta,
        dgamma (scalar decay), dw1 and dw2."""
        B.ttt_mlp_chunk_bwd(self.desc, self.q, self.k, self.v, self.beta, self.gamma, self.w1_ckpt, self.w2_ckpt,
                            self.saved, d_o, d_w1final, d_w2final, self.dq, self.dk, self.dv, self.dbeta, self.dgamma, self.dw1,
                            self.dw2, self.ws_bwd, self.ws_bwd_bytes, stream=stream)


class InplaceBuffers:
    """Device copies of In-Place inputs; w_down is reset from w0 by reset().

    With ``clip_tau`` or ``doc_lens`` in the config (or ``guarded=True``) the
    guarded entry point runs, and w0 is also the state documents restart from.
    """

    def __init__(self, inp, device="cuda", workspace=True, guarded=None):
        from .workloads import inplace_doc_starts
        torch = _torch()
        cfg = inp["cfg"]
        self.cfg = cfg
        self.guarded = bool(cfg.get("clip_tau") or cfg.get("doc_lens")) if guarded is None else guarded
        self.doc_starts = inplace_doc_starts(cfg)[1]
        self.z = to_device(inp["z_dev"], device)
        self.vhat = to_device(inp["vhat_dev"], device)
        self.w0 = to_device(inp["w0_dev"], device)
        self.w = self.w0.clone()
        Bn, T, dm = cfg["B"], cfg["T"], cfg["d_model"]
        self.o = torch.empty((Bn, T, dm), dtype=torch.bfloat16, device=device)
        size = B.inplace_ttt_guarded_workspace_size if self.guarded else B.inplace_ttt_workspace_size
        n_ws = size(Bn, T, dm, cfg["d_ff"], cfg["C"]) if workspace else 0
        self.ws = torch.empty(n_ws, dtype=torch.uint8, device=device) if n_ws else None
        self.ws_bytes = n_ws

    def reset(self):
        self.w.copy_(self.w0)

    def backward(self, d_o, d_wfinal=None, stream=None):
        """The backward from the state the last forward left in ``self.w``
        (inplace_ttt_bwd, or inplace_ttt_bwd_guarded for the guarded forward);
        returns (dz, dvhat, dw0) device tensors.  Guarded, ``self.dw_init``
        then holds dL/dw_init over the documents after each sequence's first
        (w0 is also the state they restart from, so its total derivative is
        dw0 + dw_init)."""
        torch = _torch()
        c = self.cfg
        dev = self.w.device
        Bn, T, dm, dff = c["B"], c["T"], c["d_model"], c["d_ff"]
        if not hasattr(self, "dz"):
            self.dz = torch.empty((Bn, T, dff), dtype=torch.bfloat16, device=dev)
            self.dvhat = torch.empty((Bn, T, dm), dtype=torch.bfloat16, device=dev)
            self.dw0 = torch.empty((Bn, dm, dff), dtype=torch.float32, device=dev)
            size = B.inplace_ttt_bwd_guarded_workspace_size if self.guarded else B.inplace_ttt_bwd_workspace_size
            n = size(Bn, T, dm, dff, c["C"])
            self.ws_bwd = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
            self.ws_bwd_bytes = n
            self.dw_init = torch.empty((Bn, dm, dff), dtype=torch.float32, device=dev) if self.guarded else None
        if self.guarded:
            B.inplace_ttt_bwd_guarded(Bn, T, dm, dff, c["C"], c["eta"], c.get("clip_tau") or 0.0, self.doc_starts,
                                      self.z, self.vhat, self.w0, self.w0, self.w, d_o, d_wfinal, self.dz,
                                      self.dvhat, self.dw0, self.dw_init, self.ws_bwd, self.ws_bwd_bytes,
                                      stream=stream)
        else:
            B.inplace_ttt_bwd(Bn, T, dm, dff, c["C"], c["eta"], self.z, self.vhat, self.w, d_o, d_wfinal, self.dz,
                              self.dvhat, self.dw0, self.ws_bwd, self.ws_bwd_bytes, stream=stream)
        return self.dz, self.dvhat, self.dw0

    def forward(self, stream=None):
        c = self.cfg
        if self.guarded:
            B.inplace_ttt_fwd_guarded(c["B"], c["T"], c["d_model"], c["d_ff"], c["C"], c["eta"],
                                      c.get("clip_tau") or 0.0, self.doc_starts, self.z, self.vhat, self.w0,
                                      self.w, self.o, self.ws, self.ws_bytes, stream=stream)
        else:
            B.inplace_ttt_fwd(c["B"], c["T"], c["d_model"], c["d_ff"], c["C"], c["eta"], self.z, self.vhat,
                              self.w, self.o, self.ws, self.ws_bytes, stream=stream)
