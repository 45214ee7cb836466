"""GPU side of the seeded input generator (same bits as the CPU side).

Writes straight into torch CUDA tensors; used to fill multi-gigabyte expert
stacks quickly.  Tests compare its output with the CPU generator bit for bit.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import (T_DOWN, T_GATE, T_HIDDEN, T_ROUTER, T_SHARED_DOWN, T_SHARED_GATE, T_SHARED_UP,
               T_UP, RMS_EPS)
from .configs import LayerConfig

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.path.join(_HERE, "libsynth_gpu.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(path)
        u64, u32, i32, i64, dbl, vp = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int,
                                       ctypes.c_int64, ctypes.c_double, ctypes.c_void_p)
        L.synth_gpu_quant_experts.argtypes = [u64, u32, u32, u32, i32, i32, i32, dbl, vp, vp, vp,
                                              i64, i64, vp]
        L.synth_gpu_normals.argtypes = [u64, u32, u32, u32, u64, i64, dbl, vp, vp]
        L.synth_gpu_hidden.argtypes = [u64, u32, u32, u32, i32, i32, dbl, vp, vp]
        L.synth_gpu_router.argtypes = [u64, u32, u32, i32, i32, dbl, i32, vp, vp]
        for fn in (L.synth_gpu_quant_experts, L.synth_gpu_normals, L.synth_gpu_hidden,
                   L.synth_gpu_router):
            fn.restype = i32
        _lib = L
    return _lib


def _s():
    return torch.cuda.current_stream().cuda_stream


def _ok(rc):
    if rc != 0:
        raise RuntimeError(f"GPU generator failed ({rc})")


def quant_experts_into(w, s, b, seed, layer, tensor, e0, sigma):
    """Fill w [nE, rows, cols/8] (int32), s/b [nE, rows, cols/64] (int16) in place.
    Views with an expert stride (e.g. halves of a fused gate_up) are allowed."""
    nE, rows = w.shape[0], w.shape[1]
    cols = w.shape[2] * 8
    _ok(lib().synth_gpu_quant_experts(seed, layer, tensor, e0, nE, rows, cols, sigma, w.data_ptr(),
                                      s.data_ptr(), b.data_ptr(), w.stride(0), s.stride(0), _s()))


def hidden(seed, layer, stream_id, B, d, tensor=T_HIDDEN, device="cuda"):
    out = torch.empty(B, d, dtype=torch.float32, device=device)
    _ok(lib().synth_gpu_hidden(seed, layer, tensor, stream_id, B, d, RMS_EPS, out.data_ptr(), _s()))
    return out


def normals(seed, layer, tensor, stream_id, start, n, sigma=1.0, device="cuda"):
    out = torch.empty(n, dtype=torch.float32, device=device)
    _ok(lib().synth_gpu_normals(seed, layer, tensor, stream_id, start, n, sigma, out.data_ptr(),
                                _s()))
    return out


def bf16_matrix(seed, layer, tensor, rows, cols, sigma, device="cuda"):
    """The same bits as synth.bf16_matrix, as an int16 tensor on the device."""
    out = torch.empty(rows, cols, dtype=torch.int16, device=device)
    _ok(lib().synth_gpu_router(seed, layer, tensor, rows, cols, sigma, 1, out.data_ptr(), _s()))
    return out


def router(seed, layer, E, d, sigma, bf16, device="cuda"):
    out = torch.empty(E, d, dtype=torch.int16 if bf16 else torch.float32, device=device)
    _ok(lib().synth_gpu_router(seed, layer, T_ROUTER, E, d, sigma, int(bf16), out.data_ptr(), _s()))
    return out


def _alloc(E, rows, cols, device):
    return (torch.empty(E, rows, cols // 8, dtype=torch.int32, device=device),
            torch.empty(E, rows, cols // 64, dtype=torch.int16, device=device),
            torch.empty(E, rows, cols // 64, dtype=torch.int16, device=device))


def make_layer(cfg: LayerConfig, layer: int = 0, device="cuda") -> dict:
    """Device tensors of one layer (all experts), the same bits as
    ``synth.make_layer``.  Fused configs get 'gate_up' [E, 2f, d/8] (gate rows
    on top of up rows, per expert) instead of 'gate'/'up'."""
    E, d, f, seed, sig = cfg.num_experts, cfg.d_model, cfg.ffn_dim, cfg.seed, cfg.expert_sigma
    out = {"router": router(seed, layer, E, d, cfg.router_sigma, cfg.router_bf16, device)}
    if cfg.fused:
        gu = _alloc(E, 2 * f, d, device)
        quant_experts_into(gu[0][:, :f], gu[1][:, :f], gu[2][:, :f], seed, layer, T_GATE, 0, sig)
        quant_experts_into(gu[0][:, f:], gu[1][:, f:], gu[2][:, f:], seed, layer, T_UP, 0, sig)
        out["gate_up"] = gu
    else:
        for name, tensor in (("gate", T_GATE), ("up", T_UP)):
            t = _alloc(E, f, d, device)
            quant_experts_into(*t, seed, layer, tensor, 0, sig)
            out[name] = t
    dn = _alloc(E, d, f, device)
    quant_experts_into(*dn, seed, layer, T_DOWN, 0, sig)
    out["down"] = dn
    fs = cfg.shared_ffn_dim
    if fs:
        # the shared expert: 'shared_gate_up' (fused configs) or 'shared_gate' and
        # 'shared_up', and 'shared_down', each with a leading axis of 1
        if cfg.fused:
            gu = _alloc(1, 2 * fs, d, device)
            quant_experts_into(gu[0][:, :fs], gu[1][:, :fs], gu[2][:, :fs], seed, layer,
                               T_SHARED_GATE, 0, sig)
            quant_experts_into(gu[0][:, fs:], gu[1][:, fs:], gu[2][:, fs:], seed, layer,
                               T_SHARED_UP, 0, sig)
            out["shared_gate_up"] = gu
        else:
            for name, tensor in (("shared_gate", T_SHARED_GATE), ("shared_up", T_SHARED_UP)):
                t = _alloc(1, fs, d, device)
                quant_experts_into(*t, seed, layer, tensor, 0, sig)
                out[name] = t
        sd = _alloc(1, d, fs, device)
        quant_experts_into(*sd, seed, layer, T_SHARED_DOWN, 0, sig)
        out["shared_down"] = sd
    return out
