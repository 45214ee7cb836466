"""Seeded synthetic inputs for one routed mixture-of-experts layer.

This module makes inputs only; it holds none of the layer's arithmetic.  The
CPU generator (``libsynth.so``, from ``synth.c``) and the GPU generator
(``libsynth_gpu.so``, from ``synth_gpu.hip``) share ``synth_math.h`` and make
identical bits: Philox4x32-10 counters (Salmon et al., SC'11) keyed by
(seed, layer, tensor id, stream id, element), Box-Muller normals, and a
min/max affine 4-bit quantiser with group size 64.

Element ``n`` of stream (seed, layer, tensor, stream) is a standard normal;
a matrix [rows, cols] of expert ``e`` uses stream ``e`` and ``n = r*cols + c``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .configs import LayerConfig  # noqa: F401  (re-export)

_HERE = os.path.dirname(os.path.abspath(__file__))

# Tensor ids of the counter (fixed constants of the input recipe).
T_HIDDEN = 1
T_ROUTER = 2
T_GATE = 3
T_UP = 4
T_DOWN = 5
T_DECODE = 6
T_RESIDUAL = 7
T_SHARED_GATE = 8
T_SHARED_UP = 9
T_SHARED_DOWN = 10
T_ATTN_QKV = 11
T_ATTN_O = 12
T_K_CACHE = 13
T_V_CACHE = 14

RMS_EPS = 1e-6

_lib = None


def lib():
    """The CPU generator library (built by ``synth/build.py``)."""
    global _lib
    if _lib is None:
        path = os.path.join(_HERE, "libsynth.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(path)
        u64, u32, i32, i64, dbl, vp = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int,
                                       ctypes.c_int64, ctypes.c_double, ctypes.c_void_p)
        L.synth_philox.argtypes = [vp, vp, vp]
        L.synth_normal_one.argtypes = [u64, u32, u32, u32, u64]
        L.synth_normal_one.restype = dbl
        L.synth_ln_u32.argtypes = [u64]
        L.synth_ln_u32.restype = dbl
        L.synth_sincos_turn.argtypes = [u32, vp, vp]
        L.synth_normals.argtypes = [u64, u32, u32, u32, u64, i64, dbl, vp]
        L.synth_hidden.argtypes = [u64, u32, u32, u32, i32, i32, dbl, vp]
        L.synth_router.argtypes = [u64, u32, u32, i32, i32, dbl, i32, vp]
        L.synth_quant_experts.argtypes = [u64, u32, u32, u32, i32, i32, i32, dbl, vp, vp, vp,
                                          i64, i64]
        L.synth_quant_experts.restype = i32
        L.synth_quantize_matrix.argtypes = [vp, i32, i32, vp, vp, vp]
        L.synth_quantize_matrix.restype = i32
        L.synth_num_threads.restype = i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def philox(ctr, key) -> np.ndarray:
    c = np.asarray(ctr, np.uint32)
    k = np.asarray(key, np.uint32)
    o = np.empty(4, np.uint32)
    lib().synth_philox(_ptr(c), _ptr(k), _ptr(o))
    return o


def normals(seed, layer, tensor, stream, start, n, sigma=1.0) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_normals(seed, layer, tensor, stream, start, n, sigma, _ptr(out))
    return out


def hidden(seed, layer, stream, B, d, tensor=T_HIDDEN, eps=RMS_EPS) -> np.ndarray:
    """[B, d] fp32: N(0,1) rows, each RMS-normalised (mean and root in fp64)."""
    out = np.empty((B, d), np.float32)
    lib().synth_hidden(seed, layer, tensor, stream, B, d, eps, _ptr(out))
    return out


def router(seed, layer, E, d, sigma, bf16: bool) -> np.ndarray:
    """[E, d] router gate: fp32, or bf16 bit patterns (uint16) when ``bf16``."""
    out = np.empty((E, d), np.uint16 if bf16 else np.float32)
    lib().synth_router(seed, layer, T_ROUTER, E, d, sigma, int(bf16), _ptr(out))
    return out


def bf16_matrix(seed, layer, tensor, rows, cols, sigma) -> np.ndarray:
    """[rows, cols] bf16 bit patterns (uint16) of sigma * N(0, 1), round to
    nearest even: the attention projections and the prior KV-ring contents."""
    out = np.empty((rows, cols), np.uint16)
    lib().synth_router(seed, layer, tensor, rows, cols, sigma, 1, _ptr(out))
    return out


def quant_experts(seed, layer, tensor, e0, nE, rows, cols, sigma):
    """Quantised matrices of experts e0..e0+nE-1: (w [nE,rows,cols/8] u32,
    s [nE,rows,cols/64] bf16 bits, b likewise)."""
    w = np.empty((nE, rows, cols // 8), np.uint32)
    s = np.empty((nE, rows, cols // 64), np.uint16)
    b = np.empty_like(s)
    rc = lib().synth_quant_experts(seed, layer, tensor, e0, nE, rows, cols, sigma, _ptr(w),
                                   _ptr(s), _ptr(b), rows * cols // 8, rows * cols // 64)
    if rc != 0:
        raise ValueError("bad shape for quant_experts")
    return w, s, b


def quantize_matrix(W: np.ndarray):
    """Quantise a given fp32 [rows, cols] matrix with the generator's group rule."""
    W = np.ascontiguousarray(W, np.float32)
    rows, cols = W.shape
    w = np.empty((rows, cols // 8), np.uint32)
    s = np.empty((rows, cols // 64), np.uint16)
    b = np.empty_like(s)
    if lib().synth_quantize_matrix(_ptr(W), rows, cols, _ptr(w), _ptr(s), _ptr(b)) != 0:
        raise ValueError("cols must be a multiple of 64")
    return w, s, b


def fuse_gate_up(gate, up):
    """Fused gate_up projection: per expert, gate rows on top, up rows below.

    ``gate`` and ``up`` are (w, s, b) triples with a leading expert axis.  The
    rows are concatenated per expert (axis 1), never as two whole tensors.
    """
    return tuple(np.ascontiguousarray(np.concatenate([g, u], axis=1)) for g, u in zip(gate, up))


def make_layer(cfg: "LayerConfig", layer: int = 0, experts=None):
    """Host arrays of one layer: router gate and the quantised experts.

    ``experts``: iterable of expert ids to generate (others are left zero), or
    None for all.  Returns a dict with 'router', 'gate', 'up', 'down' (each a
    (w, s, b) triple with a leading E axis) and, for fused configs, 'gate_up'.
    """
    E, d, f, seed = cfg.num_experts, cfg.d_model, cfg.ffn_dim, cfg.seed
    out = {"router": router(seed, layer, E, d, cfg.router_sigma, cfg.router_bf16)}
    ids = list(range(E)) if experts is None else sorted(set(int(e) for e in experts))

    def alloc(rows, cols):
        return (np.zeros((E, rows, cols // 8), np.uint32), np.zeros((E, rows, cols // 64), np.uint16),
                np.zeros((E, rows, cols // 64), np.uint16))

    for name, tensor, rows, cols in (("gate", T_GATE, f, d), ("up", T_UP, f, d),
                                     ("down", T_DOWN, d, f)):
        w, s, b = alloc(rows, cols)
        # contiguous runs of expert ids are generated in one call
        i = 0
        while i < len(ids):
            j = i
            while j + 1 < len(ids) and ids[j + 1] == ids[j] + 1:
                j += 1
            e0, n = ids[i], j - i + 1
            ww, ss, bb = quant_experts(seed, layer, tensor, e0, n, rows, cols, cfg.expert_sigma)
            w[e0:e0 + n], s[e0:e0 + n], b[e0:e0 + n] = ww, ss, bb
            i = j + 1
        out[name] = (w, s, b)
    if cfg.fused:
        out["gate_up"] = fuse_gate_up(out["gate"], out["up"])
    if cfg.shared_ffn_dim:
        out["shared"] = make_shared(cfg, layer)
    return out


def make_shared(cfg: "LayerConfig", layer: int = 0) -> dict:
    """The shared expert of a layer: 'gate', 'up' ([1, fs, d/8] words etc.)
    and 'down' ([1, d, fs/8]) triples, plus 'gate_up' for fused configs."""
    d, fs, seed = cfg.d_model, cfg.shared_ffn_dim, cfg.seed
    out = {}
    for name, tensor, rows, cols in (("gate", T_SHARED_GATE, fs, d), ("up", T_SHARED_UP, fs, d),
                                     ("down", T_SHARED_DOWN, d, fs)):
        out[name] = quant_experts(seed, layer, tensor, 0, 1, rows, cols, cfg.expert_sigma)
    if cfg.fused:
        out["gate_up"] = fuse_gate_up(out["gate"], out["up"])
    return out
