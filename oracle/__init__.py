"""Plain CPU reference of one routed mixture-of-experts layer (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product library
never does, and this package imports nothing from the product.

The arithmetic lives in ``oracle.cpp`` (fp32, sequential accumulation,
-ffp-contract=off); this file only marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


class QMat(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("s", ctypes.c_void_p), ("b", ctypes.c_void_p),
                ("stride_w", ctypes.c_int64), ("stride_sb", ctypes.c_int64)]


def lib():
    global _lib
    if _lib is None:
        # ORACLE_LIBRARY may name the sanitizer build (build_sanitized.py)
        path = os.environ.get("ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(path)
        vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        L.oracle_router_logits.argtypes = [vp, i32, vp, i32, i32, i32, vp]
        L.oracle_topk_softmax.argtypes = [vp, i32, i32, i32, i32, vp, vp]
        L.oracle_rank.argtypes = [vp, i32, i32, i32, vp]
        L.oracle_weights_of.argtypes = [vp, i32, i32, i32, i32, vp, vp]
        L.oracle_weights_of.restype = i32
        L.oracle_build_union.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
        L.oracle_build_union.restype = i32
        L.oracle_dequant.argtypes = [vp, vp, vp, i32, i32, vp]
        L.oracle_expert_ffn.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, vp, vp]
        qp = ctypes.POINTER(QMat)
        for fn in (L.oracle_moe_token_major, L.oracle_moe_layer_major):
            fn.argtypes = [qp, qp, qp, i32, i32, i32, vp, i32, i32, vp, vp, vp, vp, vp]
            fn.restype = i32
        L.oracle_rmsnorm.argtypes = [vp, i32, i32, f32, vp]
        L.oracle_shared_ffn.argtypes = [qp, qp, qp, i32, i32, vp, i32, vp]
        L.oracle_combine_shared.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp]
        L.oracle_num_threads.restype = i32
        L.oracle_set_num_threads.argtypes = [i32]
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))


def router_logits(Wr: np.ndarray, x: np.ndarray) -> np.ndarray:
    """logits [B, E]; Wr is fp32 [E, d] or bf16 bits (uint16) [E, d]."""
    bf16 = Wr.dtype == np.uint16
    Wr, pw = _c(Wr, Wr.dtype)
    x, px = _c(x, np.float32)
    B, d = x.shape
    E = Wr.shape[0]
    out = np.empty((B, E), np.float32)
    lib().oracle_router_logits(pw, int(bf16), px, B, d, E, out.ctypes.data)
    return out


def topk_softmax(logits: np.ndarray, K: int, norm: bool = True):
    logits, pl = _c(logits, np.float32)
    B, E = logits.shape
    idx = np.empty((B, K), np.int32)
    w = np.empty((B, K), np.float32)
    lib().oracle_topk_softmax(pl, B, E, K, int(norm), idx.ctypes.data, w.ctypes.data)
    return idx, w


def rank(logits: np.ndarray, R: int) -> np.ndarray:
    """The R highest-ranked experts of each token in rank order (logit
    descending, index ascending): [B, R] int32."""
    logits, pl = _c(logits, np.float32)
    B, E = logits.shape
    out = np.empty((B, R), np.int32)
    lib().oracle_rank(pl, B, E, R, out.ctypes.data)
    return out


def weights_of(logits: np.ndarray, idx: np.ndarray, norm: bool = True) -> np.ndarray:
    """Routing weights [B, K] of the given expert sets idx [B, K] from the
    logits' full softmax (renormalised over the set when norm)."""
    logits, pl = _c(logits, np.float32)
    idx, pi = _c(idx, np.int32)
    B, E = logits.shape
    K = idx.shape[1]
    w = np.empty((B, K), np.float32)
    if lib().oracle_weights_of(pl, B, E, K, int(norm), pi, w.ctypes.data) != 0:
        raise ValueError("expert id out of range")
    return w


def route(Wr, x, K, norm=True):
    lg = router_logits(Wr, x)
    idx, w = topk_softmax(lg, K, norm)
    return lg, idx, w


def build_union(idx: np.ndarray, E: int):
    """Returns (n_union, union_experts, offsets, pair_list, pair_pos)."""
    idx, pi = _c(idx, np.int32)
    B, K = idx.shape
    P = B * K
    m = max(1, min(E, P))
    ue = np.full(m, -1, np.int32)
    off = np.zeros(m + 1, np.int32)
    pl = np.full(max(1, P), -1, np.int32)
    pp = np.full(max(1, P), -1, np.int32)
    n = lib().oracle_build_union(pi, B, K, E, ue.ctypes.data, off.ctypes.data, pl.ctypes.data,
                                 pp.ctypes.data)
    if n < 0:
        raise ValueError("expert id out of range")
    return n, ue[:n], off[:n + 1], pl[:P], pp[:P]


def dequant(w, s, b) -> np.ndarray:
    """Dense fp32 [rows, cols] of one quantised matrix."""
    w, pw = _c(w, np.uint32)
    s, ps = _c(s, np.uint16)
    b, pb = _c(b, np.uint16)
    rows = w.shape[0]
    cols = w.shape[1] * 8
    out = np.empty((rows, cols), np.float32)
    lib().oracle_dequant(pw, ps, pb, rows, cols, out.ctypes.data)
    return out


def expert_ffn(Wg, Wu, Wd, x):
    """(g, u, h, y) of one token through one dense expert."""
    Wg, pg = _c(Wg, np.float32)
    Wu, pu = _c(Wu, np.float32)
    Wd, pd = _c(Wd, np.float32)
    x, px = _c(x, np.float32)
    f, d = Wg.shape
    g = np.empty(f, np.float32)
    u = np.empty(f, np.float32)
    h = np.empty(f, np.float32)
    y = np.empty(d, np.float32)
    lib().oracle_expert_ffn(pg, pu, pd, px, d, f, g.ctypes.data, u.ctypes.data, h.ctypes.data,
                            y.ctypes.data)
    return g, u, h, y


def _qmat(triple):
    w, s, b = (np.ascontiguousarray(a) for a in triple)
    assert w.dtype == np.uint32 and s.dtype == np.uint16 and b.dtype == np.uint16
    q = QMat(w.ctypes.data, s.ctypes.data, b.ctypes.data, w[0].size, s[0].size)
    return q, (w, s, b)


def shared_ffn(gate, up, down, x):
    """Shared-expert FFN on every token: gate/up/down are (w, s, b) triples
    of one expert (a leading axis of 1, [1, fs, d/8] etc.); x [B, d] ->
    shared_out [B, d]."""
    qg, keep_g = _qmat(gate)
    qu, keep_u = _qmat(up)
    qd, keep_d = _qmat(down)
    fs, d = keep_g[0].shape[1], keep_g[0].shape[2] * 8
    x, px = _c(x, np.float32)
    out = np.empty((x.shape[0], d), np.float32)
    lib().oracle_shared_ffn(ctypes.byref(qg), ctypes.byref(qu), ctypes.byref(qd), d, fs, px,
                            x.shape[0], out.ctypes.data)
    return out


def combine_shared(y_pairs, w, shared_out, residual=None):
    """out = residual + (shared_out + routed_out), routed_out the k-ascending
    weighted sum of the pairs' y ([B*K, d]) with w [B, K]."""
    w, pw = _c(w, np.float32)
    B, K = w.shape
    y_pairs, py = _c(y_pairs, np.float32)
    shared_out, ps = _c(shared_out, np.float32)
    d = shared_out.shape[1]
    pr = 0
    if residual is not None:
        residual, pr = _c(residual, np.float32)
    out = np.empty((B, d), np.float32)
    lib().oracle_combine_shared(py, pw, ps, pr or None, B, K, d, out.ctypes.data)
    return out


def moe(gate, up, down, x, idx, w, residual=None, layer_major=False, return_pairs=False,
        shared=None):
    """One layer: gate/up/down are (w, s, b) triples with a leading expert
    axis ([E, f, d/8] etc.); x [B, d]; idx, w [B, K].  Returns out [B, d]
    (and y per pair [B*K, d] when ``return_pairs``).  ``shared``: an optional
    (gate, up, down) of the shared expert (see shared_ffn), added as
    out = residual + (shared_out + routed_out)."""
    if shared is not None:
        _, yp = moe(gate, up, down, x, idx, w, layer_major=layer_major, return_pairs=True)
        out = combine_shared(yp, w, shared_ffn(*shared, x), residual)
        return (out, yp) if return_pairs else out
    qg, keep_g = _qmat(gate)
    qu, keep_u = _qmat(up)
    qd, keep_d = _qmat(down)
    E, f = keep_g[0].shape[0], keep_g[0].shape[1]
    d = keep_g[0].shape[2] * 8
    x, px = _c(x, np.float32)
    idx, pi = _c(idx, np.int32)
    w, pw = _c(w, np.float32)
    B, K = idx.shape
    pr = 0
    if residual is not None:
        residual, pr = _c(residual, np.float32)
    out = np.empty((B, d), np.float32)
    yp = np.empty((B * K, d), np.float32) if return_pairs else None
    fn = lib().oracle_moe_layer_major if layer_major else lib().oracle_moe_token_major
    rc = fn(ctypes.byref(qg), ctypes.byref(qu), ctypes.byref(qd), d, f, E, px, B, K, pi, pw,
            pr or None, out.ctypes.data, yp.ctypes.data if yp is not None else None)
    if rc != 0:
        raise ValueError("expert id out of range")
    return (out, yp) if return_pairs else out


def rmsnorm(v: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    v, pv = _c(v, np.float32)
    B, d = v.shape
    out = np.empty_like(v)
    lib().oracle_rmsnorm(pv, B, d, eps, out.ctypes.data)
    return out
