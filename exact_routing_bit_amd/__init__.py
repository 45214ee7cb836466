"""Python binding of libsmoe: one routed mixture-of-experts layer on MI355X.

Argument marshalling only.  Every step of the layer runs in the HIP kernels
of ``libsmoe.so`` (declared in ``include/smoe.h``); PyTorch provides device
memory and the current stream.  There is no CPU fallback: importing this
module fails when the library is missing.

Entry points (same names as the C-ABI, without the ``smoe_`` prefix):
``workspace_size``, ``workspace_init``, ``route``, ``build_union``,
``moe_forward``, ``moe_layer``, ``read_status``.  ``Layer`` bundles the
device tensors and descriptors of one layer.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SMOE_LIBRARY may name another build of the same library (the sanitizer
# build of build_sanitized.py); by default the in-tree libsmoe.so
LIB_PATH = os.environ.get("SMOE_LIBRARY") or os.path.join(_HERE, "libsmoe.so")

SMOE_OK, SMOE_EINVAL, SMOE_EUNSUPPORTED, SMOE_EWORKSPACE, SMOE_EHIP = 0, -1, -2, -3, -4
SMOE_F32, SMOE_BF16 = 0, 1
SMOE_ROUTE_LOGITS_IN = 0x1
SMOE_STATUS_BAD_EXPERT = 0x1
MAX_BATCH = 64

SMOE_STAGE_ROUTE, SMOE_STAGE_GATE_UP, SMOE_STAGE_DOWN, SMOE_STAGE_COMBINE = 0, 1, 2, 3

EXPORTED = ("smoe_workspace_size", "smoe_workspace_init", "smoe_route", "smoe_route_ranked",
            "smoe_build_union",
            "smoe_moe_forward", "smoe_moe_layer", "smoe_moe_layer_stage", "smoe_rmsnorm",
            "smoe_stack_forward", "smoe_read_status", "smoe_strerror",
            "smoe_attn_workspace_size", "smoe_attn_forward", "smoe_attn_forward_stage",
            "smoe_moe_layer_noalloc", "smoe_noalloc_scratch_bytes", "smoe_stream_read",
            "smoe_empty_launch", "smoe_grid_barrier", "smoe_dma_read", "smoe_moe_layer_single",
            "smoe_gpu_sleep", "smoe_stack_forward_chunks")


class SmoeError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what} failed: {code} ({strerror(code)})")
        self.code = code


class LayerDesc(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("ffn_dim", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("norm_topk_prob", ctypes.c_int32),
                ("router_dtype", ctypes.c_int32), ("shared_ffn_dim", ctypes.c_int32)]


class QMat(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("s", ctypes.c_void_p), ("b", ctypes.c_void_p),
                ("expert_stride_w", ctypes.c_int64), ("expert_stride_sb", ctypes.c_int64)]


class Experts(ctypes.Structure):
    _fields_ = [("gate", QMat), ("up", QMat), ("down", QMat),
                ("shared_gate", QMat), ("shared_up", QMat), ("shared_down", QMat)]


class AttnDesc(ctypes.Structure):
    _fields_ = [("rope_theta", ctypes.c_double), ("ctx", ctypes.c_int64),
                ("d_model", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("eps", ctypes.c_float), ("reserved", ctypes.c_int32)]


class Union(ctypes.Structure):
    _fields_ = [("n_union", ctypes.c_void_p), ("union_experts", ctypes.c_void_p),
                ("expert_offsets", ctypes.c_void_p), ("pair_list", ctypes.c_void_p),
                ("pair_pos", ctypes.c_void_p)]


class StackChunk(ctypes.Structure):
    _fields_ = [("h", ctypes.c_void_p), ("B", ctypes.c_int32), ("tmp", ctypes.c_void_p),
                ("topk_idx", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
                ("n_union", ctypes.c_void_p), ("un", Union), ("ws", ctypes.c_void_p),
                ("ws_bytes", ctypes.c_size_t), ("stream", ctypes.c_void_p)]


MAX_STACK_CHUNKS = 8


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
    dp = ctypes.POINTER(LayerDesc)
    L.smoe_workspace_size.argtypes = [dp, i32]
    L.smoe_workspace_size.restype = sz
    L.smoe_workspace_init.argtypes = [vp, sz, vp]
    L.smoe_route.argtypes = [dp, vp, vp, i32, vp, vp, vp, u32, vp, sz, vp]
    L.smoe_route_ranked.argtypes = [dp, vp, vp, i32, vp, i32, vp, vp, vp, u32, vp, sz, vp]
    L.smoe_build_union.argtypes = [dp, vp, i32, ctypes.POINTER(Union), vp, sz, vp]
    L.smoe_moe_forward.argtypes = [dp, ctypes.POINTER(Experts), vp, vp, vp, ctypes.POINTER(Union),
                                   i32, vp, vp, vp, sz, vp]
    L.smoe_moe_layer.argtypes = [dp, vp, ctypes.POINTER(Experts), vp, i32, vp, vp, vp, vp, vp,
                                 ctypes.POINTER(Union), vp, sz, vp]
    L.smoe_moe_layer_single.argtypes = [dp, vp, ctypes.POINTER(Experts), vp, i32, vp, vp, vp, vp,
                                        vp, ctypes.POINTER(Union), vp, sz, vp]
    L.smoe_moe_layer_noalloc.argtypes = [dp, vp, ctypes.POINTER(Experts), vp, i32, vp, vp, vp, vp,
                                         vp, ctypes.POINTER(Union), vp]
    L.smoe_stream_read.argtypes = [vp, sz, vp, i32, vp]
    L.smoe_empty_launch.argtypes = [i32, i32, vp]
    L.smoe_gpu_sleep.argtypes = [i32, vp]
    L.smoe_dma_read.argtypes = [vp, sz, i32, i32, vp, i32, vp]
    L.smoe_grid_barrier.argtypes = [i32, vp, vp, vp, vp]
    L.smoe_noalloc_scratch_bytes.argtypes = []
    L.smoe_noalloc_scratch_bytes.restype = sz
    L.smoe_moe_layer_stage.argtypes = [ctypes.c_int, dp, vp, ctypes.POINTER(Experts), vp, i32, vp,
                                       vp, vp, vp, vp, ctypes.POINTER(Union), vp, sz, vp, vp, vp]
    L.smoe_rmsnorm.argtypes = [vp, i32, i32, ctypes.c_float, vp, vp]
    L.smoe_stack_forward.argtypes = [dp, i32, ctypes.POINTER(ctypes.c_void_p),
                                     ctypes.POINTER(Experts), vp, i32, ctypes.c_float, vp, vp, vp,
                                     vp, ctypes.POINTER(Union), vp, sz, vp]
    L.smoe_stack_forward_chunks.argtypes = [dp, i32, ctypes.POINTER(ctypes.c_void_p),
                                            ctypes.POINTER(Experts), ctypes.c_float,
                                            ctypes.POINTER(StackChunk), i32]
    L.smoe_read_status.argtypes = [vp, sz, vp, ctypes.POINTER(ctypes.c_uint32)]
    L.smoe_strerror.argtypes = [ctypes.c_int]
    L.smoe_strerror.restype = ctypes.c_char_p
    ap, i64 = ctypes.POINTER(AttnDesc), ctypes.c_int64
    L.smoe_attn_workspace_size.argtypes = [ap, i32]
    L.smoe_attn_workspace_size.restype = sz
    L.smoe_attn_forward.argtypes = [ap, vp, vp, vp, i32, i64, vp, vp, vp, vp, sz, vp]
    L.smoe_attn_forward_stage.argtypes = [ctypes.c_int, ap, vp, vp, vp, i32, i64, vp, vp, vp, vp,
                                          sz, vp, vp, vp]
    for name in EXPORTED:
        if name not in ("smoe_workspace_size", "smoe_strerror", "smoe_attn_workspace_size",
                        "smoe_noalloc_scratch_bytes"):
            getattr(L, name).restype = ctypes.c_int
    return L


lib = _load()


def strerror(code: int) -> str:
    return lib.smoe_strerror(code).decode()


def _check(rc: int, what: str):
    if rc != SMOE_OK:
        raise SmoeError(rc, what)


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t, dtype=None, name="tensor"):
    """Device pointer of a contiguous CUDA tensor (or None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def make_desc(d_model, ffn_dim, num_experts, top_k, norm_topk_prob=True, router_bf16=True,
              shared_ffn_dim=0):
    return LayerDesc(d_model, ffn_dim, num_experts, top_k, 64, int(bool(norm_topk_prob)),
                     SMOE_BF16 if router_bf16 else SMOE_F32, int(shared_ffn_dim))


def workspace_size(desc: LayerDesc, max_batch: int) -> int:
    return int(lib.smoe_workspace_size(ctypes.byref(desc), max_batch))


def workspace_init(ws: torch.Tensor, stream=None):
    _check(lib.smoe_workspace_init(_ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)),
           "smoe_workspace_init")


def qmat(w: torch.Tensor, s: torch.Tensor, b: torch.Tensor, expert_stride_w=None,
         expert_stride_sb=None) -> QMat:
    """Descriptor of a quantised projection with a leading expert axis.
    w: int32/uint32 [E, rows, cols/8]; s, b: int16/uint16 bf16 bits [E, rows, cols/64].
    Strides default to the tensors' expert strides (so views into a fused
    gate_up tensor work)."""
    sw = w.stride(0) if expert_stride_w is None else expert_stride_w
    ssb = s.stride(0) if expert_stride_sb is None else expert_stride_sb
    for t, nm in ((w, "w"), (s, "s"), (b, "b")):
        if not t.is_cuda:
            raise TypeError(f"{nm} must be a CUDA tensor")
        if t.dim() == 3 and (t.stride(2) != 1 or t.stride(1) != t.shape[2]):
            raise ValueError(f"{nm}: rows must be contiguous")
    return QMat(w.data_ptr(), s.data_ptr(), b.data_ptr(), sw, ssb)


def _gate_up(weights: dict, prefix: str, f: int):
    if prefix + "gate_up" in weights:
        gw, gs, gb = weights[prefix + "gate_up"]
        return (qmat(gw[:, :f], gs[:, :f], gb[:, :f], gw.stride(0), gs.stride(0)),
                qmat(gw[:, f:], gs[:, f:], gb[:, f:], gw.stride(0), gs.stride(0)))
    return qmat(*weights[prefix + "gate"]), qmat(*weights[prefix + "up"])


def experts_of(desc: LayerDesc, weights: dict) -> Experts:
    """The Experts descriptor of a layer's weight dict (see Layer)."""
    gate, up = _gate_up(weights, "", desc.ffn_dim)
    ex = Experts(gate, up, qmat(*weights["down"]))
    if desc.shared_ffn_dim > 0:
        ex.shared_gate, ex.shared_up = _gate_up(weights, "shared_", desc.shared_ffn_dim)
        ex.shared_down = qmat(*weights["shared_down"])
    return ex


@dataclass
class UnionBuffers:
    n_union: torch.Tensor
    union_experts: torch.Tensor
    expert_offsets: torch.Tensor
    pair_list: torch.Tensor
    pair_pos: torch.Tensor

    @staticmethod
    def alloc(num_experts: int, max_pairs: int, device="cuda") -> "UnionBuffers":
        m = max(1, min(num_experts, max_pairs))
        i32 = dict(dtype=torch.int32, device=device)
        return UnionBuffers(torch.zeros(1, **i32), torch.zeros(m, **i32), torch.zeros(m + 1, **i32),
                            torch.zeros(max(1, max_pairs), **i32),
                            torch.zeros(max(1, max_pairs), **i32))

    def c(self) -> Union:
        return Union(self.n_union.data_ptr(), self.union_experts.data_ptr(),
                     self.expert_offsets.data_ptr(), self.pair_list.data_ptr(),
                     self.pair_pos.data_ptr())


def route(desc, router_w, x, topk_idx, topk_w, ws, logits=None, logits_in=False, stream=None):
    B = logits.shape[0] if logits_in else x.shape[0]
    flags = SMOE_ROUTE_LOGITS_IN if logits_in else 0
    _check(lib.smoe_route(ctypes.byref(desc), _ptr(router_w, None, "router_w"),
                          _ptr(x, torch.float32, "x"), B, _ptr(logits, torch.float32, "logits"),
                          _ptr(topk_idx, torch.int32, "topk_idx"),
                          _ptr(topk_w, torch.float32, "topk_w"), flags,
                          _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)), "smoe_route")


def route_ranked(desc, router_w, x, spec, ranked_idx, topk_idx, topk_w, ws, logits=None,
                 logits_in=False, stream=None):
    B = logits.shape[0] if logits_in else x.shape[0]
    flags = SMOE_ROUTE_LOGITS_IN if logits_in else 0
    _check(lib.smoe_route_ranked(ctypes.byref(desc), _ptr(router_w, None, "router_w"),
                                 _ptr(x, torch.float32, "x"), B,
                                 _ptr(logits, torch.float32, "logits"), int(spec),
                                 _ptr(ranked_idx, torch.int32, "ranked_idx"),
                                 _ptr(topk_idx, torch.int32, "topk_idx"),
                                 _ptr(topk_w, torch.float32, "topk_w"), flags,
                                 _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)),
           "smoe_route_ranked")


def build_union(desc, topk_idx, un: UnionBuffers, ws, stream=None):
    cu = un.c()
    _check(lib.smoe_build_union(ctypes.byref(desc), _ptr(topk_idx, torch.int32, "topk_idx"),
                                topk_idx.shape[0], ctypes.byref(cu), _ptr(ws, torch.uint8, "ws"),
                                ws.numel(), _stream(stream)), "smoe_build_union")


def moe_forward(desc, experts: Experts, x, topk_idx, topk_w, un: UnionBuffers, out, ws,
                residual=None, stream=None):
    cu = un.c()
    _check(lib.smoe_moe_forward(ctypes.byref(desc), ctypes.byref(experts),
                                _ptr(x, torch.float32, "x"), _ptr(topk_idx, torch.int32, "topk_idx"),
                                _ptr(topk_w, torch.float32, "topk_w"), ctypes.byref(cu), x.shape[0],
                                _ptr(residual, torch.float32, "residual"),
                                _ptr(out, torch.float32, "out"), _ptr(ws, torch.uint8, "ws"),
                                ws.numel(), _stream(stream)), "smoe_moe_forward")


def moe_layer(desc, router_w, experts: Experts, x, out, topk_idx, topk_w, un: UnionBuffers, ws,
              residual=None, logits=None, stream=None):
    cu = un.c()
    _check(lib.smoe_moe_layer(ctypes.byref(desc), _ptr(router_w, None, "router_w"),
                              ctypes.byref(experts), _ptr(x, torch.float32, "x"), x.shape[0],
                              _ptr(residual, torch.float32, "residual"),
                              _ptr(out, torch.float32, "out"),
                              _ptr(logits, torch.float32, "logits"),
                              _ptr(topk_idx, torch.int32, "topk_idx"),
                              _ptr(topk_w, torch.float32, "topk_w"), ctypes.byref(cu),
                              _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)),
           "smoe_moe_layer")


class PreparedCall:
    """A library call whose arguments are marshalled once (pointers, the
    descriptor structs, the stream), for loops that repeat the same call on
    the same buffers: calling it is one ctypes call.  The tensors and structs
    it points to are kept alive by the object."""

    def __init__(self, fn, what, args, keep):
        self._fn, self._what, self._args, self._keep = fn, what, args, keep

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != SMOE_OK:
            raise SmoeError(rc, self._what)


def moe_layer_single(desc, router_w, experts: Experts, x, out, topk_idx, topk_w,
                     un: UnionBuffers, ws, residual=None, logits=None, stream=None):
    """moe_layer as one cooperative launch (see smoe_moe_layer_single: B = 1
    decode layers only, SMOE_EUNSUPPORTED otherwise)."""
    cu = un.c()
    _check(lib.smoe_moe_layer_single(ctypes.byref(desc), _ptr(router_w, None, "router_w"),
                                     ctypes.byref(experts), _ptr(x, torch.float32, "x"),
                                     x.shape[0], _ptr(residual, torch.float32, "residual"),
                                     _ptr(out, torch.float32, "out"),
                                     _ptr(logits, torch.float32, "logits"),
                                     _ptr(topk_idx, torch.int32, "topk_idx"),
                                     _ptr(topk_w, torch.float32, "topk_w"), ctypes.byref(cu),
                                     _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)),
           "smoe_moe_layer_single")


def prepare_moe_layer(desc, router_w, experts: Experts, x, out, topk_idx, topk_w,
                      un: UnionBuffers, ws, residual=None, logits=None, stream=None,
                      stage=None, events=None, single=False) -> PreparedCall:
    """moe_layer (or, with ``stage``, moe_layer_stage; with ``single``,
    moe_layer_single) with its arguments marshalled once."""
    cu = un.c()
    vp = ctypes.c_void_p
    common = (vp(_ptr(x, torch.float32, "x")), x.shape[0],
              vp(_ptr(residual, torch.float32, "residual")), vp(_ptr(out, torch.float32, "out")),
              vp(_ptr(logits, torch.float32, "logits")),
              vp(_ptr(topk_idx, torch.int32, "topk_idx")),
              vp(_ptr(topk_w, torch.float32, "topk_w")), ctypes.byref(cu),
              vp(_ptr(ws, torch.uint8, "ws")), ws.numel(), vp(_stream(stream)))
    keep = (desc, experts, router_w, x, out, topk_idx, topk_w, un, ws, residual, logits, cu)
    head = (ctypes.byref(desc), vp(_ptr(router_w, None, "router_w")), ctypes.byref(experts))
    if single:
        return PreparedCall(lib.smoe_moe_layer_single, "smoe_moe_layer_single", head + common,
                            keep)
    if stage is None:
        return PreparedCall(lib.smoe_moe_layer, "smoe_moe_layer", head + common, keep)
    ev = (None, None)
    if events is not None:
        ev = tuple(vp(e.cuda_event) for e in events)
    return PreparedCall(lib.smoe_moe_layer_stage, "smoe_moe_layer_stage",
                        (int(stage),) + head + common + ev, keep + (events,))


def moe_layer_noalloc(desc, router_w, experts: Experts, x, out, topk_idx, topk_w,
                      un: UnionBuffers, residual=None, logits=None, stream=None):
    """moe_layer with the library's own device scratch: no workspace argument
    and no allocation (see smoe_moe_layer_noalloc in include/smoe.h)."""
    cu = un.c()
    _check(lib.smoe_moe_layer_noalloc(ctypes.byref(desc), _ptr(router_w, None, "router_w"),
                                      ctypes.byref(experts), _ptr(x, torch.float32, "x"),
                                      x.shape[0], _ptr(residual, torch.float32, "residual"),
                                      _ptr(out, torch.float32, "out"),
                                      _ptr(logits, torch.float32, "logits"),
                                      _ptr(topk_idx, torch.int32, "topk_idx"),
                                      _ptr(topk_w, torch.float32, "topk_w"), ctypes.byref(cu),
                                      _stream(stream)),
           "smoe_moe_layer_noalloc")


def stream_read(buf: torch.Tensor, sink: torch.Tensor, nbytes=None, stream=None):
    """Diagnostic streaming read of a device buffer (see smoe_stream_read):
    sink is an int32 tensor with one entry per workgroup."""
    n = buf.numel() * buf.element_size() if nbytes is None else int(nbytes)
    _check(lib.smoe_stream_read(_ptr(buf, None, "buf"), n, _ptr(sink, torch.int32, "sink"),
                                sink.numel(), _stream(stream)), "smoe_stream_read")


def dma_read(buf: torch.Tensor, sink: torch.Tensor, row_bytes: int, mode: int, nbytes=None,
             stream=None):
    """Diagnostic stream of a device buffer through the direct global -> LDS
    copy path (see smoe_dma_read): mode 0 the prefill FFN's pattern, 1 memory
    order; sink is an int32 tensor of at least ceil(units / 4) entries."""
    n = buf.numel() * buf.element_size() if nbytes is None else int(nbytes)
    _check(lib.smoe_dma_read(_ptr(buf, None, "buf"), n, int(row_bytes), int(mode),
                             _ptr(sink, torch.int32, "sink"), sink.numel(), _stream(stream)),
           "smoe_dma_read")


def empty_launch(blocks: int, count: int = 1, stream=None):
    """Diagnostic: `count` back-to-back launches of a kernel that does nothing
    (smoe_empty_launch)."""
    _check(lib.smoe_empty_launch(int(blocks), int(count), _stream(stream)), "smoe_empty_launch")


def gpu_sleep(us: int, stream=None):
    """Diagnostic: one wave that waits `us` microseconds on the device's clock
    (smoe_gpu_sleep), queued ahead of a timed region."""
    _check(lib.smoe_gpu_sleep(int(us), _stream(stream)), "smoe_gpu_sleep")


def grid_barrier(blocks: int, counter, stamps, timed_out, stream=None):
    """Diagnostic device-wide barrier of a cooperative grid (smoe_grid_barrier):
    counter int32 [1] cleared by the caller, stamps int64 [3 * blocks],
    timed_out int32 [1]."""
    if stamps.dtype != torch.int64 or stamps.numel() < 3 * int(blocks):
        raise ValueError("grid_barrier: stamps must be int64 with 3 * blocks entries")
    _check(lib.smoe_grid_barrier(int(blocks), _ptr(counter, torch.int32, "counter"),
                                 _ptr(stamps, torch.int64, "stamps"),
                                 _ptr(timed_out, torch.int32, "timed_out"), _stream(stream)),
           "smoe_grid_barrier")


def noalloc_scratch_bytes() -> int:
    return int(lib.smoe_noalloc_scratch_bytes())


def moe_layer_stage(stage, desc, router_w, experts: Experts, x, out, topk_idx, topk_w,
                    un: UnionBuffers, ws, residual=None, logits=None, stream=None, events=None):
    """One stage of moe_layer.  `events` = (start, stop) torch.cuda.Events
    (timing enabled, already recorded once so that they exist): they are
    submitted together with the stage's main kernel and bracket it."""
    cu = un.c()
    ev0 = ev1 = None
    if events is not None:
        ev0, ev1 = (ctypes.c_void_p(e.cuda_event) for e in events)
        if not ev0.value or not ev1.value:
            raise ValueError("moe_layer_stage: record the events once before passing them")
    _check(lib.smoe_moe_layer_stage(stage, ctypes.byref(desc), _ptr(router_w, None, "router_w"),
                                    ctypes.byref(experts), _ptr(x, torch.float32, "x"), x.shape[0],
                                    _ptr(residual, torch.float32, "residual"),
                                    _ptr(out, torch.float32, "out"),
                                    _ptr(logits, torch.float32, "logits"),
                                    _ptr(topk_idx, torch.int32, "topk_idx"),
                                    _ptr(topk_w, torch.float32, "topk_w"), ctypes.byref(cu),
                                    _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream),
                                    ev0, ev1),
           "smoe_moe_layer_stage")


def rmsnorm(v, out=None, eps=1e-6, stream=None):
    """out = v / sqrt(mean(v^2) + eps) per row (fp32 [B, d]); out may be v."""
    if out is None:
        out = torch.empty_like(v)
    if v.dim() != 2 or out.shape != v.shape:
        raise ValueError("rmsnorm takes matching [B, d] tensors")
    _check(lib.smoe_rmsnorm(_ptr(v, torch.float32, "v"), v.shape[0], v.shape[1], eps,
                            _ptr(out, torch.float32, "out"), _stream(stream)), "smoe_rmsnorm")
    return out


class StackArgs:
    """Host arrays of a stack's per-layer router pointers and expert
    descriptors, built once and passed to every stack_forward call."""

    def __init__(self, router_ws, experts):
        n = len(router_ws)
        if len(experts) != n:
            raise ValueError("one router matrix per layer of experts")
        self.n = n
        self.router = (ctypes.c_void_p * max(n, 1))(
            *[_ptr(r, name="router_w") for r in router_ws])
        self.experts = (Experts * max(n, 1))(*experts)
        self._keep = list(router_ws)


def stack_forward(desc, stack: StackArgs, h, tmp, topk_idx, topk_w, un: UnionBuffers, ws,
                  n_union=None, eps=1e-6, stream=None):
    """h <- RMSNorm(h + MoE_l(h)) for every layer l of the stack, in place.
    topk_idx/topk_w: [n_layers, B, top_k]; n_union: [n_layers] int32 or None."""
    B = h.shape[0]
    _check(lib.smoe_stack_forward(ctypes.byref(desc), stack.n, stack.router,
                                  stack.experts, _ptr(h, torch.float32, "h"), B, eps,
                                  _ptr(tmp, torch.float32, "tmp"),
                                  _ptr(topk_idx, torch.int32, "topk_idx"),
                                  _ptr(topk_w, torch.float32, "topk_w"),
                                  _ptr(n_union, torch.int32, "n_union"), ctypes.byref(un.c()),
                                  _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)),
           "smoe_stack_forward")
    return h


def stack_forward_chunks(desc, stack: StackArgs, chunks, eps=1e-6):
    """Several prompt chunks through the stack at once (smoe_stack_forward_chunks):
    chunks is a list of dicts with h, tmp, topk_idx, topk_w, un (UnionBuffers),
    ws, and optionally n_union and stream; each as for stack_forward, each with
    buffers of its own.  Ordered on the first chunk's stream."""
    arr = (StackChunk * max(len(chunks), 1))()
    for i, c in enumerate(chunks):
        h, ws = c["h"], c["ws"]
        arr[i] = StackChunk(_ptr(h, torch.float32, "h"), h.shape[0],
                            _ptr(c["tmp"], torch.float32, "tmp"),
                            _ptr(c["topk_idx"], torch.int32, "topk_idx"),
                            _ptr(c["topk_w"], torch.float32, "topk_w"),
                            _ptr(c.get("n_union"), torch.int32, "n_union"), c["un"].c(),
                            _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(c.get("stream")))
    _check(lib.smoe_stack_forward_chunks(ctypes.byref(desc), stack.n, stack.router,
                                         stack.experts, eps, arr, len(chunks)),
           "smoe_stack_forward_chunks")


def make_attn_desc(d_model, num_heads, num_kv_heads, ctx, rope_theta=1.0e6, eps=1e-6,
                   head_dim=128) -> AttnDesc:
    return AttnDesc(float(rope_theta), int(ctx), d_model, num_heads, num_kv_heads, head_dim,
                    float(eps), 0)


def attn_workspace_size(desc: AttnDesc, max_batch: int) -> int:
    return int(lib.smoe_attn_workspace_size(ctypes.byref(desc), max_batch))


def _attn_args(desc, wqkv, wo, x, pos0, k_cache, v_cache, out, ws):
    return (ctypes.byref(desc), _ptr(wqkv, None, "wqkv"), _ptr(wo, None, "wo"),
            _ptr(x, torch.float32, "x"), x.shape[0], int(pos0), _ptr(k_cache, None, "k_cache"),
            _ptr(v_cache, None, "v_cache"), _ptr(out, torch.float32, "out"),
            _ptr(ws, torch.uint8, "ws"), ws.numel())


def attn_forward(desc, wqkv, wo, x, pos0, k_cache, v_cache, out, ws, stream=None):
    """out = x + attention block of x (B tokens at positions pos0 ..); the
    K/V rings (bf16 bits, [Hkv, ctx, 128]) are updated in place."""
    _check(lib.smoe_attn_forward(*_attn_args(desc, wqkv, wo, x, pos0, k_cache, v_cache, out, ws),
                                 _stream(stream)), "smoe_attn_forward")
    return out


def attn_forward_stage(stage, desc, wqkv, wo, x, pos0, k_cache, v_cache, out, ws, stream=None,
                       events=None):
    ev0 = ev1 = None
    if events is not None:
        ev0, ev1 = (ctypes.c_void_p(e.cuda_event) for e in events)
    _check(lib.smoe_attn_forward_stage(stage, *_attn_args(desc, wqkv, wo, x, pos0, k_cache,
                                                          v_cache, out, ws),
                                       _stream(stream), ev0, ev1), "smoe_attn_forward_stage")


def read_status(ws, stream=None) -> int:
    v = ctypes.c_uint32(0)
    _check(lib.smoe_read_status(_ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream),
                                ctypes.byref(v)), "smoe_read_status")
    return int(v.value)


class Layer:
    """Device tensors and descriptors of one layer, plus its scratch buffers.

    ``weights`` maps 'router' and 'gate'/'up'/'down' (each a (w, s, b) triple
    of CUDA tensors with a leading expert axis) or 'gate_up' (fused, gate rows
    on top) + 'down'; with a shared expert (desc.shared_ffn_dim > 0) also
    'shared_gate'/'shared_up' or 'shared_gate_up', and 'shared_down' (a
    leading axis of 1).
    """

    def __init__(self, desc: LayerDesc, weights: dict, max_batch: int = MAX_BATCH,
                 device="cuda"):
        self.desc = desc
        self.w = weights
        self.router_w = weights["router"]
        self.experts = experts_of(desc, weights)
        self.max_batch = max_batch
        nbytes = workspace_size(desc, max_batch)
        if nbytes == 0:
            raise SmoeError(SMOE_EUNSUPPORTED, "smoe_workspace_size")
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        workspace_init(self.ws)
        P = max_batch * desc.top_k
        self.union = UnionBuffers.alloc(desc.num_experts, P, device)
        i = dict(device=device)
        self.topk_idx = torch.zeros(max_batch, desc.top_k, dtype=torch.int32, **i)
        self.topk_w = torch.zeros(max_batch, desc.top_k, dtype=torch.float32, **i)
        self.logits = torch.zeros(max_batch, desc.num_experts, dtype=torch.float32, **i)

    def forward(self, x, out=None, residual=None, want_logits=False, stream=None):
        B = x.shape[0]
        if out is None:
            out = torch.empty(B, self.desc.d_model, dtype=torch.float32, device=x.device)
        moe_layer(self.desc, self.router_w, self.experts, x, out, self.topk_idx[:B],
                  self.topk_w[:B], self.union, self.ws, residual=residual,
                  logits=self.logits[:B] if want_logits else None, stream=stream)
        return out
