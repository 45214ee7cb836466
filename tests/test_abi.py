"""The C-ABI library on the host: it loads, exports every declared entry point,
and rejects bad arguments before launching anything (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smoe.h")


def _lib_path():
    return os.environ.get("SMOE_LIBRARY") or os.path.join(ROOT, "exact_routing_bit_amd", "libsmoe.so")


@pytest.fixture(scope="module")
def smoe():
    if not os.path.exists(_lib_path()):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_smoe_build", os.path.join(ROOT, "exact_routing_bit_amd", "build.py"))
        b = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(b)
        b.build()
    import exact_routing_bit_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(smoe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("smoe_route", "smoe_build_union", "smoe_moe_forward", "smoe_moe_layer",
              "smoe_workspace_size", "smoe_workspace_init", "smoe_read_status", "smoe_strerror"):
        assert n in names


def test_library_exports_every_declared_symbol(smoe):
    lib = ctypes.CDLL(_lib_path())
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(smoe.EXPORTED) <= set(declared_functions())


def desc_of(smoe, **kw):
    base = dict(d_model=4096, ffn_dim=1536, num_experts=128, top_k=8, norm_topk_prob=True,
                router_bf16=True)
    base.update(kw)
    return smoe.make_desc(**base)


def test_workspace_size(smoe):
    d = desc_of(smoe)
    n1, n64 = smoe.workspace_size(d, 1), smoe.workspace_size(d, 64)
    assert 0 < n1 < n64
    # per-pair y [P, d] fp32 dominates at B=64: 512 * 4096 * 4 bytes
    assert n64 >= 512 * 4096 * 4
    assert smoe.workspace_size(d, 0) == 0 and smoe.workspace_size(d, 65) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(d_model=100), -2), (dict(ffn_dim=96), -2), (dict(d_model=16384), -2),
    (dict(num_experts=257), -2), (dict(top_k=17, num_experts=32), -2),
    (dict(top_k=9, num_experts=8), -2), (dict(num_experts=0), -2),
])
def test_descriptor_rejected(smoe, kw, code):
    d = desc_of(smoe, **kw)
    assert smoe.workspace_size(d, 8) == 0
    fake = ctypes.c_void_p(4096)
    rc = smoe.lib.smoe_route(ctypes.byref(d), fake, fake, 1, None, fake, fake, 0, fake, 1 << 30,
                             None)
    assert rc == code


def test_group_size_and_flags_rejected(smoe):
    d = desc_of(smoe)
    d.group_size = 32
    fake = ctypes.c_void_p(4096)
    assert smoe.lib.smoe_route(ctypes.byref(d), fake, fake, 1, None, fake, fake, 0, fake, 1 << 30,
                               None) == smoe.SMOE_EUNSUPPORTED
    d = desc_of(smoe)
    assert smoe.lib.smoe_route(ctypes.byref(d), fake, fake, 1, None, fake, fake, 0x10, fake,
                               1 << 30, None) == smoe.SMOE_EINVAL


def test_route_argument_errors(smoe):
    d = desc_of(smoe)
    f = ctypes.c_void_p(4096)
    r = smoe.lib.smoe_route
    big = 1 << 30
    assert r(ctypes.byref(d), f, f, -1, None, f, f, 0, f, big, None) == smoe.SMOE_EINVAL
    assert r(ctypes.byref(d), f, f, 65, None, f, f, 0, f, big, None) == smoe.SMOE_EUNSUPPORTED
    assert r(ctypes.byref(d), None, f, 1, None, f, f, 0, f, big, None) == smoe.SMOE_EINVAL
    assert r(ctypes.byref(d), ctypes.c_void_p(4097), f, 1, None, f, f, 0, f, big,
             None) == smoe.SMOE_EINVAL                                  # misaligned gate
    assert r(ctypes.byref(d), f, f, 1, None, None, f, 0, f, big, None) == smoe.SMOE_EINVAL
    assert r(ctypes.byref(d), f, f, 1, None, f, f, smoe.SMOE_ROUTE_LOGITS_IN, f, big,
             None) == smoe.SMOE_EINVAL                                  # logits_in needs logits
    assert r(ctypes.byref(d), f, f, 8, None, f, f, 0, f, 1024, None) == smoe.SMOE_EWORKSPACE
    assert r(ctypes.byref(d), f, f, 8, None, f, f, 0, ctypes.c_void_p(4096 + 16), big,
             None) == smoe.SMOE_EINVAL                                  # misaligned workspace


def test_route_ranked_argument_errors(smoe):
    d = desc_of(smoe)                                   # top_k 8 of 128
    f = ctypes.c_void_p(4096)
    r = smoe.lib.smoe_route_ranked
    big = 1 << 30

    def call(B=1, spec=4, ranked=f, idx=f, flags=0, gate=f, ws=f, n=big, desc=d):
        return r(ctypes.byref(desc), gate, f, B, None, spec, ranked, idx, f, flags, ws, n, None)

    assert call(spec=-1) == smoe.SMOE_EUNSUPPORTED
    assert call(spec=9) == smoe.SMOE_EUNSUPPORTED      # 8 + 9 > 16 ranks
    assert call(spec=8, desc=desc_of(smoe, num_experts=12)) == smoe.SMOE_EUNSUPPORTED   # > E
    assert call(B=-1) == smoe.SMOE_EINVAL
    assert call(B=65) == smoe.SMOE_EUNSUPPORTED
    assert call(B=0, ranked=None) == smoe.SMOE_OK       # nothing to do
    assert call(ranked=None) == smoe.SMOE_EINVAL
    assert call(idx=None) == smoe.SMOE_EINVAL
    assert call(gate=None) == smoe.SMOE_EINVAL
    assert call(flags=0x10) == smoe.SMOE_EINVAL
    assert call(flags=smoe.SMOE_ROUTE_LOGITS_IN) == smoe.SMOE_EINVAL   # needs logits
    assert call(B=8, n=1024) == smoe.SMOE_EWORKSPACE
    assert call(ws=ctypes.c_void_p(4096 + 16)) == smoe.SMOE_EINVAL


def test_forward_argument_errors(smoe):
    d = desc_of(smoe)
    f = 4096
    q = smoe.QMat(f, f, f, 1536 * 512, 1536 * 64)
    qd = smoe.QMat(f, f, f, 4096 * 192, 4096 * 24)
    ex = smoe.Experts(q, q, qd)
    un = smoe.Union(f, f, f, f, f)
    fw = smoe.lib.smoe_moe_forward
    big = 1 << 30
    args = lambda **o: dict(dict(desc=ctypes.byref(d), ex=ctypes.byref(ex), x=f, idx=f, w=f,
                                 un=ctypes.byref(un), B=8, res=None, out=f, ws=f, n=big), **o)

    def call(**o):
        a = args(**o)
        return fw(a["desc"], a["ex"], a["x"], a["idx"], a["w"], a["un"], a["B"], a["res"], a["out"],
                  a["ws"], a["n"], None)

    assert call(ex=None) == smoe.SMOE_EINVAL
    assert call(un=None) == smoe.SMOE_EINVAL
    assert call(x=None) == smoe.SMOE_EINVAL
    assert call(out=f + 4) == smoe.SMOE_EINVAL
    assert call(res=f + 8) == smoe.SMOE_EINVAL
    bad_stride = smoe.Experts(smoe.QMat(f, f, f, 1536 * 512 - 4, 1536 * 64), q, qd)
    assert call(ex=ctypes.byref(bad_stride)) == smoe.SMOE_EINVAL
    bad_align = smoe.Experts(smoe.QMat(f + 4, f, f, 1536 * 512, 1536 * 64), q, qd)
    assert call(ex=ctypes.byref(bad_align)) == smoe.SMOE_EINVAL
    assert call(n=4096) == smoe.SMOE_EWORKSPACE
    assert call(B=-3) == smoe.SMOE_EINVAL


def test_shared_expert_arguments(smoe):
    for fs in (-64, 32, 100, 8256):
        d = desc_of(smoe, shared_ffn_dim=fs)
        assert smoe.workspace_size(d, 8) == 0
    d0, d1 = desc_of(smoe), desc_of(smoe, shared_ffn_dim=3072)
    # the shared expert's h (f16 + group sums) and output rows per token
    grow = smoe.workspace_size(d1, 64) - smoe.workspace_size(d0, 64)
    assert grow >= 64 * (3072 * 2 + 3072 // 64 * 16 + 4096 * 4)
    f = 4096
    q = smoe.QMat(f, f, f, 1536 * 512, 1536 * 64)
    qd = smoe.QMat(f, f, f, 4096 * 192, 4096 * 24)
    un = smoe.Union(f, f, f, f, f)
    fw = smoe.lib.smoe_moe_forward
    sq = smoe.QMat(f, f, f, 0, 0)                      # one matrix: strides unused
    for ex in (smoe.Experts(q, q, qd),                 # shared matrices missing
               smoe.Experts(q, q, qd, sq, sq, smoe.QMat(f + 4, f, f, 0, 0)),   # misaligned
               smoe.Experts(q, q, qd, sq, smoe.QMat(f, None, f, 0, 0), sq)):
        assert fw(ctypes.byref(d1), ctypes.byref(ex), f, f, f, ctypes.byref(un), 8, None, f, f,
                  1 << 30, None) == smoe.SMOE_EINVAL


def test_attention_arguments(smoe):
    ok = dict(d_model=4096, num_heads=64, num_kv_heads=4, ctx=4096)
    assert smoe.attn_workspace_size(smoe.make_attn_desc(**ok), 1) > 0
    for kw, code in ((dict(head_dim=64), -2), (dict(num_heads=48), -2),          # 48*128 not 2^k*512
                     (dict(num_heads=64, num_kv_heads=3), -2), (dict(num_kv_heads=2), -2),
                     (dict(d_model=3072), -2), (dict(d_model=16384), -2), (dict(ctx=0), -2),
                     (dict(eps=0.0), -1), (dict(rope_theta=-1.0), -1)):
        d = smoe.make_attn_desc(**dict(ok, **kw))
        assert smoe.attn_workspace_size(d, 1) == 0, kw
    desc = smoe.make_attn_desc(**ok)
    f = ctypes.c_void_p(4096)
    big = 1 << 30
    fw = smoe.lib.smoe_attn_forward

    def call(B=1, pos0=0, w=f, out=f, ws=f, n=big, d=desc):
        return fw(ctypes.byref(d), w, f, f, B, pos0, f, f, out, ws, n, None)

    assert call(B=-1) == smoe.SMOE_EINVAL
    assert call(B=65) == smoe.SMOE_EUNSUPPORTED
    small = smoe.make_attn_desc(**dict(ok, ctx=4))
    assert call(B=5, d=small) == smoe.SMOE_EUNSUPPORTED        # more tokens than ring slots
    assert call(pos0=-1) == smoe.SMOE_EINVAL
    assert call(B=0, w=None, out=None) == smoe.SMOE_OK         # nothing to do
    assert call(w=None) == smoe.SMOE_EINVAL
    assert call(out=ctypes.c_void_p(4096 + 8)) == smoe.SMOE_EINVAL
    assert call(ws=ctypes.c_void_p(4096 + 16)) == smoe.SMOE_EINVAL
    assert call(n=1024) == smoe.SMOE_EWORKSPACE
    bad = smoe.make_attn_desc(**ok)
    bad.reserved = 1
    assert call(d=bad) == smoe.SMOE_EINVAL
    st = smoe.lib.smoe_attn_forward_stage
    assert st(3, ctypes.byref(desc), f, f, f, 1, 0, f, f, f, f, big, None, None, None) == smoe.SMOE_EINVAL
    assert st(0, ctypes.byref(desc), f, f, f, 1, 0, f, f, f, f, big, None, f, None) == smoe.SMOE_EINVAL


def test_stage_argument_errors(smoe):
    d = desc_of(smoe)
    f = 4096
    q = smoe.QMat(f, f, f, 1536 * 512, 1536 * 64)
    qd = smoe.QMat(f, f, f, 4096 * 192, 4096 * 24)
    ex = smoe.Experts(q, q, qd)
    un = smoe.Union(f, f, f, f, f)
    st = smoe.lib.smoe_moe_layer_stage

    def call(stage=smoe.SMOE_STAGE_GATE_UP, n=1 << 30, ev=(None, None)):
        return st(stage, ctypes.byref(d), f, ctypes.byref(ex), f, 8, None, f, None, f, f,
                  ctypes.byref(un), f, n, None, ev[0], ev[1])

    assert call(stage=-1) == smoe.SMOE_EINVAL
    assert call(stage=4) == smoe.SMOE_EINVAL
    assert call(ev=(f, None)) == smoe.SMOE_EINVAL       # events come in pairs
    assert call(ev=(None, f)) == smoe.SMOE_EINVAL
    assert call(n=4096) == smoe.SMOE_EWORKSPACE


def test_single_launch_argument_errors(smoe):
    """smoe_moe_layer_single checks its arguments as smoe_moe_layer does, then
    refuses the layers it has no single-launch kernel for (B != 1, an fp32
    router, d outside 2048/4096, a shared expert), all before any launch."""
    f = 4096
    q = smoe.QMat(f, f, f, 1536 * 512, 1536 * 64)
    qd = smoe.QMat(f, f, f, 4096 * 192, 4096 * 24)
    sq = smoe.QMat(f, f, f, 0, 0)
    ex = smoe.Experts(q, q, qd)
    un = smoe.Union(f, f, f, f, f)
    sl = smoe.lib.smoe_moe_layer_single

    def call(d=None, B=1, x=f, n=1 << 30, e=ex):
        d = desc_of(smoe) if d is None else d
        return sl(ctypes.byref(d), f, ctypes.byref(e), x, B, None, f, f, f, f, ctypes.byref(un),
                  f, n, None)

    assert call(x=None) == smoe.SMOE_EINVAL
    assert call(B=-1) == smoe.SMOE_EINVAL
    assert call(n=4096) == smoe.SMOE_EWORKSPACE
    assert call(B=0) == smoe.SMOE_OK                    # an empty batch launches nothing
    assert call(B=2) == smoe.SMOE_EUNSUPPORTED
    assert call(d=desc_of(smoe, router_bf16=False)) == smoe.SMOE_EUNSUPPORTED
    assert call(d=desc_of(smoe, d_model=1024)) == smoe.SMOE_EUNSUPPORTED
    assert call(d=desc_of(smoe, shared_ffn_dim=3072),
                e=smoe.Experts(q, q, qd, sq, sq, sq)) == smoe.SMOE_EUNSUPPORTED


def test_rmsnorm_argument_errors(smoe):
    f = ctypes.c_void_p(4096)
    rn = smoe.lib.smoe_rmsnorm
    assert rn(f, -1, 4096, 1e-6, f, None) == smoe.SMOE_EINVAL
    assert rn(f, 1, 100, 1e-6, f, None) == smoe.SMOE_EUNSUPPORTED
    assert rn(f, 1, 16384, 1e-6, f, None) == smoe.SMOE_EUNSUPPORTED
    assert rn(f, 1, 4096, 0.0, f, None) == smoe.SMOE_EINVAL
    assert rn(f, 1, 4096, float("nan"), f, None) == smoe.SMOE_EINVAL
    assert rn(None, 1, 4096, 1e-6, f, None) == smoe.SMOE_EINVAL
    assert rn(f, 1, 4096, 1e-6, ctypes.c_void_p(4100), None) == smoe.SMOE_EINVAL
    assert rn(None, 0, 4096, 1e-6, None, None) == smoe.SMOE_OK      # empty batch: no-op


def test_stack_argument_errors(smoe):
    d = desc_of(smoe)
    f = 4096
    q = smoe.QMat(f, f, f, 1536 * 512, 1536 * 64)
    qd = smoe.QMat(f, f, f, 4096 * 192, 4096 * 24)
    good = smoe.Experts(q, q, qd)
    bad = smoe.Experts(smoe.QMat(f, f, f, 1536 * 512 - 4, 1536 * 64), q, qd)
    un = smoe.Union(f, f, f, f, f)
    sf = smoe.lib.smoe_stack_forward
    big = 1 << 30

    def call(n=3, experts=(good, good, good), B=1, eps=1e-6, h=f, tmp=2 * f, un_=un, nbytes=big,
             routers=(f, f, f)):
        ra = (ctypes.c_void_p * 3)(*routers)
        ea = (smoe.Experts * 3)(*experts)
        return sf(ctypes.byref(d), n, ra, ea, h, B, eps, tmp, f, f, None,
                  ctypes.byref(un_) if un_ is not None else None, f, nbytes, None)

    assert call(n=-1) == smoe.SMOE_EINVAL
    assert call(eps=0.0) == smoe.SMOE_EINVAL
    assert call(un_=None) == smoe.SMOE_EINVAL
    assert call(B=65) == smoe.SMOE_EUNSUPPORTED
    assert call(tmp=f) == smoe.SMOE_EINVAL                       # tmp must not be h
    assert call(h=f + 4) == smoe.SMOE_EINVAL
    # a bad last layer is found before anything is launched
    assert call(experts=(good, good, bad)) == smoe.SMOE_EINVAL
    assert call(routers=(f, f, None)) == smoe.SMOE_EINVAL
    assert call(nbytes=4096) == smoe.SMOE_EWORKSPACE
    assert call(n=0) == smoe.SMOE_OK and call(B=0) == smoe.SMOE_OK


def test_stack_chunks_argument_errors(smoe):
    """smoe_stack_forward_chunks checks every chunk and layer, and that no two
    chunks share a buffer, before anything is launched."""
    d = desc_of(smoe)
    f = 4096
    q = smoe.QMat(f, f, f, 1536 * 512, 1536 * 64)
    qd = smoe.QMat(f, f, f, 4096 * 192, 4096 * 24)
    good = smoe.Experts(q, q, qd)
    bad = smoe.Experts(smoe.QMat(f, f, f, 1536 * 512 - 4, 1536 * 64), q, qd)
    sc = smoe.lib.smoe_stack_forward_chunks
    big = 1 << 30

    def chunk(base, B=64, ws=None, nbytes=big):
        # distinct 256-byte-aligned fake addresses per chunk (nothing is launched)
        a = [base + 4096 * k for k in range(12)]
        un = smoe.Union(a[5], a[6], a[7], a[8], a[9])
        return smoe.StackChunk(a[0], B, a[1], a[2], a[3], a[4], un,
                               a[10] if ws is None else ws, nbytes, None)

    def call(chunks, n=3, experts=(good, good, good), eps=1e-6, count=None):
        ra = (ctypes.c_void_p * 3)(f, f, f)
        ea = (smoe.Experts * 3)(*experts)
        arr = (smoe.StackChunk * max(len(chunks), 1))(*chunks)
        return sc(ctypes.byref(d), n, ra, ea, eps, arr, len(chunks) if count is None else count)

    c0, c1 = chunk(1 << 24), chunk(1 << 25)
    assert call([c0, c1], count=0) == smoe.SMOE_EINVAL
    assert call([c0] * 9, count=9) == smoe.SMOE_EINVAL
    assert sc(ctypes.byref(d), 3, (ctypes.c_void_p * 3)(f, f, f), (smoe.Experts * 3)(good, good, good),
              1e-6, None, 1) == smoe.SMOE_EINVAL
    assert call([c0, c1], eps=0.0) == smoe.SMOE_EINVAL
    assert call([c0, chunk(1 << 25, B=65)]) == smoe.SMOE_EUNSUPPORTED
    assert call([c0, chunk(1 << 25, nbytes=4096)]) == smoe.SMOE_EWORKSPACE
    assert call([c0, c1], experts=(good, good, bad)) == smoe.SMOE_EINVAL
    # two chunks may not share a workspace, h or any other buffer
    assert call([c0, chunk(1 << 25, ws=(1 << 24) + 4096 * 10)]) == smoe.SMOE_EINVAL
    assert call([c0, chunk((1 << 24) + 4096 * 10)]) == smoe.SMOE_EINVAL   # c1.h == c0.ws
    assert call([c0, c0]) == smoe.SMOE_EINVAL
    # nothing to do
    assert call([c0, c1], n=0) == smoe.SMOE_OK
    assert call([chunk(1 << 24, B=0), chunk(1 << 25, B=0)]) == smoe.SMOE_OK


def test_strerror(smoe):
    for c in (0, -1, -2, -3, -4):
        assert smoe.strerror(c)
    assert "unknown" in smoe.strerror(-99)


def test_diagnostics_reject_bad_arguments(smoe):
    """The calibration entry points validate before launching anything."""
    f = 4096
    sr = smoe.lib.smoe_stream_read
    assert sr(f, 64, f, 0, None) == smoe.SMOE_EINVAL           # no blocks
    assert sr(f + 4, 64, f, 8, None) == smoe.SMOE_EINVAL       # unaligned source
    assert sr(f, 60, f, 8, None) == smoe.SMOE_EINVAL           # not whole 16-byte words
    assert sr(None, 64, f, 8, None) == smoe.SMOE_EINVAL
    assert smoe.lib.smoe_empty_launch(0, 1, None) == smoe.SMOE_EINVAL
    assert smoe.lib.smoe_empty_launch((1 << 20) + 1, 1, None) == smoe.SMOE_EINVAL
    assert smoe.lib.smoe_empty_launch(8, -1, None) == smoe.SMOE_EINVAL
    assert smoe.lib.smoe_gpu_sleep(-1, None) == smoe.SMOE_EINVAL
    assert smoe.lib.smoe_gpu_sleep(100001, None) == smoe.SMOE_EINVAL
    dr = smoe.lib.smoe_dma_read
    assert dr(f, 1 << 20, 2048, 0, f, 1, None) == smoe.SMOE_EINVAL     # sink too small (2 blocks)
    assert dr(f + 4, 1 << 20, 2048, 0, f, 64, None) == smoe.SMOE_EINVAL  # unaligned source
    assert dr(f, 1 << 20, 2000, 0, f, 64, None) == smoe.SMOE_EINVAL     # row not whole 64 B
    assert dr(f, 1 << 20, 2048, 2, f, 64, None) == smoe.SMOE_EINVAL     # no such mode
    assert dr(None, 1 << 20, 2048, 0, f, 64, None) == smoe.SMOE_EINVAL
    assert dr(f, 1 << 20, 2048, 1, None, 64, None) == smoe.SMOE_EINVAL
    assert dr(f, 64 * 2048 - 1, 2048, 0, f, 1, None) == smoe.SMOE_OK    # no whole unit: nothing
    gb = smoe.lib.smoe_grid_barrier
    assert gb(0, f, f, f, None) == smoe.SMOE_EINVAL
    assert gb(4097, f, f, f, None) == smoe.SMOE_EINVAL
    assert gb(8, None, f, f, None) == smoe.SMOE_EINVAL
    assert gb(8, f, None, f, None) == smoe.SMOE_EINVAL
    assert gb(8, f, f, None, None) == smoe.SMOE_EINVAL
