"""The stacked path: the between-layer norm and a stack of routed layers.

h <- RMSNorm(h + MoE_l(h)) per layer l.  The GPU norm is checked against the
oracle's fp32 definition; smoe_stack_forward is checked to launch exactly the
chain of single-layer calls and norms (bitwise), and every layer of that
chain is checked against the oracle on the GPU's own layer input (teacher
forcing), so rounding differences do not compound down the stack.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import configs

from gpu_helpers import (assert_layer_close, desc_for, dev, device_weights, down, near_tie,
                         rel_l2, small_config, up)

pytestmark = pytest.mark.gpu
TOL = 3e-3
EPS = 1e-6


@pytest.fixture(scope="module")
def smoe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_routing_bit_amd as m
    return m


def norm_tol(d):
    """Per-element relative bound of GPU vs oracle RMSNorm: the oracle sums
    the d positive squares one after another in fp32 (relative error at most
    (d-1) u of the sum, u = 2^-24), the GPU by a short tree (at most ~32 u);
    1/sqrt halves a relative error of its argument, and the scaling adds u."""
    return (0.5 * (d + 32) + 4) * 2.0 ** -24


@pytest.mark.parametrize("B,d", [(1, 64), (3, 1024), (64, 4096), (2, 8192)])
def test_rmsnorm_parity(smoe, B, d):
    rng = np.random.default_rng(B * 7919 + d)
    v = (rng.standard_normal((B, d)) * rng.uniform(0.1, 30.0, (B, 1))).astype(np.float32)
    ref = oracle.rmsnorm(v, eps=EPS)
    g = up(v)
    out = down(smoe.rmsnorm(g, eps=EPS))
    err = np.abs(out.astype(np.float64) - ref) / np.maximum(np.abs(ref), 1e-30)
    assert err.max() <= norm_tol(d), err.max()
    # in place gives the same bits
    smoe.rmsnorm(g, out=g, eps=EPS)
    assert np.array_equal(down(g).view(np.uint32), out.view(np.uint32))


def test_rmsnorm_zero_row_and_empty(smoe):
    v = np.zeros((2, 256), np.float32)
    v[1] = 3.0
    out = down(smoe.rmsnorm(up(v), eps=EPS))
    assert np.array_equal(out[0], np.zeros(256, np.float32))     # 0 / sqrt(eps)
    assert np.allclose(out[1], 1.0, rtol=1e-6)
    empty = torch.zeros(0, 256, dtype=torch.float32, device=dev())
    smoe.rmsnorm(empty, out=empty)


class GpuStack:
    def __init__(self, smoe, cfg, n_layers, B, layers_w):
        self.smoe, self.cfg, self.B = smoe, cfg, B
        self.desc = desc_for(smoe, cfg)
        self.W = layers_w
        self.ex = [smoe.experts_of(self.desc, W) for W in layers_w]
        self.args = smoe.StackArgs([W["router"] for W in layers_w], self.ex)
        self.ws = torch.zeros(smoe.workspace_size(self.desc, B), dtype=torch.uint8, device=dev())
        smoe.workspace_init(self.ws)
        self.un = smoe.UnionBuffers.alloc(cfg.num_experts, B * cfg.top_k, dev())
        K = cfg.top_k
        i32 = dict(dtype=torch.int32, device=dev())
        self.idx = torch.full((n_layers, B, K), -7, **i32)
        self.w = torch.zeros(n_layers, B, K, dtype=torch.float32, device=dev())
        self.nu = torch.full((n_layers,), -7, **i32)
        self.tmp = torch.zeros(B, cfg.d_model, dtype=torch.float32, device=dev())

    def forward(self, h):
        self.smoe.stack_forward(self.desc, self.args, h, self.tmp, self.idx, self.w, self.un,
                                self.ws, n_union=self.nu, eps=EPS)
        return h

    def chain(self, h0):
        """The same stack as single-layer calls and norms; returns every
        layer's input, pre-norm sum h + MoE(h), routing and union size."""
        smoe, B, K = self.smoe, self.B, self.cfg.top_k
        h = h0.clone()
        ins, sums, idxs, ws_, nus = [], [], [], [], []
        idx = torch.zeros(B, K, dtype=torch.int32, device=dev())
        w = torch.zeros(B, K, dtype=torch.float32, device=dev())
        for W, ex in zip(self.W, self.ex):
            ins.append(down(h))
            s = torch.zeros_like(h)
            smoe.moe_layer(self.desc, W["router"], ex, h, s, idx, w, self.un, self.ws, residual=h)
            sums.append(down(s))
            idxs.append(down(idx))
            ws_.append(down(w))
            nus.append(int(down(self.un.n_union)[0]))
            smoe.rmsnorm(s, out=h, eps=EPS)
        return down(h), ins, sums, idxs, ws_, nus


def check_layer_vs_oracle(L, cfg, x, s_gpu, idx_gpu, w_gpu, tokens=None):
    """One layer of the chain against the oracle on the GPU's layer input x:
    routing exact (or a near-tie), MoE(x) = s - x within relative L2, and the
    norm of s within the norm's bound."""
    tokens = list(range(x.shape[0])) if tokens is None else tokens
    xs = np.ascontiguousarray(x[tokens])
    lg, idx_ref, w_ref = oracle.route(L["router"], xs, cfg.top_k, cfg.norm_topk_prob)
    idx_g = idx_gpu[tokens]
    for i in range(len(tokens)):
        if not np.array_equal(idx_g[i], idx_ref[i]):
            # a near-tie: this token takes the GPU's set, with the oracle's
            # weights for that set
            assert near_tie(lg[i], cfg.top_k), f"token {tokens[i]}: routing differs"
            idx_ref[i] = idx_g[i]
            w_ref[i] = oracle.weights_of(lg[i:i + 1], idx_g[i:i + 1], cfg.norm_topk_prob)[0]
    shared = None
    if "shared" in L:
        shared = (L["shared"]["gate"], L["shared"]["up"], L["shared"]["down"])
    moe_ref = oracle.moe(L["gate"], L["up"], L["down"], xs, idx_ref, w_ref, shared=shared)
    moe_gpu = s_gpu[tokens].astype(np.float64) - xs.astype(np.float64)
    assert_layer_close(moe_gpu, moe_ref, TOL)


# d = 2048 with B <= 2 takes the decode kernels, where each layer after the
# first normalises its input inside its router; the last cases have a shared
# expert in every layer
@pytest.mark.parametrize("d,B,shared", [(1024, 1, 0), (1024, 2, 0), (1024, 5, 0), (1024, 64, 0),
                                        (2048, 1, 0), (2048, 2, 0), (2048, 1, 2560),
                                        (1024, 5, 320)])
def test_stack_equals_chain_and_oracle(smoe, d, B, shared):
    cfg = small_config("stack", d, 32, 8, 256, B, shared=shared)
    n_layers = 3
    Ls = [synth.make_layer(cfg, layer=l) for l in range(n_layers)]
    st = GpuStack(smoe, cfg, n_layers, B, [device_weights(L) for L in Ls])
    h0 = up(synth.hidden(cfg.seed, 0, 2000 + B, B, cfg.d_model))
    final, ins, sums, idxs, wts, nus = st.chain(h0)
    h = st.forward(h0.clone())
    torch.cuda.synchronize()
    # the stack call gives the chain's bits
    assert np.array_equal(down(h).view(np.uint32), final.view(np.uint32))
    for l in range(n_layers):
        assert np.array_equal(down(st.idx[l]), idxs[l])
        assert np.array_equal(down(st.w[l]).view(np.uint32), wts[l].view(np.uint32))
        assert int(down(st.nu[l])) == nus[l] == len(np.unique(idxs[l]))
    # each layer against the oracle, teacher-forced on the GPU's layer input
    for l in range(n_layers):
        check_layer_vs_oracle(Ls[l], cfg, ins[l], sums[l], idxs[l], wts[l])
        nxt = ins[l + 1] if l + 1 < n_layers else final
        ref = oracle.rmsnorm(sums[l], eps=EPS)
        assert np.all(np.abs(nxt - ref) <= norm_tol(cfg.d_model) * np.abs(ref) + 1e-30)


@pytest.mark.parametrize("d,B,shared", [(2048, 1, 0), (1024, 5, 0), (2048, 2, 1024)])
def test_stack_graph_replays_match_eager(smoe, d, B, shared):
    """smoe_stack_forward captured once in a HIP graph: every replay, with the
    program's own eager calls and synchronisations between replays, gives the
    eager call's bits for the same input (output, routing, union sizes)."""
    cfg = small_config("stack_g", d, 32, 8, 256, B, shared=shared)
    n_layers = 3
    Ls = [synth.make_layer(cfg, layer=l) for l in range(n_layers)]
    st = GpuStack(smoe, cfg, n_layers, B, [device_weights(L) for L in Ls])
    inputs = [up(synth.hidden(cfg.seed, 0, 3000 + i, B, d)) for i in range(3)]
    refs = []
    for x in inputs:
        h = st.forward(x.clone())
        torch.cuda.synchronize()
        refs.append((down(h).copy(), down(st.idx).copy(), down(st.w).copy(), down(st.nu).copy()))
    hg = torch.zeros(B, d, dtype=torch.float32, device=dev())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        hg.copy_(inputs[0])
        st.forward(hg)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.forward(hg)
    torch.cuda.synchronize()
    for rep in range(2):
        for i, x in enumerate(inputs):
            hg.copy_(x)
            g.replay()
            torch.cuda.synchronize()
            h_ref, idx_ref, w_ref, nu_ref = refs[i]
            assert np.array_equal(down(hg).view(np.uint32), h_ref.view(np.uint32)), (rep, i)
            assert np.array_equal(down(st.idx), idx_ref)
            assert np.array_equal(down(st.w).view(np.uint32), w_ref.view(np.uint32))
            assert np.array_equal(down(st.nu), nu_ref)
            st.forward(inputs[(i + 1) % 3].clone())       # eager work between replays
            torch.cuda.synchronize()


# several prompt chunks in flight on their own streams, each a layer behind
# the previous one: every chunk's bits equal smoe_stack_forward on that chunk
# alone (routing, union sizes and the output), on the MFMA path (chunks of
# 5 and 64), the decode path (1 and 2 tokens: the norm inside the next
# layer's router) and with a shared expert; an empty chunk is skipped
@pytest.mark.parametrize("d,Bs,shared", [(1024, (64, 64, 5), 0), (2048, (2, 1), 0),
                                         (1024, (5, 0, 64, 3), 320)])
def test_stack_chunks_equal_one_chunk_at_a_time(smoe, d, Bs, shared):
    cfg = small_config("stack_c", d, 32, 8, 256, max(Bs), shared=shared)
    n_layers = 3
    Ls = [synth.make_layer(cfg, layer=l) for l in range(n_layers)]
    Wd = [device_weights(L) for L in Ls]
    sts = [GpuStack(smoe, cfg, n_layers, max(B, 1), Wd) for B in Bs]
    streams = [torch.cuda.current_stream()] + [torch.cuda.Stream() for _ in Bs[1:]]
    for rep in range(2):                               # the ordering events are reused
        h0 = [up(synth.hidden(cfg.seed, rep, 4000 + 7 * i, B, d)) if B else
              torch.zeros(0, d, dtype=torch.float32, device=dev()) for i, B in enumerate(Bs)]
        refs = []
        for st, x, B in zip(sts, h0, Bs):
            if B == 0:
                refs.append(None)
                continue
            h = st.forward(x.clone())
            torch.cuda.synchronize()
            refs.append((down(h).copy(), down(st.idx).copy(), down(st.w).copy(), down(st.nu).copy()))
            st.idx.fill_(-7)
            st.w.fill_(-7.0)
            st.nu.fill_(-7)
        hs = [x.clone() for x in h0]
        torch.cuda.synchronize()
        # (views of each stack's own buffers; for B > 0 they are those buffers)
        chunks = [dict(h=h, tmp=st.tmp[:h.shape[0]], topk_idx=st.idx[:, :h.shape[0]].contiguous(),
                       topk_w=st.w[:, :h.shape[0]].contiguous(), n_union=st.nu, un=st.un,
                       ws=st.ws, stream=s) for h, st, s in zip(hs, sts, streams)]
        smoe.stack_forward_chunks(sts[0].desc, sts[0].args, chunks, eps=EPS)
        torch.cuda.synchronize()
        for i, (h, st, ref) in enumerate(zip(hs, sts, refs)):
            if ref is None:
                continue
            assert np.array_equal(down(h).view(np.uint32), ref[0].view(np.uint32)), (rep, i)
            assert np.array_equal(down(st.idx), ref[1]), (rep, i)
            assert np.array_equal(down(st.w).view(np.uint32), ref[2].view(np.uint32)), (rep, i)
            assert np.array_equal(down(st.nu), ref[3]), (rep, i)
        assert all(smoe.read_status(st.ws) == 0 for st in sts)


def test_stack_bad_layer_leaves_h_unchanged(smoe):
    cfg = small_config("stack_bad", 1024, 32, 8, 256, 1)
    Ls = [synth.make_layer(cfg, layer=l) for l in range(2)]
    st = GpuStack(smoe, cfg, 2, 1, [device_weights(L) for L in Ls])
    q = st.ex[1].gate
    st.ex[1] = smoe.Experts(smoe.QMat(q.w + 4, q.s, q.b, q.expert_stride_w, q.expert_stride_sb),
                            st.ex[1].up, st.ex[1].down)            # misaligned: rejected
    st.args = smoe.StackArgs([W["router"] for W in st.W], st.ex)
    h = up(synth.hidden(0, 0, 9, 1, 1024))
    before = down(h)
    with pytest.raises(smoe.SmoeError):
        st.forward(h)
    torch.cuda.synchronize()
    assert np.array_equal(down(h), before)
    assert np.array_equal(down(st.idx), np.full((2, 1, 8), -7, np.int32))


@pytest.mark.parametrize("cfg,sample", [(configs.DECODE, [0]), (configs.PREFILL, [0, 33, 63])],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_full_size_stack(smoe, cfg, sample):
    """Two stacked layers at the full decode / prefill-chunk shape, in the
    launch configuration the stacked benchmark times: the stack call equals
    the chain bitwise, and sampled tokens of every layer match the oracle
    with the CPU generator's bytes of the experts they use."""
    import synth.gpu as sg
    n_layers, B = 2, cfg.batch
    Wg = [sg.make_layer(cfg, layer=l) for l in range(n_layers)]
    st = GpuStack(smoe, cfg, n_layers, B, Wg)
    h0 = up(synth.hidden(cfg.seed, 0, 3000, B, cfg.d_model))
    final, ins, sums, idxs, wts, nus = st.chain(h0)
    h = st.forward(h0.clone())
    torch.cuda.synchronize()
    assert np.array_equal(down(h).view(np.uint32), final.view(np.uint32))
    for l in range(n_layers):
        assert np.array_equal(down(st.idx[l]), idxs[l])
        experts = sorted(set(int(e) for t in sample for e in idxs[l][t]))
        Lc = synth.make_layer(cfg, layer=l, experts=experts)
        check_layer_vs_oracle(Lc, cfg, ins[l], sums[l], idxs[l], wts[l], tokens=sample)
        nxt = ins[l + 1] if l + 1 < n_layers else final
        ref = oracle.rmsnorm(sums[l][sample], eps=EPS)
        assert np.all(np.abs(nxt[sample] - ref) <= norm_tol(cfg.d_model) * np.abs(ref) + 1e-30)
