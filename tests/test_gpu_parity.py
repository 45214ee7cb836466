"""Parity of the HIP path (through the C-ABI) with the CPU oracle.

Bars: integer/index outputs bit-exact; routing indices bit-exact when both
top-k stages see the same logits; layer outputs within relative L2 3e-3
(expected ~5e-4: activations and h enter the dot products as fp16).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import configs

from gpu_helpers import (assert_layer_close, desc_for, dev, device_weights, down, near_tie,
                         oracle_layer, rel_l2, small_config, up)

pytestmark = pytest.mark.gpu
TOL = 3e-3


@pytest.fixture(scope="module")
def smoe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_routing_bit_amd as m
    return m


def new_ws(smoe, desc, B):
    ws = torch.zeros(smoe.workspace_size(desc, max(1, B)), dtype=torch.uint8, device=dev())
    smoe.workspace_init(ws)
    return ws


# ------------------------------------------------------------------ generator
def test_gpu_generator_matches_cpu_generator():
    import synth.gpu as sg
    cfg = small_config("gen", 512, 6, 2, 192, 4, fused=True)
    Lc = synth.make_layer(cfg, layer=3)
    Lg = sg.make_layer(cfg, layer=3)
    torch.cuda.synchronize()
    assert np.array_equal(down(Lg["router"]), Lc["router"])
    for k in ("gate_up", "down"):
        for a, b in zip(Lg[k], Lc[k]):
            assert np.array_equal(down(a).view(b.dtype), b), k
    # the shared expert's tensors, fused and split
    for fused in (True, False):
        cs = small_config("gen_s", 512, 6, 2, 192, 4, fused=fused, shared=320)
        Sc = synth.make_shared(cs, layer=2)
        Sg = sg.make_layer(cs, layer=2)
        keys = ("gate_up", "down") if fused else ("gate", "up", "down")
        for k in keys:
            for a, b in zip(Sg["shared_" + k], Sc[k]):
                assert np.array_equal(down(a).view(b.dtype), b), k
    xg = sg.hidden(0, 0, 5, 7, 512)
    assert np.array_equal(down(xg).view(np.uint32), synth.hidden(0, 0, 5, 7, 512).view(np.uint32))


# -------------------------------------------------------------------- routing
# B >= 3 routes through K-slice tiles of 256, 512 or 1024 inputs (at most
# eight slices): d = 2048 and below take 256, 4096 takes 512, wider 1024;
# ragged last slices at d = 640 and 6144
ROUTE_CASES = [(configs.TINY, 8), (configs.TINY, 1), (configs.DECODE, 1), (configs.DECODE, 37),
               (configs.DECODE, 64), (configs.FUSED_B64, 64),
               (small_config("k16", 256, 16, 16, 64, 5, bf16=False), 5),
               (small_config("nonorm", 512, 40, 6, 64, 9, norm=False), 9),
               (small_config("d640_e20", 640, 20, 4, 64, 6), 6),
               (small_config("d6144_b3", 6144, 64, 8, 64, 3), 3),
               (small_config("d8192_b64_f32", 8192, 48, 6, 64, 64, bf16=False), 64)]


@pytest.mark.parametrize("cfg,B", ROUTE_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_route_parity(smoe, cfg, B):
    desc = desc_for(smoe, cfg)
    Wr = synth.router(cfg.seed, 0, cfg.num_experts, cfg.d_model, cfg.router_sigma, cfg.router_bf16)
    x = synth.hidden(cfg.seed, 0, 11, B, cfg.d_model)
    lg_ref, idx_ref, w_ref = oracle.route(Wr, x, cfg.top_k, cfg.norm_topk_prob)
    ws = new_ws(smoe, desc, B)
    lg = torch.zeros(B, cfg.num_experts, dtype=torch.float32, device=dev())
    idx = torch.zeros(B, cfg.top_k, dtype=torch.int32, device=dev())
    w = torch.zeros(B, cfg.top_k, dtype=torch.float32, device=dev())
    smoe.route(desc, up(Wr), up(x), idx, w, ws, logits=lg)
    lg_g = down(lg)
    # both fp32 sums sit within a summation-error bound of the exact logits:
    # |err| <= c * sqrt(d) * 2^-24 * sum_i |w_i x_i| (random-walk growth, c = 8)
    W64 = (Wr.astype(np.uint32) << 16).view(np.float32).astype(np.float64) if cfg.router_bf16 \
        else Wr.astype(np.float64)
    exact = x.astype(np.float64) @ W64.T
    mag = np.abs(x.astype(np.float64)) @ np.abs(W64).T
    bound = 8 * np.sqrt(cfg.d_model) * 2.0**-24 * mag + 1e-12
    assert np.all(np.abs(lg_g - exact) <= bound)
    assert np.all(np.abs(lg_ref - exact) <= bound)
    # the GPU's own top-k is exact on the logits it computed
    idx_own, w_own = oracle.topk_softmax(lg_g, cfg.top_k, cfg.norm_topk_prob)
    assert np.array_equal(down(idx), idx_own)
    assert np.allclose(down(w), w_own, rtol=1e-6, atol=1e-7)
    # fed the oracle's logits, indices are bit-exact and weights match
    smoe.route(desc, None, None, idx, w, ws, logits=up(lg_ref), logits_in=True)
    assert np.array_equal(down(idx), idx_ref)
    assert np.allclose(down(w), w_ref, rtol=1e-6, atol=1e-7)
    if cfg.norm_topk_prob:
        assert np.allclose(down(w).sum(axis=1), 1.0, atol=1e-6)


def test_topk_ties_lower_index_wins(smoe):
    cfg = small_config("ties", 64, 40, 6, 64, 3)
    desc = desc_for(smoe, cfg)
    lg = np.zeros((3, 40), np.float32)
    lg[0] = 1.0                                    # all tied
    lg[1, [39, 7, 20, 3]] = 2.5                   # tie above a flat floor
    lg[2] = np.arange(40, dtype=np.float32) % 5   # repeated values
    idx_ref, w_ref = oracle.topk_softmax(lg, 6, True)
    ws = new_ws(smoe, desc, 3)
    idx = torch.zeros(3, 6, dtype=torch.int32, device=dev())
    w = torch.zeros(3, 6, dtype=torch.float32, device=dev())
    smoe.route(desc, None, None, idx, w, ws, logits=up(lg), logits_in=True)
    assert np.array_equal(down(idx), idx_ref)
    assert list(down(idx)[0]) == [0, 1, 2, 3, 4, 5]
    assert np.allclose(down(w), w_ref, rtol=1e-6)


RANKED_CASES = [(configs.DECODE, 1, 4), (configs.DECODE, 1, 8), (configs.DECODE, 37, 2),
                (configs.FUSED_B64, 64, 4), (small_config("k16r", 256, 16, 16, 64, 5, bf16=False), 5, 0),
                (small_config("nonorm_r", 512, 40, 6, 64, 9, norm=False), 9, 10)]


@pytest.mark.parametrize("cfg,B,spec", RANKED_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_route_ranked_parity(smoe, cfg, B, spec):
    desc = desc_for(smoe, cfg)
    K, R = cfg.top_k, cfg.top_k + spec
    Wr = synth.router(cfg.seed, 0, cfg.num_experts, cfg.d_model, cfg.router_sigma, cfg.router_bf16)
    x = synth.hidden(cfg.seed, 0, 12, B, cfg.d_model)
    lg_ref = oracle.route(Wr, x, K, cfg.norm_topk_prob)[0]
    ws = new_ws(smoe, desc, B)
    lg = torch.zeros(B, cfg.num_experts, dtype=torch.float32, device=dev())
    ranked = torch.full((B, R), -7, dtype=torch.int32, device=dev())
    idx = torch.zeros(B, K, dtype=torch.int32, device=dev())
    w = torch.zeros(B, K, dtype=torch.float32, device=dev())
    smoe.route_ranked(desc, up(Wr), up(x), spec, ranked, idx, w, ws, logits=lg)
    lg_g = down(lg)
    # on the logits it computed: the ranking is the oracle's, the first K
    # ranks are the top-k, and the weights are smoe_route's
    assert np.array_equal(down(ranked), oracle.rank(lg_g, R))
    assert np.array_equal(down(ranked)[:, :K], down(idx))
    idx_own, w_own = oracle.topk_softmax(lg_g, K, cfg.norm_topk_prob)
    assert np.array_equal(down(idx), idx_own)
    assert np.allclose(down(w), w_own, rtol=1e-6, atol=1e-7)
    idx2 = torch.zeros_like(idx)
    w2 = torch.zeros_like(w)
    smoe.route(desc, None, None, idx2, w2, ws, logits=lg, logits_in=True)
    assert torch.equal(idx2, idx) and torch.equal(w2, w)
    # fed the oracle's logits: bit-exact ranking
    smoe.route_ranked(desc, None, None, spec, ranked, idx, w, ws, logits=up(lg_ref), logits_in=True)
    assert np.array_equal(down(ranked), oracle.rank(lg_ref, R))


def test_route_ranked_ties_and_all_experts(smoe):
    cfg = small_config("rties", 64, 12, 4, 64, 3)
    desc = desc_for(smoe, cfg)
    lg = np.zeros((3, 12), np.float32)
    lg[0] = 1.0                                    # all tied: index order
    lg[1, [11, 2, 7]] = 3.0                        # a tied top above a flat floor
    lg[2] = np.arange(12, dtype=np.float32) % 4    # repeated values
    R = 12                                         # every expert ranked
    ws = new_ws(smoe, desc, 3)
    ranked = torch.zeros(3, R, dtype=torch.int32, device=dev())
    idx = torch.zeros(3, 4, dtype=torch.int32, device=dev())
    w = torch.zeros(3, 4, dtype=torch.float32, device=dev())
    smoe.route_ranked(desc, None, None, R - 4, ranked, idx, w, ws, logits=up(lg), logits_in=True)
    got = down(ranked)
    assert list(got[0]) == list(range(12))
    assert list(got[1][:4]) == [2, 7, 11, 0]
    assert np.array_equal(got, oracle.rank(lg, R))
    assert np.array_equal(got[:, :4], down(idx))


# ---------------------------------------------------------------------- union
@pytest.mark.parametrize("B,K,E,mode", [(1, 8, 128, "rand"), (8, 4, 16, "rand"),
                                        (64, 8, 128, "rand"), (37, 8, 256, "rand"),
                                        (64, 16, 256, "rand"), (64, 8, 128, "same"),
                                        (3, 1, 1, "rand"), (64, 16, 16, "rand")])
def test_union_parity(smoe, B, K, E, mode):
    cfg = small_config("u", 64, E, K, 64, B)
    desc = desc_for(smoe, cfg)
    rng = np.random.default_rng(B * 7 + K)
    if mode == "same":
        idx = np.tile(np.arange(K, dtype=np.int32), (B, 1))
    else:
        idx = np.stack([rng.choice(E, K, replace=False) for _ in range(B)]).astype(np.int32)
    n, ue, off, pl, pp = oracle.build_union(idx, E)
    ws = new_ws(smoe, desc, B)
    un = smoe.UnionBuffers.alloc(E, B * K, dev())
    smoe.build_union(desc, up(idx), un, ws)
    assert int(down(un.n_union)[0]) == n
    assert np.array_equal(down(un.union_experts)[:n], ue)
    assert np.array_equal(down(un.expert_offsets)[:n + 1], off)
    assert np.array_equal(down(un.pair_list)[:B * K], pl)
    assert np.array_equal(down(un.pair_pos)[:B * K], pp)
    assert smoe.read_status(ws) == 0


# -------------------------------------------------------------- expert FFN
FWD_CASES = [
    (configs.TINY, 8, False),
    (configs.TINY, 1, True),
    (small_config("odd_groups", 512, 24, 6, 192, 13), 13, True),     # f/64 = 3 groups
    (small_config("ragged", 768, 12, 4, 320, 37), 37, False),        # 12 and 5 groups
    (small_config("hot", 1024, 8, 4, 256, 64), 64, True),            # up to 4 token tiles
    (small_config("fused", 512, 32, 8, 128, 64, fused=True), 64, False),
    (small_config("wide", 2048, 16, 2, 128, 3, bf16=False), 3, True),
    (small_config("mfma_b2", 1024, 32, 12, 1536, 2), 2, True),          # B*K > 16: off the decode path
    (small_config("dec_b2", 2048, 32, 8, 1536, 2), 2, True),            # decode kernel, 32 lanes/row
    (small_config("dec_b2_f512", 4096, 64, 8, 512, 2), 2, False),       # 1 down group per lane
    (small_config("dec_b1_f192", 2048, 16, 4, 192, 1), 1, True),        # 3 groups, 1 lane per row
    (small_config("dec_b2_e8", 2048, 8, 8, 512, 2), 2, False),          # every expert, E < B*K
    (small_config("gemv_b1", 4096, 64, 8, 1536, 1), 1, False),
    (small_config("gemv_k16", 2048, 64, 16, 512, 1), 1, True),
    # the decode down kernel gives lane L words NW L .. NW L + NW - 1 of a row
    # (NW = 1, 2, 4: the fewest whose 64 lanes hold f/8 words), longer rows in
    # equal chunks of at most 256 words
    (small_config("dec_b1_f2048", 2048, 16, 4, 2048, 1), 1, True),     # NW 4, all 64 lanes
    (small_config("dec_b2_f1024", 4096, 32, 8, 1024, 2), 2, False),    # NW 2, all 64 lanes
    (small_config("dec_b1_f64", 2048, 8, 2, 64, 1), 1, True),          # NW 1, 8 lanes, one group
    (small_config("dec_b2_f320", 640, 8, 2, 320, 2), 2, True),         # NW 1, 40 lanes; d = 10 groups
    (small_config("dec_b1_f768", 3072, 16, 4, 768, 1), 1, False),      # NW 2, 48 lanes; 48 of 64 row lanes
    (small_config("b1_f2560", 2048, 16, 4, 2560, 1), 1, True),         # 2 chunks of 160 words
    (small_config("dec_b1_f2624", 2048, 16, 4, 2624, 1), 1, False),    # 2 chunks: 168 + 160 words
    (small_config("dec_b2_f3072", 2048, 16, 4, 3072, 2), 2, True),     # 2 chunks of 192 words
    (small_config("dec_b1_f8192", 1024, 8, 2, 8192, 1), 1, True),      # 4 chunks of 256 words
    # the decode gate_up kernel: 32 lanes a row up to 32 groups, 64 up to 64,
    # then two groups a lane (one j an item); lanes past the row idle
    (small_config("dec_d512", 512, 16, 4, 256, 1), 1, True),           # 8 of 32 lanes
    (small_config("dec_d1536", 1536, 32, 8, 1024, 2), 2, False),       # 24 of 32 lanes
    (small_config("dec_d6144", 6144, 16, 8, 1536, 1), 1, True),        # 96 groups: 2 a lane, 32 idle
    (small_config("dec_d8192_b2", 8192, 8, 4, 512, 2), 2, True),       # 128 groups: 2 a lane
    (small_config("dec_d8192_b1", 8192, 8, 8, 2048, 1), 1, False),
    # down with f of 512 .. 2048 (a multiple of 512): two units a wave
    (small_config("two_units_ragged", 640, 12, 4, 512, 13), 13, True),    # 10 units: second ones cut
    (small_config("two_units_f2048", 1536, 16, 4, 2048, 9, bf16=False), 9, False),
    (small_config("two_units_shared", 1024, 16, 4, 1024, 13, shared=2048), 13, True),
    (small_config("one_unit_shared_wide", 1024, 16, 4, 1024, 37, shared=2048), 37, True),
    # with a shared expert
    (small_config("s_fwd_dec2", 2048, 32, 8, 512, 2, shared=2560), 2, True),
    (small_config("s_fwd_odd", 512, 24, 6, 192, 13, shared=320), 13, True),   # 5 groups
    (small_config("s_fwd_b3", 2048, 16, 2, 128, 3, bf16=False, shared=128), 3, False),
]


@pytest.mark.parametrize("cfg,B,with_res", FWD_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_forward_parity_injected_routing(smoe, cfg, B, with_res):
    L = synth.make_layer(cfg)
    x = synth.hidden(cfg.seed, 0, 1, B, cfg.d_model)
    res = synth.hidden(cfg.seed, 0, 2, B, cfg.d_model, tensor=synth.T_RESIDUAL) if with_res else None
    _, idx, w = oracle.route(L["router"], x, cfg.top_k, cfg.norm_topk_prob)
    ref = oracle_layer(L, x, cfg, residual=res, idx=idx, w=w)[0]
    desc = desc_for(smoe, cfg)
    layer = smoe.Layer(desc, device_weights(L), max_batch=B, device=dev())
    smoe.build_union(desc, up(idx), layer.union, layer.ws)
    out = torch.empty(B, cfg.d_model, dtype=torch.float32, device=dev())
    smoe.moe_forward(desc, layer.experts, up(x), up(idx), up(w), layer.union, out, layer.ws,
                     residual=up(res) if with_res else None)
    got = down(out)
    err, worst = assert_layer_close(got, ref, TOL, residual=res if with_res else None)
    assert err <= 1.5e-3, f"precision regression: {err}"


# Skewed routing: an expert that serves more than 16 pairs takes the wide
# pass, all of its pairs (up to the chunk's 64 tokens) against one stream of
# its weights; the shared expert does too once B > 16.
SKEW_CASES = [
    (small_config("skew_all64", 1024, 32, 4, 256, 64), 64, "all"),      # 4 experts x 64 pairs
    (small_config("skew_hot48_s", 2048, 64, 8, 512, 48, shared=256), 48, "hot"),
    (small_config("skew_all17_fused", 1024, 16, 2, 192, 17, fused=True), 17, "all"),
    (small_config("skew_hot64_nof", 512, 40, 6, 320, 64, bf16=False), 64, "hot"),
    # two units a wave (f = 1024): the wide pass runs unit by unit
    (small_config("skew_hot64_two_units", 1536, 32, 4, 1024, 64), 64, "hot"),
]


def skewed_routing(cfg, B, mode, seed=7):
    """Expert ids and weights: "all" routes every token to the same K experts
    (in a different order per token); "hot" puts expert 5 first for every
    token and fills the rest at random.  Weights are random and sum to one."""
    rng = np.random.default_rng(seed)
    E, K = cfg.num_experts, cfg.top_k
    idx = np.empty((B, K), np.int32)
    for t in range(B):
        if mode == "all":
            idx[t] = rng.permutation(np.arange(K))
        else:
            others = rng.choice(np.setdiff1d(np.arange(E), [5]), K - 1, replace=False)
            idx[t] = np.concatenate([[5], others])
    w = rng.random((B, K)).astype(np.float32) + 0.05
    w /= w.sum(axis=1, keepdims=True)
    return idx, w.astype(np.float32)


@pytest.mark.parametrize("cfg,B,mode", SKEW_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_forward_parity_skewed_routing(smoe, cfg, B, mode):
    L = synth.make_layer(cfg)
    x = synth.hidden(cfg.seed, 0, 4, B, cfg.d_model)
    res = synth.hidden(cfg.seed, 0, 5, B, cfg.d_model, tensor=synth.T_RESIDUAL)
    idx, w = skewed_routing(cfg, B, mode)
    ref = oracle_layer(L, x, cfg, residual=res, idx=idx, w=w)[0]
    desc = desc_for(smoe, cfg)
    layer = smoe.Layer(desc, device_weights(L), max_batch=B, device=dev())
    smoe.build_union(desc, up(idx), layer.union, layer.ws)
    counts = np.diff(down(layer.union.expert_offsets)[:int(down(layer.union.n_union)[0]) + 1])
    assert counts.max() > 16
    out = torch.empty(B, cfg.d_model, dtype=torch.float32, device=dev())
    smoe.moe_forward(desc, layer.experts, up(x), up(idx), up(w), layer.union, out, layer.ws,
                     residual=up(res))
    err, worst = assert_layer_close(down(out), ref, TOL, residual=res)
    assert err <= 1.5e-3, f"precision regression: {err}"


# Layers with a shared expert: decode kernels (B <= 2; its down rows in one to
# sixteen chunks of up to 64 NW words, the last one partial) and prefill MFMA
# kernels (its own grid row; wider and narrower than the routed experts, the
# register and the LDS scale/bias variants), fused and split layouts.
SHARED_CASES = [
    (small_config("s_dec1_fs3072", 4096, 32, 8, 256, 1, shared=3072), 1),
    (small_config("s_dec2_fused", 2048, 64, 8, 512, 2, fused=True, shared=1024), 2),
    (small_config("s_dec1_fs8192", 2048, 16, 4, 256, 1, shared=8192), 1),
    (small_config("s_dec1_d1024", 1024, 16, 4, 128, 1, shared=192), 1),
    (small_config("s_dec1_d8192", 8192, 8, 4, 1024, 1, shared=8192), 1),    # NW 2: 8 chunks
    (small_config("s_dec2_d2560", 2560, 16, 4, 512, 2, shared=4608), 2),    # NW 1: 9 chunks
    (small_config("s_pref64", 1024, 64, 8, 256, 64, shared=512), 64),
    (small_config("s_pref37_narrow", 1024, 32, 4, 512, 37, fused=True, shared=256), 37),
    (small_config("s_pref5_fs6144", 1024, 16, 2, 128, 5, shared=6144), 5),
    # f = 1536 beside a shared expert on its wide pass: one unit a wave
    (small_config("s_pref24_fs3072", 1024, 16, 4, 1536, 24, shared=3072), 24),
]


@pytest.mark.parametrize("cfg,B", [(configs.TINY, 8), (small_config("l", 1024, 64, 8, 256, 64), 64),
                                   (small_config("l1", 1024, 64, 8, 256, 1), 1),
                                   (small_config("l_dec1", 4096, 32, 8, 256, 1), 1),
                                   (small_config("l_dec2", 2048, 64, 8, 512, 2), 2),
                                   (small_config("l_dec1_f2048", 2048, 32, 8, 2048, 1), 1),
                                   (small_config("l_dec2_nonorm", 2048, 40, 6, 192, 2, norm=False), 2)]
                         + SHARED_CASES,
                         ids=lambda v: getattr(v, "name", str(v)))
def test_layer_parity(smoe, cfg, B):
    L = synth.make_layer(cfg)
    x = synth.hidden(cfg.seed, 0, 3, B, cfg.d_model)
    ref, idx_ref, w_ref = oracle_layer(L, x, cfg)
    lg_ref = oracle.router_logits(L["router"], x)
    desc = desc_for(smoe, cfg)
    layer = smoe.Layer(desc, device_weights(L), max_batch=B, device=dev())
    out = down(layer.forward(up(x), want_logits=True))
    idx = down(layer.topk_idx[:B])
    bad = [t for t in range(B) if not np.array_equal(idx[t], idx_ref[t])]
    for t in bad:
        assert near_tie(lg_ref[t], cfg.top_k), f"routing differs for token {t}"
    if bad:
        w = oracle.weights_of(lg_ref, idx, cfg.norm_topk_prob)
        ref, _, _ = oracle_layer(L, x, cfg, idx=idx, w=w)
    assert_layer_close(out, ref, TOL)
    # the routing outputs (written by the router's tail, or for B <= 2 by the
    # gate_up kernel's prologue) are exact on the logits the GPU computed
    lg = down(layer.logits[:B])
    idx_own, w_own = oracle.topk_softmax(lg, cfg.top_k, cfg.norm_topk_prob)
    assert np.array_equal(idx, idx_own)
    assert np.allclose(down(layer.topk_w[:B]), w_own, rtol=1e-6, atol=1e-7)
    n, ue, off, pl, pp = oracle.build_union(idx, cfg.num_experts)
    un = layer.union
    assert int(down(un.n_union)[0]) == n
    assert np.array_equal(down(un.union_experts)[:n], ue)
    assert np.array_equal(down(un.expert_offsets)[:n + 1], off)
    assert np.array_equal(down(un.pair_list)[:B * cfg.top_k], pl)
    assert np.array_equal(down(un.pair_pos)[:B * cfg.top_k], pp)


def _bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("cfg,B,mode", [
    # every token on the same 4 experts: 4 experts x 64 pairs (wide pass)
    (small_config("lsk_all", 1024, 32, 4, 256, 64), 64, "all"),
    # half the tokens on 8 hot experts (32+ pairs each), the rest spread
    (small_config("lsk_half_s", 2048, 64, 8, 512, 64, shared=256), 64, "half"),
    # the 256-expert fused layout with 2 hot experts at 48 tokens
    (small_config("lsk_fused", 1024, 256, 8, 512, 48, fused=True), 48, "half"),
], ids=lambda v: getattr(v, "name", str(v)))
def test_layer_parity_skewed_router(smoe, cfg, B, mode):
    """The whole layer (the GPU's own routing) with a router that sends many
    tokens to a few experts: hot rows of the gate share a direction c that
    the hot tokens' hidden states carry, so those experts serve 17..64 pairs
    (the wide pass) while the rest serve few.  Checked against the oracle's
    routing and layer, and the union outputs against the oracle's union."""
    L = synth.make_layer(cfg)
    d, E, K = cfg.d_model, cfg.num_experts, cfg.top_k
    n_hot = K if mode == "all" else max(2, K // 4) if E > 64 else K
    z = synth.hidden(cfg.seed, 0, 6, B, d).astype(np.float64)
    c = synth.hidden(cfg.seed, 0, 7, 1, d)[0].astype(np.float64)
    hot_tok = np.arange(B) if mode == "all" else np.arange(0, B, 2)
    z[hot_tok] += 3.0 * c
    x = (z / np.sqrt(np.mean(z * z, axis=1, keepdims=True) + 1e-6)).astype(np.float32)
    rng = np.random.default_rng(11)
    wr = rng.standard_normal((E, d)) / np.sqrt(d)
    hot_exp = rng.choice(E, n_hot, replace=False)
    wr[hot_exp] = 0.5 * c / np.sqrt(d) + rng.standard_normal((n_hot, d)) / np.sqrt(d)
    L["router"] = _bf16_bits(wr)
    ref, idx_ref, w_ref = oracle_layer(L, x, cfg)
    lg_ref = oracle.router_logits(L["router"], x)
    counts = np.bincount(idx_ref.ravel(), minlength=E)
    assert counts.max() > 16, counts.max()            # some expert takes the wide pass
    desc = desc_for(smoe, cfg)
    layer = smoe.Layer(desc, device_weights(L), max_batch=B, device=dev())
    out = down(layer.forward(up(x), want_logits=True))
    idx = down(layer.topk_idx[:B])
    bad = [t for t in range(B) if not np.array_equal(idx[t], idx_ref[t])]
    for t in bad:
        assert near_tie(lg_ref[t], K), f"routing differs for token {t}"
    if bad:
        w = oracle.weights_of(lg_ref, idx, cfg.norm_topk_prob)
        ref, _, _ = oracle_layer(L, x, cfg, idx=idx, w=w)
    assert_layer_close(out, ref, TOL)
    n, ue, off, pl, pp = oracle.build_union(idx, E)
    un = layer.union
    assert int(down(un.n_union)[0]) == n
    assert np.array_equal(down(un.union_experts)[:n], ue)
    assert np.array_equal(down(un.expert_offsets)[:n + 1], off)
    assert np.array_equal(down(un.pair_list)[:B * K], pl)
    assert np.array_equal(down(un.pair_pos)[:B * K], pp)


@pytest.mark.parametrize("cfg,B", [SHARED_CASES[0], SHARED_CASES[1], SHARED_CASES[6],
                                   SHARED_CASES[8]], ids=lambda v: getattr(v, "name", str(v)))
def test_shared_zero_weights_leave_the_routed_layer(smoe, cfg, B):
    """A shared expert whose weights are all zero changes no bit of the
    layer: residual + (0 + routed_out) = residual + routed_out."""
    import dataclasses
    L = synth.make_layer(cfg)
    x = synth.hidden(cfg.seed, 0, 4, B, cfg.d_model)
    res = synth.hidden(cfg.seed, 0, 5, B, cfg.d_model, tensor=synth.T_RESIDUAL)
    plain_cfg = dataclasses.replace(cfg, shared_ffn_dim=0)
    Lp = {k: v for k, v in L.items() if k != "shared"}
    plain = smoe.Layer(desc_for(smoe, plain_cfg), device_weights(Lp), max_batch=B, device=dev())
    Lz = dict(L)
    Lz["shared"] = {k: tuple(np.zeros_like(a) for a in v) for k, v in L["shared"].items()}
    zero = smoe.Layer(desc_for(smoe, cfg), device_weights(Lz), max_batch=B, device=dev())
    live = smoe.Layer(desc_for(smoe, cfg), device_weights(L), max_batch=B, device=dev())
    a = down(plain.forward(up(x), residual=up(res)))
    b = down(zero.forward(up(x), residual=up(res)))
    c = down(live.forward(up(x), residual=up(res)))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert rel_l2(c - res, a - res) > 0.1


def test_deterministic_bitwise(smoe):
    cfg = small_config("det", 1024, 32, 8, 256, 64)
    L = synth.make_layer(cfg)
    x = up(synth.hidden(0, 0, 4, 64, 1024))
    layer = smoe.Layer(desc_for(smoe, cfg), device_weights(L), max_batch=64, device=dev())
    a = down(layer.forward(x))
    b = down(layer.forward(x))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("B", [1, 2, 64])
def test_stages_equal_layer_and_stamp_events(smoe, B):
    """The four diagnostic stages in order launch exactly one layer call's
    kernels (bitwise the same output), and the timing events given to a
    stage are stamped with its kernel's own duration."""
    import torch
    cfg = small_config("stages", 2048, 32, 8, 256, B)      # B <= 2: the decode kernels
    L = synth.make_layer(cfg)
    x = up(synth.hidden(0, 0, 5, B, 2048))
    layer = smoe.Layer(desc_for(smoe, cfg), device_weights(L), max_batch=B, device=dev())
    ref = down(layer.forward(x))
    out = torch.zeros(B, 2048, dtype=torch.float32, device=dev())
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    ev[0].record()
    ev[1].record()
    for st in (smoe.SMOE_STAGE_ROUTE, smoe.SMOE_STAGE_GATE_UP, smoe.SMOE_STAGE_DOWN,
               smoe.SMOE_STAGE_COMBINE):
        smoe.moe_layer_stage(st, layer.desc, layer.router_w, layer.experts, x, out,
                             layer.topk_idx[:B], layer.topk_w[:B], layer.union, layer.ws,
                             events=ev if st == smoe.SMOE_STAGE_GATE_UP else None)
    torch.cuda.synchronize()
    assert np.array_equal(down(out).view(np.uint32), ref.view(np.uint32))
    ms = ev[0].elapsed_time(ev[1])
    assert 0.0 < ms < 50.0


def test_integer_case_bit_exact(smoe):
    """s=1 and small integer biases, one-hot inputs, unit routing weights: every
    value on both paths is an exact integer, so GPU and oracle agree bit for
    bit.  Pins nibble order, row order, group indexing and the pair mapping."""
    d, f, E, K, B = 512, 256, 8, 2, 6
    rng = np.random.default_rng(5)

    def quant(rows, cols, lo, hi, bias):
        q = rng.integers(lo, hi + 1, (E, rows, cols)).astype(np.uint32)
        w = np.zeros((E, rows, cols // 8), np.uint32)
        for i in range(8):
            w |= q[..., i::8] << (4 * i)
        s = np.full((E, rows, cols // 64), 0x3F80, np.uint16)               # 1.0
        b = np.full((E, rows, cols // 64), np.float32(bias).view(np.uint32) >> 16, np.uint16)
        return w, s, b

    gate = quant(f, d, 0, 15, 20.0)     # g in [20, 35]: silu(g) == g in fp32
    upp = quant(f, d, 4, 11, -8.0)      # u in [-4, 3]
    dn = quant(d, f, 0, 15, 0.0)
    x = np.zeros((B, d), np.float32)
    for t in range(B):
        x[t, rng.integers(0, d)] = 1.0
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(B)]).astype(np.int32)
    w = np.ones((B, K), np.float32)
    ref = oracle.moe(gate, upp, dn, x, idx, w)
    assert np.all(ref == np.round(ref))
    cfg = small_config("int", d, E, K, f, B)
    desc = desc_for(smoe, cfg)
    W = {"router": up(np.zeros((E, d), np.uint16)), "gate": tuple(map(up, gate)),
         "up": tuple(map(up, upp)), "down": tuple(map(up, dn))}
    layer = smoe.Layer(desc, W, max_batch=B, device=dev())
    smoe.build_union(desc, up(idx), layer.union, layer.ws)
    out = torch.empty(B, d, dtype=torch.float32, device=dev())
    smoe.moe_forward(desc, layer.experts, up(x), up(idx), up(w), layer.union, out, layer.ws)
    assert np.array_equal(down(out), ref)


def test_bad_expert_sets_status_and_skips_pair(smoe):
    cfg = small_config("bad", 256, 16, 4, 128, 4)
    L = synth.make_layer(cfg)
    x = synth.hidden(0, 0, 6, 4, 256)
    _, idx, w = oracle.route(L["router"], x, 4)
    idx_bad = idx.copy()
    idx_bad[2, 1] = 999
    idx_bad[0, 3] = -1
    w_ref = w.copy()
    w_ref[2, 1] = 0.0
    w_ref[0, 3] = 0.0
    ref = oracle.moe(L["gate"], L["up"], L["down"], x, idx, w_ref)
    desc = desc_for(smoe, cfg)
    layer = smoe.Layer(desc, device_weights(L), max_batch=4, device=dev())
    assert smoe.read_status(layer.ws) == 0
    smoe.build_union(desc, up(idx_bad), layer.union, layer.ws)
    pp = down(layer.union.pair_pos)[:16]
    assert pp[2 * 4 + 1] == -1 and pp[0 * 4 + 3] == -1
    out = torch.empty(4, 256, dtype=torch.float32, device=dev())
    smoe.moe_forward(desc, layer.experts, up(x), up(idx_bad), up(w), layer.union, out, layer.ws)
    assert smoe.read_status(layer.ws) & smoe.SMOE_STATUS_BAD_EXPERT
    assert_layer_close(down(out), ref, TOL)


@pytest.mark.parametrize("B", [1, 2])
def test_decode_all_experts_bad_gives_residual(smoe, B):
    """Every routed id invalid: an empty union on the decode kernels.  Nothing
    is loaded for it, the combine adds nothing and the residual comes back."""
    cfg = small_config("allbad", 2048, 16, 4, 512, B)
    L = synth.make_layer(cfg)
    x = synth.hidden(0, 0, 7, B, 2048)
    res = synth.hidden(0, 0, 8, B, 2048, tensor=synth.T_RESIDUAL)
    idx = np.full((B, 4), 77, np.int32)
    w = np.full((B, 4), 0.25, np.float32)
    desc = desc_for(smoe, cfg)
    layer = smoe.Layer(desc, device_weights(L), max_batch=B, device=dev())
    smoe.build_union(desc, up(idx), layer.union, layer.ws)
    assert int(down(layer.union.n_union)[0]) == 0
    out = torch.empty(B, 2048, dtype=torch.float32, device=dev())
    smoe.moe_forward(desc, layer.experts, up(x), up(idx), up(w), layer.union, out, layer.ws,
                     residual=up(res))
    assert smoe.read_status(layer.ws) & smoe.SMOE_STATUS_BAD_EXPERT
    assert np.array_equal(down(out), res)


@pytest.mark.parametrize("B", [1, 2, 3])
def test_all_experts_bad_leaves_the_shared_expert(smoe, B):
    """Every routed id invalid with a shared expert: the union is empty and the
    output is residual + shared_out (decode kernels for B <= 2, MFMA rows for B = 3)."""
    cfg = small_config("allbad_s", 2048, 16, 4, 512, B, shared=1536)
    L = synth.make_layer(cfg)
    x = synth.hidden(0, 0, 7, B, 2048)
    res = synth.hidden(0, 0, 8, B, 2048, tensor=synth.T_RESIDUAL)
    idx = np.full((B, 4), 77, np.int32)
    w = np.full((B, 4), 0.25, np.float32)
    desc = desc_for(smoe, cfg)
    layer = smoe.Layer(desc, device_weights(L), max_batch=B, device=dev())
    smoe.build_union(desc, up(idx), layer.union, layer.ws)
    assert int(down(layer.union.n_union)[0]) == 0
    out = torch.empty(B, 2048, dtype=torch.float32, device=dev())
    smoe.moe_forward(desc, layer.experts, up(x), up(idx), up(w), layer.union, out, layer.ws,
                     residual=up(res))
    assert smoe.read_status(layer.ws) & smoe.SMOE_STATUS_BAD_EXPERT
    S = L["shared"]
    ref = oracle.shared_ffn(S["gate"], S["up"], S["down"], x)
    assert_layer_close(down(out), ref + res, TOL, residual=res)


def test_empty_batch_is_noop(smoe):
    cfg = configs.TINY
    L = synth.make_layer(cfg)
    desc = desc_for(smoe, cfg)
    layer = smoe.Layer(desc, device_weights(L), max_batch=8, device=dev())
    x = torch.zeros(0, cfg.d_model, dtype=torch.float32, device=dev())
    out = layer.forward(x)
    assert out.shape == (0, cfg.d_model)
    smoe.build_union(desc, torch.zeros(0, cfg.top_k, dtype=torch.int32, device=dev()), layer.union,
                     layer.ws)
    assert int(down(layer.union.n_union)[0]) == 0
