"""Parity at the full workload sizes, in the launch configuration bench.py times.

The layer's weights are made on the GPU by the seeded generator; the oracle
gets the CPU generator's bytes of the experts the sampled tokens use (the
test first checks those bytes equal the device bytes), and checks sampled
tokens one by one: routing bit-exact (or a provable near-tie) and the
layer output within relative L2 3e-3.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import configs

from gpu_helpers import desc_for, dev, down, near_tie, rel_l2, up

pytestmark = pytest.mark.gpu
TOL = 3e-3


@pytest.fixture(scope="module")
def smoe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_routing_bit_amd as m
    return m


def gpu_layer(smoe, cfg, layer_id):
    import synth.gpu as sg
    W = sg.make_layer(cfg, layer=layer_id)
    torch.cuda.synchronize()
    return smoe.Layer(desc_for(smoe, cfg), W, max_batch=cfg.batch, device=dev()), W


@pytest.mark.parametrize("cfg,sample", [(configs.DECODE, [0]), (configs.PREFILL, [0, 17, 42, 63]),
                                        (configs.FUSED_B1, [0]), (configs.FUSED_B64, [3, 31, 60]),
                                        (configs.DECODE_SHARED, [0]),
                                        (configs.PREFILL_SHARED, [0, 29, 63])],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_full_size_layer(smoe, cfg, sample):
    layer_id = 5
    layer, W = gpu_layer(smoe, cfg, layer_id)
    x = synth.hidden(cfg.seed, layer_id, 77, cfg.batch, cfg.d_model)
    out = down(layer.forward(up(x), want_logits=True))
    idx = down(layer.topk_idx[:cfg.batch])
    wts = down(layer.topk_w[:cfg.batch])
    # routing of every token, from the CPU-generated gate
    Wr = synth.router(cfg.seed, layer_id, cfg.num_experts, cfg.d_model, cfg.router_sigma,
                      cfg.router_bf16)
    assert np.array_equal(down(W["router"]), Wr)
    lg_ref, idx_ref, w_ref = oracle.route(Wr, x, cfg.top_k, cfg.norm_topk_prob)
    for t in range(cfg.batch):
        if not np.array_equal(idx[t], idx_ref[t]):
            assert near_tie(lg_ref[t], cfg.top_k), f"token {t}: routing differs"
    n_u = int(down(layer.union.n_union)[0])
    assert n_u == len(np.unique(idx))
    # sampled tokens through the oracle with CPU-generated experts
    experts = sorted(set(int(e) for t in sample for e in idx[t]))
    Lc = synth.make_layer(cfg, layer=layer_id, experts=experts)
    key = "gate_up" if cfg.fused else "gate"
    for e in experts[:2]:
        for a, b in zip(W[key], Lc[key]):
            assert np.array_equal(down(a[e]).view(b.dtype), b[e])
    xs = x[sample]
    shared = None
    if cfg.shared_ffn_dim:
        S = Lc["shared"]
        for a, b in zip(W["shared_gate"], S["gate"]):
            assert np.array_equal(down(a).view(b.dtype), b)
        shared = (S["gate"], S["up"], S["down"])
    ref = oracle.moe(Lc["gate"], Lc["up"], Lc["down"], xs, idx[sample], wts[sample],
                     shared=shared)
    err = rel_l2(out[sample], ref)
    assert err <= TOL, err
    # the GPU weights for the sampled tokens match the oracle's to 1e-6
    assert np.allclose(wts[sample], w_ref[sample], rtol=1e-5, atol=1e-6) or \
        any(not np.array_equal(idx[t], idx_ref[t]) for t in sample)
