"""The decode layer as one cooperative launch (smoe_moe_layer_single) against
the three-launch layer (smoe_moe_layer, itself checked against the oracle in
test_gpu_parity and test_gpu_fullsize): the same output, routing and union
bit for bit, twice in a row (the barriers' counters are cleared for the next
launch), no barrier timing out; shapes it does not take are refused before
anything is launched."""
import numpy as np
import pytest
import torch

import synth
from synth import configs

from gpu_helpers import desc_for, dev, device_weights, down, small_config, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def smoe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_routing_bit_amd as m
    return m


def union_state(layer, B, K):
    un = layer.union
    n = int(down(un.n_union)[0])
    return (n, down(un.union_experts)[:n].copy(), down(un.expert_offsets)[:n + 1].copy(),
            down(un.pair_list)[:B * K].copy(), down(un.pair_pos)[:B * K].copy())


def check_single(smoe, layer, cfg, xs, residual=None):
    K = cfg.top_k
    for x in xs:
        ref = down(layer.forward(x, residual=residual, want_logits=True))
        ref_idx, ref_w = down(layer.topk_idx[:1]).copy(), down(layer.topk_w[:1]).copy()
        ref_lg = down(layer.logits[:1]).copy()
        ref_un = union_state(layer, 1, K)
        out = torch.full_like(x, float("nan"))
        layer.topk_idx.fill_(-1)
        layer.topk_w.fill_(-1.0)
        smoe.moe_layer_single(layer.desc, layer.router_w, layer.experts, x, out,
                              layer.topk_idx[:1], layer.topk_w[:1], layer.union, layer.ws,
                              residual=residual, logits=layer.logits[:1])
        torch.cuda.synchronize()
        assert np.array_equal(down(out).view(np.uint32), ref.view(np.uint32))
        assert np.array_equal(down(layer.topk_idx[:1]), ref_idx)
        assert np.array_equal(down(layer.topk_w[:1]).view(np.uint32), ref_w.view(np.uint32))
        assert np.array_equal(down(layer.logits[:1]).view(np.uint32), ref_lg.view(np.uint32))
        for a, b in zip(union_state(layer, 1, K), ref_un):
            assert np.array_equal(a, b)
    assert smoe.read_status(layer.ws) == 0        # no barrier gave up


@pytest.mark.parametrize("cfg", [
    small_config("single_d4096_f1536", 4096, 32, 8, 1536, 1),    # down: 4 words a lane
    small_config("single_d2048_f512", 2048, 64, 8, 512, 1),      # 1 word a lane
    small_config("single_d2048_f1024_k4", 2048, 16, 4, 1024, 1),  # 2 words, top-4
    small_config("single_d4096_nonorm", 4096, 40, 6, 192, 1, norm=False),
    small_config("single_d2048_e255", 2048, 255, 8, 256, 1),     # more router items than blocks
], ids=lambda c: c.name)
@pytest.mark.parametrize("with_res", [False, True])
def test_single_launch_equals_three_launches(smoe, cfg, with_res):
    L = synth.make_layer(cfg)
    layer = smoe.Layer(desc_for(smoe, cfg), device_weights(L), max_batch=1, device=dev())
    xs = [up(synth.hidden(cfg.seed, 0, 40 + i, 1, cfg.d_model)) for i in range(2)]
    res = up(synth.hidden(cfg.seed, 0, 50, 1, cfg.d_model, tensor=synth.T_RESIDUAL)) if with_res else None
    check_single(smoe, layer, cfg, xs, residual=res)


@pytest.mark.parametrize("cfg", [configs.DECODE, configs.FUSED_B1], ids=lambda c: c.name)
def test_single_launch_full_size(smoe, cfg):
    import synth.gpu as sg
    W = sg.make_layer(cfg, layer=3)
    torch.cuda.synchronize()
    layer = smoe.Layer(desc_for(smoe, cfg), W, max_batch=1, device=dev())
    xs = [sg.hidden(cfg.seed, 3, 60 + i, 1, cfg.d_model) for i in range(3)]
    check_single(smoe, layer, cfg, xs)


@pytest.mark.parametrize("cfg,B", [
    (small_config("single_b2", 2048, 32, 4, 256, 2), 2),                 # two tokens
    (small_config("single_shared", 2048, 32, 4, 256, 1, shared=256), 1),  # a shared expert
    (small_config("single_d1024", 1024, 32, 4, 256, 1), 1),              # d outside 2048/4096
    (small_config("single_fp32_router", 2048, 32, 4, 256, 1, bf16=False), 1),
], ids=lambda v: getattr(v, "name", str(v)))
def test_single_launch_refuses_other_shapes(smoe, cfg, B):
    L = synth.make_layer(cfg)
    layer = smoe.Layer(desc_for(smoe, cfg), device_weights(L), max_batch=B, device=dev())
    x = up(synth.hidden(cfg.seed, 0, 1, B, cfg.d_model))
    out = torch.zeros_like(x)
    with pytest.raises(smoe.SmoeError) as e:
        smoe.moe_layer_single(layer.desc, layer.router_w, layer.experts, x, out,
                              layer.topk_idx[:B], layer.topk_w[:B], layer.union, layer.ws)
    assert e.value.code == smoe.SMOE_EUNSUPPORTED
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
