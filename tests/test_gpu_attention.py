"""Parity of the attention block (smoe_attn_forward, through the C-ABI) with
the CPU oracle (oracle/attention.py) on the same seeded inputs.

Bars: the block's contribution out - x within relative L2 3e-3 of the
oracle's; the K/V entries the call appends within one bf16 step of the
oracle's (the GPU rounds its fp32 values, the oracle its fp64 ones) plus
2e-3 of their RMS, more than 95% of them equal; every other ring slot
unchanged, bit for bit.  The absolute term is the effect of one projection
input that the GPU's fp32 input norm and the oracle's fp64 one round to
neighbouring bf16 values: one step of |x| <= 4 against a weight |w| <= 0.08
moves an entry by up to 0.08 * 4 * 2^-8 = 1.3e-3, against an RMS of 0.64
(V) or 1 (K).  Such inputs are rare (about one in 40 tokens here), so
chunks of many tokens meet them.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import attention as A

from gpu_helpers import dev, down, rel_l2, up

pytestmark = pytest.mark.gpu
TOL = 3e-3


@pytest.fixture(scope="module")
def smoe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_routing_bit_amd as m
    return m


def make_inputs(cfg, seed):
    """bf16 weights (sigma 0.02) and prior ring contents (N(0, 1), bf16)."""
    Wqkv = synth.bf16_matrix(seed, 0, synth.T_ATTN_QKV, cfg.qkv_rows, cfg.d_model, 0.02)
    Wo = synth.bf16_matrix(seed, 0, synth.T_ATTN_O, cfg.d_model, cfg.q_dim, 0.02)
    shape = (cfg.num_kv_heads, cfg.ctx, cfg.head_dim)
    Kc = synth.bf16_matrix(seed, 0, synth.T_K_CACHE, shape[0] * shape[1], shape[2], 1.0).reshape(shape)
    Vc = synth.bf16_matrix(seed, 0, synth.T_V_CACHE, shape[0] * shape[1], shape[2], 1.0).reshape(shape)
    return Wqkv, Wo, Kc, Vc


def run_both(smoe, cfg, B, pos0, seed=0):
    Wqkv, Wo, Kc, Vc = make_inputs(cfg, seed)
    x = synth.hidden(seed, 0, 40 + B, B, cfg.d_model)
    kc64, vc64 = A.bf16_bits_to_f64(Kc), A.bf16_bits_to_f64(Vc)
    ref = A.attention_block(cfg, Wqkv, Wo, x, pos0, kc64, vc64)
    desc = smoe.make_attn_desc(cfg.d_model, cfg.num_heads, cfg.num_kv_heads, cfg.ctx,
                               rope_theta=cfg.rope_theta, eps=cfg.eps)
    ws = torch.zeros(smoe.attn_workspace_size(desc, B), dtype=torch.uint8, device=dev())
    kd, vd = up(Kc), up(Vc)
    out = torch.empty(B, cfg.d_model, dtype=torch.float32, device=dev())
    smoe.attn_forward(desc, up(Wqkv), up(Wo), up(x), pos0, kd, vd, out, ws)
    torch.cuda.synchronize()
    return x, ref, down(out), (Kc, Vc), (down(kd), down(vd)), (kc64, vc64), desc


def check(cfg, B, pos0, x, ref, got, before, after, ref_cache):
    err = rel_l2(got - x, ref - x)
    assert err <= TOL, err
    written = sorted({(pos0 + t) % cfg.ctx for t in range(B)})
    keep = np.ones(cfg.ctx, bool)
    keep[written] = False
    for b, a, r in zip(before, after, ref_cache):
        assert np.array_equal(a[:, keep], b[:, keep])           # untouched slots
        got_v = A.bf16_bits_to_f64(a[:, written])
        want = r[:, written]
        # one bf16 step of the value, plus the effect of one input rounded to
        # the neighbouring bf16 value, which dominates for entries near zero
        rms = np.sqrt(np.mean(want * want))
        assert np.all(np.abs(got_v - want) <= 2.0**-7 * np.abs(want) + 2e-3 * rms)
        assert np.mean(got_v == want) > 0.95
    return err


SMALL = A.AttnConfig(d_model=512, num_heads=4, num_kv_heads=2, ctx=64)
ODD_CTX = A.AttnConfig(d_model=1024, num_heads=8, num_kv_heads=1, ctx=300)
GROUP16 = A.AttnConfig(d_model=2048, num_heads=16, num_kv_heads=1, ctx=512, rope_theta=1e4)

CASES = [
    (SMALL, 1, 0),        # first token: a window of one
    (SMALL, 1, 37),       # part of the ring filled
    (SMALL, 2, 100),      # wrapped ring, two tokens
    (SMALL, 5, 20),       # a short chunk
    (SMALL, 64, 0),       # a 64-token chunk filling the ring
    (ODD_CTX, 1, 299),    # full ring of 300: two splits, the second partial
    (ODD_CTX, 2, 1000),   # wrapped, the window crossing the ring's end
    (GROUP16, 1, 700),    # 16 query heads per key/value head
    # chunks of 3 or more tokens take the batched projections (MFMA tiles of
    # 16 tokens over 512-input slices, the slices summed in order)
    (GROUP16, 3, 10),     # the smallest batched chunk; 4 input slices
    (GROUP16, 17, 500),   # two token tiles, the second holding one token
    (ODD_CTX, 40, 280),   # three token tiles, the chunk crossing the ring's end
]


@pytest.mark.parametrize("cfg,B,pos0", CASES,
                         ids=lambda v: f"d{v.d_model}_h{v.num_heads}_kv{v.num_kv_heads}_ctx{v.ctx}"
                         if isinstance(v, A.AttnConfig) else str(v))
def test_attention_block_parity(smoe, cfg, B, pos0):
    x, ref, got, before, after, ref_cache, _ = run_both(smoe, cfg, B, pos0)
    check(cfg, B, pos0, x, ref, got, before, after, ref_cache)


FULL = A.AttnConfig(d_model=4096, num_heads=64, num_kv_heads=4, ctx=4096)


@pytest.mark.parametrize("B,pos0", [(1, 4095), (2, 5000), (64, 4032), (64, 3040)])
def test_attention_block_full_size(smoe, B, pos0):
    """The decode shape (d 4096, 64 query heads, 4 key/value heads, a 4096-slot
    ring), with the ring full and with it wrapped; a 64-token chunk that ends
    at the ring's last slot; and one that crosses a 256-position split, so that
    the early tokens of a token group do not reach the last split."""
    x, ref, got, before, after, ref_cache, _ = run_both(smoe, FULL, B, pos0)
    check(FULL, B, pos0, x, ref, got, before, after, ref_cache)


@pytest.mark.parametrize("cfg,B", [(SMALL, 2), (GROUP16, 5)], ids=["gemv_b2", "batched_b5"])
def test_stages_equal_the_whole_call(smoe, cfg, B):
    pos0 = 50
    Wqkv, Wo, Kc, Vc = make_inputs(cfg, 3)
    x = up(synth.hidden(3, 0, 9, B, cfg.d_model))
    desc = smoe.make_attn_desc(cfg.d_model, cfg.num_heads, cfg.num_kv_heads, cfg.ctx,
                               rope_theta=cfg.rope_theta)
    ws = torch.zeros(smoe.attn_workspace_size(desc, B), dtype=torch.uint8, device=dev())
    outs = []
    for staged in (False, True):
        kd, vd = up(Kc), up(Vc)
        out = torch.empty(B, cfg.d_model, dtype=torch.float32, device=dev())
        if staged:
            for st in range(3):
                smoe.attn_forward_stage(st, desc, up(Wqkv), up(Wo), x, pos0, kd, vd, out, ws)
        else:
            smoe.attn_forward(desc, up(Wqkv), up(Wo), x, pos0, kd, vd, out, ws)
        torch.cuda.synchronize()
        outs.append((down(out), down(kd), down(vd)))
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("B", [1, 4])
def test_in_place_and_empty(smoe, B):
    cfg, pos0 = SMALL, 9
    x, ref, got, *_ = run_both(smoe, cfg, B, pos0, seed=4)
    Wqkv, Wo, Kc, Vc = make_inputs(cfg, 4)
    desc = smoe.make_attn_desc(cfg.d_model, cfg.num_heads, cfg.num_kv_heads, cfg.ctx,
                               rope_theta=cfg.rope_theta)
    ws = torch.zeros(smoe.attn_workspace_size(desc, B), dtype=torch.uint8, device=dev())
    h = up(x)
    smoe.attn_forward(desc, up(Wqkv), up(Wo), h, pos0, up(Kc), up(Vc), h, ws)   # out = x
    assert np.array_equal(down(h).view(np.uint32), got.view(np.uint32))
    empty = torch.zeros(0, cfg.d_model, dtype=torch.float32, device=dev())
    smoe.attn_forward(desc, up(Wqkv), up(Wo), empty, pos0, up(Kc), up(Vc), empty, ws)
