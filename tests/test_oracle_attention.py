"""Pins of the attention-block oracle against what the pages and the
mathematics fix: hand-worked rotations, the rotation's relative-position
property, a pure-Python brute force of the attention, the GQA head mapping,
causality, chunked = token-serial ("Layer-Major Batched Prefill": the chunked
path gives the token-serial bits), the ring's window, and bf16 rounding."""
import math

import numpy as np

from oracle import attention as A


def test_bf16_round_to_nearest_even():
    one = 1.0
    got = A.bf16_round(np.array([one, one + 2.0**-8, one + 3 * 2.0**-8, one + 2.0**-8 + 2.0**-20,
                                 -2.5, 0.0], np.float32))
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties go to the even one (1)
    assert got.tolist() == [1.0, 1.0, 1.0 + 2.0**-6, 1.0 + 2.0**-7, -2.5, 0.0]


def test_rope_hand_worked():
    # hd = 4: pairs (0, 2) at angle pos * 1 and (1, 3) at pos * 10000^(-1/2)
    x = np.array([1.0, 2.0, 3.0, 4.0])
    got = A.rope(x, 1, 10000.0)
    a0, a1 = 1.0, 0.01
    want = [1 * math.cos(a0) - 3 * math.sin(a0), 2 * math.cos(a1) - 4 * math.sin(a1),
            3 * math.cos(a0) + 1 * math.sin(a0), 4 * math.cos(a1) + 2 * math.sin(a1)]
    assert np.allclose(got, want, rtol=0, atol=1e-15)
    assert np.array_equal(A.rope(x, 0, 10000.0), x)                 # position 0: identity


def test_rope_depends_on_relative_position_only():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    dots = [A.rope(q, m, 1e6) @ A.rope(k, m - 37, 1e6) for m in (37, 100, 4000)]
    assert np.allclose(dots, dots[0], rtol=1e-11)
    assert abs(np.linalg.norm(A.rope(q, 999, 1e6)) - np.linalg.norm(q)) < 1e-12


def _cfg(**kw):
    base = dict(d_model=64, num_heads=4, num_kv_heads=2, head_dim=8, ctx=16, rope_theta=1e4)
    base.update(kw)
    return A.AttnConfig(**base)


def _weights(cfg, seed):
    rng = np.random.default_rng(seed)
    def bits(rows, cols):
        w = (rng.standard_normal((rows, cols)) * 0.2).astype(np.float32)
        return (w.view(np.uint32) >> 16).astype(np.uint16)        # truncate to bf16 bits
    return bits(cfg.qkv_rows, cfg.d_model), bits(cfg.d_model, cfg.q_dim)


def test_attend_matches_brute_force_loops():
    cfg = _cfg()
    rng = np.random.default_rng(5)
    kc = rng.standard_normal((2, 16, 8))
    vc = rng.standard_normal((2, 16, 8))
    q = rng.standard_normal((4, 8))
    got = A.attend(cfg, q, kc, vc, pos=9, lo=2).reshape(4, 8)
    for h in range(4):
        g = h // 2
        s = [sum(q[h][i] * kc[g][j][i] for i in range(8)) / math.sqrt(8) for j in range(2, 10)]
        m = max(s)
        e = [math.exp(v - m) for v in s]
        z = sum(e)
        for i in range(8):
            want = sum(e[j] * vc[g][j + 2][i] for j in range(8)) / z
            assert abs(got[h][i] - want) < 1e-12


def test_gqa_head_mapping():
    """Constant V per key/value head: query head h returns its group's constant."""
    cfg = _cfg(num_heads=8, num_kv_heads=2)
    rng = np.random.default_rng(6)
    kc = rng.standard_normal((2, 16, 8))
    vc = np.stack([np.full((16, 8), 10.0), np.full((16, 8), 20.0)])
    o = A.attend(cfg, rng.standard_normal((8, 8)), kc, vc, pos=5, lo=0).reshape(8, 8)
    assert np.allclose(o[:4], 10.0) and np.allclose(o[4:], 20.0)


def test_block_is_causal_and_chunk_equals_token_serial():
    cfg = _cfg()
    Wqkv, Wo = _weights(cfg, 7)
    x = np.random.default_rng(8).standard_normal((6, cfg.d_model)).astype(np.float32)
    # three tokens of history (positions 0..2), then six more (3..8) as one
    # chunk and, on a copy of the same history, one at a time
    kc1, vc1 = A.new_cache(cfg)
    kc2, vc2 = A.new_cache(cfg)
    hist = np.random.default_rng(9).standard_normal((3, cfg.d_model)).astype(np.float32)
    A.attention_block(cfg, Wqkv, Wo, hist, 0, kc1, vc1)
    A.attention_block(cfg, Wqkv, Wo, hist, 0, kc2, vc2)
    chunk = A.attention_block(cfg, Wqkv, Wo, x, 3, kc1, vc1)
    serial = np.concatenate([A.attention_block(cfg, Wqkv, Wo, x[t:t + 1], 3 + t, kc2, vc2)
                             for t in range(6)])
    assert np.array_equal(chunk, serial)
    assert np.array_equal(kc1, kc2) and np.array_equal(vc1, vc2)
    # causality: a later token's K/V does not change an earlier token's output
    kc3, vc3 = A.new_cache(cfg)
    A.attention_block(cfg, Wqkv, Wo, hist, 0, kc3, vc3)
    first = A.attention_block(cfg, Wqkv, Wo, x[:2], 3, kc3, vc3)
    assert np.array_equal(first, chunk[:2])


def test_ring_keeps_the_last_ctx_positions():
    """20 token-serial steps through a ring of 8: the last step equals attention
    over an explicit list of the last 8 tokens' (k, v)."""
    cfg = _cfg(ctx=8)
    Wqkv, Wo = _weights(cfg, 10)
    xs = np.random.default_rng(11).standard_normal((20, cfg.d_model)).astype(np.float32)
    kc, vc = A.new_cache(cfg)
    hist_k, hist_v = [], []
    for p in range(20):
        out = A.attention_block(cfg, Wqkv, Wo, xs[p:p + 1], p, kc, vc)
        q, k, v = A.qkv_rows(cfg, Wqkv, xs[p:p + 1], p)
        hist_k.append(A.bf16_round(k[0].astype(np.float32)))
        hist_v.append(A.bf16_round(v[0].astype(np.float32)))
    K = np.stack(hist_k[-8:], axis=1)       # [Hkv, 8, hd], positions 12..19
    V = np.stack(hist_v[-8:], axis=1)
    o = A.attend(cfg, q[0], K, V, pos=7, lo=0)       # the same 8 rows, in their own slots
    want = xs[19].astype(np.float64) + A.bf16_bits_to_f64(Wo) @ A.bf16_round(o.astype(np.float32))
    assert np.allclose(out[0], want, rtol=0, atol=1e-12)


def test_qk_norm_unit_rms_and_position_zero():
    cfg = _cfg()
    Wqkv, _ = _weights(cfg, 12)
    x = np.random.default_rng(13).standard_normal((1, cfg.d_model)).astype(np.float32)
    q, k, v = A.qkv_rows(cfg, Wqkv, x, 0)             # position 0: RoPE is the identity
    assert np.allclose(np.sqrt(np.mean(q * q, axis=-1)), 1.0, atol=1e-5)
    assert np.allclose(np.sqrt(np.mean(k * k, axis=-1)), 1.0, atol=1e-5)
    assert not np.allclose(np.sqrt(np.mean(v * v, axis=-1)), 1.0, atol=1e-2)
