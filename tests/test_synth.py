"""The seeded input generator: Philox, normals, quantiser, packing, fused layout."""
import math

import numpy as np
import pytest
from scipy import stats

import synth
from synth import configs


def unpack_nibbles(w: np.ndarray) -> np.ndarray:
    """[..., cols/8] u32 -> [..., cols] codes; element c at bits 4*(c%8) of word c/8."""
    shifts = np.arange(8, dtype=np.uint32) * 4
    q = (w[..., None] >> shifts) & 0xF
    return q.reshape(*w.shape[:-1], w.shape[-1] * 8).astype(np.int64)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32)


# Known-answer vectors of Philox4x32-10 published with the Random123 library
# (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11).
PHILOX_KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,expect", PHILOX_KAT)
def test_philox_known_answers(ctr, key, expect):
    assert tuple(int(v) for v in synth.philox(ctr, key)) == expect


def test_series_ln_and_sincos_match_libm():
    import ctypes
    L = synth.lib()
    for n in [1, 2, 3, 1000, 2**31, 2**31 + 12345, 2**32 - 1, 2**32]:
        got = L.synth_ln_u32(n)
        assert abs(got - math.log(n / 2**32)) <= 2e-15 * max(1.0, abs(got)), n
    sn, cs = ctypes.c_double(), ctypes.c_double()
    for b in [0, 1, 2**29, 2**30 - 1, 2**30, 2**31 + 7, 3 * 2**30 + 99, 2**32 - 1]:
        L.synth_sincos_turn(b, ctypes.byref(sn), ctypes.byref(cs))
        th = 2 * math.pi * b / 2**32
        assert abs(sn.value - math.sin(th)) < 1e-14 and abs(cs.value - math.cos(th)) < 1e-14, b


def test_normals_distribution():
    z = synth.normals(0, 0, synth.T_GATE, 0, 0, 2_000_000).astype(np.float64)
    assert abs(z.mean()) < 5 / math.sqrt(z.size)
    assert abs(z.var() - 1) < 5 * math.sqrt(2 / z.size)
    assert abs(stats.skew(z)) < 0.01 and abs(stats.kurtosis(z)) < 0.02
    assert stats.kstest(z[:200_000], "norm").pvalue > 1e-3


def test_normals_deterministic_and_addressable():
    a = synth.normals(5, 3, synth.T_UP, 7, 1000, 4096)
    b = synth.normals(5, 3, synth.T_UP, 7, 1000, 4096)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    # element n of a stream does not depend on where the request starts
    c = synth.normals(5, 3, synth.T_UP, 7, 1500, 100)
    assert np.array_equal(a[500:600], c)
    # different tensor / stream / layer / seed give different numbers
    for args in [(5, 3, synth.T_DOWN, 7), (5, 3, synth.T_UP, 8), (5, 4, synth.T_UP, 7),
                 (6, 3, synth.T_UP, 7)]:
        d = synth.normals(*args, 1000, 4096)
        assert np.mean(a == d) < 0.01


def test_hidden_rows_are_rms_normalised():
    x = synth.hidden(0, 0, 0, 8, 256)
    rms = np.sqrt((x.astype(np.float64) ** 2).mean(axis=1))
    assert np.allclose(rms, 1.0, atol=1e-6)


def test_quantiser_bounds_and_roundtrip():
    rng = np.random.default_rng(1)
    W = (rng.standard_normal((96, 512)) * 0.02).astype(np.float32)
    W[3, :64] = 0.125                       # a constant group: scale 0, all codes 0
    w, s, b = synth.quantize_matrix(W)
    q = unpack_nibbles(w)
    assert q.min() >= 0 and q.max() <= 15
    S = np.repeat(bf16_to_f32(s), 64, axis=1).astype(np.float64)
    Bv = np.repeat(bf16_to_f32(b), 64, axis=1).astype(np.float64)
    deq = S * q + Bv
    err = np.abs(deq - W)
    # half a step, plus the bf16 rounding of scale and bias across 15 steps
    bound = 0.5 * S + 15 * S * 2.0**-8 + np.abs(Bv) * 2.0**-8 + 1e-12
    assert np.all(err <= bound)
    assert np.all(q[3, :64] == 0) and np.all(bf16_to_f32(s)[3, 0] == 0)
    # packing round trip of the codes themselves
    repacked = np.zeros_like(w)
    for i in range(8):
        repacked |= (q[:, i::8].astype(np.uint32) << (4 * i))
    assert np.array_equal(repacked, w)


def test_generated_experts_match_quantised_normals():
    rows, cols, sigma = 16, 256, 0.02
    w, s, b = synth.quant_experts(0, 2, synth.T_DOWN, 5, 2, rows, cols, sigma)
    for e in range(2):
        W = synth.normals(0, 2, synth.T_DOWN, 5 + e, 0, rows * cols, sigma).reshape(rows, cols)
        w2, s2, b2 = synth.quantize_matrix(W)
        assert np.array_equal(w[e], w2) and np.array_equal(s[e], s2) and np.array_equal(b[e], b2)


def test_fused_gate_up_interleaves_per_expert():
    cfg = configs.LayerConfig("t", 128, 4, 2, 64, 2, router_bf16=True, fused=True)
    L = synth.make_layer(cfg)
    gw, uw, fw = L["gate"][0], L["up"][0], L["gate_up"][0]
    f = cfg.ffn_dim
    assert fw.shape == (4, 2 * f, 128 // 8)
    for e in range(4):
        assert np.array_equal(fw[e, :f], gw[e]) and np.array_equal(fw[e, f:], uw[e])
    # negative control: a wholesale concat of the two [E, ...] tensors, reshaped,
    # misaligns rows (the bug the fused layout warns about)
    wrong = np.concatenate([gw, uw], axis=0).reshape(4, 2 * f, -1)
    assert not np.array_equal(wrong, fw)


def test_page_figures_of_the_layout():
    """The pages' printed sizes, from tests/golden/page_figures.txt."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "page_figures.txt")
    vals = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split("=")
            vals[k.strip()] = float(v)
    c = configs.DECODE
    packed = c.expert_packed_bytes()
    assert abs(packed / 1e6 - vals["expert_mb"]) < 0.05            # "~9.4 MB per expert"
    per_token = 94 * c.top_k * packed
    assert abs(per_token / 1e9 - vals["token_major_gb_per_token"]) < 0.1   # "≈ 7 GB"
    assert abs(c.num_experts * c.d_model / 1e6 - vals["router_macs_m"]) < 0.05  # "~0.5M MACs"
