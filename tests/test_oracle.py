"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each check uses something other than the oracle's own formulas: original
fp32 weights and the quantiser's error bound, exact integer arithmetic,
library routines in fp64 (numpy matmul, scipy softmax, stable sorts),
closed forms, and the pages' invariants (layer-major equals token-major;
swapping gate and up breaks the result).
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synth
from synth import configs


def bf16_to_f32(h):
    return (np.asarray(h).astype(np.uint32) << 16).view(np.float32)


def unpack(w):
    shifts = np.arange(8, dtype=np.uint32) * 4
    return ((w[..., None] >> shifts) & 0xF).reshape(*w.shape[:-1], w.shape[-1] * 8)


def pack(q):
    q = np.asarray(q, np.uint32)
    w = np.zeros(q.shape[:-1] + (q.shape[-1] // 8,), np.uint32)
    for i in range(8):
        w |= q[..., i::8] << (4 * i)
    return w


def rel_l2(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(a - ref) / np.linalg.norm(ref))


# ----------------------------------------------------------------- dequant
def test_dequant_recovers_original_weights_within_quantiser_bound():
    rng = np.random.default_rng(7)
    W = (rng.standard_normal((40, 320)) * 0.02).astype(np.float32)
    w, s, b = synth.quantize_matrix(W)
    D = oracle.dequant(w, s, b).astype(np.float64)
    S = np.repeat(bf16_to_f32(s), 64, axis=1).astype(np.float64)
    Bv = np.repeat(bf16_to_f32(b), 64, axis=1).astype(np.float64)
    bound = 0.5 * S + 15 * S * 2.0**-8 + np.abs(Bv) * 2.0**-8 + 1e-9
    assert np.all(np.abs(D - W) <= bound)
    # a wrong nibble order or group index would break the bound badly
    assert rel_l2(D, W) < 0.15


def test_dequant_integer_codes_exact():
    rng = np.random.default_rng(3)
    q = rng.integers(0, 16, size=(8, 128))
    s = np.full((8, 2), 0x3F80, np.uint16)          # bf16 1.0
    b = np.full((8, 2), 0xC100, np.uint16)          # bf16 -8.0
    D = oracle.dequant(pack(q), s, b)
    assert np.array_equal(D, (q - 8).astype(np.float32))


# ------------------------------------------------------------- routing
def test_router_logits_match_fp64_matmul():
    cfg = configs.TINY
    Wr = synth.router(0, 0, cfg.num_experts, cfg.d_model, cfg.router_sigma, False)
    x = synth.hidden(0, 0, 0, cfg.batch, cfg.d_model)
    lg = oracle.router_logits(Wr, x)
    ref = x.astype(np.float64) @ Wr.astype(np.float64).T
    assert np.max(np.abs(lg - ref)) < 1e-5 * np.max(np.abs(ref)) * 10
    # bf16 gates are widened exactly
    Wb = synth.router(0, 0, 32, 512, 1 / math.sqrt(512), True)
    xb = synth.hidden(0, 0, 1, 4, 512)
    ref_b = xb.astype(np.float64) @ bf16_to_f32(Wb).astype(np.float64).T
    assert np.max(np.abs(oracle.router_logits(Wb, xb) - ref_b)) < 1e-5


def test_topk_order_ties_and_weights():
    rng = np.random.default_rng(0)
    lg = rng.standard_normal((50, 40)).astype(np.float32)
    lg[0, [3, 9, 17]] = 5.0                          # three-way tie at the top
    lg[1, [30, 2]] = lg[1].max() + 1.0               # tie, higher index listed first
    for norm in (True, False):
        idx, w = oracle.topk_softmax(lg, 6, norm)
        for t in range(lg.shape[0]):
            order = np.lexsort((np.arange(40), -lg[t].astype(np.float64)))
            assert np.array_equal(idx[t], order[:6])
            p = softmax(lg[t].astype(np.float64))
            ref = p[order[:6]] / p[order[:6]].sum() if norm else p[order[:6]]
            assert np.allclose(w[t], ref, rtol=2e-6, atol=0)
        if norm:
            assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
    idx, _ = oracle.topk_softmax(lg, 6, True)
    assert list(idx[0, :3]) == [3, 9, 17] and list(idx[1, :2]) == [2, 30]


def test_topk_all_experts_is_full_softmax():
    rng = np.random.default_rng(1)
    lg = (rng.standard_normal((7, 16)) * 3).astype(np.float32)
    idx, w = oracle.topk_softmax(lg, 16, True)
    for t in range(7):
        p = softmax(lg[t].astype(np.float64))
        assert np.allclose(w[t], p[idx[t]], rtol=2e-6)
        assert sorted(idx[t]) == list(range(16))


def test_weights_of_a_given_set():
    """Weights of an arbitrary K-expert set: scipy's fp64 softmax restricted
    to the set (renormalised or not); for the top-k set, bit for bit the
    top-k weights; a permuted set permutes them; a bad id is rejected."""
    rng = np.random.default_rng(3)
    lg = (rng.standard_normal((20, 48)) * 2).astype(np.float32)
    sets = np.stack([rng.choice(48, 6, replace=False) for _ in range(20)]).astype(np.int32)
    for norm in (True, False):
        w = oracle.weights_of(lg, sets, norm)
        for t in range(20):
            p = softmax(lg[t].astype(np.float64))[sets[t]]
            ref = p / p.sum() if norm else p
            assert np.allclose(w[t], ref, rtol=2e-6, atol=0)
        idx, wt = oracle.topk_softmax(lg, 6, norm)
        assert np.array_equal(oracle.weights_of(lg, idx, norm).view(np.uint32), wt.view(np.uint32))
        # a permuted set permutes the weights (the set's sum is then added in
        # another order: equal up to its rounding)
        perm = sets[:, ::-1].copy()
        assert np.allclose(oracle.weights_of(lg, perm, norm), w[:, ::-1], rtol=1e-6, atol=0)
    assert np.allclose(oracle.weights_of(lg, sets, True).sum(axis=1), 1.0, atol=1e-6)
    bad = sets.copy()
    bad[4, 2] = 48
    with pytest.raises(ValueError):
        oracle.weights_of(lg, bad)


def test_rank_hand_worked_and_definition():
    """Ranked output ("Data Flow": ranked top-(8+spec)): by hand on ties, then
    the definition by brute force on tie-heavy rows (integer logits): the
    expert at rank k is beaten, by a larger logit or an equal one at a lower
    index, by exactly k experts; the first K are the top-K indices."""
    got = oracle.rank(np.array([[1, 3, 3, 2], [0, 0, 0, 0], [-1, 5, -1, 5]], np.float32), 4)
    assert got.tolist() == [[1, 2, 3, 0], [0, 1, 2, 3], [1, 3, 0, 2]]
    rng = np.random.default_rng(7)
    lg = rng.integers(-3, 4, size=(40, 24)).astype(np.float32)
    R = 12
    ranked = oracle.rank(lg, R)
    for t in range(lg.shape[0]):
        l = lg[t]
        assert len(set(ranked[t])) == R
        for k, r in enumerate(ranked[t]):
            beats = sum(1 for j in range(24) if l[j] > l[r] or (l[j] == l[r] and j < r))
            assert beats == k
    idx, _ = oracle.topk_softmax(lg, 5, True)
    assert np.array_equal(ranked[:, :5], idx)


# --------------------------------------------------------------- union
def brute_union(idx, E):
    flat = idx.reshape(-1)
    ue = np.unique(flat)
    lists = [np.flatnonzero(flat == e) for e in ue]
    return ue, lists


@pytest.mark.parametrize("B,K,E", [(1, 8, 128), (8, 4, 16), (64, 8, 128), (37, 8, 256),
                                   (64, 16, 16), (5, 1, 3)])
def test_union_matches_filter(B, K, E):
    rng = np.random.default_rng(B * 1000 + K)
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(B)]).astype(np.int32)
    n, ue, off, pl, pp = oracle.build_union(idx, E)
    bu, lists = brute_union(idx, E)
    assert n == len(bu) and np.array_equal(ue, bu)
    assert off[0] == 0 and off[-1] == B * K
    for u in range(n):
        assert np.array_equal(pl[off[u]:off[u + 1]], lists[u])
    assert np.array_equal(pl[pp], np.arange(B * K))
    if B == 1:
        assert n == K


def test_union_rejects_bad_expert():
    with pytest.raises(ValueError):
        oracle.build_union(np.array([[0, 16]], np.int32), 16)


def test_expected_union_closed_form_monte_carlo():
    for (E, K, B) in [(128, 8, 64), (256, 8, 64), (16, 4, 8)]:
        rng = np.random.default_rng(E + B)
        sizes = []
        for _ in range(300):
            idx = np.stack([rng.choice(E, K, replace=False) for _ in range(B)]).astype(np.int32)
            sizes.append(oracle.build_union(idx, E)[0])
        sizes = np.asarray(sizes, np.float64)
        mu = configs.expected_union(E, K, B)
        assert abs(sizes.mean() - mu) < 3 * sizes.std(ddof=1) / math.sqrt(len(sizes)) + 1e-9
    assert abs(configs.expected_union(128, 8, 64) - 125.94) < 0.01
    assert abs(configs.expected_union(256, 8, 64) - 222.44) < 0.01


# ---------------------------------------------------------- expert FFN
def test_integer_ffn_closed_form():
    """s=1, b=0 codes and small integer inputs: every pre-activation is an
    exact integer, compared with int64 arithmetic."""
    rng = np.random.default_rng(11)
    d, f = 256, 128
    qg = rng.integers(0, 16, (f, d))
    qu = rng.integers(0, 16, (f, d))
    qd = rng.integers(0, 16, (d, f))
    x = rng.integers(-3, 4, d).astype(np.float32)
    one = lambda r, c: np.full((r, c // 64), 0x3F80, np.uint16)
    zero = lambda r, c: np.zeros((r, c // 64), np.uint16)
    Wg = oracle.dequant(pack(qg), one(f, d), zero(f, d))
    Wu = oracle.dequant(pack(qu), one(f, d), zero(f, d))
    Wd = oracle.dequant(pack(qd), one(d, f), zero(d, f))
    g, u, h, y = oracle.expert_ffn(Wg, Wu, Wd, x)
    xi = x.astype(np.int64)
    assert np.array_equal(g.astype(np.int64), qg @ xi)
    assert np.array_equal(u.astype(np.int64), qu @ xi)
    # silu against the logistic function in fp64
    g64, u64 = (qg @ xi).astype(np.float64), (qu @ xi).astype(np.float64)
    h_ref = g64 / (1 + np.exp(-g64)) * u64
    assert np.allclose(h, h_ref, rtol=1e-6, atol=1e-6 * np.abs(h_ref).max())
    assert rel_l2(y, qd.astype(np.float64) @ h.astype(np.float64)) < 1e-6


def brute_force_layer(L, x, K, norm=True, swap_gate_up=False, residual=None):
    """Dense fp64 layer: every expert on every token, masked by top-k."""
    gw, gs, gb = L["gate"]
    uw, us, ub = L["up"]
    dw, ds, db = L["down"]
    if swap_gate_up:
        (gw, gs, gb), (uw, us, ub) = (uw, us, ub), (gw, gs, gb)

    def deq(w, s, b):
        q = unpack(w).astype(np.float64)
        return q * np.repeat(bf16_to_f32(s), 64, -1) + np.repeat(bf16_to_f32(b), 64, -1)

    Wr = L["router"]
    Wr64 = bf16_to_f32(Wr).astype(np.float64) if Wr.dtype == np.uint16 else Wr.astype(np.float64)
    x64 = x.astype(np.float64)
    logits = x64 @ Wr64.T
    E = Wr.shape[0]
    out = np.zeros_like(x64) if residual is None else residual.astype(np.float64).copy()
    for t in range(x.shape[0]):
        order = np.lexsort((np.arange(E), -logits[t]))[:K]
        p = softmax(logits[t])
        wk = p[order] / p[order].sum() if norm else p[order]
        for k, e in enumerate(order):
            g = deq(gw[e], gs[e], gb[e]) @ x64[t]
            u = deq(uw[e], us[e], ub[e]) @ x64[t]
            h = g / (1 + np.exp(-g)) * u
            out[t] += wk[k] * (deq(dw[e], ds[e], db[e]) @ h)
    return out


def test_layer_matches_dense_fp64_brute_force_tiny():
    cfg = configs.TINY
    L = synth.make_layer(cfg)
    x = synth.hidden(cfg.seed, 0, 0, cfg.batch, cfg.d_model)
    _, idx, w = oracle.route(L["router"], x, cfg.top_k)
    out = oracle.moe(L["gate"], L["up"], L["down"], x, idx, w)
    ref = brute_force_layer(L, x, cfg.top_k)
    assert rel_l2(out, ref) < 1e-5
    # negative control from the pages: a gate/up reorder must fail by a wide
    # margin.  With these small pre-activations silu(g)*u ~ g*u/2 is nearly
    # symmetric in g and u, so the swap costs ~37% here rather than the ~100%
    # the pages saw on a trained model; still >100x the 3e-3 tolerance.
    swapped = brute_force_layer(L, x, cfg.top_k, swap_gate_up=True)
    assert rel_l2(swapped, ref) > 0.3


def test_layer_major_equals_token_major_bitwise():
    cfg = configs.LayerConfig("mid", 512, 24, 6, 192, 13, router_bf16=True)
    L = synth.make_layer(cfg)
    x = synth.hidden(cfg.seed, 0, 0, cfg.batch, cfg.d_model)
    res = synth.hidden(cfg.seed, 0, 9, cfg.batch, cfg.d_model, tensor=synth.T_RESIDUAL)
    _, idx, w = oracle.route(L["router"], x, cfg.top_k)
    a, ya = oracle.moe(L["gate"], L["up"], L["down"], x, idx, w, residual=res, return_pairs=True)
    b, yb = oracle.moe(L["gate"], L["up"], L["down"], x, idx, w, residual=res, layer_major=True,
                       return_pairs=True)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32))
    ref = brute_force_layer(L, x, cfg.top_k, residual=res)
    assert rel_l2(a - res, ref - res) < 1e-5


def test_combine_order_and_residual():
    """out = residual + (w0*y0 + w1*y1 + ...), k ascending, checked on a case
    where the fp32 sum order matters."""
    cfg = configs.TINY
    L = synth.make_layer(cfg)
    x = synth.hidden(0, 0, 0, 2, cfg.d_model)
    idx = np.array([[1, 2, 3, 4], [5, 6, 7, 8]], np.int32)
    w = np.array([[1e8, 1.0, -1e8, 0.5], [0.25, 0.25, 0.25, 0.25]], np.float32)
    out, yp = oracle.moe(L["gate"], L["up"], L["down"], x, idx, w, return_pairs=True)
    y = yp.reshape(2, 4, -1)
    for t in range(2):
        acc = np.zeros(cfg.d_model, np.float32)
        for k in range(4):
            acc = (acc + np.float32(w[t, k]) * y[t, k]).astype(np.float32)
        assert np.array_equal(out[t], acc)


# -------------------------------------------------------- shared expert
def _shared_cfg(fs, fused=False):
    return configs.LayerConfig("sh", 256, 12, 3, 128, 5, router_bf16=True, fused=fused,
                               shared_ffn_dim=fs)


def test_shared_ffn_matches_dense_fp64_brute_force():
    """shared_out = Wd_s (silu(Wg_s x) * Wu_s x) on every token, against the
    dequantised weights in fp64; a width unlike the routed one (192 vs 128)
    and a gate/up swap as the negative control."""
    cfg = _shared_cfg(192)
    S = synth.make_shared(cfg)
    x = synth.hidden(cfg.seed, 0, 3, cfg.batch, cfg.d_model)
    got = oracle.shared_ffn(S["gate"], S["up"], S["down"], x)

    def deq(t):
        w, s, b = (a[0] for a in t)
        q = unpack(w).astype(np.float64)
        return q * np.repeat(bf16_to_f32(s), 64, -1) + np.repeat(bf16_to_f32(b), 64, -1)

    Wg, Wu, Wd = deq(S["gate"]), deq(S["up"]), deq(S["down"])
    assert Wg.shape == (192, 256) and Wd.shape == (256, 192)
    x64 = x.astype(np.float64)

    def ffn(A, Bm):
        g, u = x64 @ A.T, x64 @ Bm.T
        return (g / (1 + np.exp(-g)) * u) @ Wd.T

    ref = ffn(Wg, Wu)
    assert rel_l2(got, ref) < 1e-5
    assert rel_l2(ffn(Wu, Wg), ref) > 0.3


def test_shared_with_zero_weights_is_the_routed_layer():
    cfg = _shared_cfg(128)
    L = synth.make_layer(cfg)
    x = synth.hidden(cfg.seed, 0, 0, cfg.batch, cfg.d_model)
    res = synth.hidden(cfg.seed, 0, 9, cfg.batch, cfg.d_model, tensor=synth.T_RESIDUAL)
    _, idx, w = oracle.route(L["router"], x, cfg.top_k)
    zero = {k: tuple(np.zeros_like(a) for a in L["shared"][k]) for k in ("gate", "up", "down")}
    plain = oracle.moe(L["gate"], L["up"], L["down"], x, idx, w, residual=res)
    with_zero = oracle.moe(L["gate"], L["up"], L["down"], x, idx, w, residual=res,
                           shared=(zero["gate"], zero["up"], zero["down"]))
    assert np.array_equal(plain.view(np.uint32), with_zero.view(np.uint32))
    live = oracle.moe(L["gate"], L["up"], L["down"], x, idx, w, residual=res,
                      shared=(L["shared"]["gate"], L["shared"]["up"], L["shared"]["down"]))
    assert rel_l2(live - res, plain - res) > 0.1


def test_shared_copy_of_a_routed_expert_doubles_its_output():
    """With top-1 routing (weight exactly 1) to expert e and a shared expert
    holding e's weights, shared_out equals e's y bit for bit and
    out = residual + 2 y."""
    cfg = configs.LayerConfig("sh1", 256, 12, 1, 128, 4, router_bf16=True, shared_ffn_dim=128)
    L = synth.make_layer(cfg)
    x = synth.hidden(cfg.seed, 0, 1, cfg.batch, cfg.d_model)
    res = synth.hidden(cfg.seed, 0, 2, cfg.batch, cfg.d_model, tensor=synth.T_RESIDUAL)
    e = 7
    idx = np.full((cfg.batch, 1), e, np.int32)
    w = np.ones((cfg.batch, 1), np.float32)
    copy = tuple(tuple(a[e:e + 1] for a in L[k]) for k in ("gate", "up", "down"))
    out, yp = oracle.moe(L["gate"], L["up"], L["down"], x, idx, w, residual=res,
                         return_pairs=True, shared=copy)
    assert np.array_equal(oracle.shared_ffn(*copy, x).view(np.uint32), yp.view(np.uint32))
    assert np.array_equal(out.view(np.uint32), (res + 2 * yp).view(np.uint32))


def test_shared_combine_order():
    """out = residual + (shared_out + routed_out), routed_out formed first:
    with residual 1, shared 2^24 and routed -2^24 only this order gives 1
    ((1 + 2^24) rounds to 2^24 in fp32)."""
    big = np.float32(2.0**24)
    y = np.array([[-big / 2], [-big / 2]], np.float32).reshape(2, 1)   # [B*K, d], K = 2
    w = np.array([[1.0, 1.0]], np.float32)
    out = oracle.combine_shared(y, w, np.array([[big]], np.float32),
                                np.array([[1.0]], np.float32))
    assert out[0, 0] == 1.0
    assert np.float32(np.float32(1.0) + big) + np.float32(-big) == 0.0   # the other order
    # no residual: shared + routed
    out0 = oracle.combine_shared(y, w, np.array([[3.0]], np.float32))
    assert out0[0, 0] == np.float32(3.0) + np.float32(-big)


def test_rmsnorm_closed_form():
    v = np.full((2, 64), 3.0, np.float32)
    v[1] = -2.0
    out = oracle.rmsnorm(v, eps=1e-6)
    assert np.allclose(out[0], 3.0 / math.sqrt(9 + 1e-6), rtol=1e-7)
    assert np.allclose(out[1], -2.0 / math.sqrt(4 + 1e-6), rtol=1e-7)


def test_rmsnorm_epsilon_is_inside_the_root():
    """Rows whose mean square is comparable to eps, where eps moves the
    result by tens of percent: a dropped, misplaced or mis-scaled eps fails.
    Closed forms: a constant row c gives c / sqrt(c^2 + eps); mean square =
    eps exactly gives 1/sqrt(2) of the eps-free value; a zero row gives 0."""
    eps = 1e-6
    c = np.float32(1e-3)
    v = np.zeros((4, 256), np.float32)
    v[0] = c                                             # mean square 1e-6 = eps
    v[1, ::2], v[1, 1::2] = 2e-3, -2e-3                  # mean square 4e-6
    v[2] = 3e-4                                          # eps dominates
    out = oracle.rmsnorm(v, eps=eps)
    exp0 = float(c) / math.sqrt(float(c) ** 2 + eps)
    assert abs(exp0 - 1 / math.sqrt(2)) < 1e-6
    assert np.allclose(out[0], exp0, rtol=2e-6)
    assert np.allclose(out[1, ::2], 2e-3 / math.sqrt(4e-6 + eps), rtol=2e-6)
    assert np.allclose(out[1, 1::2], -2e-3 / math.sqrt(4e-6 + eps), rtol=2e-6)
    assert np.allclose(out[2], 3e-4 / math.sqrt(9e-8 + eps), rtol=2e-6)
    assert np.array_equal(out[3], np.zeros(256, np.float32))
    # eps is used as given: another value gives the other closed form
    out2 = oracle.rmsnorm(v[:1], eps=3e-6)
    assert np.allclose(out2[0], float(c) / math.sqrt(float(c) ** 2 + 3e-6), rtol=2e-6)
    # without eps the constant row would be exactly 1; with it, well below
    assert np.all(out[0] < 0.71)


def test_rmsnorm_random_rows_fp64():
    """Random rows of several scales against the fp64 definition
    x / sqrt(mean(x^2) + eps), within fp32 summation rounding."""
    rng = np.random.default_rng(17)
    d = 1024
    v = (rng.standard_normal((5, d)) * np.array([1e-4, 1e-3, 1.0, 30.0, 1e3])[:, None]).astype(
        np.float32)
    out = oracle.rmsnorm(v, eps=1e-6)
    v64 = v.astype(np.float64)
    ref = v64 / np.sqrt((v64 ** 2).mean(axis=1, keepdims=True) + 1e-6)
    assert np.all(np.abs(out - ref) <= (0.5 * d + 4) * 2.0 ** -24 * np.abs(ref) + 1e-30)
