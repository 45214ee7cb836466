"""Host logic of the stacked harness: union-size and adjacent-step reuse
statistics, pinned by hand-worked cases and by their closed forms under
uniform random routing (Monte Carlo within 3 sigma)."""
import numpy as np
import pytest

import bench
from synth import configs


def test_hand_worked_case():
    # 1 chunk x 2 layers x 3 tokens x K=2
    idx_pre = np.array([[[[0, 1], [1, 2], [0, 2]],
                         [[5, 4], [5, 4], [4, 5]]]], np.int32)
    nu_pre = np.array([[3, 2]], np.int32)
    # 3 decode steps x 2 layers x 1 token x K=2
    idx_dec = np.array([[[[0, 1]], [[4, 5]]],
                        [[[1, 2]], [[4, 5]]],
                        [[[3, 6]], [[5, 7]]]], np.int32)
    s = bench.stack_stats(idx_pre, nu_pre, idx_dec, E=8)
    assert s["prefill_union_mean"] == 2.5
    assert s["prefill_union_min"] == 2 and s["prefill_union_max"] == 3
    # step 1: layer0 {1}/2, layer1 {4,5}/2 -> 0.5, 1.0; step 2: 0, {5}/2 -> 0, 0.5
    assert s["decode_reuse_per_step"] == [0.75, 0.25]
    assert s["decode_reuse_mean"] == pytest.approx(0.5)
    assert s["decode_reuse_expected_uniform"] == 2 / 8


def test_device_count_mismatch_raises():
    idx_pre = np.array([[[[0, 1], [1, 2]]]], np.int32)
    with pytest.raises(RuntimeError):
        bench.stack_stats(idx_pre, np.array([[2]], np.int32), np.zeros((1, 1, 1, 2), np.int32), 8)


def _random_topk(rng, shape, E, K):
    keys = rng.random(shape + (E,))
    return np.argsort(keys, axis=-1)[..., :K].astype(np.int32)


def test_closed_forms_monte_carlo():
    """Uniform independent routing: E[|U|] = E (1 - (1 - K/E)^T) for T tokens,
    and the expected share of a step's experts reused from the step before is
    K/E (hypergeometric mean)."""
    rng = np.random.default_rng(1234)
    E, K, T, C, L, S = 128, 8, 64, 4, 50, 60
    idx_pre = _random_topk(rng, (C, L, T), E, K)
    nu_pre = np.array([[len(np.unique(idx_pre[c, l])) for l in range(L)] for c in range(C)])
    idx_dec = _random_topk(rng, (S, L, 1), E, K)
    s = bench.stack_stats(idx_pre, nu_pre, idx_dec, E)
    n = C * L
    mu_u = configs.expected_union(E, K, T)
    assert s["prefill_union_expected_uniform"] == pytest.approx(mu_u, abs=1e-3)
    # sd of |U| below sqrt(E p (1-p)) (negatively correlated indicators)
    p = (1 - K / E) ** T
    assert abs(s["prefill_union_mean"] - mu_u) <= 3 * np.sqrt(E * p * (1 - p) / n)
    # overlap of two independent K-subsets: hypergeometric, variance below K (K/E)
    m = (S - 1) * L
    sd = np.sqrt(K * (K / E) * (1 - K / E)) / K
    assert abs(s["decode_reuse_mean"] - K / E) <= 3 * sd / np.sqrt(m)
    assert mu_u == pytest.approx(125.94, abs=5e-3)
