"""Helpers shared by the GPU tests: host<->device marshalling and comparisons.
Oracle inputs come from the seeded generator: the CPU one, or host copies of
the GPU one's bytes (the same bits, which the tests check).  The layer's GPU
results are only ever compared, never fed to the oracle; the one exception is
a token at a provable near-tie of its K-th and (K+1)-th logits, which is given
the GPU's expert set (with the oracle's weights for that set)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
from synth import configs


def dev():
    return torch.device("cuda:0")


def up(a) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev())


def down(t: torch.Tensor) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a


def rel_l2(a, ref) -> float:
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(a - ref) / np.linalg.norm(ref))


def token_errors(out, ref, residual=None):
    """Relative L2 error of the whole [B, d] output and of each token's row
    (fp64).  With a residual, both sides have it subtracted first, so the
    error is measured on what the layer adds."""
    a = np.asarray(out, np.float64)
    r = np.asarray(ref, np.float64)
    if residual is not None:
        a = a - residual
        r = r - residual
    whole = float(np.linalg.norm(a - r) / np.linalg.norm(r))
    per = np.linalg.norm(a - r, axis=-1) / np.linalg.norm(r, axis=-1)
    return whole, per


def assert_layer_close(out, ref, tol, residual=None, what=""):
    """The layer bar: relative L2 <= tol over the whole output AND for every
    token's row (one bad row or lane cannot hide in a large batch)."""
    whole, per = token_errors(out, ref, residual)
    worst = int(np.argmax(per))
    assert whole <= tol, f"{what} whole-output rel L2 {whole:.3e} > {tol}"
    assert per[worst] <= tol, f"{what} token {worst}: rel L2 {per[worst]:.3e} > {tol}"
    return whole, float(per[worst])


def desc_for(smoe, cfg):
    return smoe.make_desc(cfg.d_model, cfg.ffn_dim, cfg.num_experts, cfg.top_k,
                          cfg.norm_topk_prob, cfg.router_bf16, cfg.shared_ffn_dim)


def device_weights(L: dict) -> dict:
    W = {"router": up(L["router"])}
    for k in ("gate", "up", "down", "gate_up"):
        if k in L:
            W[k] = tuple(up(a) for a in L[k])
    if "gate_up" in W:
        del W["gate"], W["up"]
    if "shared" in L:
        S = L["shared"]
        keys = ("gate_up", "down") if "gate_up" in S else ("gate", "up", "down")
        for k in keys:
            W["shared_" + k] = tuple(up(a) for a in S[k])
    return W


def small_config(name, d, E, K, f, B, bf16=True, fused=False, norm=True, shared=0):
    return configs.LayerConfig(name, d, E, K, f, B, router_bf16=bf16, fused=fused,
                               norm_topk_prob=norm, shared_ffn_dim=shared)


def near_tie(logits_row: np.ndarray, K: int) -> bool:
    """True when the oracle's K-th and (K+1)-th logits are within fp32
    rounding noise, so two correct implementations may pick either."""
    s = np.sort(logits_row.astype(np.float64))[::-1]
    if K >= len(s):
        return False
    return (s[K - 1] - s[K]) <= 1e-5 * max(1.0, np.abs(s).max())


def oracle_layer(L, x, cfg, residual=None, idx=None, w=None):
    if idx is None:
        _, idx, w = oracle.route(L["router"], x, cfg.top_k, cfg.norm_topk_prob)
    shared = None
    if "shared" in L:
        shared = (L["shared"]["gate"], L["shared"]["up"], L["shared"]["down"])
    return oracle.moe(L["gate"], L["up"], L["down"], x, idx, w, residual=residual,
                      shared=shared), idx, w
