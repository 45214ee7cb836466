"""Plain CPU reference for the attention block around the routed MoE layer.

TEST INFRASTRUCTURE ONLY, like the rest of oracle/: nothing in the product
library calls, links or loads this code; only the tests, the smoke check and
the benchmark's CPU-baseline leg do.  It shares no code with the GPU library.

numpy in float64.  Values are rounded to bf16 (round to nearest even) exactly
where the method stores bf16: the inputs of the two bf16 matrix-vector
products and the K/V entries of the cache.

The block, in the pages' order ("Data Flow", the layer loop; "Layer-Major
Batched Prefill", "Choreography Per Chunk", steps 1-4; "Surface Scout", the
model config and "KV-Cache"):
  1. RMS norm of the hidden state (input_layernorm; unit gain);
  2. Q, K and V projections, one bf16 matrix-vector product per token;
  3. per head, RMS norm of q and of k (the QK-norm; unit gain), then RoPE at
     the token's absolute stream position, the angle depending on position
     and dimension only;
  4. K and V appended to the layer's KV ring, slot = position mod ctx;
  5. causal GQA attention: query head h reads key/value head h // (H / Hkv),
     over the cached positions at or before its own (the ring holds the last
     ctx positions of the call);
  6. O projection (bf16 matrix-vector product) added to the residual.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class AttnConfig:
    d_model: int
    num_heads: int
    num_kv_heads: int
    head_dim: int = 128
    ctx: int = 4096
    rope_theta: float = 1.0e6
    eps: float = 1e-6

    @property
    def q_dim(self) -> int:
        return self.num_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.num_kv_heads * self.head_dim

    @property
    def qkv_rows(self) -> int:
        return self.q_dim + 2 * self.kv_dim


def bf16_round(a) -> np.ndarray:
    """float32 -> nearest bf16 (ties to even), returned as float64."""
    f = np.asarray(a, np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def bf16_bits_to_f64(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rmsnorm(v: np.ndarray, eps: float) -> np.ndarray:
    """v / sqrt(mean(v^2) + eps) over the last axis, unit gain."""
    v = np.asarray(v, np.float64)
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)


def rope(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotation of each pair (x_i, x_{i + hd/2}) by pos * theta^(-2i/hd)
    (the rotate-half pairing); x [..., hd]."""
    hd = x.shape[-1]
    half = hd // 2
    i = np.arange(half, dtype=np.float64)
    ang = pos * theta ** (-2.0 * i / hd)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def new_cache(cfg: AttnConfig):
    """Empty K and V rings, [Hkv, ctx, hd] each."""
    shape = (cfg.num_kv_heads, cfg.ctx, cfg.head_dim)
    return np.zeros(shape, np.float64), np.zeros(shape, np.float64)


def qkv_rows(cfg: AttnConfig, Wqkv_bits: np.ndarray, x: np.ndarray, pos0: int):
    """Steps 1-3 for tokens at positions pos0, pos0+1, ...: q [B, H, hd] after
    QK-norm and RoPE, k [B, Hkv, hd] likewise, v [B, Hkv, hd]."""
    W = bf16_bits_to_f64(Wqkv_bits)
    xb = bf16_round(rmsnorm(x, cfg.eps).astype(np.float32))
    qkv = xb @ W.T
    B = x.shape[0]
    H, G, hd = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim
    q = qkv[:, :cfg.q_dim].reshape(B, H, hd)
    k = qkv[:, cfg.q_dim:cfg.q_dim + cfg.kv_dim].reshape(B, G, hd)
    v = qkv[:, cfg.q_dim + cfg.kv_dim:].reshape(B, G, hd)
    q = rmsnorm(q, cfg.eps)
    k = rmsnorm(k, cfg.eps)
    for t in range(B):
        q[t] = rope(q[t], pos0 + t, cfg.rope_theta)
        k[t] = rope(k[t], pos0 + t, cfg.rope_theta)
    return q, k, v


def attend(cfg: AttnConfig, q: np.ndarray, k_cache, v_cache, pos: int, lo: int) -> np.ndarray:
    """Step 5 for one token at `pos`: every head over cached positions lo..pos
    (each in slot position mod ctx); returns o [H * hd]."""
    H, G, hd = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim
    group = H // G
    slots = np.arange(lo, pos + 1) % cfg.ctx
    o = np.empty((H, hd), np.float64)
    for h in range(H):
        g = h // group
        K = k_cache[g, slots]
        V = v_cache[g, slots]
        s = K @ q[h] / math.sqrt(hd)
        p = np.exp(s - s.max())
        o[h] = (p / p.sum()) @ V
    return o.reshape(H * hd)


def attention_block(cfg: AttnConfig, Wqkv_bits, Wo_bits, x, pos0: int, k_cache, v_cache):
    """The block for B tokens at positions pos0 .. pos0+B-1 (a decode step or a
    chunk); appends their K/V to the rings in place and returns
    out [B, d] = x + O (attention)."""
    x = np.asarray(x, np.float32)
    B = x.shape[0]
    q, k, v = qkv_rows(cfg, Wqkv_bits, x, pos0)
    for t in range(B):                      # all of the call's K/V first (step 4)
        slot = (pos0 + t) % cfg.ctx
        k_cache[:, slot] = bf16_round(k[t].astype(np.float32))
        v_cache[:, slot] = bf16_round(v[t].astype(np.float32))
    p_last = pos0 + B - 1
    lo = max(0, p_last - cfg.ctx + 1)       # the ring holds the last ctx positions
    Wo = bf16_bits_to_f64(Wo_bits)
    out = np.empty((B, cfg.d_model), np.float64)
    for t in range(B):
        o = attend(cfg, q[t], k_cache, v_cache, pos0 + t, lo)
        out[t] = x[t].astype(np.float64) + Wo @ bf16_round(o.astype(np.float32))
    return out
