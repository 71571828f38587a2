"""Decoder math of the talker and the code predictor, plain numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Both networks are Qwen3-style decoders (Qwen3-TTS ncnn port discussion,
section 1 "structure": 28-layer talker and 5-layer predictor, hidden 1024,
GQA 16/8, head_dim 128, QK-Norm, SwiGLU, RMSNorm, mrope). The layer internals
the pages leave open are read the standard Qwen3 way: pre-norm residual
blocks, no biases, RMSNorm epsilon 1e-6, per-head RMSNorm of q and k before
rotation, rotate-half rope, attention scale 1/sqrt(head_dim), SiLU-gated MLP.

Every function takes a numpy dtype `dt` (float32 by default, float64 for the
pins) and computes in it; weights are cast to it on the way in.
"""
from __future__ import annotations

import math

import numpy as np


def rms_norm(x, gain, eps, dt=np.float32):
    """x * (mean(x^2) + eps)^(-1/2) * gain over the last axis."""
    x = np.asarray(x, dtype=dt)
    ms = np.mean(x * x, axis=-1, keepdims=True, dtype=dt)
    return (x / np.sqrt(ms + dt(eps))) * np.asarray(gain, dtype=dt)


def silu(x):
    return x / (x.dtype.type(1) + np.exp(-x))


def rope_inv_freq(head_dim, theta):
    """theta^(-2i/d), i = 0..d/2-1, evaluated in double and kept in float32.

    The Mizuoto engine page ("Comparison results") notes that inv_freq must stay
    float32 even when the model runs in bf16; a rounded value turns later
    positions by different angles.
    """
    half = head_dim // 2
    return np.array([theta ** (-(2.0 * i) / head_dim) for i in range(half)],
                    dtype=np.float32)


def rope_tables(max_pos, head_dim, theta):
    """cos/sin tables [max_pos, head_dim/2], float32.

    angle = float32(pos) * inv_freq in float32; cos and sin of that float32
    angle evaluated in double and rounded to float32. The table row width is
    head_dim/2 (the ncnn port's section 2 convention for external rope tables).
    """
    inv = rope_inv_freq(head_dim, theta)
    cos = np.empty((max_pos, head_dim // 2), dtype=np.float32)
    sin = np.empty_like(cos)
    for p in range(max_pos):
        ang = np.float32(p) * inv  # float32 product
        for i in range(head_dim // 2):
            a = float(ang[i])
            cos[p, i] = math.cos(a)
            sin[p, i] = math.sin(a)
    return cos, sin


def apply_rope(x, positions, cos, sin, dt=np.float32):
    """Rotate-half rope: pair (i, i + d/2) is turned by angle(pos, i).

    x: [t, heads, d]; positions: [t] ints.
    """
    x = np.asarray(x, dtype=dt)
    d = x.shape[-1]
    h = d // 2
    c = np.asarray(cos, dtype=dt)[positions][:, None, :]
    s = np.asarray(sin, dtype=dt)[positions][:, None, :]
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def apply_mrope(x, pos3, cos, sin, sections, interleaved=False, dt=np.float32):
    """Multimodal rope with three position-id rows (temporal, height, width).

    pos3: [3, t]. Frequency index i takes its angle from position row j, where
    j is the section i falls in (contiguous sections of the given sizes), or
    j = i mod 3 (interleaved form).
    For text and audio rows the three position rows are equal, and this
    reduces to plain rope (ncnn port discussion, section 1, fact 1).
    """
    x = np.asarray(x, dtype=dt)
    d = x.shape[-1]
    h = d // 2
    assert sum(sections) == h
    owner = np.empty(h, dtype=np.int64)
    if interleaved:
        owner[:] = np.arange(h) % 3
    else:
        o = 0
        for j, n in enumerate(sections):
            owner[o:o + n] = j
            o += n
    c = np.empty((x.shape[0], h), dtype=dt)
    s = np.empty_like(c)
    for i in range(h):
        c[:, i] = np.asarray(cos, dtype=dt)[pos3[owner[i]], i]
        s[:, i] = np.asarray(sin, dtype=dt)[pos3[owner[i]], i]
    c = c[:, None, :]
    s = s[:, None, :]
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


class KVCache:
    """Preallocated per-layer key/value storage [layers, kv_heads, max_pos, d]."""

    def __init__(self, layers, n_kv, max_pos, head_dim, dt=np.float32):
        self.k = np.zeros((layers, n_kv, max_pos, head_dim), dtype=dt)
        self.v = np.zeros_like(self.k)


def attention(q, k_all, v_all, q_pos, n_kv, dt=np.float32):
    """Causal GQA attention of t query tokens over the cached keys.

    q: [t, nq, d]; k_all, v_all: [n_kv, L, d]; q_pos: [t]. Query head h reads
    kv head floor(h * n_kv / nq) (repeat_interleave grouping, ncnn port
    section 2); key j is visible to a query at position p iff j <= p.
    Scores are scaled by 1/sqrt(d) and normalised with a float softmax.
    """
    t, nq, d = q.shape
    L = k_all.shape[1]
    scale = dt(1.0 / math.sqrt(d))
    out = np.empty((t, nq, d), dtype=dt)
    visible = np.arange(L)[None, :] <= np.asarray(q_pos)[:, None]  # [t, L]
    for h in range(nq):
        g = (h * n_kv) // nq
        s = (q[:, h, :] @ k_all[g].T) * scale  # [t, L]
        s = np.where(visible, s, dt(-np.inf))
        s = s - np.max(s, axis=1, keepdims=True)
        p = np.exp(s)
        p = p / np.sum(p, axis=1, keepdims=True)
        out[:, h, :] = p @ v_all[g]
    return out


def decoder_layer(lw, x, cache, layer, positions, dm, cos, sin, dt=np.float32):
    """One pre-norm decoder layer over t tokens; writes their K/V into the cache."""
    nq, nkv, d = dm["n_heads"], dm["n_kv_heads"], dm["head_dim"]
    eps = dm["rms_eps"]
    t = x.shape[0]
    a = rms_norm(x, lw["attn_norm"], eps, dt)
    q = (a @ np.asarray(lw["wq"], dtype=dt).T).reshape(t, nq, d)
    k = (a @ np.asarray(lw["wk"], dtype=dt).T).reshape(t, nkv, d)
    v = (a @ np.asarray(lw["wv"], dtype=dt).T).reshape(t, nkv, d)
    q = rms_norm(q, lw["q_norm"], eps, dt)          # QK-Norm: before rotation
    k = rms_norm(k, lw["k_norm"], eps, dt)
    q = apply_rope(q, positions, cos, sin, dt)
    k = apply_rope(k, positions, cos, sin, dt)
    for i, p in enumerate(positions):
        cache.k[layer, :, p, :] = k[i]
        cache.v[layer, :, p, :] = v[i]
    L = int(np.max(positions)) + 1
    o = attention(q, cache.k[layer, :, :L], cache.v[layer, :, :L], positions, nkv, dt)
    x = x + o.reshape(t, nq * d) @ np.asarray(lw["wo"], dtype=dt).T
    m = rms_norm(x, lw["mlp_norm"], eps, dt)
    g = m @ np.asarray(lw["w_gate"], dtype=dt).T
    u = m @ np.asarray(lw["w_up"], dtype=dt).T
    x = x + (silu(g) * u) @ np.asarray(lw["w_down"], dtype=dt).T
    return x


def decoder_forward(layers, final_norm, x, cache, p0, dm, cos, sin, dt=np.float32):
    """Run t new tokens at positions p0..p0+t-1 through all layers.

    Returns the final-RMSNorm'd hidden states [t, H] (the decoder module's
    output in the ncnn port, section 4 wrapper: layers then norm).
    """
    x = np.asarray(x, dtype=dt)
    positions = np.arange(p0, p0 + x.shape[0])
    for i, lw in enumerate(layers):
        x = decoder_layer(lw, x, cache, i, positions, dm, cos, sin, dt)
    return rms_norm(x, final_norm, dm["rms_eps"], dt)


def decoder_recompute(layers, final_norm, x_all, dm, cos, sin, dt=np.float32):
    """All tokens from position 0 at once in a fresh cache (no reuse)."""
    cache = KVCache(len(layers), dm["n_kv_heads"], x_all.shape[0], dm["head_dim"], dt)
    return decoder_forward(layers, final_norm, x_all, cache, 0, dm, cos, sin, dt)
