"""The 12 Hz codec decoder: 16 codes per frame -> 1920 samples of 24 kHz audio.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix (ncnn port, section 1 "structure", Codec Decoder bullet;
Mizuoto Qwen3-TTS page, "Matching upstream" codec bullet and "Speed"
frame-streaming bullet):
  * SplitRVQ dequantisation of 16 codebooks of 2048 x 256; code 0 is the
    semantic code, codes 1..15 the acoustic ones (the ncnn codec module takes
    them as two inputs);
  * an 8-layer transformer, hidden 512, head_dim 64, rope theta 1e4,
    LayerScale, whose attention sees a 72-frame window;
  * two (transposed convolution + ConvNeXt) upsampling stages;
  * a DAC-style vocoder with SnakeBeta activations (parameters stored in log
    space and exponentiated), upsampling by 8, 5, 4 and 3: x1920 overall;
  * one feed-forward pass, causal throughout;
  * decoding runs in chunks of 300 frames, each with 25 frames of left
    context whose samples are dropped;
  * streaming decodes after 4 frames and then every 12, each time from the
    current chunk's regular start, and emits the samples not emitted yet.

Readings where the pages are silent (each one a plain choice the rest
supports): the two codebook groups are summed separately and each projected
256 -> 512 by its own linear map, the projections added; pre-norm transformer
blocks with LayerNorm (gain and bias, eps 1e-5) and a 512 -> 2048 -> 512 GELU
(erf) MLP, no biases in the linear maps, rotate-half rope at chunk-local
positions 0.. , window: query t sees keys t-71 .. t; LayerScale = a gain per
channel on each residual branch; a final LayerNorm; upsampling stage = causal
transposed convolution (kernel 2, stride 2) then a ConvNeXt block (depthwise
causal convolution, kernel 7 -> LayerNorm -> 512 -> 2048 -> 512 GELU MLP ->
LayerScale -> residual); vocoder = causal convolution (kernel 7) to 1536
channels, four blocks (SnakeBeta -> causal transposed convolution, kernel
2 x stride, channels halved -> three residual units with dilations 1, 3, 9:
SnakeBeta -> causal dilated convolution kernel 7 -> SnakeBeta -> convolution
kernel 1 -> residual add), SnakeBeta, causal convolution kernel 7 to one
channel, tanh. SnakeBeta(x) = x + sin(e^a x)^2 / (e^b + 1e-9) per channel.
Causal convolution: output t sees inputs t - (k-1) d .. t (zeros before the
start); causal transposed convolution with stride s and kernel K (2 in the
upsampling stages, 2 s in the vocoder): output m s + p = sum_i W_(p + i s)
x[m - i] (the last K - s outputs of the full transposed convolution
trimmed). Convolution weights are stored tap-major,
[k][out][in]. Computed in float32 by default (float64 for the pins).
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

from . import model


def layer_norm(x, g, b, eps=1e-5, dt=np.float32):
    x = np.asarray(x, dtype=dt)
    mu = np.mean(x, axis=-1, keepdims=True, dtype=dt)
    var = np.mean((x - mu) * (x - mu), axis=-1, keepdims=True, dtype=dt)
    return (x - mu) / np.sqrt(var + dt(eps)) * np.asarray(g, dtype=dt) + np.asarray(b, dtype=dt)


def gelu(x):
    return (0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))).astype(x.dtype)


def snake_beta(x, a, b, dt=np.float32):
    """x + sin(e^a x)^2 / (e^b + 1e-9), per channel (last axis)."""
    x = np.asarray(x, dtype=dt)
    alpha = np.exp(np.asarray(a, dtype=dt))
    beta = np.exp(np.asarray(b, dtype=dt))
    s = np.sin(alpha * x)
    return x + s * s / (beta + dt(1e-9))


def conv1d_causal(x, W, dilation=1, dt=np.float32):
    """x [T, Cin], W [k, Cout, Cin] -> [T, Cout]; tap j reads x[t - (k-1-j) d]."""
    x = np.asarray(x, dtype=dt)
    W = np.asarray(W, dtype=dt)
    k = W.shape[0]
    T = x.shape[0]
    out = np.zeros((T, W.shape[1]), dtype=dt)
    for j in range(k):
        sh = (k - 1 - j) * dilation
        if sh >= T:
            continue
        out[sh:] += x[:T - sh] @ W[j].T
    return out


def conv_transpose_causal(x, W, stride, dt=np.float32):
    """x [T, Cin], W [K, Cout, Cin] with K a multiple of the stride s ->
    [T s, Cout]: output m s + p = sum_i W_(p + i s) x[m - i] (x before the
    start is zero): the transposed convolution with its last K - s outputs
    trimmed."""
    x = np.asarray(x, dtype=dt)
    W = np.asarray(W, dtype=dt)
    s = stride
    K, T = W.shape[0], x.shape[0]
    y = np.zeros((T, s, W.shape[1]), dtype=dt)
    for p in range(s):
        for i in range(K // s):
            if i >= T:
                break
            y[i:, p] += x[:T - i] @ W[p + i * s].T
    return y.reshape(T * s, W.shape[1])


def depthwise_causal(x, w, dt=np.float32):
    """x [T, C], w [k, C]: out[t, c] = sum_j w[j, c] x[t - (k-1-j), c]."""
    x = np.asarray(x, dtype=dt)
    w = np.asarray(w, dtype=dt)
    k = w.shape[0]
    T = x.shape[0]
    out = np.zeros_like(x)
    for j in range(k):
        sh = k - 1 - j
        if sh >= T:
            continue
        out[sh:] += x[:T - sh] * w[j]
    return out


def dequantize(codes, w, dt=np.float32):
    """codes [T, 16] -> [T, hidden]: W_s C_0[c_0] + W_a sum_{j>=1} C_j[c_j]."""
    codes = np.asarray(codes)
    C = np.asarray(w["codebooks"], dtype=dt)            # [16, codebook, dim]
    sem = C[0][codes[:, 0]]
    ac = np.zeros_like(sem)
    for j in range(1, C.shape[0]):
        ac = ac + C[j][codes[:, j]]
    return sem @ np.asarray(w["proj_sem"], dtype=dt).T + ac @ np.asarray(w["proj_ac"], dtype=dt).T


def window_attention(q, k, v, window, dt=np.float32):
    """q, k, v [T, heads, d] (rotated): query t attends keys t-window+1 .. t."""
    T, H, d = q.shape
    out = np.zeros_like(q)
    sc = dt(1.0 / np.sqrt(d))
    for t in range(T):
        j0 = max(0, t - window + 1)
        s = np.einsum("hd,jhd->hj", q[t], k[j0:t + 1]) * sc
        s = s - np.max(s, axis=1, keepdims=True)
        p = np.exp(s)
        p = p / np.sum(p, axis=1, keepdims=True)
        out[t] = np.einsum("hj,jhd->hd", p, v[j0:t + 1])
    return out


def transformer(x, w, cd, dt=np.float32):
    x = np.asarray(x, dtype=dt)
    T = x.shape[0]
    H, d = cd["heads"], cd["head_dim"]
    cos, sin = model.rope_tables(max(T, 1), d, cd["rope_theta"])
    pos = np.arange(T)
    for lw in w["layers"]:
        a = layer_norm(x, lw["ln1_g"], lw["ln1_b"], dt=dt)
        qkv = a @ np.asarray(lw["wqkv"], dtype=dt).T
        q = model.apply_rope(qkv[:, :H * d].reshape(T, H, d), pos, cos, sin, dt)
        k = model.apply_rope(qkv[:, H * d:2 * H * d].reshape(T, H, d), pos, cos, sin, dt)
        v = qkv[:, 2 * H * d:].reshape(T, H, d)
        o = window_attention(q, k, v, cd["window"], dt).reshape(T, H * d)
        x = x + np.asarray(lw["ls1"], dtype=dt) * (o @ np.asarray(lw["wo"], dtype=dt).T)
        m = layer_norm(x, lw["ln2_g"], lw["ln2_b"], dt=dt)
        h = gelu(m @ np.asarray(lw["fc1"], dtype=dt).T)
        x = x + np.asarray(lw["ls2"], dtype=dt) * (h @ np.asarray(lw["fc2"], dtype=dt).T)
    return layer_norm(x, w["ln_f_g"], w["ln_f_b"], dt=dt)


def convnext(x, bw, dt=np.float32):
    h = depthwise_causal(x, bw["dw"], dt)
    h = layer_norm(h, bw["ln_g"], bw["ln_b"], dt=dt)
    h = gelu(h @ np.asarray(bw["fc1"], dtype=dt).T)
    h = h @ np.asarray(bw["fc2"], dtype=dt).T
    return x + np.asarray(bw["gamma"], dtype=dt) * h


def vocoder(x, w, cd, dt=np.float32):
    x = conv1d_causal(x, w["voc_in"], 1, dt)
    for bw, s in zip(w["voc_blocks"], cd["strides"]):
        x = snake_beta(x, bw["snake_a"], bw["snake_b"], dt)
        x = conv_transpose_causal(x, bw["up"], s, dt)
        for uw, dil in zip(bw["units"], cd["dilations"]):
            h = snake_beta(x, uw["a1"], uw["b1"], dt)
            h = conv1d_causal(h, uw["conv7"], dil, dt)
            h = snake_beta(h, uw["a2"], uw["b2"], dt)
            x = x + conv1d_causal(h, uw["conv1"], 1, dt)
    x = snake_beta(x, w["voc_out_a"], w["voc_out_b"], dt)
    y = conv1d_causal(x, w["voc_out"], 1, dt)
    return np.tanh(y[:, 0])


def decode(codes, w, cd, dt=np.float32):
    """One causal pass over codes [T, 16] (positions from 0): audio [T * hop]."""
    z = dequantize(codes, w, dt)
    x = transformer(z, w, cd, dt)
    for uw in w["up_blocks"]:
        x = conv_transpose_causal(x, uw["up"], 2, dt)
        x = convnext(x, uw, dt)
    return vocoder(x, w, cd, dt)


def hop(cd):
    return 4 * int(np.prod(cd["strides"]))


def decode_chunked(codes, w, cd, dt=np.float32):
    """The chunk grid: chunk c covers frames [c N, c N + N), decoded from
    frame max(0, c N - ctx) with the context's samples dropped."""
    codes = np.asarray(codes)
    T, N, ctx, hp = codes.shape[0], cd["chunk"], cd["context"], hop(cd)
    out = []
    for c0 in range(0, T, N):
        s0 = max(0, c0 - ctx)
        a = decode(codes[s0:min(T, c0 + N)], w, cd, dt)
        out.append(a[(c0 - s0) * hp:])
    return np.concatenate(out) if out else np.zeros(0, dt)


def stream_schedule(T, first=4, every=12):
    """Frame counts at which streaming decodes: first, first + every, ...,
    and the final count T (the end of the request)."""
    marks = []
    n = first
    while n < T:
        marks.append(n)
        n += every
    marks.append(T)
    return marks


def decode_stream(codes, w, cd, first=4, every=12, dt=np.float32):
    """Streaming decode: at each mark n, decode the current chunk from its
    regular start (with context) up to frame n and emit the samples not
    emitted before. Returns the list of emitted pieces."""
    codes = np.asarray(codes)
    N, ctx, hp = cd["chunk"], cd["context"], hop(cd)
    sent = 0
    pieces = []
    for n in stream_schedule(codes.shape[0], first, every):
        while sent < n * hp:
            c0 = (sent // hp) // N * N            # the chunk that holds the next unsent sample
            s0 = max(0, c0 - ctx)
            end = min(n, c0 + N)
            a = decode(codes[s0:end], w, cd, dt)
            piece = a[sent - s0 * hp:]
            pieces.append(piece)
            sent += piece.size
    return pieces
