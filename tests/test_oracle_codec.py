"""Pins of the oracle's 12 Hz codec decoder (ncnn port section 1, Codec
Decoder bullet; Mizuoto page, codec and frame-streaming bullets).

  * building blocks against library routines in float64: causal and dilated
    convolutions vs torch conv1d with left padding, the causal transposed
    convolution vs torch conv_transpose1d with its tail trimmed, the
    depthwise convolution vs a grouped torch conv1d, LayerNorm and GELU vs
    torch, the window attention vs torch scaled_dot_product_attention with a
    band mask; SnakeBeta by hand values;
  * the window is enforced: keys older than 72 frames do not change a query;
  * dequantisation in closed form (one-hot codebooks, identity projections):
    a wrong codebook index or a mixed-up group fails;
  * causality of the whole decoder: decoding the first t frames gives the
    first t x 1920 samples of the full decode (float64, to rounding);
  * the chunk grid: a request within one chunk is one decode; across the
    300-frame boundary the second chunk is decoded from 25 frames of context
    with their samples dropped;
  * streaming (after 4 frames, then every 12) emits exactly the chunked
    decode's samples, piece by piece.
"""
import numpy as np
import torch
import torch.nn.functional as F

from codec_lm_autoregressive_amd import synth
from oracle import codec as oc

D64 = np.float64


def test_conv_blocks_match_torch():
    g = np.random.default_rng(1)
    x = g.standard_normal((23, 5))
    for k, d in ((7, 1), (7, 3), (7, 9), (1, 1)):
        W = g.standard_normal((k, 6, 5))
        ref = F.conv1d(F.pad(torch.from_numpy(x.T)[None], ((k - 1) * d, 0)),
                       torch.from_numpy(np.transpose(W, (1, 2, 0)).copy()), dilation=d)[0].numpy().T
        np.testing.assert_allclose(oc.conv1d_causal(x, W, d, D64), ref, rtol=0, atol=1e-12)
    for K, s in ((2, 2), (16, 8), (10, 5), (6, 3)):
        W = g.standard_normal((K, 6, 5))
        full = F.conv_transpose1d(torch.from_numpy(x.T)[None],
                                  torch.from_numpy(np.transpose(W, (2, 1, 0)).copy()), stride=s)[0].numpy().T
        np.testing.assert_allclose(oc.conv_transpose_causal(x, W, s, D64), full[:23 * s], rtol=0, atol=1e-12)
    w = g.standard_normal((7, 5))
    ref = F.conv1d(F.pad(torch.from_numpy(x.T)[None], (6, 0)), torch.from_numpy(w.T.copy())[:, None, :],
                   groups=5)[0].numpy().T
    np.testing.assert_allclose(oc.depthwise_causal(x, w, D64), ref, rtol=0, atol=1e-12)


def test_norm_gelu_snake():
    g = np.random.default_rng(2)
    x = g.standard_normal((9, 12))
    ga, be = g.standard_normal(12), g.standard_normal(12)
    ref = F.layer_norm(torch.from_numpy(x), (12,), torch.from_numpy(ga), torch.from_numpy(be), 1e-5).numpy()
    np.testing.assert_allclose(oc.layer_norm(x, ga, be, dt=D64), ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(oc.gelu(x), F.gelu(torch.from_numpy(x)).numpy(), rtol=0, atol=1e-12)
    # SnakeBeta with a = b = 0 (alpha = beta = 1): x + sin(x)^2 / (1 + 1e-9)
    for v in (0.0, 1.0, -2.0, np.pi / 2):
        want = v + np.sin(v) ** 2 / (1.0 + 1e-9)
        assert abs(oc.snake_beta(np.array([[v]]), [0.0], [0.0], D64)[0, 0] - want) < 1e-14
    # alpha = e, beta = e^-1 at x = 1: 1 + sin(e)^2 * e / (1 + 1e-9 e)
    got = oc.snake_beta(np.array([[1.0]]), [1.0], [-1.0], D64)[0, 0]
    assert abs(got - (1.0 + np.sin(np.e) ** 2 / (np.exp(-1.0) + 1e-9))) < 1e-13


def test_window_attention_matches_sdpa_and_is_windowed():
    g = np.random.default_rng(3)
    T, H, d, win = 40, 2, 8, 7
    q, k, v = (g.standard_normal((T, H, d)) for _ in range(3))
    i = np.arange(T)
    band = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - win)
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(a.transpose(1, 0, 2)) for a in (q, k, v)),
                                         attn_mask=torch.from_numpy(band)).numpy().transpose(1, 0, 2)
    out = oc.window_attention(q, k, v, win, D64)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    k2, v2 = k.copy(), v.copy()
    k2[:20] += 5.0
    v2[:20] -= 3.0
    out2 = oc.window_attention(q, k2, v2, win, D64)
    np.testing.assert_array_equal(out2[20 + win - 1:], out[20 + win - 1:])   # keys older than the window
    assert np.abs(out2[20] - out[20]).max() > 1e-3                          # inside the window they matter


def test_dequantize_closed_form():
    cd = synth.codec_dims("tiny")
    C, dim = 64, cd["codebook_dim"]
    rng = np.random.default_rng(4)
    books = np.zeros((16, C, dim))
    for j in range(16):
        books[j, np.arange(C), (np.arange(C) + 3 * j) % dim] = float(j + 1)   # row c of book j: (j+1) e_((c+3j) % dim)
    w = dict(codebooks=books, proj_sem=np.eye(dim), proj_ac=2.0 * np.eye(dim))
    codes = rng.integers(0, C, (5, 16))
    z = oc.dequantize(codes, w, D64)
    for t in range(5):
        want = np.zeros(dim)
        want[(codes[t, 0]) % dim] += 1.0
        for j in range(1, 16):
            want[(codes[t, j] + 3 * j) % dim] += 2.0 * (j + 1)
        np.testing.assert_array_equal(z[t], want)


def _tiny():
    cd = synth.codec_dims("tiny")
    return cd, synth.make_codec_weights(cd, seed=7, dtype="f32")


def test_decoder_is_causal():
    cd, w = _tiny()
    codes = synth.make_codes(11, seed=8)
    hp = oc.hop(cd)
    full = oc.decode(codes, w, cd, D64)
    assert full.shape == (11 * hp,)
    for t in (1, 4, 7):
        part = oc.decode(codes[:t], w, cd, D64)
        np.testing.assert_allclose(part, full[:t * hp], rtol=0, atol=1e-11)
    later = codes.copy()
    later[6:] = (later[6:] + 1) % 2048
    np.testing.assert_allclose(oc.decode(later, w, cd, D64)[:6 * hp], full[:6 * hp], rtol=0, atol=1e-11)


def test_chunk_grid():
    cd, w = _tiny()                      # chunk 12 frames, context 3
    hp, N, ctx = oc.hop(cd), cd["chunk"], cd["context"]
    codes = synth.make_codes(30, seed=9)
    one = synth.make_codes(10, seed=10)
    np.testing.assert_array_equal(oc.decode_chunked(one, w, cd, D64), oc.decode(one, w, cd, D64))
    ch = oc.decode_chunked(codes, w, cd, D64)
    assert ch.shape == (30 * hp,)
    np.testing.assert_array_equal(ch[:N * hp], oc.decode(codes[:N], w, cd, D64))
    second = oc.decode(codes[N - ctx:2 * N], w, cd, D64)[ctx * hp:]
    np.testing.assert_array_equal(ch[N * hp:2 * N * hp], second)
    # the grid is load-bearing: the chunked decode is not one pass over the whole request
    assert np.abs(ch - oc.decode(codes, w, cd, D64)).max() > 1e-6


def test_streaming_emits_the_chunked_decode():
    cd, w = _tiny()
    codes = synth.make_codes(31, seed=11)
    assert oc.stream_schedule(31, 4, 12) == [4, 16, 28, 31]
    pieces = oc.decode_stream(codes, w, cd, 4, 12, D64)
    got = np.concatenate(pieces)
    np.testing.assert_allclose(got, oc.decode_chunked(codes, w, cd, D64), rtol=0, atol=1e-11)
    assert pieces[0].size == 4 * oc.hop(cd)
