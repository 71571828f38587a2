"""Pins of the oracle's token-id frontend (text embedding, ResizeMLP,
dual-track prompt assembly; ncnn port section 1, Talker and generation-loop
bullets, and section 8 on built-in voices).

  * ResizeMLP against torch's nn.Linear -> nn.SiLU -> nn.Linear in float64
    (non-square layers, so a transposed weight fails), with and without
    biases;
  * the text-track gather in closed form: one-hot embedding rows, a scaled
    identity first layer and a permutation second layer make the output of
    id t a known one-hot of height 8 sigma(8) at a known coordinate;
  * the assembly: position-by-position sums, empty tracks (-1) as zero rows,
    a built-in voice's speaker row equal to its codec-table row, extra rows
    (x-vectors) added on top.
"""
import math

import numpy as np
import torch

from oracle import frontend


def _fw(g, V, Tin, Hm, H, bias=True, scale=0.05):
    return dict(text_embed=g.standard_normal((V, Tin)),
                fc1_w=g.standard_normal((Hm, Tin)) * scale, fc1_b=g.standard_normal(Hm) * scale if bias else None,
                fc2_w=g.standard_normal((H, Hm)) * scale, fc2_b=g.standard_normal(H) * scale if bias else None)


def test_resize_mlp_matches_torch():
    g = np.random.default_rng(1)
    for bias in (True, False):
        fw = _fw(g, 50, 64, 96, 48, bias)
        x = g.standard_normal((7, 64))
        mlp = torch.nn.Sequential(torch.nn.Linear(64, 96, bias=bias), torch.nn.SiLU(),
                                  torch.nn.Linear(96, 48, bias=bias)).double()
        with torch.no_grad():
            mlp[0].weight.copy_(torch.from_numpy(fw["fc1_w"]))
            mlp[2].weight.copy_(torch.from_numpy(fw["fc2_w"]))
            if bias:
                mlp[0].bias.copy_(torch.from_numpy(fw["fc1_b"]))
                mlp[2].bias.copy_(torch.from_numpy(fw["fc2_b"]))
            ref = mlp(torch.from_numpy(x)).numpy()
        out = frontend.resize_mlp(x, fw, np.float64)
        assert np.max(np.abs(out - ref)) < 1e-12
    # the 0.6B shape (2048 -> 2048 -> 1024) on a few rows
    fw = _fw(g, 10, 2048, 2048, 1024, True, 0.02)
    x = g.standard_normal((3, 2048))
    mlp = torch.nn.Sequential(torch.nn.Linear(2048, 2048), torch.nn.SiLU(), torch.nn.Linear(2048, 1024)).double()
    with torch.no_grad():
        mlp[0].weight.copy_(torch.from_numpy(fw["fc1_w"]))
        mlp[0].bias.copy_(torch.from_numpy(fw["fc1_b"]))
        mlp[2].weight.copy_(torch.from_numpy(fw["fc2_w"]))
        mlp[2].bias.copy_(torch.from_numpy(fw["fc2_b"]))
        ref = mlp(torch.from_numpy(x)).numpy()
    assert np.max(np.abs(frontend.resize_mlp(x, fw, np.float64) - ref)) < 1e-11


def test_text_track_gather_closed_form():
    V, D = 64, 64
    g = np.random.default_rng(2)
    pi, sig = g.permutation(V), g.permutation(D)
    eye = np.eye(D)
    fw = dict(text_embed=eye[pi], fc1_w=8.0 * eye, fc1_b=None, fc2_w=eye[np.argsort(sig)], fc2_b=None)
    ids = np.array([5, -1, 63, 0, 5])
    out = frontend.text_track(ids, fw, np.float64)
    h = 8.0 / (1.0 + math.exp(-8.0))             # silu(8)
    for i, t in enumerate(ids):
        if t < 0:
            assert np.all(out[i] == 0.0)
            continue
        want = np.zeros(D)
        want[sig[pi[t]]] = h                       # row t -> e_pi(t) -> 8 e_pi(t) -> silu -> W2 row sig^-1
        assert np.max(np.abs(out[i] - want)) < 1e-12


def test_assembly_sums_tracks_position_by_position():
    g = np.random.default_rng(3)
    fw = _fw(g, 40, 32, 48, 16, True)
    codec = g.standard_normal((3072, 16))
    text_ids = np.array([3, 7, -1, 39, -1])
    codec_ids = np.array([-1, 2149, 3066, 2148, -1])   # none, codec_bos, a built-in speaker id, codec_pad, none
    extra = g.standard_normal((5, 16))
    rows = frontend.assemble(text_ids, codec_ids, fw, codec, extra=None, dt=np.float64)
    tt = frontend.resize_mlp(fw["text_embed"][[3, 7, 39]], fw, np.float64)
    np.testing.assert_allclose(rows[0], tt[0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(rows[1], tt[1] + codec[2149], rtol=0, atol=1e-14)
    np.testing.assert_array_equal(rows[2], codec[3066])           # the speaker row is the codec-table row
    np.testing.assert_allclose(rows[3], tt[2] + codec[2148], rtol=0, atol=1e-14)
    np.testing.assert_array_equal(rows[4], np.zeros(16))
    with_x = frontend.assemble(text_ids, codec_ids, fw, codec, extra=extra, dt=np.float64)
    np.testing.assert_allclose(with_x - rows, extra, rtol=0, atol=1e-14)
