"""Token-id frontend of the talker: text embedding, ResizeMLP and the
dual-track prompt assembly.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix (ncnn port, section 1 "structure", Talker and generation-
loop bullets; section 8 on built-in voices):
  * text ids index a text embedding table (Qwen2 BPE vocabulary, 2048-wide
    rows); a ResizeMLP 2048 -> 2048 -> talker width with SiLU between the two
    layers maps each row to the talker's width (the text track);
  * every prompt position adds a text-track row and a codec-track row
    position by position; the codec track is the talker's codec embedding of
    a codec id (role / language / think prefixes, codec_bos, codec_pad), and
    a built-in voice's speaker row is the codec embedding of its speaker id,
    placed where an x-vector would go;
  * after the prompt, each frame adds the next trailing text-track row, and
    tts_pad's text-track row once the text is used up.

Readings where the pages are silent: the two MLP layers are affine
(weight and bias; a missing bias is zero); a position may leave a track empty
(id -1), which contributes a zero row; an extra row per position (an x-vector)
may be added on top. Computed in float32 by default (float64 for the pins).
"""
from __future__ import annotations

import numpy as np


def silu(x):
    return x / (x.dtype.type(1) + np.exp(-x))


def resize_mlp(x, fw, dt=np.float32):
    """W2 · silu(W1 · x + b1) + b2 over rows of x."""
    x = np.asarray(x, dtype=dt)
    W1, W2 = np.asarray(fw["fc1_w"], dtype=dt), np.asarray(fw["fc2_w"], dtype=dt)
    b1 = np.zeros(W1.shape[0], dt) if fw.get("fc1_b") is None else np.asarray(fw["fc1_b"], dtype=dt)
    b2 = np.zeros(W2.shape[0], dt) if fw.get("fc2_b") is None else np.asarray(fw["fc2_b"], dtype=dt)
    h = silu(x @ W1.T + b1)
    return h @ W2.T + b2


def text_track(ids, fw, dt=np.float32):
    """ResizeMLP(text_embed[id]) per id; zero rows for id -1."""
    ids = np.asarray(ids, dtype=np.int64)
    E = np.asarray(fw["text_embed"])
    H = np.asarray(fw["fc2_w"]).shape[0]
    out = np.zeros((ids.size, H), dtype=dt)
    keep = ids >= 0
    if keep.any():
        out[keep] = resize_mlp(E[ids[keep]], fw, dt)
    return out


def codec_track(ids, codec_embed, dt=np.float32):
    """talker_codec_embed[id] per id; zero rows for id -1."""
    ids = np.asarray(ids, dtype=np.int64)
    T = np.asarray(codec_embed, dtype=dt)
    out = np.zeros((ids.size, T.shape[1]), dtype=dt)
    keep = ids >= 0
    out[keep] = T[ids[keep]]
    return out


def assemble(text_ids, codec_ids, fw, codec_embed, extra=None, dt=np.float32):
    """Dual-track prompt rows: text track + codec track (+ extra rows), position by position."""
    rows = text_track(text_ids, fw, dt) + codec_track(codec_ids, codec_embed, dt)
    if extra is not None:
        rows = rows + np.asarray(extra, dtype=dt)
    return rows
