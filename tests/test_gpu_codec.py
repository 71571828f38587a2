"""The 12 Hz codec decoder on the GPU against the oracle (ncnn port section 1,
Codec Decoder bullet; Mizuoto page, codec and frame-streaming bullets).

The oracle runs in float64 on the same weights (bf16-rounded for bf16). The
GPU computes in float32 with every linear map and convolution on the
projection kernels (bf16 hi + lo activations against exact bf16 weights, or
fp32 FMA), so the two agree to float32 rounding accumulated over the ~45
layers of the path; the bar is an SNR of at least 70 dB and max |d| <= 2e-4
on samples in [-1, 1] (tanh output).

  * one causal pass at the tiny shape (fp32 and bf16 weights) for 1, 5 and 15
    frames (the last = chunk + context) and at the full shape (hidden 512,
    8 layers, channels 1536 .. 96, x1920) for 6 frames;
  * the chunk grid: at the tiny shape over 31 frames (three chunks) against
    the oracle's chunked decode; at the full shape over 305 frames, the first
    frames of chunk 0 and the 5 frames of chunk 1 (decoded from 25 frames of
    context) against the oracle's decodes of those spans;
  * streaming: steps after 4 frames and then every 12 return, piece by piece,
    the chunked decode;
  * codes out of range are refused before any device work.
"""
import functools

import numpy as np
import pytest

from codec_lm_autoregressive_amd import binding, synth
from oracle import codec as oc
from test_gpu_parity import log

pytestmark = pytest.mark.gpu


def snr_db(got, ref):
    err = np.sum((got - ref) ** 2)
    return float("inf") if err == 0 else 10 * np.log10(np.sum(ref ** 2) / err)


def check(got, ref, what):
    s = snr_db(got, ref)
    m = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    log(f"{what}: {ref.size} samples, SNR {s:.1f} dB, max|d| {m:.2e}")
    assert s >= 70.0 and m <= 2e-4, (what, s, m)


@functools.lru_cache(maxsize=3)
def _model(name, dtype):
    cd = synth.codec_dims(name)
    return cd, synth.make_codec_weights(cd, seed=3, dtype=dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_codec_decode_tiny(dtype):
    cd, w = _model("tiny", dtype)
    cod = binding.Codec(cd, w, dtype)
    for T in (1, 5, cd["chunk"] + cd["context"]):
        codes = synth.make_codes(T, seed=T)
        got = cod.decode(codes).cpu().numpy()
        check(got, oc.decode(codes, w, cd, np.float64), f"tiny {dtype} decode T={T}")
    with pytest.raises(binding.QtError) as e:
        cod.decode(synth.make_codes(cd["chunk"] + cd["context"] + 1, seed=1))
    assert e.value.status == binding.QT_E_CAPACITY
    bad = synth.make_codes(3, seed=2)
    bad[1, 7] = cd["codebook"]
    with pytest.raises(binding.QtError) as e:
        cod.decode(bad)
    assert e.value.status == binding.QT_E_RANGE
    cod.close()


def test_codec_chunked_and_streaming_tiny():
    cd, w = _model("tiny", "bf16")
    cod = binding.Codec(cd, w, "bf16")
    T = 31
    codes = synth.make_codes(T, seed=9)
    ref = oc.decode_chunked(codes, w, cd, np.float64)
    got = cod.decode_chunked(codes).cpu().numpy()
    check(got, ref, "tiny chunked T=31")
    pieces, sent = [], 0
    for n in oc.stream_schedule(T, 4, 12):
        p = cod.stream_step(codes[:n], sent).cpu().numpy()
        pieces.append(p)
        sent += p.size
    assert [p.size for p in pieces] == [4 * cod.hop, 12 * cod.hop, 12 * cod.hop, 3 * cod.hop]
    check(np.concatenate(pieces), ref, "tiny streamed T=31")
    cod.close()


@pytest.mark.timeout(900)
def test_codec_full_shape():
    cd, w = _model("12hz", "bf16")
    log("codec 12 Hz: weights ready")
    cod = binding.Codec(cd, w, "bf16")
    hp = cod.hop
    assert hp == 1920
    codes = synth.make_codes(6, seed=5)
    check(cod.decode(codes).cpu().numpy(), oc.decode(codes, w, cd), "12hz decode T=6")
    # chunk grid over 305 frames: chunk 0's first 8 frames, all of chunk 1
    T = 305
    codes = synth.make_codes(T, seed=6)
    got = cod.decode_chunked(codes).cpu().numpy()
    assert got.shape == (T * hp,)
    check(got[:8 * hp], oc.decode(codes[:8], w, cd), "12hz chunk 0, frames 0..7")
    s0 = cd["chunk"] - cd["context"]
    check(got[cd["chunk"] * hp:], oc.decode(codes[s0:T], w, cd)[cd["context"] * hp:], "12hz chunk 1 (25-frame context)")
    # streaming inside chunk 0: after 4 frames, then every 12, up to 40
    pieces, sent = [], 0
    for n in oc.stream_schedule(40, 4, 12):
        p = cod.stream_step(codes[:n], sent).cpu().numpy()
        pieces.append(p)
        sent += p.size
    check(np.concatenate(pieces), oc.decode(codes[:40], w, cd), "12hz streamed 40 frames")
    cod.close()
