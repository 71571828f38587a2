"""The token-id frontend on the GPU against the oracle (ncnn port section 1,
Talker and generation-loop bullets; section 8 on built-in voices).

  * qt_embed_ids against oracle.frontend.assemble in float64 on the same
    (bf16-rounded or fp32) weights: 1, 7, 40 and 300 rows, so that the
    ResizeMLP's two projections take the register GEMV, the 8-row and
    row-block matrix-core kernels and the split-activation GEMM; empty
    tracks, codec-only rows, extra rows; bound from the fp32 arithmetic
    (float32 accumulation over K <= 2048 and the hi/lo bf16 split of the
    activations: relative 1e-4 of the row scale);
  * qt_prefill_ids end to end: the oracle assembles the prompt, trailing
    text and tts_pad rows from the same ids and runs its loop; the GPU loop
    is teacher-forced with the oracle's codes (logits and choices under the
    parity rules of test_gpu_parity), at the tiny fp32 shape and at the
    0.6B bf16 shape with the full 151936 x 2048 text embedding;
  * ids out of range are refused before any device work.
"""
import functools

import numpy as np
import pytest

from codec_lm_autoregressive_amd import binding, synth
import oracle
from oracle import frontend
from test_gpu_parity import log, teacher_forced_check

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=2)
def _model(name, dtype):
    dm = synth.dims(name)
    return dm, synth.make_weights(dm, seed=0, dtype=dtype)


@functools.lru_cache(maxsize=2)
def _frontend(name, H, dtype):
    return synth.make_frontend_weights(synth.frontend_dims(name), H, seed=5, dtype=dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_embed_ids_matches_oracle(dtype):
    dm, w = _model("tiny", dtype)
    H = dm["talker"]["hidden"]
    fw = _frontend("tiny", H, dtype)
    V = fw["text_embed"].shape[0]
    eng = binding.Engine(dm, w, dtype, max_batch=1, max_positions=64)
    eng.attach_frontend(fw, max_rows=400)
    g = np.random.default_rng(9)
    for n in (1, 7, 40, 300):
        ti = g.integers(-1, V, n).astype(np.int32)
        ci = g.integers(-1, 3072, n).astype(np.int32)
        ti[0], ci[0] = 17, -1                      # a text-only row
        if n > 1:
            ti[1], ci[1] = -1, 3066                # a codec-only row (a built-in speaker id)
        extra = (g.standard_normal((n, H)) * 0.1).astype(np.float32) if n in (7, 300) else None
        got = eng.embed_ids(ti, ci, extra).cpu().numpy()
        ref = frontend.assemble(ti, ci, fw, w["talker_codec_embed"], extra=extra, dt=np.float64)
        scale = float(np.max(np.abs(ref)))
        err = float(np.max(np.abs(got - ref)))
        log(f"embed_ids {dtype} n={n}: max|d| {err:.2e} (row scale {scale:.2f})")
        assert err <= 1e-4 * max(scale, 1.0), (n, err)
        both_empty = (ti < 0) & (ci < 0)
        if extra is None:
            assert np.all(got[both_empty] == 0.0)
        if n > 1 and extra is None:   # the codec-only row is the codec-table row itself
            np.testing.assert_array_equal(got[1], ref[1].astype(np.float32))
    with pytest.raises(binding.QtError) as e:
        eng.embed_ids(np.array([V], np.int32), np.array([0], np.int32))
    assert e.value.status == binding.QT_E_RANGE
    with pytest.raises(binding.QtError) as e:
        eng.embed_ids(np.array([0], np.int32), np.array([3072], np.int32))
    assert e.value.status == binding.QT_E_RANGE
    eng.close()


def _ids_request(dm, fw, lens, trailing_lens, seed):
    V = fw["text_embed"].shape[0]
    ti, ci = synth.make_prompt_ids(lens, V, seed)
    g = np.random.default_rng(seed + 1)
    tr = g.integers(0, V, int(np.sum(trailing_lens))).astype(np.int32)
    pad_id = int(g.integers(0, V))
    return ti, ci, tr, pad_id


def _oracle_rows(w, fw, ti, ci, tr, pad_id, lens, trailing_lens):
    prompts = frontend.assemble(ti, ci, fw, w["talker_codec_embed"])
    texts = frontend.text_track(tr, fw) if tr.size else np.zeros((0, prompts.shape[1]), np.float32)
    pad = frontend.text_track([pad_id], fw)[0]
    return (synth.split_rows(prompts, lens), synth.split_rows(texts, trailing_lens), pad)


def test_prefill_ids_tiny_fp32_parity():
    dm, w = _model("tiny", "f32")
    fw = _frontend("tiny", dm["talker"]["hidden"], "f32")
    lens = np.array([9, 14], dtype=np.int32)
    tlens = np.array([4, 0], dtype=np.int32)
    ti, ci, tr, pad_id = _ids_request(dm, fw, lens, tlens, 3)
    prompts, texts, pad = _oracle_rows(w, fw, ti, ci, tr, pad_id, lens, tlens)
    eng = binding.Engine(dm, w, "f32", max_batch=2, max_positions=64)
    eng.attach_frontend(fw, max_rows=64)
    samp, psamp = synth.workload("tiny_fp32_b1")["talker"], synth.workload("tiny_fp32_b1")["predictor"]
    teacher_forced_check(eng, w, dm, prompts, lens, pad, samp, psamp, 0, 8, 2e-3, texts=texts,
                         prefill=lambda: eng.prefill_ids(ti, ci, lens, tr, tlens, pad_id, samp, psamp, 0, 8))
    eng.close()


@pytest.mark.timeout(900)
def test_prefill_ids_qwen06b_full_vocabulary_parity():
    """0.6B bf16 talker behind the full-size frontend (151936 x 2048 text
    embedding, ResizeMLP 2048 -> 2048 -> 1024), batch 4 with sampling,
    prompts of 20..90 ids, trailing text on two rows, 4 frames."""
    wl = synth.workload("qwen06b_bf16_b8_sampling")
    dm, w = _model("qwen06b", "bf16")
    log("generating the 151936 x 2048 text embedding")
    fw = _frontend("qwen06b", dm["talker"]["hidden"], "bf16")
    lens = synth.prompt_lengths(4, 20, 90, seed=7)
    tlens = np.array([6, 0, 3, 0], dtype=np.int32)
    ti, ci, tr, pad_id = _ids_request(dm, fw, lens, tlens, 11)
    prompts, texts, pad = _oracle_rows(w, fw, ti, ci, tr, pad_id, lens, tlens)
    eng = binding.Engine(dm, w, "bf16", max_batch=4, max_positions=wl["max_positions"])
    eng.attach_frontend(fw, max_rows=512)
    teacher_forced_check(eng, w, dm, prompts, lens, pad, wl["talker"], wl["predictor"], 0, 4, 5e-2, texts=texts,
                         prefill=lambda: eng.prefill_ids(ti, ci, lens, tr, tlens, pad_id, wl["talker"],
                                                         wl["predictor"], 0, 4))
    eng.close()
