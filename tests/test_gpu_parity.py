"""End-to-end parity of the HIP frame loop with the oracle, through the C ABI.

Rules (spec tolerances): raw logits max|d| <= 2e-3 for fp32 weights,
<= 5e-2 for bf16 weights (the oracle holds the same bf16-rounded weights in
fp32 with fp32 accumulation); teacher-forced choices agree 100 % except where
the oracle's decision margin is below that tolerance (greedy: top-2 gap of the
processed logits; sampling: the race gap in logit units, or the top-k / top-p
cut within reach). Integer work (frame counts, stop reasons, code ranges,
determinism, graph replay vs eager) is exact.
"""
import functools
import sys

import numpy as np
import pytest

from codec_lm_autoregressive_amd import binding, synth
import oracle

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=2)
def weights(model, dtype, seed=0):
    return synth.make_weights(synth.dims(model), seed=seed, dtype=dtype)


def margins_exempt(info, tol):
    return info["margin"] < tol or info.get("topp_gap", np.inf) < tol


def teacher_forced_check(eng, w, dm, prompts, lens, pad, tsamp, psamp, seed, frames, tol, rows=None, texts=None,
                         text_packed=None, text_lens=None):
    """Oracle free run -> force its codes into the GPU loop, compare logits and choices."""
    B = len(lens)
    rows = list(range(B)) if rows is None else rows
    ref = oracle.generate(w, dm, [prompts[r] for r in rows], pad, tsamp, psamp, seed, frames, rows=rows,
                          texts=None if texts is None else [texts[r] for r in rows])
    eng.prefill(np.concatenate(prompts), lens, pad, tsamp, psamp, seed, frames, text=text_packed,
                text_lens=text_lens)
    tl0 = eng.talker_logits()
    worst = 0.0
    n_cmp = n_exempt = 0
    for j, r in enumerate(rows):
        d = float(np.max(np.abs(tl0[r] - ref[j]["talker_logits"][0])))
        worst = max(worst, d)
    F = max(x["n_frames"] for x in ref)
    for k in range(F):
        forced = np.zeros((B, 16), dtype=np.int32)
        forced[:, 0] = dm["eos_id"]
        for j, r in enumerate(rows):
            if k < ref[j]["n_frames"]:
                forced[r] = ref[j]["codes"][k]
        tl, pl, ch = eng.step_forced(forced)
        for j, r in enumerate(rows):
            x = ref[j]
            if k >= x["n_frames"]:
                continue
            worst = max(worst, float(np.max(np.abs(pl[r] - x["pred_logits"][k]))))
            worst = max(worst, float(np.max(np.abs(tl[r] - x["talker_logits"][k + 1]))))
            for s in range(15):
                n_cmp += 1
                if ch[r, s + 1] != x["pred_choice"][k][s]:
                    assert margins_exempt(x["pred_info"][k][s], tol), (r, k, s, ch[r, s + 1], x["pred_choice"][k][s],
                                                                       x["pred_info"][k][s])
                    n_exempt += 1
            n_cmp += 1
            if ch[r, 0] != x["talker_choice"][k + 1]:
                assert margins_exempt(x["talker_info"][k + 1], tol), (r, k, ch[r, 0], x["talker_choice"][k + 1])
                n_exempt += 1
    log(f"teacher-forced: {F} frames, max|dlogit| {worst:.3e} (tol {tol}), choices {n_cmp - n_exempt}/{n_cmp} equal")
    assert worst <= tol, worst
    return ref, worst


def test_tiny_fp32_greedy_parity():
    wl = synth.workload("tiny_fp32_b1")
    dm = synth.dims(wl["model"])
    w = weights(wl["model"], "f32")
    lens = synth.prompt_lengths(1, *wl["prompt"], seed=2)
    prompts = synth.split_rows(synth.make_prompts(lens, dm["talker"]["hidden"], seed=1), lens)
    pad = synth.make_tts_pad(dm["talker"]["hidden"], seed=3)
    eng = binding.Engine(dm, w, "f32", max_batch=1, max_positions=wl["max_positions"])
    codes, n, fin = eng.generate(np.concatenate(prompts), lens, pad, wl["talker"], wl["predictor"], 0, wl["frames"])
    ref = oracle.generate(w, dm, prompts, pad, wl["talker"], wl["predictor"], 0, wl["frames"])[0]
    assert int(n[0]) == ref["n_frames"]
    assert {1: "stop", 2: "length"}[int(fin[0])] == ref["finish"]
    np.testing.assert_array_equal(codes[0, :ref["n_frames"]], ref["codes"])
    teacher_forced_check(eng, w, dm, prompts, lens, pad, wl["talker"], wl["predictor"], 0, wl["frames"], 2e-3)
    eng.close()


@pytest.mark.parametrize("kv", ["bf16", "f16"])
def test_tiny_bf16_parity(kv):
    """head_dim 64, bf16 weights, a bf16 or fp16 KV cache."""
    wl = synth.workload("tiny_fp32_b1")
    dm = synth.dims(wl["model"])
    w = weights(wl["model"], "bf16")
    lens = np.array([8, 3, 13], dtype=np.int32)
    prompts = synth.split_rows(synth.make_prompts(lens, dm["talker"]["hidden"], seed=21), lens)
    pad = synth.make_tts_pad(dm["talker"]["hidden"], seed=22)
    eng = binding.Engine(dm, w, "bf16", kv_dtype=kv, max_batch=3, max_positions=96)
    teacher_forced_check(eng, w, dm, prompts, lens, pad, synth.SAMPLING, synth.PRED_SAMPLING, 5, 70, 5e-2)
    eng.close()


def test_tiny_trailing_text_parity():
    wl = synth.workload("tiny_fp32_b1")
    dm = synth.dims(wl["model"])
    w = weights(wl["model"], "f32")
    H = dm["talker"]["hidden"]
    lens = np.array([8, 5], dtype=np.int32)
    prompts = synth.split_rows(synth.make_prompts(lens, H, seed=11), lens)
    tlens = np.array([3, 0], dtype=np.int32)
    text = synth.make_text(tlens, H, seed=12)
    texts = synth.split_rows(text, tlens)
    pad = synth.make_tts_pad(H, seed=13)
    eng = binding.Engine(dm, w, "f32", max_batch=2, max_positions=32)
    codes, n, fin = eng.generate(np.concatenate(prompts), lens, pad, wl["talker"], wl["predictor"], 0, 6,
                                 text=text, text_lens=tlens)
    ref = oracle.generate(w, dm, prompts, pad, wl["talker"], wl["predictor"], 0, 6, texts=texts)
    for r in range(2):
        assert int(n[r]) == ref[r]["n_frames"]
        np.testing.assert_array_equal(codes[r, :ref[r]["n_frames"]], ref[r]["codes"])
    teacher_forced_check(eng, w, dm, prompts, lens, pad, wl["talker"], wl["predictor"], 0, 6, 2e-3,
                         texts=texts, text_packed=text, text_lens=tlens)
    eng.close()


def test_small_sampling_batch_parity():
    dm = synth.small_dims(layers_t=3, layers_p=2, hidden=128, n_heads=4, n_kv_heads=2, head_dim=32, intermediate=256)
    w = synth.make_weights(dm, seed=4, dtype="f32")
    lens = synth.prompt_lengths(3, 3, 40, seed=5)
    prompts = synth.split_rows(synth.make_prompts(lens, 128, seed=6), lens)
    pad = synth.make_tts_pad(128, seed=7)
    eng = binding.Engine(dm, w, "f32", max_batch=4, max_positions=64)
    teacher_forced_check(eng, w, dm, prompts, lens, pad, synth.SAMPLING, synth.PRED_SAMPLING, 77, 8, 2e-3)
    eng.close()


def test_qwen06b_bf16_b1_parity():
    wl = synth.workload("qwen06b_bf16_b1")
    dm = synth.dims(wl["model"])
    log("generating 0.6B weights")
    w = weights(wl["model"], "bf16")
    lens = synth.prompt_lengths(1, *wl["prompt"], seed=2)
    prompts = synth.split_rows(synth.make_prompts(lens, 1024, seed=1), lens)
    pad = synth.make_tts_pad(1024, seed=3)
    eng = binding.Engine(dm, w, "bf16", max_batch=1, max_positions=wl["max_positions"])
    log("engine ready")
    teacher_forced_check(eng, w, dm, prompts, lens, pad, wl["talker"], wl["predictor"], 0, 12, 5e-2)
    eng.close()


def test_qwen06b_bf16_b8_sampling_parity():
    wl = synth.workload("qwen06b_bf16_b8_sampling")
    dm = synth.dims(wl["model"])
    w = weights(wl["model"], "bf16")
    lens = synth.prompt_lengths(8, *wl["prompt"], seed=2)
    prompts = synth.split_rows(synth.make_prompts(lens, 1024, seed=1), lens)
    pad = synth.make_tts_pad(1024, seed=3)
    eng = binding.Engine(dm, w, "bf16", max_batch=8, max_positions=wl["max_positions"])
    teacher_forced_check(eng, w, dm, prompts, lens, pad, wl["talker"], wl["predictor"], 0, 4, 5e-2, rows=[0, 5, 7])
    eng.close()


def test_qwen06b_bf16_b16_sampling_parity():
    """Batch 16 (between the benchmarked sizes): the talker attention runs
    over 4 key ranges, 16-row projections take the 16-row matrix-core GEMV and
    the skinny kernel, the predictor's two-token pass the 32-row paths; rows
    0 and 15 are checked against the oracle over 2 frames."""
    wl = synth.workload("qwen06b_bf16_b8_sampling")
    dm = synth.dims(wl["model"])
    w = weights(wl["model"], "bf16")
    lens = synth.prompt_lengths(16, *wl["prompt"], seed=5)
    prompts = synth.split_rows(synth.make_prompts(lens, 1024, seed=1), lens)
    pad = synth.make_tts_pad(1024, seed=3)
    eng = binding.Engine(dm, w, "bf16", max_batch=16, max_positions=wl["max_positions"])
    teacher_forced_check(eng, w, dm, prompts, lens, pad, wl["talker"], wl["predictor"], 0, 2, 5e-2, rows=[0, 15])
    eng.close()


def test_qwen06b_b8_sampling_200_frames_stay_finite():
    """The whole batch-8 sampling request (200 frames, contexts up to 450
    keys, the talker attention split over key ranges) completes without a
    non-finite logit and with codes in range. A split block whose range ends
    at the new key once read the new-key rows it does not own from stale LDS
    (0 x NaN in the masked P.V products) at frame 130 of this request."""
    wl = synth.workload("qwen06b_bf16_b8_sampling")
    dm = synth.dims(wl["model"])
    w = weights(wl["model"], "bf16")
    lens = synth.prompt_lengths(8, *wl["prompt"], seed=2)
    prompt = synth.make_prompts(lens, 1024, seed=1)
    pad = synth.make_tts_pad(1024, seed=3)
    eng = binding.Engine(dm, w, "bf16", max_batch=8, max_positions=wl["max_positions"])
    codes, n, _ = eng.generate(prompt, lens, pad, wl["talker"], wl["predictor"], 0, wl["frames"])
    eng.close()
    assert int(n.max()) > 130
    for r in range(8):
        c = codes[r, : int(n[r])]
        assert np.all((c[:, 1:] >= 0) & (c[:, 1:] < 2048))
        assert np.all((c[:, 0] >= 0) & ((c[:, 0] < 2048) | (c[:, 0] == dm["eos_id"])))


def _full_size(name, rows, frames, seed=0, lens=None):
    wl = synth.workload(name)
    dm = synth.dims(wl["model"])
    H = dm["talker"]["hidden"]
    log(f"{name}: generating weights")
    w = weights(wl["model"], "bf16")
    if lens is None:
        lens = synth.prompt_lengths(wl["B"], *wl["prompt"], seed=2)
    prompts = synth.split_rows(synth.make_prompts(lens, H, seed=1), lens)
    pad = synth.make_tts_pad(H, seed=3)
    eng = binding.Engine(dm, w, "bf16", max_batch=len(lens), max_positions=wl["max_positions"])
    log(f"{name}: engine ready, prompt lengths {list(lens)[:8]}..., rows {rows}")
    teacher_forced_check(eng, w, dm, prompts, lens, pad, wl["talker"], wl["predictor"], seed, frames, 5e-2,
                         rows=rows)
    return eng, dm, prompts, lens, pad, wl


def test_qwen06b_bf16_b64_sampling_parity():
    """Batch 64 with prompts of 128..512 tokens: the prefill runs 8192-token
    chunks through the split-activation MFMA GEMM, decode runs 64 / 128 rows
    through the split-K GEMM; rows 0, 29 and 63 are checked against the
    oracle, and so is the row whose prompt straddles the first chunk boundary
    (its keys come from two prefill chunks)."""
    wl = synth.workload("qwen06b_bf16_b64_sampling")
    lens = synth.prompt_lengths(wl["B"], *wl["prompt"], seed=2)
    ends = np.cumsum(lens)
    straddle = int(np.nonzero((ends - lens < 8192) & (ends > 8192))[0][0])
    eng, *_ = _full_size("qwen06b_bf16_b64_sampling", sorted({0, straddle, 29, 63}), 2)
    eng.close()


def test_qwen06b_b64_graph_replay_equals_forced_eager():
    """At the full batch-64 shape, free-run codes (frames 2.. from graph
    replays) equal the eager forced replay bit for bit."""
    wl = synth.workload("qwen06b_bf16_b64_sampling")
    dm = synth.dims(wl["model"])
    w = weights(wl["model"], "bf16")
    lens = synth.prompt_lengths(64, *wl["prompt"], seed=2)
    prompt = synth.make_prompts(lens, 1024, seed=1)
    pad = synth.make_tts_pad(1024, seed=3)
    eng = binding.Engine(dm, w, "bf16", max_batch=64, max_positions=wl["max_positions"])
    codes, n, _ = eng.generate(prompt, lens, pad, wl["talker"], wl["predictor"], 11, 4)
    assert np.all((codes[:, :, 1:] >= 0) & (codes[:, :, 1:] < 2048))
    eng.prefill(prompt, lens, pad, wl["talker"], wl["predictor"], 11, 4)
    for k in range(int(n.max())):
        forced = codes[:, k].copy()
        forced[n <= k] = 0
        forced[n <= k, 0] = dm["eos_id"]
        _, _, ch = eng.step_forced(forced)
        live = n > k
        np.testing.assert_array_equal(ch[live, 1:], codes[live, k, 1:])
        if k + 1 < codes.shape[1]:
            nxt = n > k + 1
            np.testing.assert_array_equal(ch[nxt, 0], codes[nxt, k + 1, 0])
    eng.close()


def test_long_context_parity():
    """Talker attention over the batch-64 workload's full KV extent: a
    1500-token prompt (prefill attention over up to 1500 keys, decode at
    positions 1500..1501) next to a 700-token one."""
    eng, *_ = _full_size("qwen06b_bf16_b64_sampling", [0, 1], 2, lens=np.array([1500, 700], dtype=np.int32))
    eng.close()


def test_qwen17b_bf16_b1_parity():
    """1.7B-class talker (hidden 2048, I 6144) with the 2048 -> 1024 predictor
    input projection, batch 1 greedy."""
    eng, *_ = _full_size("qwen17b_bf16_b1", [0], 3)
    eng.close()


def test_qwen17b_bf16_b8_parity():
    eng, *_ = _full_size("qwen17b_bf16_b8", [0, 7], 2)
    eng.close()


def test_determinism_and_graph_replay_equals_eager():
    dm = synth.small_dims(layers_t=2, layers_p=2, hidden=128, n_heads=4, n_kv_heads=2, head_dim=32, intermediate=256)
    w = synth.make_weights(dm, seed=8, dtype="bf16")
    lens = np.array([5, 9], dtype=np.int32)
    prompt = synth.make_prompts(lens, 128, seed=9)
    pad = synth.make_tts_pad(128, seed=10)
    eng = binding.Engine(dm, w, "bf16", max_batch=2, max_positions=40)
    a = eng.generate(prompt, lens, pad, synth.SAMPLING, synth.PRED_SAMPLING, 3, 12)
    b = eng.generate(prompt, lens, pad, synth.SAMPLING, synth.PRED_SAMPLING, 3, 12)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    c = eng.generate(prompt, lens, pad, synth.SAMPLING, synth.PRED_SAMPLING, 4, 12)
    assert not np.array_equal(a[0], c[0])
    # frames 2.. above came from graph replays; the forced path is eager
    codes, n, _ = a
    eng.prefill(prompt, lens, pad, synth.SAMPLING, synth.PRED_SAMPLING, 3, 12)
    F = int(n.max())
    for k in range(F):
        forced = codes[:, k].copy()
        forced[n <= k] = 0
        forced[n <= k, 0] = dm["eos_id"]
        _, _, ch = eng.step_forced(forced)
        for r in range(2):
            if k < n[r]:
                np.testing.assert_array_equal(ch[r, 1:], codes[r, k, 1:])
                if k + 1 < n[r]:
                    assert ch[r, 0] == codes[r, k + 1, 0]
    eng.close()


def test_frame_states_and_abi_errors():
    dm = synth.small_dims(layers_t=1, layers_p=1, hidden=64, n_heads=2, n_kv_heads=1, head_dim=32, intermediate=64)
    w = synth.make_weights(dm, seed=12, dtype="f32")
    # EOS wins as soon as it is unmasked: the talker head row of EOS reads a large coordinate
    w["talker_codec_head"][2150] = 0
    w["talker_codec_head"][2150, 0] = 50.0
    w["talker_norm"][0] = 1.0
    lens = np.array([4, 6], dtype=np.int32)
    prompt = synth.make_prompts(lens, 64, seed=13)
    prompt[:, 0] = 30.0
    pad = synth.make_tts_pad(64, seed=14)
    pad[0] = 30.0
    eng = binding.Engine(dm, w, "f32", max_batch=2, max_positions=16)
    with pytest.raises(binding.QtError) as e:
        eng.step_frame()
    assert e.value.status == binding.QT_E_STATE
    with pytest.raises(binding.QtError) as e:
        eng.prefill(prompt, lens, pad, synth.GREEDY, synth.PRED_GREEDY, 0, 11)   # 6 + 11 > 16
    assert e.value.status == binding.QT_E_CAPACITY
    with pytest.raises(binding.QtError) as e:
        eng.prefill(np.concatenate([prompt, prompt[:4]]), np.array([4, 6, 4], np.int32), pad, synth.GREEDY,
                    synth.PRED_GREEDY, 0, 3)
    assert e.value.status == binding.QT_E_CAPACITY
    # min_new_tokens 3: EOS masked at selections 0..2, chosen at selection 3 -> 3 frames, stop
    samp = dict(synth.GREEDY, min_new_tokens=3)
    eng.prefill(prompt, lens, pad, samp, synth.PRED_GREEDY, 0, 8)
    states = []
    for k in range(3):
        codes, st = eng.step_frame()
        states.append(st.copy())
        assert np.all((codes[:, 1:] >= 0) & (codes[:, 1:] < 2048))
    assert list(states[0]) == [0, 0] and list(states[1]) == [0, 0] and list(states[2]) == [1, 1]
    with pytest.raises(binding.QtError) as e:
        eng.step_frame()
    assert e.value.status == binding.QT_E_STATE
    # length stop: 2 frames with EOS masked throughout
    samp = dict(synth.GREEDY, min_new_tokens=100)
    codes, n, fin = eng.generate(prompt, lens, pad, samp, synth.PRED_GREEDY, 0, 2)
    assert list(n) == [2, 2] and list(fin) == [2, 2]
    # forced ids are range-checked before any device work
    eng.prefill(prompt, lens, pad, synth.GREEDY, synth.PRED_GREEDY, 0, 4)
    bad = np.zeros((2, 16), np.int32)
    bad[1, 5] = 2048
    with pytest.raises(binding.QtError) as e:
        eng.step_forced(bad)
    assert e.value.status == binding.QT_E_RANGE
    # a NaN prompt row fails closed at the prefill sync
    p2 = prompt.copy()
    p2[5, 3] = np.nan
    with pytest.raises(binding.QtError) as e:
        eng.prefill(p2, lens, pad, synth.GREEDY, synth.PRED_GREEDY, 0, 4)
    assert e.value.status == binding.QT_E_NAN
    eng.close()
