"""Pins of the oracle's frame loop.

  * frame schedule: N frames <=> N+1 talker selections and 15 N predictor
    passes, natural stop on an EOS lookahead, length stop at max_frames
    (tests/golden/frame_schedule.json, ncnn CustomVoice port sections 3.1
    and 4);
  * table/head offsets and the feedback sum in closed form: with every
    decoder layer zeroed (each layer is then the identity on the residual)
    and one-hot tables / permutation heads, every code of a frame is a
    permutation lookup of the previous one (ncnn port section 1: step s embeds
    with table s-1 and applies head s), and the next code 0 is the most
    frequent one-hot index of the feedback sum;
  * the trailing-text switch (text row k for frame k, tts_pad afterwards);
  * determinism, the prefix property and batch independence (ncnn CustomVoice
    port section 4: repeatable oracle, a 25-frame run is a prefix of the
    54-frame run);
  * teacher forcing with the oracle's own codes reproduces the free run.
"""
import json
import os

import numpy as np
import pytest

from codec_lm_autoregressive_amd import synth
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
GREEDY = dict(do_sample=False, temperature=1.0, top_k=0, top_p=1.0, repetition_penalty=1.0, min_new_tokens=0)


def _zero_layers(w):
    for key in ("talker_layers", "pred_layers"):
        for lw in w[key]:
            for n, a in lw.items():
                lw[n] = np.zeros_like(a) if a.ndim == 2 else np.ones_like(a)
    w["talker_norm"] = np.ones_like(w["talker_norm"])
    w["pred_norm"] = np.ones_like(w["pred_norm"])
    return w


def _eos_model(H=64):
    """Identity layers; tts_pad and the last prompt row carry a large coordinate 0,
    and the EOS head row reads it, so EOS wins as soon as it is not masked."""
    dm = synth.small_dims(layers_t=2, layers_p=2, hidden=H)
    w = _zero_layers(synth.make_weights(dm, seed=21, dtype="f32"))
    w["talker_codec_head"][2150] = 0
    w["talker_codec_head"][2150, 0] = 1.0
    pad = synth.make_tts_pad(H, 22)
    pad[0] = 100.0
    prompt = synth.make_prompts([5], H, 23)
    prompt[-1, 0] = 100.0
    return dm, w, [prompt], pad


def test_frame_schedule_golden():
    gold = json.load(open(os.path.join(GOLD, "frame_schedule.json")))
    dm, w, prompts, pad = _eos_model()
    for case in gold["cases"]:
        N = case["frames"]
        if case.get("finish") == "stop":
            samp = dict(GREEDY, min_new_tokens=N)  # EOS masked for selections 0..N-1
            r = oracle.generate(w, dm, prompts, pad, samp, GREEDY, 0, max_frames=100)[0]
            assert r["finish"] == "stop"
            assert int(r["talker_choice"][-1]) == case["last_lookahead"]
        else:
            samp = dict(GREEDY, min_new_tokens=10_000)  # never stops on EOS
            r = oracle.generate(w, dm, prompts, pad, samp, GREEDY, 0, max_frames=N)[0]
            assert r["finish"] == "length"
        assert r["n_frames"] == N
        assert r["codes"].size == case["codes"]
        assert r["n_talker_selections"] == case["talker_selections"]
        assert r["n_predictor_passes"] == case["predictor_passes"]
        assert len(r["talker_choice"]) == N + 1


def _perm_model(seed=31):
    C = H = 64
    dm = synth.small_dims(layers_t=1, layers_p=2, hidden=H, codebook=C)
    w = _zero_layers(synth.make_weights(dm, seed=seed, dtype="f32"))
    g = np.random.default_rng(seed)
    tau = [g.permutation(C) for _ in range(15)]
    sig = [g.permutation(C) for _ in range(15)]
    eye = np.eye(C, dtype=np.float32)
    w["talker_codec_embed"] = eye[np.arange(3072) % C]
    w["talker_codec_head"] = eye[np.arange(3072) % C]
    w["pred_embeds"] = np.concatenate([eye[tau[j]] for j in range(15)])     # Tab[j][c] = e_tau_j(c)
    w["pred_heads"] = np.concatenate([eye[sig[s]] for s in range(15)])      # Head[s][i] = e_sig_s(i)
    return dm, w, tau, sig


def _closed_form_frames(code0, tau, sig, n_frames, C=64, texts=None):
    inv = [np.argsort(s) for s in sig]
    frames, sel = [], [code0]
    for k in range(n_frames):
        c = [code0]
        c.append(int(inv[0][code0 % C]))
        for s in range(1, 15):
            c.append(int(inv[s][tau[s - 1][c[s]]]))
        frames.append(c)
        counts = np.zeros(C)
        counts[code0 % C] += 1
        for j in range(1, 16):
            counts[tau[j - 1][c[j]]] += 1
        if texts is not None and k < len(texts):
            code0 = int(texts[k])
        else:
            code0 = int(np.argmax(counts))  # lowest index among the most frequent
        sel.append(code0)
    return np.array(frames), np.array(sel)


def test_table_head_offsets_closed_form():
    dm, w, tau, sig = _perm_model()
    prompt = np.zeros((4, 64), dtype=np.float32)
    prompt[:, 9] = 1.0  # selection 0 reads the last prompt row: code 0 = 9
    pad = np.zeros(64, dtype=np.float32)
    r = oracle.generate(w, dm, [prompt], pad, GREEDY, GREEDY, 0, max_frames=6)[0]
    frames, sel = _closed_form_frames(9, tau, sig, 6)
    np.testing.assert_array_equal(r["codes"], frames)
    np.testing.assert_array_equal(r["talker_choice"], sel)


def test_trailing_text_switch():
    dm, w, tau, sig = _perm_model(seed=32)
    prompt = np.zeros((3, 64), dtype=np.float32)
    prompt[-1, 20] = 1.0
    pad = np.zeros(64, dtype=np.float32)
    marks = [41, 3, 60]
    text = np.zeros((3, 64), dtype=np.float32)
    for k, m in enumerate(marks):
        text[k, m] = 100.0
    r = oracle.generate(w, dm, [prompt], pad, GREEDY, GREEDY, 0, max_frames=6, texts=[text])[0]
    frames, sel = _closed_form_frames(20, tau, sig, 6, texts=marks)
    np.testing.assert_array_equal(r["talker_choice"], sel)
    np.testing.assert_array_equal(r["codes"], frames)
    assert list(r["talker_choice"][1:4]) == marks


def test_predictor_input_projection_closed_form():
    """The 1.7B-class predictor sits behind a [Hp, H] input projection that
    applies to every predictor input: the talker hidden and the talker table
    row of pass 0 and every table row of steps 1..14; the feedback sum stays
    at talker width. Talker width 128, predictor width 64; W_proj selects the
    coordinates rho(0..63) (W[i, rho(i)] = 1), table j maps code c to the talker
    one-hot e_rho(kappa_j(c)), so its projection is the predictor one-hot
    e_kappa_j(c), and head s is a permutation sigma_s. With identity layers
    every code is then c_{s+1} = sigma_s^-1(kappa_{s-1}(c_s)) and the next code 0
    is the most frequent coordinate of the feedback sum. An input left
    unprojected, or the projection applied to the feedback, has the wrong
    width and fails; a transposed projection fails the same way."""
    C, H, Hp = 64, 128, 64
    dm = synth.small_dims(layers_t=1, layers_p=2, hidden=H, codebook=C, pred_in_proj=True, pred_hidden=Hp)
    w = _zero_layers(synth.make_weights(dm, seed=33, dtype="f32"))
    g = np.random.default_rng(33)
    rho = g.permutation(H)[:Hp]                 # injective map of predictor coords into talker coords
    kappa = [g.permutation(C) for _ in range(15)]
    sig = [g.permutation(C) for _ in range(15)]
    eyeH = np.eye(H, dtype=np.float32)
    eyeC = np.eye(C, dtype=np.float32)
    proj = np.zeros((Hp, H), dtype=np.float32)
    proj[np.arange(Hp), rho] = 1.0
    w["pred_in_proj"] = proj
    w["talker_codec_embed"] = eyeH[rho[np.arange(3072) % C]]
    w["talker_codec_head"] = eyeH[rho[np.arange(3072) % C]]
    w["pred_embeds"] = np.concatenate([eyeH[rho[kappa[j]]] for j in range(15)])
    w["pred_heads"] = np.concatenate([eyeC[sig[s]] for s in range(15)])
    prompt = np.zeros((4, H), dtype=np.float32)
    prompt[:, rho[17]] = 1.0                    # selection 0: code 0 = 17
    pad = np.zeros(H, dtype=np.float32)
    r = oracle.generate(w, dm, [prompt], pad, GREEDY, GREEDY, 0, max_frames=5)[0]
    frames, sel = _closed_form_frames(17, kappa, sig, 5)
    np.testing.assert_array_equal(r["codes"], frames)
    np.testing.assert_array_equal(r["talker_choice"], sel)
    # the projection is load-bearing: without it the predictor sees 128-wide rows
    w_bad = dict(w, pred_in_proj=None)
    with pytest.raises(ValueError):
        oracle.generate(w_bad, dm, [prompt], pad, GREEDY, GREEDY, 0, max_frames=1)
    # and a different projection (another coordinate choice) changes the codes
    w_perm = dict(w, pred_in_proj=proj[g.permutation(Hp)])
    r2 = oracle.generate(w_perm, dm, [prompt], pad, GREEDY, GREEDY, 0, max_frames=5)[0]
    assert not np.array_equal(r2["codes"], r["codes"])


SAMPLING = dict(do_sample=True, temperature=0.9, top_k=50, top_p=0.8, repetition_penalty=1.05, min_new_tokens=2)
PSAMP = dict(do_sample=True, temperature=0.9, top_k=50, top_p=0.8, repetition_penalty=1.0, min_new_tokens=0)


def _small_run(B=3, frames=5, samp=SAMPLING, psamp=PSAMP, rows=None, which=None, forced=None, seed=7):
    dm = synth.small_dims(layers_t=2, layers_p=2, hidden=64)
    w = synth.make_weights(dm, seed=41, dtype="bf16")
    lens = synth.prompt_lengths(B, 3, 9, seed=42)
    pr = synth.split_rows(synth.make_prompts(lens, 64, 43), lens)
    pad = synth.make_tts_pad(64, 44)
    if which is not None:
        pr = [pr[i] for i in which]
    return oracle.generate(w, dm, pr, pad, samp, psamp, seed, max_frames=frames, rows=rows, forced=forced)


def test_determinism_and_prefix():
    a = _small_run(frames=6)
    b = _small_run(frames=6)
    c = _small_run(frames=3)
    for x, y, z in zip(a, b, c):
        np.testing.assert_array_equal(x["codes"], y["codes"])
        np.testing.assert_array_equal(x["talker_logits"], y["talker_logits"])
        n = z["n_frames"]
        np.testing.assert_array_equal(x["codes"][:n], z["codes"])
        np.testing.assert_array_equal(x["talker_logits"][:n + 1], z["talker_logits"])
        np.testing.assert_array_equal(x["pred_logits"][:n], z["pred_logits"])
    # a different seed changes the sampled codes
    d = _small_run(frames=6, seed=8)
    assert any(not np.array_equal(x["codes"], y["codes"]) for x, y in zip(a, d))


def test_batch_independence():
    full = _small_run(B=3, frames=4)
    for r in range(3):
        one = _small_run(B=3, frames=4, which=[r], rows=[r])[0]
        np.testing.assert_array_equal(one["codes"], full[r]["codes"])
        np.testing.assert_array_equal(one["talker_logits"], full[r]["talker_logits"])


def test_teacher_forcing_with_own_codes_reproduces_run():
    free = _small_run(B=2, frames=5)
    forced = [f["codes"] for f in free]
    tf = _small_run(B=2, frames=5, forced=forced)
    for f, t in zip(free, tf):
        n = f["n_frames"]
        np.testing.assert_array_equal(t["talker_logits"][:n + 1], f["talker_logits"][:n + 1])
        np.testing.assert_array_equal(t["pred_logits"], f["pred_logits"])
        np.testing.assert_array_equal(t["pred_choice"], f["codes"][:, 1:])
        np.testing.assert_array_equal(t["talker_choice"][:n], f["codes"][:, 0])


def test_codes_in_range():
    for r in _small_run(B=3, frames=8):
        c = r["codes"]
        assert np.all((c[:, 0] < 2048) | (c[:, 0] == 2150))
        assert np.all((c[:, 1:] >= 0) & (c[:, 1:] < 2048))
