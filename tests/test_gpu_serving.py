"""Continuous batching (qt_admit) against the oracle: a queue of requests
flows through a fixed number of slots; whenever a slot's request finishes
(EOS lookahead or its own frame cap), the next request is admitted into it
between two frames while the other slots keep generating (Mizuoto engine
page, "Matching upstream", sampler bullet; the SGLang-Omni case's talker
serving stage). Every request must produce the oracle's free run of that
request alone (its prompt, trailing text, seed, noise row and frame cap),
frame by frame, up to a decision inside the margin; rows are independent
sequences, so the admission order and slot cannot matter.
"""
import numpy as np
import pytest

from codec_lm_autoregressive_amd import binding, synth
import oracle
from test_gpu_parity import free_run_agreement, log, weights

pytestmark = pytest.mark.gpu


def _serve(eng, reqs, slots, tsamp, psamp, pad, seed0, cap0):
    """Run the queue: the first `slots` requests start with qt_prefill (seed
    seed0, noise rows 0..slots-1, frame cap cap0); the rest are admitted into
    slots as they free up. Returns {request index: codes [n, 16]}."""
    first = reqs[:slots]
    lens = np.array([r["prompt"].shape[0] for r in first], np.int32)
    tl = np.array([0 if r["text"] is None else r["text"].shape[0] for r in first], np.int32)
    text = np.concatenate([r["text"] for r in first if r["text"] is not None]) if tl.sum() else None
    eng.prefill(np.concatenate([r["prompt"] for r in first]), lens, pad, tsamp, psamp, seed0, cap0,
                text=text, text_lens=tl if tl.sum() else None)
    holder = list(range(slots))
    out = {i: [] for i in range(len(reqs))}
    nxt = slots
    done = set()
    frames = 0
    while len(done) < len(reqs):
        codes, st = eng.step_frame()
        frames += 1
        for s in range(slots):
            q = holder[s]
            if q is None or st[s] == 3:
                continue
            out[q].append(codes[s].copy())
            if st[s] in (1, 2):
                done.add(q)
                holder[s] = None
                if nxt < len(reqs):
                    r = reqs[nxt]
                    eng.admit(s, r["prompt"], r["text"], r["seed"], r["noise_row"], r["cap"])
                    holder[s] = nxt
                    nxt += 1
        if all(h is None for h in holder):
            break
        assert frames < 10_000
    log(f"served {len(reqs)} requests through {slots} slots in {frames} frames")
    return {q: np.array(v, np.int32).reshape(-1, 16) for q, v in out.items()}


def _requests(dm, n, slots, seed0, cap0, caps, prompt_range, text_every, H):
    g = np.random.default_rng(41)
    reqs = []
    for i in range(n):
        P = int(g.integers(*prompt_range))
        prompt = synth.make_prompts([P], H, seed=100 + i)
        nt = int(g.integers(1, 5)) if i % text_every == 1 else 0
        text = synth.make_text(np.array([nt]), H, seed=200 + i) if nt else None
        if i < slots:
            reqs.append(dict(prompt=prompt, text=text, seed=seed0, noise_row=i, cap=cap0))
        else:
            reqs.append(dict(prompt=prompt, text=text, seed=int(g.integers(0, 2**63)), noise_row=int(g.integers(0, 1000)),
                             cap=int(caps[i % len(caps)])))
    return reqs


def _check(eng, w, dm, reqs, got, tsamp, psamp, pad, tol, min_equal_frac):
    equal = total = 0
    for i, r in enumerate(reqs):
        ref = oracle.generate(w, dm, [r["prompt"]], pad, tsamp, psamp, r["seed"], r["cap"], rows=[r["noise_row"]],
                              texts=None if r["text"] is None else [r["text"]])[0]
        e = free_run_agreement(got[i], got[i].shape[0], ref, dm, tsamp, psamp, r["seed"], r["noise_row"], tol)
        equal += e
        total += ref["n_frames"]
    log(f"frames equal to the oracle's runs of each request alone: {equal}/{total}")
    assert equal >= min_equal_frac * total


def test_tiny_fp32_continuous_batching():
    wl = synth.workload("tiny_fp32_b1")
    dm = synth.dims(wl["model"])
    H = dm["talker"]["hidden"]
    w = weights(wl["model"], "f32")
    pad = synth.make_tts_pad(H, seed=3)
    slots = 3
    reqs = _requests(dm, 9, slots, 5, 4, caps=[3, 7, 2, 9, 5], prompt_range=(4, 20), text_every=2, H=H)
    eng = binding.Engine(dm, w, "f32", max_batch=slots, max_positions=64)
    got = _serve(eng, reqs, slots, synth.SAMPLING, synth.PRED_SAMPLING, pad, 5, 4)
    # the slot / state rules of the ABI
    with pytest.raises(binding.QtError) as e:
        eng.admit(slots, reqs[0]["prompt"], max_frames=2)
    assert e.value.status in (binding.QT_E_RANGE, binding.QT_E_STATE)
    eng.close()
    _check(eng, w, dm, reqs, got, synth.SAMPLING, synth.PRED_SAMPLING, pad, 2e-3, 0.9)


def test_admit_refuses_an_active_slot():
    dm = synth.small_dims(layers_t=1, layers_p=1, hidden=64, n_heads=2, n_kv_heads=1, head_dim=32, intermediate=64)
    w = synth.make_weights(dm, seed=12, dtype="f32")
    lens = np.array([4, 6], dtype=np.int32)
    prompt = synth.make_prompts(lens, 64, seed=13)
    pad = synth.make_tts_pad(64, seed=14)
    eng = binding.Engine(dm, w, "f32", max_batch=2, max_positions=16)
    samp = dict(synth.GREEDY, min_new_tokens=100)
    eng.prefill(prompt, lens, pad, samp, synth.PRED_GREEDY, 0, 3)
    with pytest.raises(binding.QtError) as e:
        eng.admit(0, prompt[:4], max_frames=2)            # still active
    assert e.value.status == binding.QT_E_STATE
    for _ in range(3):
        eng.step_frame()                                   # both rows reach their cap of 3
    with pytest.raises(binding.QtError) as e:
        eng.admit(1, prompt[:6], max_frames=11)           # 6 + 11 > 16 positions
    assert e.value.status == binding.QT_E_CAPACITY
    eng.admit(1, prompt[:6], max_frames=5)
    codes, st = eng.step_frame()
    assert st[0] == 3 and st[1] == 0
    eng.close()


@pytest.mark.timeout(900)
def test_qwen06b_bf16_b8_continuous_batching():
    """0.6B bf16, 8 slots with sampling, 16 requests (prompts 32..96, caps
    6..20, trailing text on some) through the captured frame graph."""
    wl = synth.workload("qwen06b_bf16_b8_sampling")
    dm = synth.dims(wl["model"])
    H = dm["talker"]["hidden"]
    w = weights(wl["model"], "bf16")
    pad = synth.make_tts_pad(H, seed=3)
    slots = 8
    reqs = _requests(dm, 16, slots, 7, 12, caps=[6, 20, 9, 14, 11], prompt_range=(32, 96), text_every=3, H=H)
    eng = binding.Engine(dm, w, "bf16", max_batch=slots, max_positions=wl["max_positions"])
    got = _serve(eng, reqs, slots, wl["talker"], wl["predictor"], pad, 7, 12)
    eng.close()
    _check(eng, w, dm, reqs, got, wl["talker"], wl["predictor"], pad, 5e-2, 0.6)
