"""Pins of the oracle's processors, warpers, race and Philox.

  * processors and warpers vs the transformers classes the Mizuoto page
    ("Matching upstream", sampler bullet) says the talker chain follows, on
    24 random logit sets (the ncnn port's section 7 sampler check);
  * the penalty sign rule and min-new masking vs the values in
    tests/golden/processors.json (ncnn CustomVoice port section 3.2; ncnn
    port section 1 fact 3);
  * lowest-index ties, the suppress range, NaN fail-closed;
  * the exponential race: P(choose i) = p_i, checked by chi-square;
  * top-p against brute-force subset enumeration;
  * Philox4x64-10 vs numpy's own Philox bit generator.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import philox, sampling

GOLD = os.path.join(os.path.dirname(__file__), "golden")
CFG = dict(eos_id=2150, suppress_begin=2048, suppress_end=3072)
TALK = dict(do_sample=True, temperature=0.9, top_k=50, top_p=0.8, repetition_penalty=1.05, min_new_tokens=2)


def test_penalty_golden():
    g = json.load(open(os.path.join(GOLD, "processors.json")))
    rp = g["repetition_penalty"]
    for c in rp["cases"]:
        l = np.array([c["logit"], 0.5], dtype=np.float32)
        out = sampling.repetition_penalty(l, [0] if c["seen"] else [], rp["rho"])
        assert abs(float(out[0]) - c["expected"]) < 1e-6
        assert out[1] == np.float32(0.5)


def test_min_new_masks_not_resamples():
    g = json.load(open(os.path.join(GOLD, "processors.json")))["min_new_tokens"]
    samp = dict(TALK, do_sample=False, repetition_penalty=1.0)
    l = np.zeros(3072, dtype=np.float32)
    l[2150] = 5.0   # EOS is the best logit
    l[17] = 3.0     # runner-up
    for sel in g["eos_masked_at_selection"]:
        p = sampling.talker_process(l, [], sel, samp, CFG)
        assert p[2150] == -np.inf
        assert sampling.greedy(p) == 17
    for sel in g["eos_allowed_at_selection"]:
        p = sampling.talker_process(l, [], sel, samp, CFG)
        assert sampling.greedy(p) == 2150


def test_suppress_range_and_ties():
    samp = dict(TALK, do_sample=False, repetition_penalty=1.0)
    l = np.zeros(3072, dtype=np.float32)
    l[2048:3072] = 10.0          # control ids would win if not suppressed
    p = sampling.talker_process(l, [], 5, samp, CFG)
    assert np.all(p[2048:2150] == -np.inf) and np.all(p[2151:] == -np.inf)
    assert p[2150] == 10.0       # EOS survives the suppress processor
    assert sampling.greedy(p) == 2150
    l2 = np.zeros(3072, dtype=np.float32)
    l2[[7, 3, 900]] = 1.0        # three-way tie -> lowest index
    assert sampling.greedy(sampling.talker_process(l2, [], 5, samp, CFG)) == 3
    assert sampling.greedy(np.zeros(2048, np.float32)) == 0


def test_nan_fails_closed():
    l = np.zeros(3072, dtype=np.float32)
    l[5] = np.nan
    with pytest.raises(sampling.NonFinite):
        sampling.talker_process(l, [], 0, TALK, CFG)
    l[5] = np.inf
    with pytest.raises(sampling.NonFinite):
        sampling.talker_process(l, [], 0, TALK, CFG)


def test_processors_match_transformers():
    from transformers.generation.logits_process import (
        MinNewTokensLengthLogitsProcessor, RepetitionPenaltyLogitsProcessor,
        SuppressTokensLogitsProcessor, TemperatureLogitsWarper, TopKLogitsWarper,
        TopPLogitsWarper)
    sup = [i for i in range(2048, 3072) if i != 2150]
    for trial in range(24):
        g = np.random.default_rng(100 + trial)
        l = (g.standard_normal(3072) * 2).astype(np.float32)
        n_sel = int(g.integers(0, 4))
        seen = list(g.integers(0, 2048, size=int(g.integers(0, 30))))
        prompt_len = 7
        ids = torch.tensor([[1] * prompt_len + [int(s) for s in seen][:n_sel] + [0] * max(0, n_sel - len(seen))])
        # transformers counts new tokens from input length; our penalty set is `seen`
        ref = torch.from_numpy(l.copy())[None]
        ref = RepetitionPenaltyLogitsProcessor(1.05)(torch.tensor([seen if seen else [0]]), ref) if seen else ref
        ref = MinNewTokensLengthLogitsProcessor(prompt_len, 2, 2150)(ids[:, :prompt_len + n_sel], ref)
        ref = SuppressTokensLogitsProcessor(sup, device="cpu")(ids, ref)
        ours = sampling.talker_process(l, seen, n_sel, TALK, CFG)
        np.testing.assert_array_equal(ours, ref[0].numpy())
        # warpers: temperature -> top-k -> top-p; compare the surviving id set
        w = TemperatureLogitsWarper(0.9)(ids, ref.clone())
        w = TopKLogitsWarper(50)(ids, w)
        w = TopPLogitsWarper(0.8)(ids, w)
        ref_keep = set(np.nonzero(np.isfinite(w[0].numpy()))[0].tolist())
        _, _, keep = sampling.warp(ours, TALK)
        assert set(keep) == ref_keep, trial


def test_topk_ties_kept():
    l = np.array([3, 2, 2, 2, 1, 0], dtype=np.float32)
    _, _, keep = sampling.warp(l, dict(temperature=1.0, top_k=2, top_p=1.0))
    assert sorted(keep) == [0, 1, 2, 3]


def test_top_p_brute_force():
    import itertools
    g = np.random.default_rng(9)
    for trial in range(20):
        V = 8
        # dyadic target probabilities (multiples of 1/64), all distinct
        raw = g.choice(np.arange(1, 40), size=V, replace=False).astype(np.float64)
        p = raw / raw.sum()
        l = np.log(p).astype(np.float32)
        tp = float(g.choice([0.3, 0.5, 0.7, 0.8, 0.9]))
        _, pp, keep = sampling.warp(l, dict(temperature=1.0, top_k=0, top_p=tp))
        # brute force: smallest subset whose mass reaches top_p; among those of that
        # size, the one of largest mass (unique here: distinct probabilities)
        best = None
        for r in range(1, V + 1):
            cands = [s for s in itertools.combinations(range(V), r) if p[list(s)].sum() >= tp - 1e-6]
            if cands:
                best = max(cands, key=lambda s: p[list(s)].sum())
                break
        assert sorted(keep) == sorted(best), (trial, tp)


def test_race_distribution_chi_square():
    from scipy import stats
    p = np.array([0.4, 0.2, 0.15, 0.1, 0.08, 0.04, 0.02, 0.01], dtype=np.float32)
    n = 20000
    counts = np.zeros(8)
    for j in range(n):
        c, _ = sampling.race(p, list(range(8)), lambda i, j=j: philox.exp_noise(1234, 0, 0, j, i))
        counts[c] += 1
    chi2, pv = stats.chisquare(counts, n * p.astype(np.float64) / p.sum())
    assert pv > 1e-4, (counts, pv)


def test_race_lowest_id_on_tie():
    p = np.array([0.5, 0.5], dtype=np.float32)
    c, _ = sampling.race(p, [0, 1], lambda i: np.float32(1.0))
    assert c == 0


def test_philox_matches_numpy():
    g = np.random.default_rng(11)
    for _ in range(16):
        key = [int(x) for x in g.integers(0, 2**63, size=2, dtype=np.int64)]
        ctr = [int(x) for x in g.integers(0, 2**63, size=4, dtype=np.int64)]
        ctr[0] += 1  # numpy increments the counter before producing a block
        ours = philox.philox4x64_10(ctr, key)
        bg = np.random.Philox(key=np.array(key, dtype=np.uint64),
                              counter=np.array([ctr[0] - 1] + ctr[1:], dtype=np.uint64))
        assert tuple(int(x) for x in bg.random_raw(4)) == ours


def test_uniform_open_interval():
    assert philox.uniform_open(0) > 0.0
    assert philox.uniform_open((1 << 64) - 1) < 1.0
    # the noise is positive and finite at both ends
    for x in (0, (1 << 64) - 1):
        e = -np.log(philox.uniform_open(x))
        assert np.isfinite(e) and e > 0
