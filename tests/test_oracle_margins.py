"""Pins of the oracle's decision-margin helpers, which decide when a GPU
choice that differs from the oracle's is excused in the parity tests.

The rule they implement (the parity tolerance rule, restated): a teacher-forced
choice may differ from the oracle's only where the oracle's decision could
change under a perturbation of the logits of the size the tolerance allows.
Each pin below fixes a value by hand or checks the helper against brute
force, so that a dropped factor (2 delta, the temperature), a wrong sign, or
a gap measured in the wrong units fails here:

  * top2_margin on hand-built logits (ties, -inf, a single finite value);
  * greedy flips: exactly at l_a - l_b = 2 delta;
  * the race: dyadic probabilities and hand-picked Exp(1) values, the flip
    threshold at delta = T ln 2 / 2;
  * top-k membership: an id 0.1 below the k-th value enters at delta = 0.05;
  * top-p membership: the worst-case mass ahead S r / (S r + 1 - S) reaches
    top_p at exactly delta = ln(4/3) / 2 in a dyadic case, checked against
    the explicit worst-case perturbation;
  * soundness by brute force: random perturbations within delta that change
    the selection are always reported as possible flips;
  * non-vacuity: well-separated decisions are never excused.
"""
import math

import numpy as np

from oracle import sampling

GREEDY = dict(do_sample=False, temperature=1.0, top_k=0, top_p=1.0, repetition_penalty=1.0, min_new_tokens=0)


def samp(T=1.0, k=0, p=1.0):
    return dict(do_sample=True, temperature=T, top_k=k, top_p=p, repetition_penalty=1.0, min_new_tokens=0)


def test_top2_margin_hand_values():
    l = np.array([0.5, 2.0, 1.25, -np.inf, 1.75], dtype=np.float32)
    assert sampling.top2_margin(l) == 0.25
    l2 = np.array([1.0, 3.0, 3.0], dtype=np.float32)
    assert sampling.top2_margin(l2) == 0.0
    l3 = np.array([-np.inf, 4.0, -np.inf], dtype=np.float32)
    assert sampling.top2_margin(l3) == float("inf")
    l4 = np.array([-2.0, -0.5, -1.5], dtype=np.float32)
    assert sampling.top2_margin(l4) == 1.0


def test_greedy_flip_threshold():
    l = np.array([0.0, 1.0, 0.7, -np.inf], dtype=np.float32)
    a = sampling.greedy(l)
    assert a == 1
    gap = float(l[1]) - float(l[2])
    assert not sampling.flip_possible(l, GREEDY, None, a, 2, gap / 2 * 0.99)
    assert sampling.flip_possible(l, GREEDY, None, a, 2, gap / 2 * 1.01)
    assert not sampling.flip_possible(l, GREEDY, None, a, 3, 100.0)   # masked ids never win


def test_race_flip_threshold_dyadic():
    T = 0.9
    p = np.array([0.5, 0.25, 0.125, 0.125])
    l = (T * np.log(p)).astype(np.float32)
    E = {0: np.float32(1.0), 1: np.float32(1.0), 2: np.float32(0.5), 3: np.float32(2.0)}
    s = samp(T)
    a, info = sampling.select(l, s, lambda i: E[i])
    # scores p/E: 0.5, 0.25, 0.25, 0.0625 -> id 0, ids 1 and 2 second, ln 2 below in log units
    assert a == 0
    assert abs(info["race_gap"] - T * math.log(2.0)) < 1e-5
    thr = T * math.log(2.0) / 2.0      # (l_a - l_b)/T + ln(E_b / E_a) = ln 2  <=  2 delta / T
    assert not sampling.flip_possible(l, s, lambda i: E[i], 0, 1, thr * 0.99)
    assert sampling.flip_possible(l, s, lambda i: E[i], 0, 1, thr * 1.01)
    assert sampling.flip_possible(l, s, lambda i: E[i], 0, 2, thr * 1.01)
    # id 3 is ln 8 behind: needs delta >= T ln 8 / 2
    assert not sampling.flip_possible(l, s, lambda i: E[i], 0, 3, thr * 2.9)
    assert sampling.flip_possible(l, s, lambda i: E[i], 0, 3, thr * 3.01)


def test_topk_membership_threshold():
    l = np.array([5.0, 4.0, 3.0, 2.9, 1.0, 0.0], dtype=np.float32)
    s = samp(1.0, k=3)
    gap = float(l[2]) - float(l[3])           # 0.1 (in float32)
    assert not sampling.member_can_flip(l, s, 3, gap / 2 * 0.98)
    assert sampling.member_can_flip(l, s, 3, gap / 2 * 1.02)
    assert not sampling.member_can_flip(l, s, 2, gap / 2 * 0.98)
    assert sampling.member_can_flip(l, s, 2, gap / 2 * 1.02)
    assert not sampling.member_can_flip(l, s, 0, 0.4)   # 1.0 above the k-th
    assert not sampling.member_can_flip(l, s, 5, 0.9)   # 3.0 below the k-th


def _keep_after(l, s):
    return set(sampling.warp(np.asarray(l, np.float32), s)[2])


def test_topp_membership_threshold_dyadic():
    p = np.array([0.5, 0.25, 0.125, 0.0625, 0.0625])
    l = np.log(p).astype(np.float32)
    s = samp(1.0, p=0.8)
    assert _keep_after(l, s) == {0, 1, 2}          # running sums 0.5, 0.75, 0.875
    thr = math.log(4.0 / 3.0) / 2.0               # 0.75 r / (0.75 r + 0.25) = 0.8 at r = 4/3
    assert not sampling.member_can_flip(l, s, 2, thr * 0.97)
    assert sampling.member_can_flip(l, s, 2, thr * 1.03)
    # the worst case it describes is real: ids 0 and 1 up by delta, the rest down
    for d, out in ((thr * 1.03, True), (thr * 0.97, False)):
        lp = l.astype(np.float64) + np.array([d, d, -d, -d, -d])
        assert (2 not in _keep_after(lp, s)) == out
    # id 3 (dropped, mass ahead 0.875): enters when 0.875 / (0.875 + 0.125 r) < 0.8,
    # with every id behind the cut (3 and 4) up by delta and the rest down
    thr3 = math.log(0.875 * 0.2 / (0.8 * 0.125)) / 2.0
    assert not sampling.member_can_flip(l, s, 3, thr3 * 0.97)
    lp = l.astype(np.float64) + np.array([-1, -1, -1, 1, 1]) * thr3 * 1.03
    assert 3 in _keep_after(lp, s)
    assert sampling.member_can_flip(l, s, 3, thr3 * 1.03)


def test_flip_possible_is_sound_by_brute_force():
    """Random logits with near-ties; whenever a perturbation within delta
    changes the selection, flip_possible must say so."""
    g = np.random.default_rng(5)
    settings = [samp(0.9, k=5, p=0.7), samp(1.0, k=0, p=0.6), samp(0.7, k=4, p=1.0), GREEDY]
    checked = 0
    for trial in range(60):
        V = 10
        l = (g.standard_normal(V) * 0.6).astype(np.float32)
        l[g.integers(V)] = -np.inf
        E = {i: np.float32(-math.log(g.uniform(1e-3, 1.0))) for i in range(V)}
        for s in settings:
            noise = (lambda i: E[i])
            a, _ = sampling.select(l, s, noise)
            for delta in (0.02, 0.1):
                for _ in range(40):
                    d = g.uniform(-delta, delta, V)
                    d[g.random(V) < 0.5] = np.sign(d[g.random(V) < 0.5].sum() + 1e-9) * delta
                    lp = (l.astype(np.float64) + d).astype(np.float32)
                    b, _ = sampling.select(lp, s, noise)
                    if b != a:
                        checked += 1
                        assert sampling.flip_possible(l, s, noise, a, b, delta * 1.0001), (trial, s, a, b, delta)
    assert checked > 50


def test_well_separated_decisions_are_never_excused():
    T = 0.9
    l = np.array([4.0, 3.0, 2.0, 1.0, 0.0, -1.0, -2.0, -3.0], dtype=np.float32)
    E = {i: np.float32(1.0) for i in range(8)}
    for s in (samp(T, k=4, p=0.95), samp(T, k=0, p=0.99), GREEDY):
        a, _ = sampling.select(l, s, lambda i: E[i])
        assert a == 0
        for b in range(1, 8):
            assert not sampling.flip_possible(l, s, lambda i: E[i], a, b, 0.01)
