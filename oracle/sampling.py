"""Logits processors, warpers and the single-sample race.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Order of the talker chain (Mizuoto engine page, "Matching upstream",
sampler bullet; ncnn port section 6): repetition penalty -> min-new-tokens
EOS mask -> suppress control ids -> (greedy argmax | temperature -> top-k ->
top-p -> one multinomial draw). The draw is computed as
argmax over kept ids of p_i / E_i with E_i ~ Exp(1) (Mizuoto "Speed": the
computation multinomial itself performs, without its checks).

Processor rules (ncnn CustomVoice port, section 3.2; ncnn port section 1,
fact 3):
  * repetition penalty rho: an id already drawn has its logit divided by rho
    when positive and multiplied by rho when negative;
  * min_new_tokens: while fewer selections than min_new_tokens have been
    made, the EOS logit is -inf and the next best id wins (no resampling);
  * suppress [suppress_begin, suppress_end) except EOS: -inf;
  * NaN (or +inf) logits fail closed; argmax ties go to the lowest index.
The code predictor has only the warpers (no penalty, min-new or suppress).
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
NEG_INF = F32(-np.inf)


class NonFinite(Exception):
    pass


def check_finite(logits):
    l = np.asarray(logits)
    if np.isnan(l).any() or np.isposinf(l).any():
        raise NonFinite("non-finite logit")


def repetition_penalty(l, seen_ids, rho):
    """Divide positive / multiply negative logits of seen ids by rho (once per id)."""
    l = l.copy()
    rho = F32(rho)
    for i in sorted(set(int(s) for s in seen_ids)):
        l[i] = l[i] * rho if l[i] < 0 else l[i] / rho
    return l


def talker_process(logits, seen_ids, n_selected, samp, cfg):
    """Processors of the talker, in order. Returns float32 processed logits."""
    l = np.array(logits, dtype=F32)
    check_finite(l)
    if samp["repetition_penalty"] != 1.0:
        l = repetition_penalty(l, seen_ids, samp["repetition_penalty"])
    eos = cfg["eos_id"]
    if n_selected < samp["min_new_tokens"]:
        l[eos] = NEG_INF
    for i in range(cfg["suppress_begin"], cfg["suppress_end"]):
        if i != eos:
            l[i] = NEG_INF
    return l


def greedy(l):
    """Lowest-index argmax (numpy returns the first maximum)."""
    return int(np.argmax(l))


def top2_margin(l):
    """Gap between the largest and second-largest finite values (inf if only one)."""
    f = np.sort(l[np.isfinite(l)])[::-1]
    if f.size < 2:
        return float("inf")
    return float(f[0] - f[1])


def tempered_softmax(l, samp):
    """Temperature -> top-k -> softmax. Returns (z, p), both float32.

    Top-k keeps every id whose value is >= the k-th largest (ties at the
    threshold kept); the others get -inf and probability 0.
    """
    z = l / F32(samp["temperature"])
    k = int(samp["top_k"])
    if 0 < k < z.size:
        kth = np.sort(z)[::-1][k - 1]
        z = np.where(z < kth, NEG_INF, z).astype(F32)
    m = np.max(z)
    e = np.exp(z - m)
    s = np.sum(e, dtype=F32)
    p = (e / s).astype(F32)
    return z, p


def top_p_keep(p, top_p):
    """Ids that survive top-p, ordered by (p desc, id asc).

    Keeps the shortest prefix of that order whose float32 running sum reaches
    top_p (the crossing id included, at least one id); top_p >= 1 keeps every
    id with p > 0.
    """
    ids = [i for i in range(p.size) if p[i] > 0]
    ids.sort(key=lambda i: (-p[i], i))
    if float(top_p) >= 1.0:
        return ids
    csum = np.cumsum(p[ids], dtype=F32)
    hit = np.nonzero(csum >= F32(top_p))[0]
    n = int(hit[0]) + 1 if hit.size else len(ids)
    return ids[:n]


def warp(l, samp):
    """Temperature -> top-k -> softmax -> top-p: returns (z, p, keep)."""
    z, p = tempered_softmax(l, samp)
    return z, p, top_p_keep(p, samp["top_p"])


def race(p, keep, noise):
    """argmax over kept ids of p_i / E_i, float32, lowest id on ties.

    noise(i) returns E_i (float32). Also returns the gap, in log units, between
    the best and second-best ln p - ln E (inf when one id is kept).
    """
    best, best_s = None, None
    scores = []
    for i in sorted(keep):
        s = F32(p[i] / noise(i))
        scores.append((float(np.log(np.float64(p[i]))) - float(np.log(np.float64(noise(i)))), i))
        if best is None or s > best_s:
            best, best_s = i, s
    scores.sort(reverse=True)
    gap = scores[0][0] - scores[1][0] if len(scores) > 1 else float("inf")
    return best, gap


def select(processed, samp, noise):
    """Choose one id from processed logits.

    Returns (id, info). info['margin'] is the decision margin that the
    parity tests use: greedy -> top-2 gap of the processed logits; sampling ->
    min(race gap / temperature-free log units converted back to logit units,
    top-k threshold gap), all in units of raw logits.
    """
    if not samp["do_sample"]:
        return greedy(processed), dict(margin=top2_margin(processed))
    z, p, keep = warp(processed, samp)
    cid, gap = race(p, keep, noise)
    T = float(samp["temperature"])
    info = dict(race_gap=gap * T, keep=len(keep))
    # threshold gaps: how far the k-th value sits from the (k+1)-th, and how far
    # the top-p running sum sits from top_p at the cut (both in logit units)
    k = int(samp["top_k"])
    fz = np.sort(processed[np.isfinite(processed)])[::-1]
    info["topk_gap"] = float(fz[k - 1] - fz[k]) if 0 < k < fz.size else float("inf")
    tp = float(samp["top_p"])
    if tp < 1.0:
        ids = sorted([i for i in range(p.size) if p[i] > 0], key=lambda i: (-p[i], i))
        csum = np.cumsum(p[ids], dtype=np.float64)
        n = len(keep)
        # distance of top_p from the running sums on either side of the cut
        lo = csum[n - 2] if n >= 2 else 0.0
        hi = csum[n - 1]
        info["topp_gap"] = float(min(abs(tp - lo), abs(hi - tp)))
    else:
        info["topp_gap"] = float("inf")
    info["margin"] = min(info["race_gap"], info["topk_gap"])
    return cid, info
