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

    Returns (id, info). Greedy: info['margin'] is the top-2 gap of the
    processed logits. Sampling: info['race_gap'] is the gap between the two
    best race scores ln p - ln E, times the temperature (logit units), and
    info['keep'] the number of ids that survive top-k and top-p.
    """
    if not samp["do_sample"]:
        return greedy(processed), dict(margin=top2_margin(processed))
    z, p, keep = warp(processed, samp)
    cid, gap = race(p, keep, noise)
    return cid, dict(race_gap=gap * float(samp["temperature"]), keep=len(keep))


# ---------------------------------------------------------------- decision margins
# A selection made from logits l' with max_i |l'_i - l_i| <= delta can differ
# from the selection made from l only if the perturbation can move one of the
# comparisons the selection rests on. flip_possible() answers, for a given
# pair of ids (a = the choice from l, b = another id), whether some such
# perturbation could make b the choice; it errs only towards True (a
# sufficient test for "cannot flip"). Every bound is in raw-logit units:
# temperature divides the logits, so tempered logits move by delta / T.

def _topk_member_can_flip(l, k, i, delta):
    """Can top-k membership of id i (kept iff fewer than k ids are strictly
    above it) change when every finite logit moves by at most delta?"""
    others = np.delete(l, i)
    others = others[np.isfinite(others)]
    if l[i] >= np.sort(np.concatenate([others, [l[i]]]))[::-1][k - 1]:
        # kept: drops out only if k others can end strictly above it
        return int(np.sum(others >= l[i] - 2.0 * delta)) >= k
    # dropped: enters only if fewer than k others can stay strictly above it
    return int(np.sum(others > l[i] + 2.0 * delta)) < k


def _topp_member_can_flip(l, samp, i, delta):
    """Can top-p membership of id i change under a delta perturbation?

    i is kept iff the probability mass S of the ids ordered ahead of it
    (p desc, id asc) is below top_p. With the set ahead of it fixed, a
    perturbation scales each tempered weight by at most e^(delta/T) either
    way, so S' lies within [S / (S + (1 - S) r), S r / (S r + 1 - S)] with
    r = e^(2 delta / T). Ids whose logits lie within 2 delta of l_i may change
    sides, and ids within 2 delta of the top-k threshold may enter or leave
    the normalising set; both widen the interval.
    """
    T = float(samp["temperature"])
    top_p = float(samp["top_p"])
    k = int(samp["top_k"])
    z, p = tempered_softmax(l, samp)
    p = p.astype(np.float64)
    ids = [j for j in range(p.size) if p[j] > 0]
    ids.sort(key=lambda j: (-p[j], j))
    pos = ids.index(i)
    S = float(np.sum(p[ids[:pos]]))
    near = [j for j in ids if j != i and abs(float(l[j]) - float(l[i])) <= 2.0 * delta]
    ahead_near = sum(p[j] for j in near if ids.index(j) < pos)
    behind_near = sum(p[j] for j in near if ids.index(j) > pos)
    # mass that may leave / enter the top-k set (tail ids near its threshold)
    p_out = p_in = 0.0
    fin = l[np.isfinite(l)]
    if 0 < k < fin.size:
        srt = np.sort(fin)[::-1]
        kth, nxt = float(srt[k - 1]), float(srt[k])
        m = float(np.max(z[np.isfinite(z)]))
        Z = float(np.sum(np.exp(z[np.isfinite(z)].astype(np.float64) - m)))
        for j in range(l.size):
            if j == i or not np.isfinite(l[j]):
                continue
            if p[j] > 0 and float(l[j]) - nxt <= 2.0 * delta:
                p_out += p[j]
            elif p[j] == 0 and kth - float(l[j]) <= 2.0 * delta:
                p_in += float(np.exp(np.float64(l[j]) / T - m)) / Z
    r = float(np.exp(2.0 * delta / T))
    if S < top_p:   # kept: can the mass ahead reach top_p?
        s_plus = S + behind_near
        rest = max(0.0, 1.0 - s_plus - p_out)
        return s_plus * r / (s_plus * r + rest) >= top_p if s_plus > 0 else False
    s_minus = max(0.0, S - ahead_near)
    rest = 1.0 - s_minus + p_in * r
    return s_minus / (s_minus + rest * r) < top_p


def member_can_flip(l, samp, i, delta):
    """Can the survival of id i through top-k and top-p change under a delta
    perturbation of the processed logits l? (-inf ids never survive.)"""
    l = np.asarray(l, dtype=np.float64)
    if not np.isfinite(l[i]):
        return False
    k = int(samp["top_k"])
    n_fin = int(np.sum(np.isfinite(l)))
    if 0 < k < n_fin:
        if _topk_member_can_flip(l, k, i, delta):
            return True
        kth = np.sort(l[np.isfinite(l)])[::-1][k - 1]
        if l[i] < kth:
            return False          # out of top-k and cannot enter
    if float(samp["top_p"]) >= 1.0:
        return False
    return _topp_member_can_flip(np.asarray(l, dtype=np.float32), samp, i, delta)


def flip_possible(processed, samp, noise, a, b, delta):
    """Could logits within delta (max norm) of `processed` make the selection
    b instead of a (a = the selection from `processed`)?

    Greedy: only if l_a - l_b <= 2 delta. Sampling (exponential race): b can
    win only if both race scores ln p - ln E can meet, i.e.
    (l_a - l_b) / T - ln E_a + ln E_b <= 2 delta / T (the normaliser is common
    to both), and b survives top-k / top-p on the perturbed side; or a itself
    can drop out of the survivors, after which any survivor may win.
    """
    l = np.asarray(processed, dtype=np.float32)
    if a == b:
        return True
    if not np.isfinite(l[b]):
        return False
    if not samp["do_sample"]:
        return float(l[a]) - float(l[b]) <= 2.0 * delta
    if member_can_flip(l, samp, a, delta):
        return True
    T = float(samp["temperature"])
    ds = (float(l[a]) - float(l[b])) / T - float(np.log(np.float64(noise(a)))) + float(np.log(np.float64(noise(b))))
    if ds > 2.0 * delta / T:
        return False
    _, _, keep = warp(l, samp)
    return b in keep or member_can_flip(l, samp, b, delta)
