"""The per-frame generation loop of the Qwen3-TTS 12 Hz model.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Per row, independently (rows of a batch never interact; finished rows of a
GPU batch are fed EOS, which changes nothing for the other rows):

  prefill   talker over the prompt embeddings at positions 0..P-1; the
            final-norm hidden of the last position, h, goes through the codec
            head and selection 0 picks the first code 0.
  frame k   stop if code 0 is EOS (reason "stop") or k == max_frames (reason
            "length"; the lookahead is discarded). Otherwise:
            * code predictor, fresh cache: a 2-token prefill [h ; talker
              table(code 0)] at positions 0,1, head[0] on the last position
              -> code 1; then for s = 1..14 one token table[s-1](code s) at
              position s+1, head[s] -> code s+1 (ncnn port section 1: step s
              embeds with table s-1 and applies head s);
            * the frame is (code 0, codes 1..15), assembled one step late;
            * feedback e = talker table(code 0) + sum of table[j-1](code j),
              j = 1..15, + the next trailing text embedding (tts_pad once the
              text is used up), summed left to right (Mizuoto "How it works";
              ncnn port section 1);
            * talker step on e at position P + k -> h, codec head, selection
              k + 1 picks the next code 0.
  So N frames take N + 1 talker selections and 15 N predictor passes (ncnn
  CustomVoice port, section 3.1).

Sampling noise: stream 0 is the talker (index = selection number), stream s
(1..15) the predictor's code s (index = frame number); see philox.py.

Teacher forcing: with forced[r] of shape [F, 16], frame k commits
forced[r][k][0] as its code 0 and feeds forced[r][k][s] as code s to the
predictor chain and the feedback sum; the oracle's own choices are still
recorded. Exactly F frames are run.
"""
from __future__ import annotations

import numpy as np

from . import model, sampling
from .philox import exp_noise
from .sampling import NonFinite as OracleNonFinite


def _select(logits, samp, seen, n_sel, cfg, noise, talker):
    if talker:
        l = sampling.talker_process(logits, seen, n_sel, samp, cfg)
    else:
        l = np.array(logits, dtype=np.float32)
        sampling.check_finite(l)
    return sampling.select(l, samp, noise)


def prefill_row(w, dm, prompt, max_pos, dt=np.float32, tabs=None):
    """Talker over one row's prompt. Returns (cache, h, logits)."""
    t = dm["talker"]
    cos, sin = tabs if tabs is not None else model.rope_tables(max_pos, t["head_dim"], t["rope_theta"])
    cache = model.KVCache(t["layers"], t["n_kv_heads"], max_pos, t["head_dim"], dt)
    y = model.decoder_forward(w["talker_layers"], w["talker_norm"], prompt, cache, 0, t, cos, sin, dt)
    h = y[-1]
    logits = h @ np.asarray(w["talker_codec_head"], dtype=dt).T
    return cache, h, logits


def _pred_input(w, x, dt):
    if w.get("pred_in_proj") is None:
        return np.asarray(x, dtype=dt)
    return np.asarray(x, dtype=dt) @ np.asarray(w["pred_in_proj"], dtype=dt).T


def generate(w, dm, prompts, tts_pad, talker_samp, pred_samp, seed, max_frames,
             texts=None, rows=None, forced=None, dt=np.float32, record=True):
    """Generate frames for each row. Returns one result dict per row.

    prompts: list of [P_r, H] arrays; texts: list of [n_r, H] arrays or None;
    rows: global row ids (for the noise counters), default 0..B-1;
    forced: list of [F_r, 16] int arrays or None (teacher forcing).
    """
    t, p = dm["talker"], dm["predictor"]
    C = dm["codebook"]
    eos = dm["eos_id"]
    cfg = dict(eos_id=eos, suppress_begin=dm["suppress_begin"], suppress_end=dm["suppress_end"])
    B = len(prompts)
    rows = list(range(B)) if rows is None else list(rows)
    T_emb = np.asarray(w["talker_codec_embed"], dtype=dt)
    T_head = np.asarray(w["talker_codec_head"], dtype=dt)
    P_tab = np.asarray(w["pred_embeds"], dtype=dt)
    P_head = np.asarray(w["pred_heads"], dtype=dt)
    pad = np.asarray(tts_pad, dtype=dt)
    max_pos_t = max(int(pr.shape[0]) for pr in prompts) + max_frames + 1
    tab_t = model.rope_tables(max_pos_t, t["head_dim"], t["rope_theta"])
    tab_p = model.rope_tables(16, p["head_dim"], p["rope_theta"])
    out = []
    for b in range(B):
        row = rows[b]
        prompt = np.asarray(prompts[b], dtype=dt)
        P = prompt.shape[0]
        text = None if texts is None else np.asarray(texts[b], dtype=dt)
        n_text = 0 if text is None else text.shape[0]
        fz = None if forced is None else np.asarray(forced[b])
        n_force = None if fz is None else fz.shape[0]

        cache, h, logits = prefill_row(w, dm, prompt, max_pos_t, dt, tab_t)
        seen = []
        n_sel = 0
        code0, info = _select(logits, talker_samp, seen, n_sel,
                              cfg, lambda i: exp_noise(seed, row, 0, 0, i), True)
        n_sel += 1
        rec = dict(talker_logits=[logits.astype(np.float32)] if record else [],
                   talker_choice=[code0], talker_info=[info],
                   pred_logits=[], pred_choice=[], pred_info=[], codes=[],
                   n_predictor_passes=0)
        k = 0
        finish = None
        while True:
            if fz is not None:
                if k == n_force:
                    finish = "forced"
                    break
                code0 = int(fz[k][0])
            else:
                if code0 == eos:
                    finish = "stop"
                    break
                if k == max_frames:
                    finish = "length"
                    break
            seen.append(code0)
            codes = [code0]
            own = []
            plog, pinf = [], []
            # predictor pass 0: [h ; talker table(code 0)] at positions 0, 1
            pc = model.KVCache(p["layers"], p["n_kv_heads"], 16, p["head_dim"], dt)
            x = _pred_input(w, np.stack([h, T_emb[code0]]), dt)
            z = model.decoder_forward(w["pred_layers"], w["pred_norm"], x, pc, 0, p, *tab_p, dt=dt)
            rec["n_predictor_passes"] += 1
            for s in range(0, 15):
                if s > 0:
                    # step s: table[s-1](code s) at position s+1
                    x = _pred_input(w, P_tab[(s - 1) * C + codes[s]][None, :], dt)
                    z = model.decoder_forward(w["pred_layers"], w["pred_norm"], x, pc, s + 1, p, *tab_p, dt=dt)
                    rec["n_predictor_passes"] += 1
                lg = z[-1] @ P_head[s * C:(s + 1) * C].T
                c, inf = _select(lg, pred_samp, None, 0, cfg,
                                 lambda i, s=s: exp_noise(seed, row, s + 1, k, i), False)
                own.append(c)
                if record:
                    plog.append(lg.astype(np.float32))
                pinf.append(inf)
                codes.append(int(fz[k][s + 1]) if fz is not None else c)
            rec["codes"].append(codes)
            rec["pred_choice"].append(own)
            rec["pred_logits"].append(plog)
            rec["pred_info"].append(pinf)
            # feedback sum, left to right
            e = T_emb[codes[0]].copy()
            for j in range(1, 16):
                e = e + P_tab[(j - 1) * C + codes[j]]
            e = e + (text[k] if k < n_text else pad)
            y = model.decoder_forward(w["talker_layers"], w["talker_norm"], e[None, :], cache, P + k, t, *tab_t, dt=dt)
            h = y[0]
            logits = h @ T_head.T
            code0, info = _select(logits, talker_samp, seen, n_sel, cfg,
                                  lambda i, j=n_sel: exp_noise(seed, row, 0, j, i), True)
            n_sel += 1
            if record:
                rec["talker_logits"].append(logits.astype(np.float32))
            rec["talker_choice"].append(code0)
            rec["talker_info"].append(info)
            k += 1
        rec["finish"] = finish
        rec["n_frames"] = len(rec["codes"])
        rec["n_talker_selections"] = n_sel
        rec["codes"] = np.array(rec["codes"], dtype=np.int32).reshape(-1, 16)
        rec["pred_choice"] = np.array(rec["pred_choice"], dtype=np.int32).reshape(-1, 15)
        rec["talker_choice"] = np.array(rec["talker_choice"], dtype=np.int32)
        if record:
            rec["talker_logits"] = np.stack(rec["talker_logits"])
            rec["pred_logits"] = (np.array(rec["pred_logits"], dtype=np.float32)
                                  if rec["pred_logits"] else np.zeros((0, 15, C), np.float32))
        out.append(rec)
    return out
