"""Seeded synthetic inputs for the Qwen3-TTS 12 Hz frame step.

This module only draws random numbers and lays them out: model dimensions,
weights, prompt embeddings, prompt lengths. It holds none of the method's
arithmetic. Both the HIP path (through the tests and the benchmark) and the
CPU oracle are fed from here, so that they see the same inputs.

Recipe (the pages publish no weights, so random ones of the right shape stand
in for the checkpoints):
  * linear weights, embedding tables and heads ~ N(0, 0.02);
  * RMSNorm gains = 1 + N(0, 0.02) (a literal N(0, 0.02) gain would shrink
    every activation ~50x per norm and turn every logit into a near-tie);
  * prompt embeddings ~ N(0, 1);
  * trailing text embeddings and tts_pad ~ N(0, 0.02), the scale of the code
    embedding rows they are summed with in the feedback (at N(0, 1) the pad
    row would swamp the 16 code rows and the talker input would barely depend
    on the codes just drawn);
  * for bf16 configurations every weight tensor is rounded to bf16
    (round-to-nearest-even) and handed out as float32 holding the bf16 value.
Each tensor family draws from its own PCG64 stream, derived from the seed and
the tensor's name, so one tensor never depends on the order others are drawn.
"""
from __future__ import annotations

import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Codec ids of the 12 Hz talker vocabulary (Qwen3-TTS ncnn port discussion,
# section 1 "structure"): 0..2047 acoustic codes, pad 2148, bos 2149, eos 2150.
TALKER_VOCAB = 3072
CODEBOOK = 2048
N_GROUPS = 16
EOS_ID = 2150
SUPPRESS_BEGIN = 2048
SUPPRESS_END = 3072


def _dec(layers, hidden, n_heads, n_kv_heads, head_dim, intermediate,
         rope_theta=1.0e6, rms_eps=1.0e-6):
    return dict(layers=layers, hidden=hidden, n_heads=n_heads,
                n_kv_heads=n_kv_heads, head_dim=head_dim,
                intermediate=intermediate, rope_theta=rope_theta,
                rms_eps=rms_eps)


def dims(name: str) -> dict:
    """Model dimensions of a named workload.

    tiny     - 4-layer talker / 2-layer predictor, hidden 512, GQA 8/4, d 64
    qwen06b  - 0.6B-shaped: 28/5 layers, hidden 1024, GQA 16/8, d 128, I 3072
    qwen17b  - 1.7B-class talker (hidden 2048, I 6144) with a 1024-wide
               predictor behind a 2048->1024 input projection
    """
    base = dict(talker_vocab=TALKER_VOCAB, codebook=CODEBOOK,
                n_groups=N_GROUPS, eos_id=EOS_ID,
                suppress_begin=SUPPRESS_BEGIN, suppress_end=SUPPRESS_END)
    if name == "tiny":
        t = _dec(4, 512, 8, 4, 64, 1536)
        p = _dec(2, 512, 8, 4, 64, 1536)
        return dict(base, talker=t, predictor=p, pred_in_proj=False)
    if name == "qwen06b":
        t = _dec(28, 1024, 16, 8, 128, 3072)
        p = _dec(5, 1024, 16, 8, 128, 3072)
        return dict(base, talker=t, predictor=p, pred_in_proj=False)
    if name == "qwen17b":
        t = _dec(28, 2048, 16, 8, 128, 6144)
        p = _dec(5, 1024, 16, 8, 128, 3072)
        return dict(base, talker=t, predictor=p, pred_in_proj=True)
    raise KeyError(name)


def small_dims(layers_t=2, layers_p=2, hidden=64, n_heads=4, n_kv_heads=2,
               head_dim=16, intermediate=96, vocab=TALKER_VOCAB,
               codebook=CODEBOOK, pred_in_proj=False, pred_hidden=None):
    """A reduced shape for fast tests (vocabulary kept at its real size)."""
    hp = hidden if pred_hidden is None else pred_hidden
    return dict(talker_vocab=vocab, codebook=codebook, n_groups=N_GROUPS,
                eos_id=EOS_ID, suppress_begin=SUPPRESS_BEGIN,
                suppress_end=SUPPRESS_END,
                talker=_dec(layers_t, hidden, n_heads, n_kv_heads, head_dim,
                            intermediate),
                predictor=_dec(layers_p, hp, n_heads, n_kv_heads, head_dim,
                               intermediate),
                pred_in_proj=pred_in_proj)


def _stream(seed: int, name: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([seed, zlib.crc32(name.encode())]))


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    return _bf16_round_inplace(np.array(a, dtype=np.float32, copy=True, order="C"))


def _bf16_round_inplace(a: np.ndarray) -> np.ndarray:
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return a


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that already hold bf16 values."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


class _Normal:
    """A weight tensor still to be drawn: N(mean, std^2) from its own stream."""

    def __init__(self, name, shape, std, mean=0.0):
        self.name, self.shape, self.std, self.mean = name, shape, std, mean

    def draw(self, seed, bf16):
        g = _stream(seed, self.name)
        x = g.standard_normal(size=self.shape, dtype=np.float32)
        if self.std != 1.0:
            x *= np.float32(self.std)
        if self.mean != 0.0:
            x += np.float32(self.mean)
        return _bf16_round_inplace(x) if bf16 else x


def _normal(seed, name, shape, std, mean=0.0):
    return _Normal(name, shape, std, mean).draw(seed, False)


def _decoder_weights(prefix, d, in_hidden=None):
    H = d["hidden"]
    nq, nkv, hd, inter = d["n_heads"], d["n_kv_heads"], d["head_dim"], d["intermediate"]
    layers = []
    for i in range(d["layers"]):
        p = f"{prefix}.{i}."
        layers.append(dict(
            attn_norm=_Normal(p + "attn_norm", (H,), 0.02, 1.0),
            wq=_Normal(p + "wq", (nq * hd, H), 0.02),
            wk=_Normal(p + "wk", (nkv * hd, H), 0.02),
            wv=_Normal(p + "wv", (nkv * hd, H), 0.02),
            q_norm=_Normal(p + "q_norm", (hd,), 0.02, 1.0),
            k_norm=_Normal(p + "k_norm", (hd,), 0.02, 1.0),
            wo=_Normal(p + "wo", (H, nq * hd), 0.02),
            mlp_norm=_Normal(p + "mlp_norm", (H,), 0.02, 1.0),
            w_gate=_Normal(p + "w_gate", (inter, H), 0.02),
            w_up=_Normal(p + "w_up", (inter, H), 0.02),
            w_down=_Normal(p + "w_down", (H, inter), 0.02),
        ))
    return layers


def make_weights(dm: dict, seed: int = 0, dtype: str = "bf16") -> dict:
    """All weights of talker + code predictor, float32 arrays.

    Layout is nn.Linear's [out, in], row-major.  pred_embeds holds the 15
    predictor tables stacked as [15*codebook, talker_hidden]; pred_heads the
    15 heads stacked as [15*codebook, pred_hidden].
    """
    t, p = dm["talker"], dm["predictor"]
    H, Hp = t["hidden"], p["hidden"]
    V, C, G = dm["talker_vocab"], dm["codebook"], dm["n_groups"]
    w = dict(
        talker_layers=_decoder_weights("talker", t),
        talker_norm=_Normal("talker.norm", (H,), 0.02, 1.0),
        talker_codec_embed=_Normal("talker.codec_embed", (V, H), 0.02),
        talker_codec_head=_Normal("talker.codec_head", (V, H), 0.02),
        pred_layers=_decoder_weights("pred", p),
        pred_norm=_Normal("pred.norm", (Hp,), 0.02, 1.0),
        pred_embeds=_Normal("pred.embeds", ((G - 1) * C, H), 0.02),
        pred_heads=_Normal("pred.heads", ((G - 1) * C, Hp), 0.02),
        pred_in_proj=(_Normal("pred.in_proj", (Hp, H), 0.02)
                      if dm["pred_in_proj"] else None),
    )
    if dtype not in ("bf16", "f32"):
        raise ValueError(dtype)
    # every tensor has its own stream, so drawing them in parallel threads
    # gives the same values as drawing them one after another
    leaves = []
    map_arrays(w, lambda x: leaves.append(x) or x)
    workers = max(1, min(16, os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        drawn = dict(zip(map(id, leaves), ex.map(lambda x: x.draw(seed, dtype == "bf16"), leaves)))
    return map_arrays(w, lambda x: drawn[id(x)])


def map_arrays(w, fn):
    """Apply fn to every array of a weight tree (dicts / lists / None kept)."""
    if isinstance(w, dict):
        return {k: map_arrays(v, fn) for k, v in w.items()}
    if isinstance(w, list):
        return [map_arrays(v, fn) for v in w]
    if w is None:
        return None
    return fn(w)


def prompt_lengths(B: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Per-row prompt lengths, uniform on the integers lo..hi inclusive."""
    if lo == hi:
        return np.full(B, lo, dtype=np.int32)
    g = _stream(seed, "prompt_lengths")
    return g.integers(lo, hi + 1, size=B).astype(np.int32)


def make_prompts(lens, hidden: int, seed: int) -> np.ndarray:
    """Packed prompt embeddings [sum(lens), hidden], N(0, 1)."""
    return _normal(seed, "prompt", (int(np.sum(lens)), hidden), 1.0)


def make_text(lens, hidden: int, seed: int) -> np.ndarray:
    """Packed trailing text embeddings [sum(lens), hidden], N(0, 0.02)."""
    return _normal(seed, "text", (int(np.sum(lens)), hidden), 0.02)


def make_tts_pad(hidden: int, seed: int) -> np.ndarray:
    """The tts_pad embedding [hidden], N(0, 0.02)."""
    return _normal(seed, "tts_pad", (hidden,), 0.02)


def split_rows(packed: np.ndarray, lens) -> list:
    """Cut a packed [sum(lens), H] array into per-row views."""
    out, o = [], 0
    for n in lens:
        out.append(packed[o:o + int(n)])
        o += int(n)
    return out


# Sampling settings of the workloads (Qwen3-TTS pages: repetition penalty 1.05,
# min_new_tokens 2, suppress 2048..3071 except EOS; temperature 0.9, top-k 50,
# top-p 0.8 for the sampling workloads).
GREEDY = dict(do_sample=False, temperature=1.0, top_k=0, top_p=1.0,
              repetition_penalty=1.05, min_new_tokens=2)
SAMPLING = dict(do_sample=True, temperature=0.9, top_k=50, top_p=0.8,
                repetition_penalty=1.05, min_new_tokens=2)
# The code predictor has no penalty, min-new or suppress processors.
PRED_GREEDY = dict(do_sample=False, temperature=1.0, top_k=0, top_p=1.0,
                   repetition_penalty=1.0, min_new_tokens=0)
PRED_SAMPLING = dict(do_sample=True, temperature=0.9, top_k=50, top_p=0.8,
                     repetition_penalty=1.0, min_new_tokens=0)


def workload(name: str) -> dict:
    """The five synthetic workloads (shape, batch, prompt lengths, frames, sampling)."""
    if name == "tiny_fp32_b1":
        return dict(model="tiny", dtype="f32", B=1, prompt=(8, 8), frames=4,
                    talker=GREEDY, predictor=PRED_GREEDY, max_positions=64)
    if name == "qwen06b_bf16_b1":
        return dict(model="qwen06b", dtype="bf16", B=1, prompt=(32, 32),
                    frames=100, talker=GREEDY, predictor=PRED_GREEDY,
                    max_positions=160)
    if name == "qwen06b_bf16_b8_sampling":
        return dict(model="qwen06b", dtype="bf16", B=8, prompt=(32, 256),
                    frames=200, talker=SAMPLING, predictor=PRED_SAMPLING,
                    max_positions=512)
    if name == "qwen17b_bf16_b1":
        return dict(model="qwen17b", dtype="bf16", B=1, prompt=(64, 64),
                    frames=250, talker=GREEDY, predictor=PRED_GREEDY,
                    max_positions=320)
    if name == "qwen17b_bf16_b8":
        return dict(model="qwen17b", dtype="bf16", B=8, prompt=(64, 64),
                    frames=250, talker=GREEDY, predictor=PRED_GREEDY,
                    max_positions=320)
    if name == "qwen06b_bf16_b64_sampling":
        return dict(model="qwen06b", dtype="bf16", B=64, prompt=(128, 512),
                    frames=1024, talker=SAMPLING, predictor=PRED_SAMPLING,
                    max_positions=1536)
    raise KeyError(name)


# ---------------------------------------------------------------- token-id frontend
def frontend_dims(name: str) -> dict:
    """Text embedding and ResizeMLP shapes (ncnn port section 1: Qwen2 BPE
    vocabulary of 151936 ids, 2048-wide rows, ResizeMLP 2048 -> 2048 -> talker
    width); "tiny" is a reduced vocabulary and width for fast tests."""
    if name == "tiny":
        return dict(text_vocab=3000, text_hidden=256, mlp_hidden=384)
    return dict(text_vocab=151936, text_hidden=2048, mlp_hidden=2048)


def make_frontend_weights(fd: dict, talker_hidden: int, seed: int = 0, dtype: str = "bf16") -> dict:
    """Text embedding rows ~ N(0, 1) (so the MLP sees its SiLU's curved range),
    the two layers' weights and biases ~ N(0, 0.02)."""
    V, Ti, Hm = fd["text_vocab"], fd["text_hidden"], fd["mlp_hidden"]
    w = dict(text_embed=_Normal("frontend.text_embed", (V, Ti), 1.0),
             fc1_w=_Normal("frontend.fc1_w", (Hm, Ti), 0.02), fc1_b=_Normal("frontend.fc1_b", (Hm,), 0.02),
             fc2_w=_Normal("frontend.fc2_w", (talker_hidden, Hm), 0.02),
             fc2_b=_Normal("frontend.fc2_b", (talker_hidden,), 0.02))
    leaves = []
    map_arrays(w, lambda x: leaves.append(x) or x)
    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        drawn = dict(zip(map(id, leaves), ex.map(lambda x: x.draw(seed, dtype == "bf16"), leaves)))
    return map_arrays(w, lambda x: drawn[id(x)])


def make_prompt_ids(lens, text_vocab: int, seed: int):
    """Dual-track id arrays for prompts of the given lengths, packed row after
    row, laid out like the pages' prompts: a few text-only positions (a role
    prefix: codec track empty, -1), then language-prefix codec ids
    (2050..2071), one built-in speaker id (3063..3071, a codec-table row),
    codec_pad (2148) under the rest of the text, and codec_bos (2149) last.
    Text ids are uniform over the vocabulary. Returns (text_ids, codec_ids)."""
    g = np.random.default_rng(seed)
    tids, cids = [], []
    for P in np.asarray(lens):
        P = int(P)
        t = g.integers(0, text_vocab, P).astype(np.int32)
        c = np.full(P, 2148, dtype=np.int32)
        c[:min(3, P)] = -1
        if P > 5:
            c[3] = g.integers(2050, 2072)
            c[4] = g.integers(3063, 3072)
        c[-1] = 2149
        tids.append(t)
        cids.append(c)
    return np.concatenate(tids), np.concatenate(cids)


# ---------------------------------------------------------------- 12 Hz codec decoder
def codec_dims(name: str) -> dict:
    """Shapes of the codec decoder (ncnn port section 1, Codec Decoder bullet:
    16 codebooks of 2048 x 256, an 8-layer window-72 transformer with hidden
    512, head_dim 64 and rope theta 1e4, two upsampling stages, a vocoder
    upsampling by 8, 5, 4, 3; Mizuoto page: 300-frame chunks with 25 frames
    of left context). "tiny" is a reduced shape for fast tests."""
    if name == "tiny":
        return dict(n_q=16, codebook=2048, codebook_dim=16, hidden=64, layers=2, heads=2, head_dim=32, ffn=128,
                    window=8, rope_theta=1.0e4, up_ffn=128, voc_channels=[96, 48, 24], strides=[2, 3],
                    dilations=[1, 3, 9], chunk=12, context=3)
    return dict(n_q=16, codebook=2048, codebook_dim=256, hidden=512, layers=8, heads=8, head_dim=64, ffn=2048,
                window=72, rope_theta=1.0e4, up_ffn=2048, voc_channels=[1536, 768, 384, 192, 96],
                strides=[8, 5, 4, 3], dilations=[1, 3, 9], chunk=300, context=25)


def make_codec_weights(cd: dict, seed: int = 0, dtype: str = "bf16") -> dict:
    """Random codec-decoder weights: codebook rows ~ N(0, 1); linear and
    convolution weights ~ N(0, 1 / fan_in) (the residual branches' 1x1
    convolutions and the output convolution smaller, so the residual stream
    stays O(1) and the final tanh works mostly in its linear range);
    LayerNorm gains 1 + N(0, 0.02), biases N(0, 0.02); LayerScale gains
    N(0.1, 0.02); SnakeBeta log-parameters N(0, 0.1). Convolution weights
    tap-major [k][out][in]."""
    D, Hd, F = cd["hidden"], cd["heads"] * cd["head_dim"], cd["ffn"]
    cdim = cd["codebook_dim"]
    w = dict(codebooks=_Normal("codec.codebooks", (cd["n_q"], cd["codebook"], cdim), 1.0),
             proj_sem=_Normal("codec.proj_sem", (D, cdim), cdim ** -0.5),
             proj_ac=_Normal("codec.proj_ac", (D, cdim), (15 * cdim) ** -0.5),
             layers=[], up_blocks=[], voc_blocks=[])
    for i in range(cd["layers"]):
        p = f"codec.tf.{i}."
        w["layers"].append(dict(
            ln1_g=_Normal(p + "ln1_g", (D,), 0.02, 1.0), ln1_b=_Normal(p + "ln1_b", (D,), 0.02),
            wqkv=_Normal(p + "wqkv", (3 * Hd, D), D ** -0.5), wo=_Normal(p + "wo", (D, Hd), Hd ** -0.5),
            ls1=_Normal(p + "ls1", (D,), 0.02, 0.1),
            ln2_g=_Normal(p + "ln2_g", (D,), 0.02, 1.0), ln2_b=_Normal(p + "ln2_b", (D,), 0.02),
            fc1=_Normal(p + "fc1", (F, D), D ** -0.5), fc2=_Normal(p + "fc2", (D, F), F ** -0.5),
            ls2=_Normal(p + "ls2", (D,), 0.02, 0.1)))
    w["ln_f_g"] = _Normal("codec.ln_f_g", (D,), 0.02, 1.0)
    w["ln_f_b"] = _Normal("codec.ln_f_b", (D,), 0.02)
    for i in range(2):
        p = f"codec.up.{i}."
        w["up_blocks"].append(dict(
            up=_Normal(p + "up", (2, D, D), D ** -0.5), dw=_Normal(p + "dw", (7, D), 7 ** -0.5),
            ln_g=_Normal(p + "ln_g", (D,), 0.02, 1.0), ln_b=_Normal(p + "ln_b", (D,), 0.02),
            fc1=_Normal(p + "fc1", (cd["up_ffn"], D), D ** -0.5),
            fc2=_Normal(p + "fc2", (D, cd["up_ffn"]), cd["up_ffn"] ** -0.5),
            gamma=_Normal(p + "gamma", (D,), 0.02, 0.1)))
    ch = cd["voc_channels"]
    w["voc_in"] = _Normal("codec.voc_in", (7, ch[0], D), (7 * D) ** -0.5)
    for b, s in enumerate(cd["strides"]):
        p = f"codec.voc.{b}."
        ci, co = ch[b], ch[b + 1]
        units = []
        for u in range(len(cd["dilations"])):
            q = p + f"u{u}."
            units.append(dict(a1=_Normal(q + "a1", (co,), 0.1), b1=_Normal(q + "b1", (co,), 0.1),
                              conv7=_Normal(q + "conv7", (7, co, co), (7 * co) ** -0.5),
                              a2=_Normal(q + "a2", (co,), 0.1), b2=_Normal(q + "b2", (co,), 0.1),
                              conv1=_Normal(q + "conv1", (1, co, co), 0.3 * co ** -0.5)))
        w["voc_blocks"].append(dict(snake_a=_Normal(p + "snake_a", (ci,), 0.1),
                                    snake_b=_Normal(p + "snake_b", (ci,), 0.1),
                                    up=_Normal(p + "up", (2 * s, co, ci), (2 * ci) ** -0.5), units=units))
    w["voc_out_a"] = _Normal("codec.voc_out_a", (ch[-1],), 0.1)
    w["voc_out_b"] = _Normal("codec.voc_out_b", (ch[-1],), 0.1)
    w["voc_out"] = _Normal("codec.voc_out", (7, 1, ch[-1]), 0.15 * (7 * ch[-1]) ** -0.5)
    leaves = []
    map_arrays(w, lambda x: leaves.append(x) or x)
    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        drawn = dict(zip(map(id, leaves), ex.map(lambda x: x.draw(seed, dtype == "bf16"), leaves)))
    return map_arrays(w, lambda x: drawn[id(x)])


def make_codes(T: int, seed: int, codebook: int = CODEBOOK) -> np.ndarray:
    """Random frames of 16 codes, [T, 16] int32, uniform over the codebook."""
    return np.random.default_rng(seed).integers(0, codebook, (T, N_GROUPS)).astype(np.int32)
