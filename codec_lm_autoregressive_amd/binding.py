"""ctypes binding of libqt.so (include/qt.h), argument marshalling only.

Every step of the frame runs in the HIP library; this module only turns
Python / numpy / torch objects into the C structures and device pointers the
ABI takes. torch provides device memory and the stream. The library must be
built (codec_lm_autoregressive_amd.build); importing the binding without it
raises - there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqt.so")

QT_OK, QT_E_INVALID, QT_E_RANGE, QT_E_CAPACITY, QT_E_NOMEM, QT_E_HIP, QT_E_NAN, QT_E_STATE = range(8)
QT_DTYPE_F32, QT_DTYPE_BF16, QT_DTYPE_F16 = 0, 1, 2
_DTYPES = {"f32": QT_DTYPE_F32, "bf16": QT_DTYPE_BF16, "f16": QT_DTYPE_F16}
STATUS_NAMES = {0: "QT_OK", 1: "QT_E_INVALID", 2: "QT_E_RANGE", 3: "QT_E_CAPACITY", 4: "QT_E_NOMEM",
                5: "QT_E_HIP", 6: "QT_E_NAN", 7: "QT_E_STATE"}


class QtError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class DecoderDims(C.Structure):
    _fields_ = [("layers", C.c_int32), ("hidden", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("intermediate", C.c_int32),
                ("rope_theta", C.c_float), ("rms_eps", C.c_float)]


class Config(C.Structure):
    _fields_ = [("talker", DecoderDims), ("predictor", DecoderDims), ("talker_vocab", C.c_int32),
                ("n_groups", C.c_int32), ("codebook", C.c_int32), ("eos_id", C.c_int32),
                ("suppress_begin", C.c_int32), ("suppress_end", C.c_int32), ("pred_in_proj", C.c_int32),
                ("weight_dtype", C.c_int32), ("kv_dtype", C.c_int32), ("max_batch", C.c_int32),
                ("max_positions", C.c_int32)]


class LayerWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo",
                                          "mlp_norm", "w_gate", "w_up", "w_down")]


class Weights(C.Structure):
    _fields_ = [("talker_layers", C.POINTER(LayerWeights)), ("talker_norm", C.c_void_p),
                ("talker_codec_embed", C.c_void_p), ("talker_codec_head", C.c_void_p),
                ("pred_layers", C.POINTER(LayerWeights)), ("pred_norm", C.c_void_p),
                ("pred_embeds", C.c_void_p), ("pred_heads", C.c_void_p), ("pred_in_proj", C.c_void_p)]


class Sampling(C.Structure):
    _fields_ = [("do_sample", C.c_int32), ("temperature", C.c_float), ("top_k", C.c_int32),
                ("top_p", C.c_float), ("repetition_penalty", C.c_float), ("min_new_tokens", C.c_int32)]


class FrontendConfig(C.Structure):
    _fields_ = [("text_vocab", C.c_int32), ("text_hidden", C.c_int32), ("mlp_hidden", C.c_int32),
                ("max_rows", C.c_int32)]


class FrontendWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("text_embed", "fc1_w", "fc1_b", "fc2_w", "fc2_b")]


CODEC_MAX_BLOCKS, CODEC_UNITS = 6, 3


class CodecConfig(C.Structure):
    _fields_ = [("n_q", C.c_int32), ("codebook", C.c_int32), ("codebook_dim", C.c_int32), ("hidden", C.c_int32),
                ("layers", C.c_int32), ("heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
                ("window", C.c_int32), ("rope_theta", C.c_float), ("up_ffn", C.c_int32), ("n_blocks", C.c_int32),
                ("channels", C.c_int32 * (CODEC_MAX_BLOCKS + 1)), ("strides", C.c_int32 * CODEC_MAX_BLOCKS),
                ("dilations", C.c_int32 * CODEC_UNITS), ("chunk", C.c_int32), ("context", C.c_int32),
                ("weight_dtype", C.c_int32)]


class CodecLayerWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("ln1_g", "ln1_b", "wqkv", "wo", "ls1", "ln2_g", "ln2_b", "fc1", "fc2",
                                          "ls2")]


class CodecUpWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("up", "dw", "ln_g", "ln_b", "fc1", "fc2", "gamma")]


class CodecUnitWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("a1", "b1", "conv7", "a2", "b2", "conv1")]


class CodecBlockWeights(C.Structure):
    _fields_ = [("snake_a", C.c_void_p), ("snake_b", C.c_void_p), ("up", C.c_void_p),
                ("units", CodecUnitWeights * CODEC_UNITS)]


class CodecWeights(C.Structure):
    _fields_ = [("codebooks", C.c_void_p), ("proj_sem", C.c_void_p), ("proj_ac", C.c_void_p),
                ("layers", C.POINTER(CodecLayerWeights)), ("ln_f_g", C.c_void_p), ("ln_f_b", C.c_void_p),
                ("up", CodecUpWeights * 2), ("voc_in", C.c_void_p), ("blocks", CodecBlockWeights * CODEC_MAX_BLOCKS),
                ("voc_out_a", C.c_void_p), ("voc_out_b", C.c_void_p), ("voc_out", C.c_void_p)]


_lib = None


def lib():
    """The loaded library (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with python -m codec_lm_autoregressive_amd.build")
        L = C.CDLL(LIB_PATH)
        vp, i32, u64, f32 = C.c_void_p, C.c_int32, C.c_uint64, C.c_float
        sig = {
            "qt_config_check": ([C.POINTER(Config)], i32),
            "qt_workspace_bytes": ([C.POINTER(Config), C.POINTER(C.c_size_t)], i32),
            "qt_create": ([C.POINTER(Config), C.POINTER(Weights), vp, C.c_size_t, vp, C.POINTER(vp)], i32),
            "qt_prefill": ([vp, i32, vp, vp, vp, vp, vp, C.POINTER(Sampling), C.POINTER(Sampling), u64, i32], i32),
            "qt_step_frame": ([vp, vp, vp], i32),
            "qt_generate": ([vp, i32, vp, vp, vp, vp, vp, C.POINTER(Sampling), C.POINTER(Sampling), u64, i32,
                             vp, vp, vp], i32),
            "qt_destroy": ([vp], None),
            "qt_last_error": ([vp], C.c_char_p),
            "qt_debug_step_forced": ([vp, vp, vp, vp, vp], i32),
            "qt_debug_talker_logits": ([vp, vp], i32),
            "qt_debug_select": ([vp, i32, i32, vp, vp, vp, vp, i32, i32, i32, i32, C.POINTER(Sampling), u64, i32,
                                 i32, vp, vp, vp], i32),
            "qt_admit": ([vp, i32, vp, i32, vp, i32, u64, i32, i32], i32),
            "qt_frontend_bytes": ([C.POINTER(Config), C.POINTER(FrontendConfig), C.POINTER(C.c_size_t)], i32),
            "qt_attach_frontend": ([vp, C.POINTER(FrontendConfig), C.POINTER(FrontendWeights), vp, C.c_size_t], i32),
            "qt_embed_ids": ([vp, i32, vp, vp, vp, vp], i32),
            "qt_prefill_ids": ([vp, i32, vp, vp, vp, vp, vp, i32, C.POINTER(Sampling), C.POINTER(Sampling), u64, i32],
                               i32),
            "qt_codec_workspace_bytes": ([C.POINTER(CodecConfig), C.POINTER(C.c_size_t)], i32),
            "qt_codec_create": ([C.POINTER(CodecConfig), C.POINTER(CodecWeights), vp, C.c_size_t, vp, C.POINTER(vp)],
                                i32),
            "qt_codec_destroy": ([vp], None),
            "qt_codec_last_error": ([vp], C.c_char_p),
            "qt_codec_decode": ([vp, vp, i32, vp], i32),
            "qt_codec_decode_chunked": ([vp, vp, i32, vp], i32),
            "qt_codec_stream": ([vp, vp, i32, C.c_int64, vp], i32),
            "qt_debug_exp_noise": ([vp, i32, vp, C.c_int64, u64, vp], i32),
            "qt_debug_linear": ([vp, i32, vp, i32, i32, vp, i32, vp, f32, i32, vp, vp, C.c_int64, i32, i32,
                                 C.c_int64], i32),
            "qt_linear_noalloc": ([vp, i32, vp, i32, i32, vp, i32, vp, f32, i32, vp], i32),
            "qt_debug_prefill_attention": ([vp, i32, i32, i32, i32, i32, vp, i32, vp, vp, vp, f32, vp, vp, vp, vp,
                                            vp, i32, vp, C.c_int64], i32),
            "qt_debug_decode_attention": ([vp, i32, i32, i32, i32, i32, i32, vp, vp, i32, vp, vp, vp, f32, vp, vp, vp,
                                           vp, vp, i32, vp], i32),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(status, ctx=None):
    if status != QT_OK:
        raise QtError(status, lib().qt_last_error(ctx).decode())


def _dec(d):
    return DecoderDims(d["layers"], d["hidden"], d["n_heads"], d["n_kv_heads"], d["head_dim"],
                       d["intermediate"], d["rope_theta"], d["rms_eps"])


def make_config(dm, weight_dtype="bf16", kv_dtype=None, max_batch=1, max_positions=256):
    wd = QT_DTYPE_BF16 if weight_dtype == "bf16" else QT_DTYPE_F32
    # default cache: fp16 next to bf16 weights (same bytes as bf16, three more
    # mantissa bits: K is RMS-normalised and V small, far inside fp16 range)
    if kv_dtype is None:
        kv_dtype = "f16" if weight_dtype == "bf16" else "f32"
    kd = _DTYPES[kv_dtype]
    return Config(_dec(dm["talker"]), _dec(dm["predictor"]), dm["talker_vocab"], dm["n_groups"], dm["codebook"],
                  dm["eos_id"], dm["suppress_begin"], dm["suppress_end"], int(bool(dm["pred_in_proj"])),
                  wd, kd, max_batch, max_positions)


def sampling(s):
    return Sampling(int(bool(s["do_sample"])), s["temperature"], s["top_k"], s["top_p"],
                    s["repetition_penalty"], s["min_new_tokens"])


def config_check(cfg):
    return lib().qt_config_check(C.byref(cfg))


def workspace_bytes(cfg):
    n = C.c_size_t(0)
    _check(lib().qt_workspace_bytes(C.byref(cfg), C.byref(n)))
    return n.value


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else None


def _np_ptr(a):
    return a.ctypes.data_as(C.c_void_p) if a is not None else None


def to_device_weight(a, dtype, device="cuda"):
    """numpy float32 array (holding bf16 values for bf16) -> device tensor of the ABI element type."""
    import torch
    if dtype == "bf16":
        from .synth import bf16_bits
        return torch.from_numpy(bf16_bits(a).view(np.int16)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


class Engine:
    """One qt_ctx on the current device, on a private torch stream."""

    def __init__(self, dm, weights, dtype="bf16", kv_dtype=None, max_batch=1, max_positions=256,
                 use_workspace=True):
        import torch
        self.torch = torch
        self.dm = dm
        self.dtype = dtype
        self.cfg = make_config(dm, dtype, kv_dtype, max_batch, max_positions)
        self.stream = torch.cuda.Stream()
        L = lib()
        dev = {}

        def up(a):
            t = to_device_weight(a, dtype)
            dev[id(t)] = t
            return _ptr(t)

        def layers(ws):
            arr = (LayerWeights * len(ws))()
            for i, lw in enumerate(ws):
                arr[i] = LayerWeights(*[up(lw[n]) for n in ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm",
                                                              "wo", "mlp_norm", "w_gate", "w_up", "w_down")])
            return arr

        with torch.cuda.stream(self.stream):
            tl = layers(weights["talker_layers"])
            pl = layers(weights["pred_layers"])
            w = Weights(tl, up(weights["talker_norm"]), up(weights["talker_codec_embed"]),
                        up(weights["talker_codec_head"]), pl, up(weights["pred_norm"]),
                        up(weights["pred_embeds"]), up(weights["pred_heads"]),
                        up(weights["pred_in_proj"]) if weights.get("pred_in_proj") is not None else None)
            torch.cuda.synchronize()
            self.ws_bytes = workspace_bytes(self.cfg)
            self.workspace = (torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
                              if use_workspace else None)
            ctx = C.c_void_p()
            _check(L.qt_create(C.byref(self.cfg), C.byref(w), _ptr(self.workspace),
                               self.ws_bytes if use_workspace else 0,
                               C.c_void_p(self.stream.cuda_stream), C.byref(ctx)))
        self.ctx = ctx
        dev.clear()  # the library holds its own repacked copy
        torch.cuda.synchronize()
        self.B = 0
        self._keep = []

    def close(self):
        if getattr(self, "ctx", None):
            lib().qt_destroy(self.ctx)
            self.ctx = None

    __del__ = close

    # ---- generation
    def prefill(self, prompt, lens, tts_pad, talker, predictor, seed, max_frames, text=None, text_lens=None):
        """prompt: packed [sum(lens), H] (numpy or device tensor); tts_pad [H]; text packed or None."""
        torch = self.torch
        dev = lambda a: a if isinstance(a, torch.Tensor) else torch.from_numpy(  # noqa: E731
            np.ascontiguousarray(a, dtype=np.float32)).cuda()
        with torch.cuda.stream(self.stream):
            p = dev(prompt)
            pad = dev(tts_pad)
            tx = dev(text) if text is not None else None
        torch.cuda.synchronize()
        self._keep = [p, pad, tx]  # the library reads text / pad in every frame
        lens = np.ascontiguousarray(lens, dtype=np.int32)
        tl = np.ascontiguousarray(text_lens, dtype=np.int32) if text_lens is not None else None
        self.B = int(lens.size)
        ts, ps = sampling(talker), sampling(predictor)
        _check(lib().qt_prefill(self.ctx, self.B, _ptr(p), _np_ptr(lens), _ptr(tx), _np_ptr(tl), _ptr(pad),
                                C.byref(ts), C.byref(ps), C.c_uint64(seed), int(max_frames)), self.ctx)

    def step_frame(self):
        codes = np.zeros((self.B, 16), dtype=np.int32)
        state = np.zeros(self.B, dtype=np.uint8)
        _check(lib().qt_step_frame(self.ctx, _np_ptr(codes), _np_ptr(state)), self.ctx)
        return codes, state

    def generate(self, prompt, lens, tts_pad, talker, predictor, seed, max_frames, text=None, text_lens=None):
        torch = self.torch
        with torch.cuda.stream(self.stream):
            p = prompt if isinstance(prompt, torch.Tensor) else torch.from_numpy(
                np.ascontiguousarray(prompt, dtype=np.float32)).cuda()
            pad = tts_pad if isinstance(tts_pad, torch.Tensor) else torch.from_numpy(
                np.ascontiguousarray(tts_pad, dtype=np.float32)).cuda()
            tx = None if text is None else (text if isinstance(text, torch.Tensor) else torch.from_numpy(
                np.ascontiguousarray(text, dtype=np.float32)).cuda())
        torch.cuda.synchronize()
        self._keep = [p, pad, tx]
        lens = np.ascontiguousarray(lens, dtype=np.int32)
        tl = np.ascontiguousarray(text_lens, dtype=np.int32) if text_lens is not None else None
        B = int(lens.size)
        self.B = B
        codes = np.zeros((B, max_frames, 16), dtype=np.int32)
        n = np.zeros(B, dtype=np.int32)
        fin = np.zeros(B, dtype=np.uint8)
        ts, ps = sampling(talker), sampling(predictor)
        _check(lib().qt_generate(self.ctx, B, _ptr(p), _np_ptr(lens), _ptr(tx), _np_ptr(tl), _ptr(pad),
                                 C.byref(ts), C.byref(ps), C.c_uint64(seed), int(max_frames),
                                 _np_ptr(codes), _np_ptr(n), _np_ptr(fin)), self.ctx)
        return codes, n, fin

    def admit(self, slot, prompt, text=None, seed=0, noise_row=None, max_frames=1):
        """Start a new request in a finished slot (continuous batching)."""
        torch = self.torch
        dev = lambda a: a if isinstance(a, torch.Tensor) else torch.from_numpy(  # noqa: E731
            np.ascontiguousarray(a, dtype=np.float32)).cuda()
        with torch.cuda.stream(self.stream):
            p = dev(prompt)
            tx = dev(text) if text is not None and len(text) else None
        torch.cuda.synchronize()
        self._keep_slot = getattr(self, "_keep_slot", {})
        self._keep_slot[slot] = (p, tx)   # trailing text is read during the request's frames
        _check(lib().qt_admit(self.ctx, int(slot), _ptr(p), int(p.shape[0]), _ptr(tx),
                              0 if tx is None else int(tx.shape[0]), C.c_uint64(seed),
                              int(slot if noise_row is None else noise_row), int(max_frames)), self.ctx)

    # ---- token-id frontend
    def attach_frontend(self, fw, max_rows):
        """fw: dict text_embed, fc1_w, fc1_b, fc2_w, fc2_b (numpy, biases may be None)."""
        torch = self.torch
        V, Ti = fw["text_embed"].shape
        Hm = fw["fc1_w"].shape[0]
        self.fcfg = FrontendConfig(V, Ti, Hm, int(max_rows))
        keep = []

        def up(a):
            if a is None:
                return None
            x = to_device_weight(a, self.dtype)
            keep.append(x)
            return _ptr(x)
        with torch.cuda.stream(self.stream):
            w = FrontendWeights(up(fw["text_embed"]), up(fw["fc1_w"]), up(fw.get("fc1_b")), up(fw["fc2_w"]),
                                up(fw.get("fc2_b")))
        torch.cuda.synchronize()
        _check(lib().qt_attach_frontend(self.ctx, C.byref(self.fcfg), C.byref(w), None, 0), self.ctx)
        keep.clear()   # the library holds its own repacked copy

    def embed_ids(self, text_ids, codec_ids, extra=None):
        """Dual-track rows [n, H] (device tensor) for host id arrays."""
        torch = self.torch
        ti = np.ascontiguousarray(text_ids, dtype=np.int32)
        ci = np.ascontiguousarray(codec_ids, dtype=np.int32)
        n = int(ti.size)
        out = torch.empty((n, self.dm["talker"]["hidden"]), dtype=torch.float32, device="cuda")
        ex = None
        if extra is not None:
            ex = extra if isinstance(extra, torch.Tensor) else torch.from_numpy(
                np.ascontiguousarray(extra, dtype=np.float32)).cuda()
        torch.cuda.synchronize()
        _check(lib().qt_embed_ids(self.ctx, n, _np_ptr(ti), _np_ptr(ci), _ptr(ex), _ptr(out)), self.ctx)
        torch.cuda.synchronize()
        return out

    def prefill_ids(self, text_ids, codec_ids, lens, trailing_ids, trailing_lens, tts_pad_id, talker, predictor, seed,
                    max_frames):
        ti = np.ascontiguousarray(text_ids, dtype=np.int32)
        ci = np.ascontiguousarray(codec_ids, dtype=np.int32)
        lens = np.ascontiguousarray(lens, dtype=np.int32)
        tr = np.ascontiguousarray(trailing_ids, dtype=np.int32) if trailing_ids is not None else None
        tl = np.ascontiguousarray(trailing_lens, dtype=np.int32) if trailing_lens is not None else None
        self.B = int(lens.size)
        self._keep = []
        ts, ps = sampling(talker), sampling(predictor)
        _check(lib().qt_prefill_ids(self.ctx, self.B, _np_ptr(ti), _np_ptr(ci), _np_ptr(lens), _np_ptr(tr),
                                    _np_ptr(tl), int(tts_pad_id), C.byref(ts), C.byref(ps), C.c_uint64(seed),
                                    int(max_frames)), self.ctx)

    # ---- test entry points
    def step_forced(self, forced):
        forced = np.ascontiguousarray(forced, dtype=np.int32)
        tl = np.zeros((self.B, self.dm["talker_vocab"]), dtype=np.float32)
        pl = np.zeros((self.B, 15, self.dm["codebook"]), dtype=np.float32)
        ch = np.zeros((self.B, 16), dtype=np.int32)
        _check(lib().qt_debug_step_forced(self.ctx, _np_ptr(forced), _np_ptr(tl), _np_ptr(pl), _np_ptr(ch)),
               self.ctx)
        return tl, pl, ch

    def talker_logits(self):
        out = np.zeros((self.B, self.dm["talker_vocab"]), dtype=np.float32)
        _check(lib().qt_debug_talker_logits(self.ctx, _np_ptr(out)), self.ctx)
        return out

    def last_error(self):
        return lib().qt_last_error(self.ctx).decode()


def debug_linear(W, X, gain=None, eps=1e-6, epilogue=0, Y=None, wdtype="bf16", reps=1, stream=None,
                 matrix_cores=True, copies=1):
    """Y = op(W · norm(X)) on the device (torch tensors: W int16 bf16 bits or float32).

    matrix_cores: give the library its row and split-K scratch, so bf16
    weights with many rows take the MFMA kernels as in the frame.
    copies: W may hold [copies, N, K] stacked weight copies; launch i of the
    reps uses copy i % copies (timing from HBM instead of a cache)."""
    import torch
    if W.dim() == 3:
        copies, N, K = W.shape
    else:
        N, K = W.shape
        copies = 1
    M = X.shape[0]
    if Y is None:
        Y = torch.zeros((M, N // 2 if epilogue == 2 else N), dtype=torch.float32, device=X.device)
    # row denominators; split-K partial sums (<= 128 rows) or the hi/lo split of the rows (more rows)
    n_scratch = (M + 63) // 64 * 64 + ((K // 256) * M * (N + 1) if M <= 128 else M * K)
    scratch = torch.empty(n_scratch, dtype=torch.float32, device=X.device) if matrix_cores else None
    s = stream.cuda_stream if stream is not None else torch.cuda.current_stream().cuda_stream
    _check(lib().qt_debug_linear(C.c_void_p(s), QT_DTYPE_BF16 if wdtype == "bf16" else QT_DTYPE_F32,
                                 _ptr(W), N, K, _ptr(X), M, _ptr(gain), eps, epilogue, _ptr(Y), _ptr(scratch),
                                 n_scratch if matrix_cores else 0, reps, copies, N * K * W.element_size()))
    return Y


def linear_noalloc(W, X, gain=None, eps=1e-6, epilogue=0, Y=None, wdtype="bf16", stream=None):
    """Y = op(W · norm(X)) through qt_linear_noalloc (the library's static
    scratch; nothing allocated by the library). torch tensors as debug_linear."""
    import torch
    N, K = W.shape
    M = X.shape[0]
    if Y is None:
        Y = torch.zeros((M, N // 2 if epilogue == 2 else N), dtype=torch.float32, device=X.device)
    s = stream.cuda_stream if stream is not None else torch.cuda.current_stream().cuda_stream
    _check(lib().qt_linear_noalloc(C.c_void_p(s), QT_DTYPE_BF16 if wdtype == "bf16" else QT_DTYPE_F32, _ptr(W), N,
                                   K, _ptr(X), M, _ptr(gain), eps, epilogue, _ptr(Y)))
    return Y


def debug_prefill_attention(qkv, lens, q_gain, k_gain, cos, sin, kc, vc, nq, nkv, eps=1e-6, kv_dtype="f16",
                            tiled=True):
    """Prefill attention of one layer on device tensors; returns out [T, nq d].

    qkv [T, (nq + 2 nkv) d] float32; kc, vc [B, nkv, max_pos, d] of the cache
    type (written); cos, sin [max_pos, d / 2]."""
    import torch
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    T = int(lens.sum())
    d = qkv.shape[1] // (nq + 2 * nkv)
    max_pos = kc.shape[2]
    out = torch.zeros((T, nq * d), dtype=torch.float32, device=qkv.device)
    n_runs = 4 * (T + T // 32 + lens.size)
    runs = torch.zeros(n_runs, dtype=torch.int32, device=qkv.device)
    s = torch.cuda.current_stream().cuda_stream
    _check(lib().qt_debug_prefill_attention(C.c_void_p(s), _DTYPES[kv_dtype], d, nq, nkv, int(lens.size),
                                            _np_ptr(lens), max_pos, _ptr(qkv), _ptr(q_gain), _ptr(k_gain), eps,
                                            _ptr(cos), _ptr(sin), _ptr(kc), _ptr(vc), _ptr(out), int(bool(tiled)),
                                            _ptr(runs), n_runs))
    return out


def debug_decode_attention(qkv, pos, q_gain, k_gain, cos, sin, kc, vc, nq, nkv, eps=1e-6, kv_dtype="f16",
                           kv_split=1, ntok=1):
    """One decode step of one layer's attention on device tensors for ntok
    (1 or 2) new tokens per row; returns out [B ntok, nq d].

    qkv [B ntok, (nq + 2 nkv) d] float32 (row r ntok + t: token t of row r, at
    position pos[r] + t); pos host int [B]; kc, vc [B, nkv, max_pos, d] of the
    cache type (positions below pos[r] hold the cache, pos[r] .. pos[r] +
    ntok - 1 are written); cos, sin [max_pos, d / 2]."""
    import torch
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    B = int(pos.size)
    d = qkv.shape[1] // (nq + 2 * nkv)
    max_pos = kc.shape[2]
    if qkv.shape[0] != B * ntok:
        raise ValueError("qkv must hold B * ntok rows")
    out = torch.zeros((B * ntok, nq * d), dtype=torch.float32, device=qkv.device)
    pos_dev = torch.zeros(B, dtype=torch.int32, device=qkv.device)
    split = None
    if kv_split > 1:
        split = torch.zeros(B * nkv * kv_split * (nq // nkv) * (d + 2), dtype=torch.float32, device=qkv.device)
    s = torch.cuda.current_stream().cuda_stream
    _check(lib().qt_debug_decode_attention(C.c_void_p(s), _DTYPES[kv_dtype], d, nq, nkv, B, int(ntok), _np_ptr(pos),
                                           _ptr(pos_dev), max_pos, _ptr(qkv), _ptr(q_gain), _ptr(k_gain), eps,
                                           _ptr(cos), _ptr(sin), _ptr(kc), _ptr(vc), _ptr(out), int(kv_split),
                                           _ptr(split) if split is not None else None))
    return out


def debug_exp_noise(words, mode=0, seed=0):
    """Device Exp(1) noise: words is a device uint64 tensor ([n, 4] counters
    (vocab id, stream, index, row) for mode 0, [n] raw words for mode 1)
    stored as int64; returns a float32 tensor [n]."""
    import torch
    n = words.shape[0]
    out = torch.zeros(n, dtype=torch.float32, device=words.device)
    s = torch.cuda.current_stream().cuda_stream
    _check(lib().qt_debug_exp_noise(C.c_void_p(s), int(mode), _ptr(words), n, C.c_uint64(seed), _ptr(out)))
    torch.cuda.synchronize()
    return out


def debug_select(logits, samp, seen=None, noise=None, probs=None, processors=False, eos=2150,
                 suppress=(2048, 3072), seed=0, stream_id=0, sel_index=0, want_processed=False):
    """Run the selection kernel on device tensors [B, V]; returns (codes, processed, status)."""
    import torch
    B, V = logits.shape
    out = torch.zeros(B, dtype=torch.int32, device=logits.device)
    st = torch.zeros(1, dtype=torch.int32, device=logits.device)
    proc = torch.zeros((B, V), dtype=torch.float32, device=logits.device) if want_processed else None
    sm = sampling(samp)
    s = torch.cuda.current_stream().cuda_stream
    _check(lib().qt_debug_select(C.c_void_p(s), B, V, _ptr(logits), _ptr(seen), _ptr(noise), _ptr(probs),
                                 int(bool(processors)), eos, suppress[0], suppress[1], C.byref(sm),
                                 C.c_uint64(seed), stream_id, sel_index, _ptr(out), _ptr(proc), _ptr(st)))
    torch.cuda.synchronize()
    return out, proc, st


def codec_config(cd, dtype="bf16"):
    ch = list(cd["voc_channels"]) + [0] * (CODEC_MAX_BLOCKS + 1 - len(cd["voc_channels"]))
    st = list(cd["strides"]) + [0] * (CODEC_MAX_BLOCKS - len(cd["strides"]))
    return CodecConfig(cd["n_q"], cd["codebook"], cd["codebook_dim"], cd["hidden"], cd["layers"], cd["heads"],
                       cd["head_dim"], cd["ffn"], cd["window"], cd["rope_theta"], cd["up_ffn"], len(cd["strides"]),
                       (C.c_int32 * (CODEC_MAX_BLOCKS + 1))(*ch), (C.c_int32 * CODEC_MAX_BLOCKS)(*st),
                       (C.c_int32 * CODEC_UNITS)(*cd["dilations"]), cd["chunk"], cd["context"],
                       QT_DTYPE_BF16 if dtype == "bf16" else QT_DTYPE_F32)


class Codec:
    """One qt_codec on the current device, on a private torch stream."""

    def __init__(self, cd, w, dtype="bf16"):
        import torch
        self.torch = torch
        self.cd = cd
        self.hop = 4 * int(np.prod(cd["strides"]))
        self.cfg = codec_config(cd, dtype)
        self.stream = torch.cuda.Stream()
        keep = []

        def up(a):
            x = to_device_weight(a, dtype)
            keep.append(x)
            return _ptr(x)
        with torch.cuda.stream(self.stream):
            layers = (CodecLayerWeights * max(1, len(w["layers"])))()
            for i, lw in enumerate(w["layers"]):
                layers[i] = CodecLayerWeights(*[up(lw[n]) for n in ("ln1_g", "ln1_b", "wqkv", "wo", "ls1", "ln2_g",
                                                                     "ln2_b", "fc1", "fc2", "ls2")])
            ups = (CodecUpWeights * 2)(*[CodecUpWeights(*[up(u[n]) for n in ("up", "dw", "ln_g", "ln_b", "fc1", "fc2",
                                                                             "gamma")]) for u in w["up_blocks"]])
            blocks = (CodecBlockWeights * CODEC_MAX_BLOCKS)()
            for b, bw in enumerate(w["voc_blocks"]):
                units = (CodecUnitWeights * CODEC_UNITS)(*[CodecUnitWeights(*[up(u[n]) for n in (
                    "a1", "b1", "conv7", "a2", "b2", "conv1")]) for u in bw["units"]])
                blocks[b] = CodecBlockWeights(up(bw["snake_a"]), up(bw["snake_b"]), up(bw["up"]), units)
            cw = CodecWeights(up(w["codebooks"]), up(w["proj_sem"]), up(w["proj_ac"]), layers, up(w["ln_f_g"]),
                              up(w["ln_f_b"]), ups, up(w["voc_in"]), blocks, up(w["voc_out_a"]), up(w["voc_out_b"]),
                              up(w["voc_out"]))
        torch.cuda.synchronize()
        n = C.c_size_t(0)
        _check(lib().qt_codec_workspace_bytes(C.byref(self.cfg), C.byref(n)))
        self.ws_bytes = n.value
        ctx = C.c_void_p()
        st = lib().qt_codec_create(C.byref(self.cfg), C.byref(cw), None, 0, C.c_void_p(self.stream.cuda_stream),
                                   C.byref(ctx))
        if st != QT_OK:
            raise QtError(st, lib().qt_codec_last_error(None).decode())
        self.ctx = ctx
        keep.clear()
        torch.cuda.synchronize()

    def _run(self, fn, codes, *extra, n_out):
        torch = self.torch
        codes = np.ascontiguousarray(codes, dtype=np.int32)
        out = torch.zeros(n_out, dtype=torch.float32, device="cuda")
        st = fn(self.ctx, _np_ptr(codes), int(codes.shape[0]), *extra, _ptr(out))
        if st != QT_OK:
            raise QtError(st, lib().qt_codec_last_error(self.ctx).decode())
        torch.cuda.synchronize()
        return out

    def decode(self, codes):
        """One causal pass over codes [T, 16] -> device float [T * hop]."""
        return self._run(lib().qt_codec_decode, codes, n_out=len(codes) * self.hop)

    def decode_chunked(self, codes):
        return self._run(lib().qt_codec_decode_chunked, codes, n_out=len(codes) * self.hop)

    def stream_step(self, codes, sent):
        """New samples sent .. T * hop - 1 for all frames so far (DecodeStream rule)."""
        return self._run(lib().qt_codec_stream, codes, C.c_int64(int(sent)), n_out=len(codes) * self.hop - int(sent))

    def close(self):
        if getattr(self, "ctx", None):
            lib().qt_codec_destroy(self.ctx)
            self.ctx = None

    __del__ = close
