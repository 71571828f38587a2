"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/qt.h declares, and rejects bad arguments before any device work
(ncnn CustomVoice port section 3.6: fail-closed checks of lengths, ids and
overflow before any access)."""
import ctypes as C
import os
import re

import pytest

from codec_lm_autoregressive_amd import binding, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qt.h")


@pytest.fixture(scope="module", autouse=True)
def built_library():
    """The library these checks load: built in-tree first when it is missing."""
    if not os.path.exists(binding.LIB_PATH):
        from codec_lm_autoregressive_amd import build
        build.build()
    yield


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qt_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared()
    assert "qt_create" in names and "qt_step_frame" in names and "qt_generate" in names
    lib = C.CDLL(binding.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def cfg06(**kw):
    c = binding.make_config(synth.dims("qwen06b"), "bf16", max_batch=1, max_positions=160)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_valid_configs_pass():
    assert binding.config_check(cfg06()) == binding.QT_OK
    tiny = binding.make_config(synth.dims("tiny"), "f32", max_batch=1, max_positions=64)
    assert binding.config_check(tiny) == binding.QT_OK
    big = binding.make_config(synth.dims("qwen17b"), "bf16", max_batch=8, max_positions=320)
    assert binding.config_check(big) == binding.QT_OK


@pytest.mark.parametrize("field,value", [
    ("n_groups", 15), ("talker_vocab", 1), ("codebook", 9000), ("eos_id", 3072), ("eos_id", -1),
    ("suppress_begin", 3000), ("suppress_end", 4000), ("weight_dtype", 7), ("kv_dtype", -1),
    ("max_batch", 0), ("max_positions", 1), ("pred_in_proj", 2),
])
def test_bad_config_rejected(field, value):
    c = cfg06(**{field: value})
    if field == "suppress_begin":
        c.suppress_end = 2900
    assert binding.config_check(c) == binding.QT_E_INVALID
    assert binding.lib().qt_last_error(None)


@pytest.mark.parametrize("field,value", [("head_dim", 96), ("n_kv_heads", 3), ("hidden", 1000), ("layers", 0),
                                         ("intermediate", 100), ("rope_theta", 0.0), ("rms_eps", -1.0)])
def test_bad_dims_rejected(field, value):
    c = cfg06()
    setattr(c.talker, field, value)
    assert binding.config_check(c) == binding.QT_E_INVALID


def test_predictor_width_needs_projection():
    dm = synth.dims("qwen17b")
    c = binding.make_config(dm, "bf16")
    c.pred_in_proj = 0
    assert binding.config_check(c) == binding.QT_E_INVALID


def test_workspace_bytes():
    dm = synth.dims("qwen06b")
    n = binding.workspace_bytes(cfg06())
    # packed bf16 weights alone: 33 layers of 15.73 M params + tables and heads
    params = 33 * (4096 * 1024 + 1024 * 2048 + 2 * 3072 * 1024 + 1024 * 3072) + 2 * 3072 * 1024 + 2 * 15 * 2048 * 1024
    # the predictor's code-indexed first-layer q/k/v tables: 14 steps x 2048 codes x 4096 fp32
    lut = 14 * 2048 * 4096 * 4
    assert n >= 2 * params + lut
    assert n < 2 * params + lut + (1 << 30)
    # KV grows linearly with max_batch * max_positions
    n2 = binding.workspace_bytes(cfg06(max_batch=2))
    kv_row = 28 * 8 * 160 * 128 * 2 * 2
    assert n2 - n >= kv_row
    del dm


def test_workspace_overflow_reported():
    c = cfg06(max_batch=4096, max_positions=1 << 20)
    c.talker.layers = 1024
    c.talker.hidden = 16384
    c.talker.intermediate = 65536
    c.pred_in_proj = 1
    s = C.c_size_t(0)
    st = binding.lib().qt_workspace_bytes(C.byref(c), C.byref(s))
    assert st in (binding.QT_OK, binding.QT_E_CAPACITY)
    if st == binding.QT_OK:
        assert s.value > (1 << 40)


def test_create_rejects_null_weights_without_device():
    L = binding.lib()
    w = binding.Weights()
    ctx = C.c_void_p()
    st = L.qt_create(C.byref(cfg06()), C.byref(w), None, 0, None, C.byref(ctx))
    assert st == binding.QT_E_INVALID
    assert not ctx.value
    assert b"NULL" in L.qt_last_error(None)


def test_null_ctx_calls_rejected():
    L = binding.lib()
    ts = binding.sampling(synth.GREEDY)
    assert L.qt_prefill(None, 1, None, None, None, None, None, C.byref(ts), C.byref(ts), 0, 1) == binding.QT_E_INVALID
    assert L.qt_step_frame(None, None, None) == binding.QT_E_INVALID
    assert L.qt_debug_step_forced(None, None, None, None, None) == binding.QT_E_INVALID
    L.qt_destroy(None)


def test_debug_entry_points_validate_before_launch():
    L = binding.lib()
    # bad shapes are rejected before any device pointer is touched
    assert L.qt_debug_linear(None, 1, None, 10, 7, None, 1, None, 1e-6, 0, None, None, 0, 1, 1, 0) == binding.QT_E_INVALID
    assert L.qt_debug_linear(None, 1, C.c_void_p(16), 10, 12, C.c_void_p(16), 1, None, 1e-6, 0,
                             C.c_void_p(16), None, 0, 1, 1, 0) == binding.QT_E_INVALID  # K not a multiple of 8
    sm = binding.sampling(dict(synth.SAMPLING, temperature=0.0))
    assert L.qt_debug_select(None, 1, 3072, C.c_void_p(16), None, None, None, 1, 2150, 2048, 3072, C.byref(sm), 0,
                             0, 0, C.c_void_p(16), None, C.c_void_p(16)) == binding.QT_E_INVALID
    fake = C.c_void_p(256)
    fc = binding.FrontendConfig(151936, 2048, 2048, 4096)
    n = C.c_size_t(0)
    assert L.qt_frontend_bytes(C.byref(cfg06()), C.byref(fc), C.byref(n)) == binding.QT_OK
    assert n.value > 151936 * 2048 * 2 + 2048 * 2048 * 2 + 1024 * 2048 * 2   # packed bf16 weights and buffers
    for bad in (binding.FrontendConfig(0, 2048, 2048, 16), binding.FrontendConfig(10, 2044, 2048, 16),
                binding.FrontendConfig(10, 2048, 2048, 0)):
        assert L.qt_frontend_bytes(C.byref(cfg06()), C.byref(bad), C.byref(n)) == binding.QT_E_INVALID
    ids = (C.c_int32 * 1)(0)
    assert L.qt_embed_ids(None, 1, ids, ids, None, fake) == binding.QT_E_INVALID
    assert L.qt_prefill_ids(None, 1, ids, ids, ids, None, None, 0, None, None, 0, 1) == binding.QT_E_INVALID
    ccfg = binding.codec_config(synth.codec_dims("12hz"))
    assert L.qt_codec_workspace_bytes(C.byref(ccfg), C.byref(n)) == binding.QT_OK
    assert n.value > 16 * 2048 * 256 * 2
    ccfg.dilations[2] = 11                                            # 6 x 11 rows > the zeroed padding
    assert L.qt_codec_workspace_bytes(C.byref(ccfg), C.byref(n)) == binding.QT_E_INVALID
    ccfg = binding.codec_config(synth.codec_dims("12hz"))
    ccfg.channels[2] = 100                                            # not a multiple of 8
    assert L.qt_codec_workspace_bytes(C.byref(ccfg), C.byref(n)) == binding.QT_E_INVALID
    assert L.qt_codec_decode(None, fake, 1, fake) == binding.QT_E_INVALID
    assert L.qt_codec_stream(None, fake, 1, 0, fake) == binding.QT_E_INVALID
    assert L.qt_debug_exp_noise(None, 2, fake, 4, 0, fake) == binding.QT_E_INVALID    # mode
    assert L.qt_debug_exp_noise(None, 0, None, 4, 0, fake) == binding.QT_E_INVALID    # NULL input
    assert L.qt_debug_exp_noise(None, 1, fake, -1, 0, fake) == binding.QT_E_INVALID   # n < 0
    lens = (C.c_int32 * 2)(5, 9)

    def pa(kv, d, nq, nkv, tiled, lens=lens, max_pos=64, runs_ints=1000):
        return L.qt_debug_prefill_attention(None, kv, d, nq, nkv, 2, lens, max_pos, fake, fake, fake, 1e-6, fake,
                                            fake, fake, fake, fake, tiled, fake, runs_ints)
    assert pa(binding.QT_DTYPE_F16, 64, 4, 2, 1) == binding.QT_E_INVALID     # no tiled kernel for head_dim 64
    assert pa(binding.QT_DTYPE_F32, 128, 4, 2, 1) == binding.QT_E_INVALID    # nor for an fp32 cache
    assert pa(binding.QT_DTYPE_F16, 128, 8, 2, 1) == binding.QT_E_INVALID    # nor for 4 q heads per kv head
    assert pa(binding.QT_DTYPE_F16, 96, 4, 2, 0) == binding.QT_E_INVALID     # head_dim
    assert pa(binding.QT_DTYPE_F16, 128, 6, 4, 0) == binding.QT_E_INVALID    # nq not a multiple of nkv
    assert pa(binding.QT_DTYPE_F16, 128, 4, 2, 1, max_pos=8) == binding.QT_E_INVALID   # a row longer than max_pos
    assert pa(binding.QT_DTYPE_F16, 128, 4, 2, 1, runs_ints=50) == binding.QT_E_INVALID  # run scratch too small
    pos = (C.c_int32 * 2)(5, 9)

    def da(kv, d, nq, nkv, split, pos=pos, max_pos=64, split_buf=fake, B=2, ntok=1):
        return L.qt_debug_decode_attention(None, kv, d, nq, nkv, B, ntok, pos, fake, max_pos, fake, fake, fake, 1e-6, fake,
                                           fake, fake, fake, fake, split, split_buf)
    assert da(7, 128, 4, 2, 1) == binding.QT_E_INVALID                         # kv_dtype
    assert da(binding.QT_DTYPE_F16, 96, 4, 2, 1) == binding.QT_E_INVALID       # head_dim
    assert da(binding.QT_DTYPE_F16, 128, 6, 4, 1) == binding.QT_E_INVALID      # nq not a multiple of nkv
    assert da(binding.QT_DTYPE_F16, 128, 4, 2, 3) == binding.QT_E_INVALID      # kv_split not a power of two
    assert da(binding.QT_DTYPE_F16, 128, 4, 2, 4, split_buf=None) == binding.QT_E_INVALID   # split without scratch
    assert da(binding.QT_DTYPE_F16, 64, 4, 2, 4) == binding.QT_E_INVALID       # split needs head_dim 128
    assert da(binding.QT_DTYPE_F16, 128, 16, 2, 2) == binding.QT_E_INVALID     # and at most 4 q heads per kv head
    assert da(binding.QT_DTYPE_F16, 128, 4, 2, 1, max_pos=9) == binding.QT_E_INVALID   # a position past max_pos - 1
    assert da(binding.QT_DTYPE_F16, 128, 4, 2, 1, B=0) == binding.QT_E_INVALID          # no rows
    assert da(binding.QT_DTYPE_F16, 128, 4, 2, 1, ntok=3) == binding.QT_E_INVALID       # one or two new tokens
    assert da(binding.QT_DTYPE_F16, 128, 4, 2, 2, ntok=2) == binding.QT_E_INVALID       # two tokens: no key ranges
    assert da(binding.QT_DTYPE_F16, 256, 4, 2, 1, ntok=2) == binding.QT_E_INVALID       # nor head_dim above 128
    assert da(binding.QT_DTYPE_F16, 128, 4, 2, 1, max_pos=10, ntok=2) == binding.QT_E_INVALID   # pos + 1 past max_pos - 1
