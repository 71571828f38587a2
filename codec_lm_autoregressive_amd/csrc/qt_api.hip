// C-ABI layer of the Qwen3-TTS 12 Hz frame step: validation, workspace
// layout, weight repacking, prompt prefill, the per-frame kernel sequence
// (replayed as one hipGraph per batch size), and the test entry points.
#include "qt.h"
#include "qt_internal.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

using namespace qt;

namespace {

thread_local char g_err[512] = "";

constexpr int kGroups = 16;       // codes per frame
constexpr int kPredPositions = 16;
constexpr int kPrefillChunk = 8192;
constexpr int kMaxVocab = 6144;
constexpr int kMaxKvSplit = 16;   // key ranges of one decode attention row

// Key ranges for the talker's single-token decode attention at `rows` batch
// rows: about 512 blocks (a power of two ranges, at most kMaxKvSplit) when
// the batch gives 64..256 blocks. Measured at 8 rows: 850 keys 12.5 us
// instead of 24.6, 400 keys 10.1 instead of 14, 130 keys even. Fewer rows
// keep one range (the combine launch costs more than the ranges save at
// short contexts), and so do 64 rows (512 blocks already; two ranges were
// slower at every context).
static int kv_split_for(int rows, int nkv) {
  if (rows < 8 || (long)rows * nkv > 256) return 1;
  int sp = 1;
  while (sp < kMaxKvSplit && (long)rows * nkv * sp * 2 <= 512) sp *= 2;
  return sp;
}

void set_err(char* buf, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, 512, fmt, ap);
  va_end(ap);
}

size_t esize(int dt) { return dt == QT_DTYPE_F32 ? 4 : 2; }

// overflow-checked size arithmetic
struct Sz {
  bool ovf = false;
  size_t mul(size_t a, size_t b) {
    size_t r;
    if (__builtin_mul_overflow(a, b, &r)) { ovf = true; return 0; }
    return r;
  }
  size_t mul(std::initializer_list<size_t> xs) {
    size_t r = 1;
    for (size_t x : xs) r = mul(r, x);
    return r;
  }
};

bool dims_ok(const qt_decoder_dims& d, char* err, const char* who) {
  if (d.layers < 1 || d.layers > 1024) { set_err(err, "%s.layers must be in 1..1024", who); return false; }
  if (d.hidden < 64 || d.hidden > 16384 || d.hidden % 64) { set_err(err, "%s.hidden must be a multiple of 64 in 64..16384", who); return false; }
  if (d.n_kv_heads < 1 || d.n_heads < 1 || d.n_heads % d.n_kv_heads) { set_err(err, "%s.n_heads must be a positive multiple of n_kv_heads", who); return false; }
  {
    const int gq = d.n_heads / d.n_kv_heads;
    if (gq != 1 && gq != 2 && gq != 4 && gq != 8) { set_err(err, "%s: n_heads / n_kv_heads must be 1, 2, 4 or 8", who); return false; }
  }
  if (d.head_dim != 16 && d.head_dim != 32 && d.head_dim != 64 && d.head_dim != 128 && d.head_dim != 256) {
    set_err(err, "%s.head_dim must be 16, 32, 64, 128 or 256", who); return false;
  }
  if ((d.n_heads * d.head_dim) % 64 || (d.n_heads * d.head_dim) > 65536) { set_err(err, "%s: n_heads*head_dim must be a multiple of 64", who); return false; }
  if (d.intermediate < 64 || d.intermediate > 65536 || d.intermediate % 64) { set_err(err, "%s.intermediate must be a multiple of 64 in 64..65536", who); return false; }
  if (!(d.rope_theta > 0.f) || !std::isfinite(d.rope_theta)) { set_err(err, "%s.rope_theta must be positive", who); return false; }
  if (!(d.rms_eps > 0.f) || !std::isfinite(d.rms_eps)) { set_err(err, "%s.rms_eps must be positive", who); return false; }
  return true;
}

qt_status check_config(const qt_config* c, char* err) {
  if (!c) { set_err(err, "config is NULL"); return QT_E_INVALID; }
  if (!dims_ok(c->talker, err, "talker") || !dims_ok(c->predictor, err, "predictor")) return QT_E_INVALID;
  if (c->n_groups != kGroups) { set_err(err, "n_groups must be 16"); return QT_E_INVALID; }
  if (c->talker_vocab < 2 || c->talker_vocab > kMaxVocab) { set_err(err, "talker_vocab must be in 2..%d", kMaxVocab); return QT_E_INVALID; }
  if (c->codebook < 2 || c->codebook > kMaxVocab) { set_err(err, "codebook must be in 2..%d", kMaxVocab); return QT_E_INVALID; }
  if (c->codebook > c->talker_vocab) { set_err(err, "codebook must not exceed talker_vocab"); return QT_E_INVALID; }
  if (c->eos_id < 0 || c->eos_id >= c->talker_vocab) { set_err(err, "eos_id out of range"); return QT_E_INVALID; }
  if (c->suppress_begin < 0 || c->suppress_begin > c->suppress_end || c->suppress_end > c->talker_vocab) {
    set_err(err, "suppress range must satisfy 0 <= begin <= end <= talker_vocab"); return QT_E_INVALID;
  }
  if (c->pred_in_proj != 0 && c->pred_in_proj != 1) { set_err(err, "pred_in_proj must be 0 or 1"); return QT_E_INVALID; }
  if (!c->pred_in_proj && c->predictor.hidden != c->talker.hidden) {
    set_err(err, "predictor.hidden must equal talker.hidden without pred_in_proj"); return QT_E_INVALID;
  }
  if ((c->weight_dtype != QT_DTYPE_F32 && c->weight_dtype != QT_DTYPE_BF16) ||
      (c->kv_dtype != QT_DTYPE_F32 && c->kv_dtype != QT_DTYPE_BF16 && c->kv_dtype != QT_DTYPE_F16)) {
    set_err(err, "weight_dtype must be QT_DTYPE_F32 or QT_DTYPE_BF16; kv_dtype also QT_DTYPE_F16");
    return QT_E_INVALID;
  }
  if (c->max_batch < 1 || c->max_batch > 4096) { set_err(err, "max_batch must be in 1..4096"); return QT_E_INVALID; }
  if (c->max_positions < 2 || c->max_positions > (1 << 20)) { set_err(err, "max_positions must be in 2..2^20"); return QT_E_INVALID; }
  return QT_OK;
}

bool sampling_ok(const qt_sampling* s, char* err, const char* who) {
  if (!s) { set_err(err, "%s sampling settings are NULL", who); return false; }
  if (s->do_sample != 0 && s->do_sample != 1) { set_err(err, "%s.do_sample must be 0 or 1", who); return false; }
  if (!(s->temperature > 0.f) || !std::isfinite(s->temperature)) { set_err(err, "%s.temperature must be > 0", who); return false; }
  if (s->top_k < 0) { set_err(err, "%s.top_k must be >= 0", who); return false; }
  if (!(s->top_p > 0.f) || s->top_p > 1.f) { set_err(err, "%s.top_p must be in (0, 1]", who); return false; }
  if (!(s->repetition_penalty > 0.f) || !std::isfinite(s->repetition_penalty)) { set_err(err, "%s.repetition_penalty must be > 0", who); return false; }
  if (s->min_new_tokens < 0) { set_err(err, "%s.min_new_tokens must be >= 0", who); return false; }
  return true;
}

struct Dec {
  int L, H, nq, nkv, d, I, qkv, nqd;
  float theta, eps;
  static Dec of(const qt_decoder_dims& x) {
    Dec d;
    d.L = x.layers; d.H = x.hidden; d.nq = x.n_heads; d.nkv = x.n_kv_heads; d.d = x.head_dim;
    d.I = x.intermediate; d.qkv = (x.n_heads + 2 * x.n_kv_heads) * x.head_dim; d.nqd = x.n_heads * x.head_dim;
    d.theta = x.rope_theta; d.eps = x.rms_eps;
    return d;
  }
};

// Workspace plan: every buffer's byte offset, 256-byte aligned.
struct Plan {
  Sz sz;
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    size_t b = (bytes + 255) & ~(size_t)255;
    if (__builtin_add_overflow(off, b, &off)) sz.ovf = true;
    return o;
  }
};

struct LayerBuf { size_t wqkv, wo, wgu, wd, attn_norm, q_norm, k_norm, mlp_norm; };

struct Layout {
  std::vector<LayerBuf> tl, pl;
  size_t talker_norm, temb, thead, pred_norm, pemb, phead, pproj, plut, pxlut, lut_stage;
  size_t cos_t, sin_t, cos_p, sin_p, kc_t, vc_t, kc_p, vc_p;
  size_t x_t, qkv, attn, act, x_p, xin_w, h, xlast, logits_t, logits_p, rope_rows, row_den, part, xsplit, ksplit;
  long part_floats, xsplit_floats;
  size_t rowstate, row64, seen, runs, idx, frame_out, req;
  size_t total;
  int tmax, seen_words, max_runs;
  bool ovf;
};

Layout plan_layout(const qt_config& c) {
  Layout L;
  Plan p;
  const Dec t = Dec::of(c.talker), q = Dec::of(c.predictor);
  const size_t es = esize(c.weight_dtype), kvs = esize(c.kv_dtype);
  const size_t V = c.talker_vocab, C = c.codebook, B = c.max_batch, MP = c.max_positions;
  auto layer = [&](const Dec& d) {
    LayerBuf b;
    b.wqkv = p.take(p.sz.mul({(size_t)d.qkv, (size_t)d.H, es}));
    b.wo = p.take(p.sz.mul({(size_t)d.H, (size_t)d.nqd, es}));
    b.wgu = p.take(p.sz.mul({2, (size_t)d.I, (size_t)d.H, es}));
    b.wd = p.take(p.sz.mul({(size_t)d.H, (size_t)d.I, es}));
    b.attn_norm = p.take((size_t)d.H * 4);
    b.q_norm = p.take((size_t)d.d * 4);
    b.k_norm = p.take((size_t)d.d * 4);
    b.mlp_norm = p.take((size_t)d.H * 4);
    return b;
  };
  for (int i = 0; i < t.L; ++i) L.tl.push_back(layer(t));
  for (int i = 0; i < q.L; ++i) L.pl.push_back(layer(q));
  L.talker_norm = p.take((size_t)t.H * 4);
  L.temb = p.take(p.sz.mul({V, (size_t)t.H, es}));
  L.thead = p.take(p.sz.mul({V, (size_t)t.H, es}));
  L.pred_norm = p.take((size_t)q.H * 4);
  L.pemb = p.take(p.sz.mul({15, C, (size_t)t.H, es}));
  L.phead = p.take(p.sz.mul({15, C, (size_t)q.H, es}));
  L.pproj = c.pred_in_proj ? p.take(p.sz.mul({(size_t)q.H, (size_t)t.H, es})) : 0;
  // code-indexed input side of the predictor's first layer for steps 1..14:
  // the q/k/v rows of every code of tables 0..13 (with the input projection
  // also the projected rows), fp32, and one table as fp32 rows to build them
  L.plut = p.take(p.sz.mul({14, C, (size_t)q.qkv, 4}));
  L.pxlut = c.pred_in_proj ? p.take(p.sz.mul({14, C, (size_t)q.H, 4})) : 0;
  L.lut_stage = p.take(p.sz.mul({C, (size_t)t.H, 4}));
  L.cos_t = p.take(p.sz.mul({MP, (size_t)t.d / 2, 4}));
  L.sin_t = p.take(p.sz.mul({MP, (size_t)t.d / 2, 4}));
  L.cos_p = p.take((size_t)kPredPositions * q.d / 2 * 4);
  L.sin_p = p.take((size_t)kPredPositions * q.d / 2 * 4);
  const size_t kvt = p.sz.mul({(size_t)t.L, B, (size_t)t.nkv, MP, (size_t)t.d, kvs});
  L.kc_t = p.take(kvt);
  L.vc_t = p.take(kvt);
  const size_t kvp = p.sz.mul({(size_t)q.L, B, (size_t)q.nkv, (size_t)kPredPositions, (size_t)q.d, kvs});
  L.kc_p = p.take(kvp);
  L.vc_p = p.take(kvp);
  // activation rows: one prefill chunk (never more than the prompt tokens
  // max_batch * max_positions can hold) or the predictor's two-token pass
  L.tmax = (int)std::max<long>(std::min<long>(kPrefillChunk, (long)c.max_batch * c.max_positions), 2L * c.max_batch);
  const size_t T = L.tmax;
  const size_t Hm = std::max(t.H, q.H), QKVm = std::max(t.qkv, q.qkv), NQm = std::max(t.nqd, q.nqd),
               Im = std::max(t.I, q.I);
  L.x_t = p.take(p.sz.mul({T, (size_t)t.H, 4}));
  L.qkv = p.take(p.sz.mul({T, QKVm, 4}));
  L.attn = p.take(p.sz.mul({T, NQm, 4}));
  L.act = p.take(p.sz.mul({T, Im, 4}));
  L.x_p = p.take(p.sz.mul({2 * B, (size_t)q.H, 4}));
  L.xin_w = c.pred_in_proj ? p.take(p.sz.mul({2 * B, (size_t)t.H, 4})) : 0;
  L.h = p.take(p.sz.mul({B, (size_t)t.H, 4}));
  L.xlast = p.take(p.sz.mul({B, (size_t)t.H, 4}));
  L.logits_t = p.take(p.sz.mul({B, V, 4}));
  L.logits_p = p.take(p.sz.mul({15, B, C, 4}));
  L.rope_rows = p.take(p.sz.mul({B, (size_t)t.d, 4}));
  L.row_den = p.take(p.sz.mul({T, 4}));
  // K-range partial sums (and per-row sums of squares): (K / 256) x rows x (N + 1)
  // for the largest projection at up to 128 rows
  {
    const size_t rows = std::min<size_t>(128, T);
    size_t need = 0;
    auto lin = [&](size_t n, size_t k) { need = std::max(need, (k / 256) * rows * (n + 1)); };
    for (const Dec* d : {&t, &q}) {
      lin(d->qkv, d->H); lin(d->H, d->nqd); lin(2 * (size_t)d->I, d->H); lin(d->H, d->I);
    }
    lin(V, t.H); lin(C, q.H);
    if (c.pred_in_proj) lin(q.H, t.H);
    need = std::min<size_t>(need, (size_t)16 << 20);
    L.part_floats = (long)need;
    L.part = p.take(p.sz.mul({need, 4}));
  }
  // bf16 hi/lo split of the activations of one prefill chunk (projections of more than 128 rows)
  {
    const size_t kmax = std::max({(size_t)t.H, (size_t)q.H, (size_t)t.nqd, (size_t)q.nqd, Im});
    L.xsplit_floats = T > 128 ? (long)(T * kmax) : 0;
    L.xsplit = T > 128 ? p.take(p.sz.mul({T, kmax, 4})) : 0;
  }
  // key-range partials of the talker's decode attention (see kv_split_for)
  L.ksplit = p.take(p.sz.mul({B, (size_t)t.nkv, (size_t)kMaxKvSplit, (size_t)(t.nq / std::max(t.nkv, 1)),
                              (size_t)t.d + 2, 4}));
  (void)Hm;
  // row state: code0_next, finished, pos, noise_row, text_len, max_frames,
  // frame_k [B]; own / forced [B, 16]; then the 64-bit seed and trailing-text
  // pointer of each row
  L.rowstate = p.take(p.sz.mul({B, 7 + 2 * kGroups, 4}));
  L.row64 = p.take(p.sz.mul({B, 2, 8}));
  L.seen_words = (int)((V + 31) / 32);
  L.seen = p.take(p.sz.mul({B, (size_t)L.seen_words, 4}));
  // decode runs, one per prompt token, and the prefill's tiles: at most
  // total / kAttnTileTokens + one partial tile per (row, chunk) piece
  const size_t BMP = (size_t)B * MP;
  L.max_runs = (int)std::min<size_t>((size_t)1 << 30, 3 * B + BMP + BMP / kAttnTileTokens + B + BMP / kPrefillChunk + 1);
  L.runs = p.take(p.sz.mul({(size_t)L.max_runs, sizeof(Run)}));
  L.idx = p.take(B * 4);
  L.frame_out = p.take(p.sz.mul({1 + B + B * kGroups, 4}));
  L.req = p.take(sizeof(ReqParams));
  L.total = p.off;
  L.ovf = p.sz.ovf;
  return L;
}

// Workspace of the token-id frontend: packed weights, id arrays, the MLP's
// row buffers for chunks of up to kFrontendChunk rows with the projections'
// matrix-core scratch, and the assembled rows of qt_prefill_ids (prompt
// rows, then trailing text rows, then tts_pad's row).
constexpr int kFrontendChunk = 8192;
struct FeLayout {
  size_t embed, fc1, fc2, b1, b2, tids, cids, x0, h1, y, scratch, rows, total;
  long scratch_floats;
  int chunk;
  bool ovf;
};

bool frontend_ok(const qt_config& c, const qt_frontend_config* f, char* err) {
  if (!f) { set_err(err, "frontend config is NULL"); return false; }
  if (f->text_vocab < 1 || f->text_vocab > (1 << 24)) { set_err(err, "text_vocab must be in 1..2^24"); return false; }
  if (f->text_hidden < 8 || f->text_hidden > 24576 || f->text_hidden % 8) {
    set_err(err, "text_hidden must be a multiple of 8 in 8..24576"); return false;
  }
  if (f->mlp_hidden < 8 || f->mlp_hidden > 24576 || f->mlp_hidden % 8) {
    set_err(err, "mlp_hidden must be a multiple of 8 in 8..24576"); return false;
  }
  if (f->max_rows < 1 || f->max_rows > (1 << 24)) { set_err(err, "max_rows must be in 1..2^24"); return false; }
  (void)c;
  return true;
}

FeLayout plan_frontend(const qt_config& c, const qt_frontend_config& f) {
  FeLayout L;
  Plan p;
  const size_t es = esize(c.weight_dtype), H = c.talker.hidden, Ti = f.text_hidden, Hm = f.mlp_hidden;
  const size_t R = f.max_rows, ch = std::min<size_t>(R, kFrontendChunk);
  L.chunk = (int)ch;
  L.embed = p.take(p.sz.mul({(size_t)f.text_vocab, Ti, es}));
  L.fc1 = p.take(p.sz.mul({Hm, Ti, es}));
  L.fc2 = p.take(p.sz.mul({H, Hm, es}));
  L.b1 = p.take(Hm * 4);
  L.b2 = p.take(H * 4);
  L.tids = p.take(p.sz.mul(R, 4));
  L.cids = p.take(p.sz.mul(R, 4));
  L.x0 = p.take(p.sz.mul({ch, Ti, 4}));
  L.h1 = p.take(p.sz.mul({ch, Hm, 4}));
  L.y = p.take(p.sz.mul({ch, H, 4}));
  // row denominators + the larger of: the hi/lo planes of a full chunk, or
  // the K-range partial sums of a chunk of up to 128 rows
  const size_t kmax = std::max(Ti, Hm), nmax = std::max(Hm, H);
  const size_t need = (ch + 63) / 64 * 64 + std::max(ch > 128 ? ch * kmax : 0, (kmax / 256) * std::min<size_t>(ch, 128) * (nmax + 1));
  L.scratch_floats = (long)need;
  L.scratch = p.take(p.sz.mul(need, 4));
  L.rows = p.take(p.sz.mul({R, H, 4}));
  L.total = p.off;
  L.ovf = p.sz.ovf;
  return L;
}

struct DevLayer {
  void *wqkv, *wo, *wgu, *wd;
  float *attn_norm, *q_norm, *k_norm, *mlp_norm;
};

}  // namespace

struct qt_ctx {
  qt_config cfg;
  Dec t, p;
  Layout lay;
  hipStream_t stream = nullptr;       // caller's stream
  hipStream_t cap = nullptr;          // private stream for graph capture
  hipEvent_t ev = nullptr;
  int device = 0;
  char err[512] = "";
  char* ws = nullptr;
  bool own_ws = false;
  std::vector<DevLayer> tl, pl;
  float *talker_norm, *pred_norm;
  void *temb, *thead, *pemb, *phead, *pproj;
  float *plut, *pxlut, *lut_stage;     // code-indexed first-layer tables of predictor steps 1..14
  float *cos_t, *sin_t, *cos_p, *sin_p;
  void *kc_t, *vc_t, *kc_p, *vc_p;
  float *x_t, *qkv, *attn, *act, *x_p, *xin_w, *h, *xlast, *logits_t, *logits_p, *rope_rows, *row_den, *part, *xsplit, *ksplit;
  long part_floats, xsplit_floats;
  int *code0_next, *finished, *pos, *noise_row, *text_len, *max_frames_row, *frame_k, *own, *forced;
  uint64_t* row_seed;
  const float** text_ptr;
  uint32_t* seen;
  Run* runs;
  int* idx;
  int* frame_out;                     // [status | state B | codes B*16]
  ReqParams* req;                     // per-request settings (device)
  int* hout = nullptr;                // pinned host mirror of frame_out
  // generation state
  int B = 0;
  bool prefilled = false, failed = false;
  int frames_done = 0, max_frames = 0;
  std::vector<uint8_t> done;
  qt_sampling ts{}, ps{};
  uint64_t seed = 0;
  const float* text = nullptr;
  const float* pad = nullptr;
  bool has_text = false;
  // graph of one frame for the current B
  hipGraphExec_t gexec = nullptr;
  int graph_B = -1;
  int graph_pred_sample = -1;         // the predictor's do_sample the graph was taken with
  int eager_frames = 0;
  // token-id frontend (qt_attach_frontend)
  struct Frontend {
    bool on = false;
    qt_frontend_config fc{};
    char* ws = nullptr;
    bool own_ws = false;
    void *embed = nullptr, *fc1 = nullptr, *fc2 = nullptr;
    float *b1 = nullptr, *b2 = nullptr;
    int *tids = nullptr, *cids = nullptr;
    float *x0 = nullptr, *h1 = nullptr, *y = nullptr, *scratch = nullptr;
    long scratch_floats = 0;
    int chunk = 0;
    float *prompt = nullptr, *trail = nullptr, *pad = nullptr;   // qt_prefill_ids outputs
  } fe;
};

namespace {

template <typename T> T* at(qt_ctx* c, size_t off) { return (T*)(c->ws + off); }

#define HIPCK(call)                                                                   \
  do {                                                                                \
    hipError_t e_ = (call);                                                           \
    if (e_ != hipSuccess) {                                                           \
      set_err(ctx->err, "%s failed: %s", #call, hipGetErrorString(e_));               \
      return QT_E_HIP;                                                                \
    }                                                                                 \
  } while (0)

#define QTCK(call)                \
  do {                            \
    qt_status r_ = (call);        \
    if (r_ != QT_OK) return r_;   \
  } while (0)

void host_rope(int max_pos, int d, float theta, std::vector<float>& cs, std::vector<float>& sn) {
  const int half = d / 2;
  std::vector<float> inv(half);
  for (int i = 0; i < half; ++i) inv[i] = (float)std::pow((double)theta, -(2.0 * i) / d);
  cs.resize((size_t)max_pos * half);
  sn.resize((size_t)max_pos * half);
  for (int p = 0; p < max_pos; ++p)
    for (int i = 0; i < half; ++i) {
      const float ang = (float)p * inv[i];  // float32 product
      cs[(size_t)p * half + i] = (float)std::cos((double)ang);
      sn[(size_t)p * half + i] = (float)std::sin((double)ang);
    }
}

qt_status pack_layer(qt_ctx* ctx, const qt_layer_weights& w, const Dec& d, DevLayer& o, hipStream_t s) {
  const int wd = ctx->cfg.weight_dtype;
  const size_t es = esize(wd);
  if (!w.attn_norm || !w.wq || !w.wk || !w.wv || !w.q_norm || !w.k_norm || !w.wo || !w.mlp_norm || !w.w_gate ||
      !w.w_up || !w.w_down) {
    set_err(ctx->err, "a layer weight pointer is NULL");
    return QT_E_INVALID;
  }
  // fused q/k/v rows
  HIPCK(launch_convert(w.wq, wd, d.H, o.wqkv, wd, d.H, (long)d.nq * d.d, d.H, s));
  HIPCK(launch_convert(w.wk, wd, d.H, (char*)o.wqkv + (size_t)d.nq * d.d * d.H * es, wd, d.H, (long)d.nkv * d.d, d.H, s));
  HIPCK(launch_convert(w.wv, wd, d.H, (char*)o.wqkv + (size_t)(d.nq + d.nkv) * d.d * d.H * es, wd, d.H,
                       (long)d.nkv * d.d, d.H, s));
  HIPCK(launch_convert(w.wo, wd, d.nqd, o.wo, wd, d.nqd, d.H, d.nqd, s));
  // gate / up interleaved by row: row 2j = gate j, row 2j+1 = up j
  HIPCK(launch_convert(w.w_gate, wd, d.H, o.wgu, wd, 2L * d.H, d.I, d.H, s));
  HIPCK(launch_convert(w.w_up, wd, d.H, (char*)o.wgu + (size_t)d.H * es, wd, 2L * d.H, d.I, d.H, s));
  HIPCK(launch_convert(w.w_down, wd, d.I, o.wd, wd, d.I, d.H, d.I, s));
  HIPCK(launch_convert(w.attn_norm, wd, d.H, o.attn_norm, DT_F32, d.H, 1, d.H, s));
  HIPCK(launch_convert(w.q_norm, wd, d.d, o.q_norm, DT_F32, d.d, 1, d.d, s));
  HIPCK(launch_convert(w.k_norm, wd, d.d, o.k_norm, DT_F32, d.d, 1, d.d, s));
  HIPCK(launch_convert(w.mlp_norm, wd, d.H, o.mlp_norm, DT_F32, d.H, 1, d.H, s));
  return QT_OK;
}

// A code predictor step's input from the code-indexed tables of the first
// layer: q/k/v rows (row stride lut_ld, `rows` codes) and, with the input
// projection, the projected rows. sel: the step's greedy selection is folded
// into the attention (batch 1); else the codes are codes[r * code_ld] and
// the attention reads the table rows itself or they are gathered first.
struct StepIn {
  const float* lut; long lut_ld; const float* xlut; const SelFold* sel;
  const int* codes; int code_ld; int rows;
};

// ---- the decoder stack over M tokens
// pass0: the code predictor's 2-token pass (row r's tokens are activation rows
// 2r and 2r + 1 at positions 0 and 1).
// prefill: tiles (n_tiles > 0) are the runs of up to kAttnTileTokens tokens
// the attend pass takes instead of one run per token.
// in: a code predictor step whose first layer reads the code-indexed tables.

qt_status run_layers(qt_ctx* ctx, bool talker, float* x, int M, const Run* runs, int n_runs, const int* row_pos,
                     int pos_base, hipStream_t s, bool prefill = false, bool single_token = false, bool pass0 = false,
                     const Run* tiles = nullptr, int n_tiles = 0, const StepIn* in = nullptr) {
  const Dec& d = talker ? ctx->t : ctx->p;
  std::vector<DevLayer>& layers = talker ? ctx->tl : ctx->pl;
  const int maxpos = talker ? ctx->cfg.max_positions : kPredPositions;
  const size_t kvs = esize(ctx->cfg.kv_dtype);
  const long row_stride = (long)d.nkv * maxpos * d.d;
  const size_t layer_kv = (size_t)ctx->cfg.max_batch * row_stride * kvs;
  char* kc = (char*)(talker ? ctx->kc_t : ctx->kc_p);
  char* vc = (char*)(talker ? ctx->vc_t : ctx->vc_p);
  for (int l = 0; l < d.L; ++l) {
    const DevLayer& w = layers[l];
    LinearArgs a{};
    a.wdtype = ctx->cfg.weight_dtype;
    a.eps = d.eps;
    a.row_den = ctx->row_den; a.xs = ctx->xsplit; a.xs_floats = ctx->xsplit_floats;
    a.part = ctx->part; a.part_floats = ctx->part_floats;
    // q/k/v = W_qkv · RMSNorm(x)
    a.W = w.wqkv; a.N = d.qkv; a.K = d.H; a.X = x; a.ldx = d.H; a.M = M; a.gain = w.attn_norm;
    a.Y = ctx->qkv; a.ldy = d.qkv; a.epi = EPI_STORE;
    // single-token decode attention adds split-K partial sums itself, so a
    // split projection needs no reduce launch
    const bool decode_attn = !prefill && (single_token || pass0) && d.d <= 128;
    // a code predictor step's first layer takes its q/k/v rows from the
    // code-indexed table (gathered into qkv, or read by the attention itself)
    const bool from_lut = in && l == 0;
    const int zq = decode_attn && !from_lut ? linear_split_ranges(a) : 1;
    a.defer = zq > 1;
    if (!from_lut) HIPCK(launch_linear(a, s));
    a.defer = 0;
    AttnArgs t{};
    if (zq > 1) { t.part = ctx->part; t.part_z = zq; t.part_rows = M; t.part_k = d.H; t.part_eps = d.eps; }
    t.qkv = ctx->qkv; t.ld_qkv = d.qkv; t.out = ctx->attn; t.ld_out = d.nqd;
    t.q_gain = w.q_norm; t.k_gain = w.k_norm; t.eps = d.eps; t.scale = (float)(1.0 / std::sqrt((double)d.d));
    t.cos = talker ? ctx->cos_t : ctx->cos_p; t.sin = talker ? ctx->sin_t : ctx->sin_p;
    t.kc = kc + l * layer_kv; t.vc = vc + l * layer_kv; t.kvdtype = ctx->cfg.kv_dtype;
    t.row_stride = row_stride; t.max_pos = maxpos;
    t.runs = runs; t.n_runs = n_runs; t.row_pos = row_pos; t.pos_base = pos_base;
    t.nq = d.nq; t.nkv = d.nkv; t.d = d.d;
    // x += W_o · attn
    LinearArgs ao = a;
    ao.W = w.wo; ao.N = d.H; ao.K = d.nqd; ao.X = ctx->attn; ao.ldx = d.nqd; ao.gain = nullptr;
    ao.Y = x; ao.ldy = d.H; ao.epi = EPI_RESIDUAL;
    bool fused = false;
    if (prefill) {
      // every key of the chunk first, then one block per (kv head, query token)
      t.mode = ATT_WRITE;
      HIPCK(launch_attention(t, s));
      t.mode = ATT_ATTEND;
      if (n_tiles > 0) { t.runs = tiles; t.n_runs = n_tiles; t.max_ntok = kAttnTileTokens; }
      HIPCK(launch_attention(t, s));
    } else if (pass0 && d.d <= 128) {
      // tokens 0 and 1 of every row (positions 0 and 1); token 1 attends to
      // token 0's key and value
      t.mode = ATT_WRITE_ATTEND;
      t.single_token = 1;
      t.ntok = 2;
      t.tok_stride = 2;
      t.tok_off = 0;
      t.row_pos = nullptr;
      t.pos_base = 0;
    } else {
      t.mode = ATT_WRITE_ATTEND;
      t.single_token = single_token;
      t.rope_rows = (single_token && talker) ? ctx->rope_rows : nullptr;
      if (single_token && talker) { t.kv_split = kv_split_for(n_runs, d.nkv); t.split_buf = ctx->ksplit; }
    }
    if (from_lut && !in->sel) {
      if (!in->xlut && attention_reads_lut(t)) {
        t.lut = in->lut; t.lut_ld = in->lut_ld;
        t.lut_codes = in->codes; t.lut_code_ld = in->code_ld; t.lut_rows = in->rows;
      } else {
        HIPCK(launch_lut_rows(in->codes, in->code_ld, M, in->rows, in->lut, (int)in->lut_ld, ctx->qkv, d.qkv, in->xlut,
                              d.H, x, d.H, s));
      }
    }
    if (!prefill) {
      // the code predictor at one row: attention and o-projection in one launch
      if (!talker) {
        if (from_lut && in->sel) {
          // the folded selection: the attention reads the selected code's table rows
          t.lut = in->lut; t.lut_ld = in->lut_ld; t.xlut = in->xlut; t.sel = *in->sel;
          HIPCK(launch_attention_oproj(t, ao, s));
          fused = true;
        } else {
          const hipError_t e = launch_attention_oproj(t, ao, s);
          if (e != hipErrorNotSupported) { HIPCK(e); fused = true; }
        }
      }
      if (!fused) HIPCK(launch_attention(t, s));
    }
    if (!fused) HIPCK(launch_linear(ao, s));
    // act = silu(W_g · RMSNorm(x)) * (W_u · RMSNorm(x))
    a.W = w.wgu; a.N = 2 * d.I; a.K = d.H; a.X = x; a.ldx = d.H; a.gain = w.mlp_norm;
    a.Y = ctx->act; a.ldy = d.I; a.epi = EPI_SWIGLU;
    HIPCK(launch_linear(a, s));
    // x += W_d · act
    a.W = w.wd; a.N = d.H; a.K = d.I; a.X = ctx->act; a.ldx = d.I; a.gain = nullptr;
    a.Y = x; a.ldy = d.H; a.epi = EPI_RESIDUAL;
    HIPCK(launch_linear(a, s));
  }
  return QT_OK;
}

SelectArgs select_base(qt_ctx* ctx, const qt_sampling& sm, bool talker) {
  SelectArgs a{};
  a.req = ctx->req; a.which = talker ? 0 : 1;
  a.B = ctx->B;
  a.V = talker ? ctx->cfg.talker_vocab : ctx->cfg.codebook;
  a.processors = talker ? 1 : 0;
  a.seen = ctx->seen; a.seen_words = ctx->lay.seen_words;
  a.penalty = sm.repetition_penalty; a.min_new = sm.min_new_tokens;
  a.eos = ctx->cfg.eos_id; a.sup_b = ctx->cfg.suppress_begin; a.sup_e = ctx->cfg.suppress_end;
  a.do_sample = sm.do_sample; a.temperature = sm.temperature; a.top_k = sm.top_k; a.top_p = sm.top_p;
  a.seed = ctx->seed; a.row_seed = ctx->row_seed; a.noise_row = ctx->noise_row;
  a.status = ctx->frame_out;
  return a;
}

// The greedy selection of predictor head st - 1 (code st), folded into the
// fused attention of predictor step st at batch 1.
static SelFold pred_sel_fold(qt_ctx* ctx, int st) {
  const int C = ctx->cfg.codebook;
  SelFold f{};
  f.logits = ctx->logits_p + (size_t)(st - 1) * ctx->cfg.max_batch * C; f.V = C;
  f.tab = ctx->pemb; f.tab_off = (long)(st - 1) * C; f.tab_dim = ctx->t.H;
  f.used = ctx->frame_out + 1 + ctx->cfg.max_batch; f.own = ctx->own; f.col = st;
  f.fb = ctx->x_t;
  f.status = ctx->frame_out;
  return f;
}

// Whether a free-running frame folds the predictor's selections 1..14 into
// the next step's fused attention: batch 1, greedy predictor, and a
// predictor shape the fused kernel serves.
static bool pred_folds(qt_ctx* ctx) {
  const qt_config& c = ctx->cfg;
  return ctx->B == 1 && !ctx->ps.do_sample &&
         attention_oproj_sel_ok(ctx->p.nq, ctx->p.nkv, ctx->p.d, c.kv_dtype, c.weight_dtype, c.codebook, ctx->t.H) &&
         (c.pred_in_proj || ctx->t.H == ctx->p.H);
}

// One frame for all rows; forced != nullptr selects teacher forcing.
qt_status enqueue_frame(qt_ctx* ctx, hipStream_t s, const int* forced) {
  const int B = ctx->B;
  const Dec &T = ctx->t, &P = ctx->p;
  const int C = ctx->cfg.codebook;
  const bool proj = ctx->cfg.pred_in_proj != 0;
  const int wd = ctx->cfg.weight_dtype;
  int* codes = ctx->frame_out + 1 + ctx->cfg.max_batch;
  int* state = ctx->frame_out + 1;
  Run* runs_decode = ctx->runs;
  Run* runs_pass0 = ctx->runs + ctx->cfg.max_batch;
  Run* runs_step = ctx->runs + 2 * ctx->cfg.max_batch;

  FrameStartArgs fs{};
  fs.B = B; fs.eos = ctx->cfg.eos_id; fs.V = ctx->cfg.talker_vocab;
  fs.code0_next = ctx->code0_next; fs.finished = ctx->finished; fs.forced = forced; fs.forced_ld = kGroups;
  fs.seen = ctx->seen; fs.seen_words = ctx->lay.seen_words; fs.codes = codes;
  fs.temb = ctx->temb; fs.tdtype = wd; fs.H = T.H; fs.h = ctx->h;
  fs.pass0 = proj ? ctx->xin_w : ctx->x_p; fs.pass0_ld = T.H;
  fs.fb = ctx->x_t; fs.fb_ld = T.H; fs.status = ctx->frame_out;
  fs.cos = ctx->cos_t; fs.sin = ctx->sin_t; fs.pos = ctx->pos; fs.half = T.d / 2; fs.rope_rows = ctx->rope_rows;
  HIPCK(launch_frame_start(fs, s));

  LinearArgs pa{};
  pa.row_den = ctx->row_den; pa.xs = ctx->xsplit; pa.xs_floats = ctx->xsplit_floats;
  pa.part = ctx->part; pa.part_floats = ctx->part_floats;
  pa.wdtype = wd; pa.W = ctx->pproj; pa.N = P.H; pa.K = T.H; pa.X = ctx->xin_w; pa.ldx = T.H;
  pa.Y = ctx->x_p; pa.ldy = P.H; pa.epi = EPI_STORE;

  const bool fold = !forced && pred_folds(ctx);
  for (int st = 0; st < 15; ++st) {
    const int M = st == 0 ? 2 * B : B;
    if (st == 0) {
      if (proj) { pa.M = M; HIPCK(launch_linear(pa, s)); }
      QTCK(run_layers(ctx, false, ctx->x_p, M, runs_pass0, B, nullptr, 0, s, false, false, true));
    } else {
      // step st's input row is the embedding of code st: its first-layer
      // q/k/v (and projected row) come from the tables built at create
      const float* lut = ctx->plut + (size_t)(st - 1) * C * P.qkv;
      const float* xlut = proj ? ctx->pxlut + (size_t)(st - 1) * C * P.H : nullptr;
      const SelFold sf = fold ? pred_sel_fold(ctx, st) : SelFold{};
      const StepIn in{lut, (long)P.qkv, xlut, fold ? &sf : nullptr, codes + st, kGroups, C};
      QTCK(run_layers(ctx, false, ctx->x_p, M, runs_step, B, nullptr, st + 1, s, false, true, false, nullptr, 0, &in));
    }
    // head st on the last token of each row
    LinearArgs ha{};
    ha.row_den = ctx->row_den; ha.xs = ctx->xsplit; ha.xs_floats = ctx->xsplit_floats;
    ha.part = ctx->part; ha.part_floats = ctx->part_floats;
    ha.wdtype = wd; ha.W = (const char*)ctx->phead + (size_t)st * C * P.H * esize(wd); ha.N = C; ha.K = P.H;
    ha.X = st == 0 ? ctx->x_p + P.H : ctx->x_p; ha.ldx = st == 0 ? 2L * P.H : P.H; ha.M = B;
    ha.gain = ctx->pred_norm; ha.eps = P.eps;
    ha.Y = ctx->logits_p + (size_t)st * ctx->cfg.max_batch * C; ha.ldy = C; ha.epi = EPI_STORE;
    HIPCK(launch_linear(ha, s));
    SelectArgs sa = select_base(ctx, ctx->ps, false);
    sa.logits = ha.Y; sa.ld = C;
    sa.stream = st + 1; sa.ctr = ctx->frame_k; sa.ctr_add = 0;
    sa.forced = forced; sa.forced_ld = kGroups; sa.forced_col = st + 1;
    sa.used = codes; sa.used_ld = kGroups; sa.used_col = st + 1;
    sa.own = ctx->own; sa.own_ld = kGroups; sa.own_col = st + 1;
    sa.epi = 1;
    sa.tab = ctx->pemb; sa.tab_dtype = wd; sa.tab_dim = T.H; sa.tab_off = (long)st * C;
    sa.next_in = st < 14 ? (proj ? ctx->xin_w : ctx->x_p) : nullptr; sa.next_ld = T.H;
    sa.fb = ctx->x_t; sa.fb_ld = T.H;
    sa.add_text = st == 14; sa.text_ptr = ctx->text_ptr; sa.text_len = ctx->text_len;
    sa.frame_k = ctx->frame_k;
    if (!(fold && st < 14)) HIPCK(launch_select(sa, s));
  }
  // talker step at position P_r + k
  QTCK(run_layers(ctx, true, ctx->x_t, B, runs_decode, B, ctx->pos, 0, s, false, true));
  LinearArgs ta{};
  ta.row_den = ctx->row_den; ta.xs = ctx->xsplit; ta.xs_floats = ctx->xsplit_floats;
  ta.part = ctx->part; ta.part_floats = ctx->part_floats;
  ta.wdtype = wd; ta.W = ctx->thead; ta.N = ctx->cfg.talker_vocab; ta.K = T.H; ta.X = ctx->x_t; ta.ldx = T.H; ta.M = B;
  ta.gain = ctx->talker_norm; ta.eps = T.eps; ta.Y = ctx->logits_t; ta.ldy = ctx->cfg.talker_vocab; ta.epi = EPI_STORE;
  ta.norm_out = ctx->h; ta.ld_norm = T.H;
  HIPCK(launch_linear(ta, s));
  SelectArgs sa = select_base(ctx, ctx->ts, true);
  sa.logits = ctx->logits_t; sa.ld = ctx->cfg.talker_vocab;
  sa.stream = 0; sa.ctr = ctx->frame_k; sa.ctr_add = 1;
  sa.used = ctx->code0_next; sa.used_ld = 1; sa.used_col = 0;
  sa.own = ctx->own; sa.own_ld = kGroups; sa.own_col = 0;
  sa.epi = forced ? 0 : 2; sa.finished = ctx->finished; sa.state = state; sa.row_max = ctx->max_frames_row;
  sa.frame_k = ctx->frame_k;
  HIPCK(launch_select(sa, s));
  HIPCK(launch_frame_advance(ctx->frame_k, ctx->pos, ctx->finished, B, s));
  return QT_OK;
}

// The code-indexed first-layer tables of predictor steps 1..14. Step st's
// input row is row c of embedding table st - 1 (through the input
// projection when there is one), so its first-layer q/k/v are a function of
// c alone: for every c, lut row c = W_qkv RMSNorm(x_c) and xlut row c = x_c.
// Built once from the packed weights with the scratch-free fp32 projection.
qt_status build_pred_lut(qt_ctx* ctx, hipStream_t s) {
  const Dec &T = ctx->t, &P = ctx->p;
  const int wd = ctx->cfg.weight_dtype;
  const long C = ctx->cfg.codebook;
  for (int st = 1; st < 15; ++st) {
    HIPCK(launch_convert((const char*)ctx->pemb + (size_t)(st - 1) * C * T.H * esize(wd), wd, T.H, ctx->lut_stage,
                         DT_F32, T.H, C, T.H, s));
    LinearArgs a{};
    a.wdtype = wd; a.M = (int)C; a.epi = EPI_STORE; a.eps = P.eps;
    const float* x = ctx->lut_stage;
    if (ctx->cfg.pred_in_proj) {
      a.W = ctx->pproj; a.N = P.H; a.K = T.H; a.X = x; a.ldx = T.H;
      a.Y = ctx->pxlut + (size_t)(st - 1) * C * P.H; a.ldy = P.H;
      HIPCK(launch_linear(a, s));
      x = a.Y;
    }
    a.W = ctx->pl[0].wqkv; a.N = P.qkv; a.K = P.H; a.X = x; a.ldx = P.H; a.gain = ctx->pl[0].attn_norm;
    a.Y = ctx->plut + (size_t)(st - 1) * C * P.qkv; a.ldy = P.qkv;
    HIPCK(launch_linear(a, s));
  }
  return QT_OK;
}

qt_status read_status(qt_ctx* ctx) {
  const int st = ctx->hout[0];
  if (st & ST_NONFINITE) {
    ctx->failed = true;
    set_err(ctx->err, "non-finite logit on the device (frame %d)", ctx->frames_done);
    return QT_E_NAN;
  }
  if (st & ST_RANGE) {
    ctx->failed = true;
    set_err(ctx->err, "code id out of range on the device (frame %d)", ctx->frames_done);
    return QT_E_RANGE;
  }
  return QT_OK;
}

}  // namespace

// ---- scratch of the allocation-free projection entry point (qt_linear_noalloc)
// One array per device, held until the process ends. In host code `scratch`
// names only a host-side stand-in: kernels get the device address that
// hipGetSymbolAddress returns for the current device, cached per device.
constexpr long kNoallocScratchFloats = 8L << 20;   // 32 MiB
static __device__ __align__(256) float scratch[kNoallocScratchFloats];
constexpr int kMaxDevices = 64;
static float* g_scratch_dev[kMaxDevices];
static std::mutex g_scratch_mu;

static qt_status noalloc_scratch(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    set_err(g_err, "no current HIP device (or device index >= %d)", kMaxDevices);
    return QT_E_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      set_err(g_err, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
      return QT_E_HIP;
    }
    g_scratch_dev[dev] = (float*)ptr;
  }
  *out = g_scratch_dev[dev];
  return QT_OK;
}

// Scratch floats a projection of M rows needs for the matrix-core paths:
// the row denominators (rounded up to 64 floats) and either the K-range
// partial sums (up to 128 rows) or the hi/lo split planes of the rows.
static long linear_scratch_floats(long M, long N, long K) {
  return (M + 63) / 64 * 64 + (M <= 128 ? (K / 256) * M * (N + 1) : M * K);
}

extern "C" {

qt_status qt_config_check(const qt_config* cfg) { return check_config(cfg, g_err); }

qt_status qt_workspace_bytes(const qt_config* cfg, size_t* bytes) {
  qt_status s = check_config(cfg, g_err);
  if (s != QT_OK) return s;
  if (!bytes) { set_err(g_err, "bytes is NULL"); return QT_E_INVALID; }
  Layout L = plan_layout(*cfg);
  if (L.ovf) { set_err(g_err, "workspace size overflows size_t"); return QT_E_CAPACITY; }
  *bytes = L.total;
  return QT_OK;
}

const char* qt_last_error(const qt_ctx* ctx) { return ctx ? ctx->err : g_err; }

qt_status qt_create(const qt_config* cfg, const qt_weights* w, void* workspace, size_t ws_bytes, void* hip_stream,
                    qt_ctx** out) {
  qt_status s = check_config(cfg, g_err);
  if (s != QT_OK) return s;
  if (!out) { set_err(g_err, "out is NULL"); return QT_E_INVALID; }
  *out = nullptr;
  if (!w || !w->talker_layers || !w->pred_layers || !w->talker_norm || !w->talker_codec_embed ||
      !w->talker_codec_head || !w->pred_norm || !w->pred_embeds || !w->pred_heads) {
    set_err(g_err, "a weight pointer is NULL");
    return QT_E_INVALID;
  }
  if (cfg->pred_in_proj && !w->pred_in_proj) { set_err(g_err, "pred_in_proj weights are NULL"); return QT_E_INVALID; }
  Layout L = plan_layout(*cfg);
  if (L.ovf) { set_err(g_err, "workspace size overflows size_t"); return QT_E_CAPACITY; }
  if (workspace && ws_bytes < L.total) {
    set_err(g_err, "workspace too small: %zu < %zu bytes", ws_bytes, L.total);
    return QT_E_NOMEM;
  }
  qt_ctx* ctx = new (std::nothrow) qt_ctx();
  if (!ctx) { set_err(g_err, "out of host memory"); return QT_E_NOMEM; }
  ctx->cfg = *cfg;
  ctx->t = Dec::of(cfg->talker);
  ctx->p = Dec::of(cfg->predictor);
  ctx->lay = L;
  ctx->stream = (hipStream_t)hip_stream;
  auto fail = [&](qt_status st) {
    snprintf(g_err, sizeof g_err, "%s", ctx->err);
    qt_destroy(ctx);
    return st;
  };
  if (hipGetDevice(&ctx->device) != hipSuccess) { set_err(ctx->err, "no HIP device"); return fail(QT_E_HIP); }
  if (workspace) {
    ctx->ws = (char*)workspace;
  } else {
    if (hipMalloc((void**)&ctx->ws, L.total) != hipSuccess) {
      set_err(ctx->err, "hipMalloc of %zu bytes failed", L.total);
      return fail(QT_E_NOMEM);
    }
    ctx->own_ws = true;
  }
  if (hipStreamCreateWithFlags(&ctx->cap, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&ctx->ev, hipEventDisableTiming) != hipSuccess) {
    set_err(ctx->err, "stream/event creation failed");
    return fail(QT_E_HIP);
  }
  if (hipHostMalloc((void**)&ctx->hout, (1 + cfg->max_batch + (size_t)cfg->max_batch * kGroups) * sizeof(int)) !=
      hipSuccess) {
    set_err(ctx->err, "pinned host allocation failed");
    return fail(QT_E_NOMEM);
  }
  for (const LayerBuf& b : L.tl)
    ctx->tl.push_back({at<void>(ctx, b.wqkv), at<void>(ctx, b.wo), at<void>(ctx, b.wgu), at<void>(ctx, b.wd),
                       at<float>(ctx, b.attn_norm), at<float>(ctx, b.q_norm), at<float>(ctx, b.k_norm),
                       at<float>(ctx, b.mlp_norm)});
  for (const LayerBuf& b : L.pl)
    ctx->pl.push_back({at<void>(ctx, b.wqkv), at<void>(ctx, b.wo), at<void>(ctx, b.wgu), at<void>(ctx, b.wd),
                       at<float>(ctx, b.attn_norm), at<float>(ctx, b.q_norm), at<float>(ctx, b.k_norm),
                       at<float>(ctx, b.mlp_norm)});
  ctx->talker_norm = at<float>(ctx, L.talker_norm);
  ctx->temb = at<void>(ctx, L.temb);
  ctx->thead = at<void>(ctx, L.thead);
  ctx->pred_norm = at<float>(ctx, L.pred_norm);
  ctx->pemb = at<void>(ctx, L.pemb);
  ctx->phead = at<void>(ctx, L.phead);
  ctx->pproj = cfg->pred_in_proj ? at<void>(ctx, L.pproj) : nullptr;
  ctx->plut = at<float>(ctx, L.plut);
  ctx->pxlut = cfg->pred_in_proj ? at<float>(ctx, L.pxlut) : nullptr;
  ctx->lut_stage = at<float>(ctx, L.lut_stage);
  ctx->cos_t = at<float>(ctx, L.cos_t); ctx->sin_t = at<float>(ctx, L.sin_t);
  ctx->cos_p = at<float>(ctx, L.cos_p); ctx->sin_p = at<float>(ctx, L.sin_p);
  ctx->kc_t = at<void>(ctx, L.kc_t); ctx->vc_t = at<void>(ctx, L.vc_t);
  ctx->kc_p = at<void>(ctx, L.kc_p); ctx->vc_p = at<void>(ctx, L.vc_p);
  ctx->x_t = at<float>(ctx, L.x_t); ctx->qkv = at<float>(ctx, L.qkv); ctx->attn = at<float>(ctx, L.attn);
  ctx->act = at<float>(ctx, L.act); ctx->x_p = at<float>(ctx, L.x_p);
  ctx->xin_w = cfg->pred_in_proj ? at<float>(ctx, L.xin_w) : nullptr;
  ctx->h = at<float>(ctx, L.h); ctx->xlast = at<float>(ctx, L.xlast);
  ctx->logits_t = at<float>(ctx, L.logits_t); ctx->logits_p = at<float>(ctx, L.logits_p);
  ctx->rope_rows = at<float>(ctx, L.rope_rows);
  ctx->row_den = at<float>(ctx, L.row_den);
  ctx->part = at<float>(ctx, L.part);
  ctx->part_floats = L.part_floats;
  ctx->xsplit = L.xsplit_floats > 0 ? at<float>(ctx, L.xsplit) : nullptr;
  ctx->xsplit_floats = L.xsplit_floats;
  ctx->ksplit = at<float>(ctx, L.ksplit);
  int* rs = at<int>(ctx, L.rowstate);
  const int MB = cfg->max_batch;
  ctx->code0_next = rs; ctx->finished = rs + MB; ctx->pos = rs + 2 * MB; ctx->noise_row = rs + 3 * MB;
  ctx->text_len = rs + 4 * MB; ctx->max_frames_row = rs + 5 * MB; ctx->frame_k = rs + 6 * MB;
  ctx->own = rs + 7 * MB; ctx->forced = rs + 7 * MB + kGroups * MB;
  ctx->row_seed = at<uint64_t>(ctx, L.row64);
  ctx->text_ptr = (const float**)(ctx->row_seed + MB);
  ctx->seen = at<uint32_t>(ctx, L.seen);
  ctx->runs = at<Run>(ctx, L.runs);
  ctx->idx = at<int>(ctx, L.idx);
  ctx->frame_out = at<int>(ctx, L.frame_out);
  ctx->req = at<ReqParams>(ctx, L.req);

  hipStream_t st = ctx->stream;
  for (int i = 0; i < ctx->t.L; ++i) {
    qt_status r = pack_layer(ctx, w->talker_layers[i], ctx->t, ctx->tl[i], st);
    if (r != QT_OK) return fail(r);
  }
  for (int i = 0; i < ctx->p.L; ++i) {
    qt_status r = pack_layer(ctx, w->pred_layers[i], ctx->p, ctx->pl[i], st);
    if (r != QT_OK) return fail(r);
  }
  const int wd = cfg->weight_dtype;
  const Dec &T = ctx->t, &P = ctx->p;
  const long V = cfg->talker_vocab, C = cfg->codebook;
  auto conv = [&](const void* src, void* dst, int ddt, long rows, int n) -> bool {
    return launch_convert(src, wd, n, dst, ddt, n, rows, n, st) == hipSuccess;
  };
  bool ok = conv(w->talker_norm, ctx->talker_norm, DT_F32, 1, T.H) && conv(w->talker_codec_embed, ctx->temb, wd, V, T.H) &&
            conv(w->talker_codec_head, ctx->thead, wd, V, T.H) && conv(w->pred_norm, ctx->pred_norm, DT_F32, 1, P.H) &&
            conv(w->pred_embeds, ctx->pemb, wd, 15 * C, T.H) && conv(w->pred_heads, ctx->phead, wd, 15 * C, P.H) &&
            (!cfg->pred_in_proj || conv(w->pred_in_proj, ctx->pproj, wd, P.H, T.H));
  if (!ok) { set_err(ctx->err, "weight repack launch failed"); return fail(QT_E_HIP); }
  {
    qt_status r = build_pred_lut(ctx, st);
    if (r != QT_OK) return fail(r);
  }
  std::vector<float> cs, sn;
  host_rope(cfg->max_positions, T.d, T.theta, cs, sn);
  if (hipMemcpyAsync(ctx->cos_t, cs.data(), cs.size() * 4, hipMemcpyHostToDevice, st) != hipSuccess ||
      hipMemcpyAsync(ctx->sin_t, sn.data(), sn.size() * 4, hipMemcpyHostToDevice, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess) {
    set_err(ctx->err, "rope table upload failed");
    return fail(QT_E_HIP);
  }
  host_rope(kPredPositions, P.d, P.theta, cs, sn);
  if (hipMemcpyAsync(ctx->cos_p, cs.data(), cs.size() * 4, hipMemcpyHostToDevice, st) != hipSuccess ||
      hipMemcpyAsync(ctx->sin_p, sn.data(), sn.size() * 4, hipMemcpyHostToDevice, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess) {
    set_err(ctx->err, "rope table upload failed");
    return fail(QT_E_HIP);
  }
  *out = ctx;
  return QT_OK;
}

void qt_destroy(qt_ctx* ctx) {
  if (!ctx) return;
  if (ctx->stream || ctx->cap) (void)hipDeviceSynchronize();
  if (ctx->gexec) (void)hipGraphExecDestroy(ctx->gexec);
  if (ctx->own_ws && ctx->ws) (void)hipFree(ctx->ws);
  if (ctx->fe.own_ws && ctx->fe.ws) (void)hipFree(ctx->fe.ws);
  if (ctx->hout) (void)hipHostFree(ctx->hout);
  if (ctx->ev) (void)hipEventDestroy(ctx->ev);
  if (ctx->cap) (void)hipStreamDestroy(ctx->cap);
  delete ctx;
}

// Device state of rows row0 .. row0 + n - 1 for a new request each: code 0
// pending, not finished, talker position at the prompt's end, frame counter
// 0, the noise key and row, the frame cap, the trailing text; seen bits,
// own codes and the frame output slots cleared.
static qt_status init_rows(qt_ctx* ctx, int row0, int n, const int32_t* lens, const float* const* text,
                           const int32_t* text_lens, uint64_t seed, const int32_t* noise_rows, int32_t max_frames) {
  const hipStream_t s = ctx->stream;
  std::vector<int> pos(n), nrow(n), tlen(n), mf(n, max_frames);
  std::vector<uint64_t> sd(n, seed);
  std::vector<const float*> tp(n, nullptr);
  for (int i = 0; i < n; ++i) {
    pos[i] = lens[i];
    nrow[i] = noise_rows ? noise_rows[i] : row0 + i;
    tlen[i] = text_lens ? text_lens[i] : 0;
    tp[i] = tlen[i] > 0 ? text[i] : nullptr;
  }
  const size_t ib = (size_t)n * sizeof(int);
  HIPCK(launch_fill_i32(ctx->code0_next + row0, 0, n, s));
  HIPCK(launch_fill_i32(ctx->finished + row0, 0, n, s));
  HIPCK(launch_fill_i32(ctx->frame_k + row0, 0, n, s));
  HIPCK(hipMemcpyAsync(ctx->pos + row0, pos.data(), ib, hipMemcpyHostToDevice, s));
  HIPCK(hipMemcpyAsync(ctx->noise_row + row0, nrow.data(), ib, hipMemcpyHostToDevice, s));
  HIPCK(hipMemcpyAsync(ctx->text_len + row0, tlen.data(), ib, hipMemcpyHostToDevice, s));
  HIPCK(hipMemcpyAsync(ctx->max_frames_row + row0, mf.data(), ib, hipMemcpyHostToDevice, s));
  HIPCK(hipMemcpyAsync(ctx->row_seed + row0, sd.data(), (size_t)n * 8, hipMemcpyHostToDevice, s));
  HIPCK(hipMemcpyAsync((void*)(ctx->text_ptr + row0), tp.data(), (size_t)n * 8, hipMemcpyHostToDevice, s));
  HIPCK(launch_fill_i32((int*)ctx->seen + (size_t)row0 * ctx->lay.seen_words, 0, (long)n * ctx->lay.seen_words, s));
  HIPCK(launch_fill_i32(ctx->own + (size_t)row0 * kGroups, 0, (long)n * kGroups, s));
  HIPCK(launch_fill_i32(ctx->frame_out + 1 + row0, 0, n, s));
  HIPCK(launch_fill_i32(ctx->frame_out + 1 + ctx->cfg.max_batch + (size_t)row0 * kGroups, 0, (long)n * kGroups, s));
  // the pageable host vectors above must outlive their copies
  HIPCK(hipStreamSynchronize(s));
  return QT_OK;
}

// The prompt prefill of rows row0 .. row0 + n - 1 (their rows' state
// initialised): the talker over each prompt at positions 0..P_r-1 in chunks
// of up to kPrefillChunk tokens (K/V rows into the rows' caches), the codec
// head at each row's last position and talker selection 0 (ncnn CustomVoice
// port section 3.1). Synchronises; states of the rows in ctx->hout[1 + row].
static qt_status prefill_rows(qt_ctx* ctx, int row0, int n, const float* prompt, const int32_t* lens) {
  const qt_config& c = ctx->cfg;
  const Dec& T = ctx->t;
  const hipStream_t s = ctx->stream;
  const int MB = c.max_batch;
  long total = 0;
  std::vector<long> start(n + 1, 0);
  for (int r = 0; r < n; ++r) start[r + 1] = start[r] + lens[r];
  total = start[n];
  // run tables after the 3 MB fixed decode entries
  std::vector<Run> runs;
  struct Chunk { long t0; int n; int run0, nrun; int last0, nlast, lastrow0; int tile0, ntile; };
  const bool tiled = attn_prefill_tiles(T.d, T.nq, T.nkv, c.kv_dtype);
  std::vector<Chunk> chunks;
  std::vector<int> lastidx;
  const int base = 3 * MB;
  for (long t0 = 0; t0 < total; t0 += kPrefillChunk) {
    Chunk ch{t0, (int)std::min<long>(kPrefillChunk, total - t0), base + (int)runs.size(), 0, (int)lastidx.size(), 0,
             -1, 0, 0};
    for (int r = 0; r < n; ++r) {
      const long a = std::max(start[r], t0), b = std::min(start[r + 1], t0 + ch.n);
      if (a >= b) continue;
      for (long tk = a; tk < b; ++tk)  // one run per prompt token
        runs.push_back(Run{row0 + r, (int)(tk - t0), 1, (int)(tk - start[r])});
      ch.nrun += (int)(b - a);
      if (start[r + 1] - 1 >= t0 && start[r + 1] - 1 < t0 + ch.n) {
        if (ch.lastrow0 < 0) ch.lastrow0 = row0 + r;
        lastidx.push_back((int)(start[r + 1] - 1 - t0));
        ch.nlast++;
      }
    }
    if (tiled) {   // the attend pass: runs of up to kAttnTileTokens tokens of one row
      ch.tile0 = base + (int)runs.size();
      const size_t first = runs.size();
      for (int r = 0; r < n; ++r) {
        const long a = std::max(start[r], t0), b = std::min(start[r + 1], t0 + ch.n);
        for (long tk = a; tk < b; tk += kAttnTileTokens)
          runs.push_back(Run{row0 + r, (int)(tk - t0), (int)std::min<long>(kAttnTileTokens, b - tk),
                             (int)(tk - start[r])});
      }
      ch.ntile = (int)(runs.size() - first);
      // longest first (a tile's keys end at its last position), so the
      // heaviest blocks do not form the tail of the grid
      std::stable_sort(runs.begin() + first, runs.end(),
                       [](const Run& x, const Run& y) { return x.pos0 + x.ntok > y.pos0 + y.ntok; });
    }
    chunks.push_back(ch);
  }
  if (base + (long)runs.size() > ctx->lay.max_runs) { set_err(ctx->err, "internal: run table overflow"); return QT_E_CAPACITY; }
  HIPCK(hipMemcpyAsync(ctx->runs + base, runs.data(), runs.size() * sizeof(Run), hipMemcpyHostToDevice, s));
  HIPCK(hipMemcpyAsync(ctx->idx, lastidx.data(), lastidx.size() * sizeof(int), hipMemcpyHostToDevice, s));
  for (const Chunk& ch : chunks) {
    HIPCK(hipMemcpyAsync(ctx->x_t, prompt + ch.t0 * T.H, (size_t)ch.n * T.H * 4, hipMemcpyDeviceToDevice, s));
    qt_status r = run_layers(ctx, true, ctx->x_t, ch.n, ctx->runs + ch.run0, ch.nrun, nullptr, 0, s, true, false,
                             false, ctx->runs + ch.tile0, ch.ntile);
    if (r != QT_OK) return r;
    if (ch.nlast > 0)
      HIPCK(launch_copy_rows(ctx->x_t, T.H, ctx->idx + ch.last0, ch.nlast, ctx->xlast + (size_t)ch.lastrow0 * T.H, T.H,
                             T.H, s));
  }
  LinearArgs ta{};
  ta.row_den = ctx->row_den; ta.xs = ctx->xsplit; ta.xs_floats = ctx->xsplit_floats;
  ta.part = ctx->part; ta.part_floats = ctx->part_floats;
  ta.wdtype = c.weight_dtype; ta.W = ctx->thead; ta.N = c.talker_vocab; ta.K = T.H;
  ta.X = ctx->xlast + (size_t)row0 * T.H; ta.ldx = T.H; ta.M = n; ta.gain = ctx->talker_norm; ta.eps = T.eps;
  ta.Y = ctx->logits_t + (size_t)row0 * c.talker_vocab; ta.ldy = c.talker_vocab;
  ta.epi = EPI_STORE; ta.norm_out = ctx->h + (size_t)row0 * T.H; ta.ld_norm = T.H;
  HIPCK(launch_linear(ta, s));
  SelectArgs sa = select_base(ctx, ctx->ts, true);
  sa.B = n; sa.row0 = row0;
  sa.logits = ctx->logits_t; sa.ld = c.talker_vocab; sa.stream = 0; sa.ctr = nullptr; sa.ctr_add = 0;
  sa.used = ctx->code0_next; sa.used_ld = 1; sa.used_col = 0;
  sa.own = ctx->own; sa.own_ld = kGroups; sa.own_col = 0;
  sa.epi = 2; sa.finished = ctx->finished; sa.state = ctx->frame_out + 1;
  sa.frame_k = nullptr;
  HIPCK(launch_select(sa, s));
  HIPCK(hipMemcpyAsync(ctx->hout, ctx->frame_out, (1 + MB) * sizeof(int), hipMemcpyDeviceToHost, s));
  HIPCK(hipStreamSynchronize(s));
  return read_status(ctx);
}

qt_status qt_prefill(qt_ctx* ctx, int32_t B, const float* prompt, const int32_t* prompt_lens, const float* text,
                     const int32_t* text_lens, const float* tts_pad, const qt_sampling* talker,
                     const qt_sampling* predictor, uint64_t seed, int32_t max_frames) {
  if (!ctx) { set_err(g_err, "ctx is NULL"); return QT_E_INVALID; }
  const qt_config& c = ctx->cfg;
  if (B < 1 || B > c.max_batch) { set_err(ctx->err, "B=%d outside 1..max_batch=%d", B, c.max_batch); return QT_E_CAPACITY; }
  if (!prompt || !prompt_lens || !tts_pad) { set_err(ctx->err, "prompt, prompt_lens and tts_pad must not be NULL"); return QT_E_INVALID; }
  if (max_frames < 1) { set_err(ctx->err, "max_frames must be >= 1"); return QT_E_INVALID; }
  if (!sampling_ok(talker, ctx->err, "talker") || !sampling_ok(predictor, ctx->err, "predictor")) return QT_E_INVALID;
  long total = 0, text_total = 0;
  for (int r = 0; r < B; ++r) {
    if (prompt_lens[r] < 1) { set_err(ctx->err, "prompt_lens[%d]=%d must be >= 1", r, prompt_lens[r]); return QT_E_RANGE; }
    if ((long)prompt_lens[r] + max_frames > c.max_positions) {
      set_err(ctx->err, "row %d: prompt %d + max_frames %d exceeds max_positions %d", r, prompt_lens[r], max_frames, c.max_positions);
      return QT_E_CAPACITY;
    }
    total += prompt_lens[r];
    if (text_lens) {
      if (text_lens[r] < 0) { set_err(ctx->err, "text_lens[%d] must be >= 0", r); return QT_E_RANGE; }
      text_total += text_lens[r];
    }
  }
  if (text_total > 0 && !text) { set_err(ctx->err, "text is NULL but text_lens are positive"); return QT_E_INVALID; }
  if (total > (1L << 30)) { set_err(ctx->err, "total prompt length too large"); return QT_E_CAPACITY; }

  ctx->B = B; ctx->prefilled = false; ctx->failed = false; ctx->frames_done = 0; ctx->max_frames = max_frames;
  ctx->done.assign(B, 0); ctx->ts = *talker; ctx->ps = *predictor; ctx->seed = seed;
  ctx->text = text; ctx->pad = tts_pad; ctx->has_text = text_total > 0;
  ctx->eager_frames = 0;
  const Dec& T = ctx->t;
  hipStream_t s = ctx->stream;
  const int MB = c.max_batch;
  // fixed run tables of the frame: one token per row
  std::vector<Run> runs((size_t)3 * MB, Run{0, 0, 0, 0});
  for (int r = 0; r < MB; ++r) {
    runs[r] = Run{r, r, 1, 0};                 // talker decode (pos from the device)
    runs[MB + r] = Run{r, 2 * r, 2, 0};        // predictor pass 0: positions 0, 1
    runs[2 * MB + r] = Run{r, r, 1, 0};        // predictor step s: position s + 1
  }
  HIPCK(hipMemcpyAsync(ctx->runs, runs.data(), runs.size() * sizeof(Run), hipMemcpyHostToDevice, s));
  ReqParams rq{};
  const qt_sampling* sm[2] = {talker, predictor};
  for (int i = 0; i < 2; ++i)
    rq.samp[i] = SampParams{sm[i]->do_sample, sm[i]->temperature, sm[i]->top_k, sm[i]->top_p,
                            sm[i]->repetition_penalty, sm[i]->min_new_tokens};
  rq.pad = tts_pad;
  HIPCK(hipMemcpyAsync(ctx->req, &rq, sizeof rq, hipMemcpyHostToDevice, s));
  HIPCK(launch_fill_i32(ctx->frame_out, 0, 1 + MB + (long)MB * kGroups, s));
  std::vector<const float*> tp(B, nullptr);
  long to = 0;
  for (int r = 0; r < B; ++r) {
    tp[r] = text ? text + to * T.H : nullptr;
    to += text_lens ? text_lens[r] : 0;
  }
  QTCK(init_rows(ctx, 0, B, prompt_lens, tp.data(), text_lens, seed, nullptr, max_frames));
  qt_status r = prefill_rows(ctx, 0, B, prompt, prompt_lens);
  if (r != QT_OK) return r;
  for (int i = 0; i < B; ++i) ctx->done[i] = ctx->hout[1 + i] == 1;
  ctx->prefilled = true;
  return QT_OK;
}

qt_status qt_admit(qt_ctx* ctx, int32_t slot, const float* prompt, int32_t prompt_len, const float* text,
                   int32_t text_len, uint64_t seed, int32_t noise_row, int32_t max_frames) {
  if (!ctx) { set_err(g_err, "ctx is NULL"); return QT_E_INVALID; }
  const qt_config& c = ctx->cfg;
  if (!ctx->prefilled || ctx->failed) { set_err(ctx->err, "qt_admit needs a successful qt_prefill first"); return QT_E_STATE; }
  if (slot < 0 || slot >= ctx->B) { set_err(ctx->err, "slot %d outside 0..B-1=%d", slot, ctx->B - 1); return QT_E_RANGE; }
  if (!ctx->done[slot]) { set_err(ctx->err, "slot %d still holds an active request", slot); return QT_E_STATE; }
  if (!prompt) { set_err(ctx->err, "prompt must not be NULL"); return QT_E_INVALID; }
  if (prompt_len < 1) { set_err(ctx->err, "prompt_len must be >= 1"); return QT_E_RANGE; }
  if (max_frames < 1) { set_err(ctx->err, "max_frames must be >= 1"); return QT_E_INVALID; }
  if ((long)prompt_len + max_frames > c.max_positions) {
    set_err(ctx->err, "prompt %d + max_frames %d exceeds max_positions %d", prompt_len, max_frames, c.max_positions);
    return QT_E_CAPACITY;
  }
  if (text_len < 0) { set_err(ctx->err, "text_len must be >= 0"); return QT_E_RANGE; }
  if (text_len > 0 && !text) { set_err(ctx->err, "text is NULL but text_len is positive"); return QT_E_INVALID; }
  if (noise_row < 0) { set_err(ctx->err, "noise_row must be >= 0"); return QT_E_RANGE; }
  const float* tp[1] = {text};
  QTCK(init_rows(ctx, slot, 1, &prompt_len, tp, &text_len, seed, &noise_row, max_frames));
  qt_status r = prefill_rows(ctx, slot, 1, prompt, &prompt_len);
  if (r != QT_OK) return r;
  ctx->done[slot] = ctx->hout[1 + slot] == 1;
  return QT_OK;
}

static qt_status frame_common(qt_ctx* ctx, const int* forced_dev) {
  hipStream_t s = ctx->stream;
  const int MB = ctx->cfg.max_batch;
  if (forced_dev) {
    qt_status r = enqueue_frame(ctx, s, forced_dev);
    if (r != QT_OK) return r;
  } else {
    // the first frame after a prefill runs eagerly; later frames replay one captured graph
    if (ctx->gexec && ctx->graph_B == ctx->B && ctx->graph_pred_sample == ctx->ps.do_sample) {
      HIPCK(hipGraphLaunch(ctx->gexec, s));
    } else if (ctx->eager_frames == 0) {
      qt_status r = enqueue_frame(ctx, s, nullptr);
      if (r != QT_OK) return r;
      ctx->eager_frames++;
    } else {
      if (ctx->gexec) { (void)hipGraphExecDestroy(ctx->gexec); ctx->gexec = nullptr; }
      HIPCK(hipStreamSynchronize(s));
      hipGraph_t g = nullptr;
      HIPCK(hipStreamBeginCapture(ctx->cap, hipStreamCaptureModeThreadLocal));
      qt_status r = enqueue_frame(ctx, ctx->cap, nullptr);
      hipError_t e = hipStreamEndCapture(ctx->cap, &g);
      if (r != QT_OK) { if (g) (void)hipGraphDestroy(g); return r; }
      if (e != hipSuccess) { set_err(ctx->err, "graph capture failed: %s", hipGetErrorString(e)); return QT_E_HIP; }
      e = hipGraphInstantiate(&ctx->gexec, g, nullptr, nullptr, 0);
      (void)hipGraphDestroy(g);
      if (e != hipSuccess) { ctx->gexec = nullptr; set_err(ctx->err, "graph instantiate failed: %s", hipGetErrorString(e)); return QT_E_HIP; }
      ctx->graph_B = ctx->B;
      ctx->graph_pred_sample = ctx->ps.do_sample;
      HIPCK(hipGraphLaunch(ctx->gexec, s));
    }
  }
  HIPCK(hipMemcpyAsync(ctx->hout, ctx->frame_out, (1 + MB + (size_t)MB * kGroups) * sizeof(int), hipMemcpyDeviceToHost, s));
  HIPCK(hipEventRecord(ctx->ev, s));
  HIPCK(hipEventSynchronize(ctx->ev));
  return read_status(ctx);
}

qt_status qt_step_frame(qt_ctx* ctx, int32_t* codes, uint8_t* state) {
  if (!ctx) { set_err(g_err, "ctx is NULL"); return QT_E_INVALID; }
  if (!codes || !state) { set_err(ctx->err, "codes and state must not be NULL"); return QT_E_INVALID; }
  if (!ctx->prefilled || ctx->failed) { set_err(ctx->err, "qt_step_frame needs a successful qt_prefill first"); return QT_E_STATE; }
  bool any = false;
  for (int r = 0; r < ctx->B; ++r) any |= !ctx->done[r];
  if (!any) { set_err(ctx->err, "every row has finished"); return QT_E_STATE; }
  qt_status r = frame_common(ctx, nullptr);
  if (r != QT_OK) return r;
  const int MB = ctx->cfg.max_batch;
  for (int i = 0; i < ctx->B; ++i) {
    const int st = ctx->hout[1 + i];
    state[i] = (uint8_t)(ctx->done[i] ? 3 : st);
    if (!ctx->done[i] && (st == 1 || st == 2)) ctx->done[i] = 1;
    memcpy(codes + (size_t)i * kGroups, ctx->hout + 1 + MB + (size_t)i * kGroups, kGroups * sizeof(int));
  }
  ctx->frames_done++;
  return QT_OK;
}

qt_status qt_generate(qt_ctx* ctx, int32_t B, const float* prompt, const int32_t* prompt_lens, const float* text,
                      const int32_t* text_lens, const float* tts_pad, const qt_sampling* talker,
                      const qt_sampling* predictor, uint64_t seed, int32_t max_frames, int32_t* codes,
                      int32_t* n_frames, uint8_t* finish) {
  if (!ctx) { set_err(g_err, "ctx is NULL"); return QT_E_INVALID; }
  if (!codes || !n_frames || !finish) { set_err(ctx->err, "codes, n_frames and finish must not be NULL"); return QT_E_INVALID; }
  qt_status r = qt_prefill(ctx, B, prompt, prompt_lens, text, text_lens, tts_pad, talker, predictor, seed, max_frames);
  if (r != QT_OK) return r;
  std::vector<int32_t> fc((size_t)B * kGroups);
  std::vector<uint8_t> st(B);
  for (int i = 0; i < B; ++i) {
    n_frames[i] = 0;
    finish[i] = ctx->done[i] ? 1 : 0;
  }
  while (true) {
    bool any = false;
    for (int i = 0; i < B; ++i) any |= !ctx->done[i];
    if (!any) break;
    r = qt_step_frame(ctx, fc.data(), st.data());
    if (r != QT_OK) return r;
    for (int i = 0; i < B; ++i) {
      if (st[i] == 3) continue;
      memcpy(codes + ((size_t)i * max_frames + n_frames[i]) * kGroups, fc.data() + (size_t)i * kGroups,
             kGroups * sizeof(int32_t));
      n_frames[i]++;
      if (st[i] == 1 || st[i] == 2) finish[i] = st[i];
    }
  }
  return QT_OK;
}

// ---- token-id frontend

// out[i] = ResizeMLP(text_embed[tids[i]]) + codec_embed[cids[i]] (+ extra[i]),
// empty tracks (-1) as zero rows; ids already validated, n <= max_rows.
static qt_status fe_embed(qt_ctx* ctx, int n, const int* tids, const int* cids, const float* extra, float* out) {
  auto& fe = ctx->fe;
  const hipStream_t s = ctx->stream;
  const int H = ctx->t.H, Ti = fe.fc.text_hidden, Hm = fe.fc.mlp_hidden, wd = ctx->cfg.weight_dtype;
  HIPCK(hipMemcpyAsync(fe.tids, tids, (size_t)n * 4, hipMemcpyHostToDevice, s));
  HIPCK(hipMemcpyAsync(fe.cids, cids, (size_t)n * 4, hipMemcpyHostToDevice, s));
  HIPCK(hipStreamSynchronize(s));   // the host id arrays may go away after this call
  for (int r0 = 0; r0 < n; r0 += fe.chunk) {
    const int m = std::min(fe.chunk, n - r0);
    HIPCK(launch_gather_rows(fe.embed, wd, Ti, fe.tids + r0, m, fe.x0, s));
    LinearArgs a{};
    a.wdtype = wd; a.eps = 1e-6f; a.M = m; a.epi = EPI_STORE;
    const long den = ((long)m + 63) / 64 * 64;
    a.row_den = fe.scratch; a.part = fe.scratch + den; a.part_floats = fe.scratch_floats - den;
    a.xs = a.part; a.xs_floats = a.part_floats;
    a.W = fe.fc1; a.N = Hm; a.K = Ti; a.X = fe.x0; a.ldx = Ti; a.Y = fe.h1; a.ldy = Hm;
    HIPCK(launch_linear(a, s));
    HIPCK(launch_bias_silu(fe.h1, m, Hm, fe.b1, s));
    a.W = fe.fc2; a.N = H; a.K = Hm; a.X = fe.h1; a.ldx = Hm; a.Y = fe.y; a.ldy = H;
    HIPCK(launch_linear(a, s));
    HIPCK(launch_assemble_rows(fe.y, fe.b2, fe.tids + r0, fe.cids + r0, ctx->temb, wd,
                               extra ? extra + (size_t)r0 * H : nullptr, out + (size_t)r0 * H, m, H, s));
  }
  return QT_OK;
}

static qt_status check_ids(qt_ctx* ctx, int n, const int* ids, int hi, const char* who) {
  for (int i = 0; i < n; ++i)
    if (ids[i] < -1 || ids[i] >= hi) {
      set_err(ctx->err, "%s[%d]=%d outside -1..%d", who, i, ids[i], hi - 1);
      return QT_E_RANGE;
    }
  return QT_OK;
}

qt_status qt_frontend_bytes(const qt_config* cfg, const qt_frontend_config* fc, size_t* bytes) {
  qt_status s = check_config(cfg, g_err);
  if (s != QT_OK) return s;
  if (!frontend_ok(*cfg, fc, g_err)) return QT_E_INVALID;
  if (!bytes) { set_err(g_err, "bytes is NULL"); return QT_E_INVALID; }
  FeLayout L = plan_frontend(*cfg, *fc);
  if (L.ovf) { set_err(g_err, "frontend workspace size overflows size_t"); return QT_E_CAPACITY; }
  *bytes = L.total;
  return QT_OK;
}

qt_status qt_attach_frontend(qt_ctx* ctx, const qt_frontend_config* fc, const qt_frontend_weights* fw, void* workspace,
                             size_t ws_bytes) {
  if (!ctx) { set_err(g_err, "ctx is NULL"); return QT_E_INVALID; }
  if (!frontend_ok(ctx->cfg, fc, ctx->err)) return QT_E_INVALID;
  if (!fw || !fw->text_embed || !fw->fc1_w || !fw->fc2_w) {
    set_err(ctx->err, "frontend weights (text_embed, fc1_w, fc2_w) must not be NULL");
    return QT_E_INVALID;
  }
  FeLayout L = plan_frontend(ctx->cfg, *fc);
  if (L.ovf) { set_err(ctx->err, "frontend workspace size overflows size_t"); return QT_E_CAPACITY; }
  if (workspace && ws_bytes < L.total) {
    set_err(ctx->err, "frontend workspace too small: %zu < %zu bytes", ws_bytes, L.total);
    return QT_E_NOMEM;
  }
  auto& fe = ctx->fe;
  HIPCK(hipStreamSynchronize(ctx->stream));
  if (fe.own_ws && fe.ws) (void)hipFree(fe.ws);
  fe = qt_ctx::Frontend{};
  if (workspace) {
    fe.ws = (char*)workspace;
  } else {
    if (hipMalloc((void**)&fe.ws, L.total) != hipSuccess) {
      set_err(ctx->err, "hipMalloc of %zu frontend bytes failed", L.total);
      fe.ws = nullptr;
      return QT_E_NOMEM;
    }
    fe.own_ws = true;
  }
  fe.fc = *fc;
  fe.embed = fe.ws + L.embed; fe.fc1 = fe.ws + L.fc1; fe.fc2 = fe.ws + L.fc2;
  fe.b1 = (float*)(fe.ws + L.b1); fe.b2 = (float*)(fe.ws + L.b2);
  fe.tids = (int*)(fe.ws + L.tids); fe.cids = (int*)(fe.ws + L.cids);
  fe.x0 = (float*)(fe.ws + L.x0); fe.h1 = (float*)(fe.ws + L.h1); fe.y = (float*)(fe.ws + L.y);
  fe.scratch = (float*)(fe.ws + L.scratch); fe.scratch_floats = L.scratch_floats; fe.chunk = L.chunk;
  fe.prompt = (float*)(fe.ws + L.rows);
  const int wd = ctx->cfg.weight_dtype, H = ctx->t.H, Ti = fc->text_hidden, Hm = fc->mlp_hidden;
  const hipStream_t s = ctx->stream;
  HIPCK(launch_convert(fw->text_embed, wd, Ti, fe.embed, wd, Ti, fc->text_vocab, Ti, s));
  HIPCK(launch_convert(fw->fc1_w, wd, Ti, fe.fc1, wd, Ti, Hm, Ti, s));
  HIPCK(launch_convert(fw->fc2_w, wd, Hm, fe.fc2, wd, Hm, H, Hm, s));
  if (fw->fc1_b) HIPCK(launch_convert(fw->fc1_b, wd, Hm, fe.b1, DT_F32, Hm, 1, Hm, s));
  else HIPCK(launch_fill_i32((int*)fe.b1, 0, Hm, s));
  if (fw->fc2_b) HIPCK(launch_convert(fw->fc2_b, wd, H, fe.b2, DT_F32, H, 1, H, s));
  else HIPCK(launch_fill_i32((int*)fe.b2, 0, H, s));
  HIPCK(hipStreamSynchronize(s));
  fe.on = true;
  return QT_OK;
}

qt_status qt_embed_ids(qt_ctx* ctx, int32_t n, const int32_t* text_ids, const int32_t* codec_ids, const float* extra,
                       float* out) {
  if (!ctx) { set_err(g_err, "ctx is NULL"); return QT_E_INVALID; }
  if (!ctx->fe.on) { set_err(ctx->err, "no frontend attached (qt_attach_frontend)"); return QT_E_STATE; }
  if (n < 1 || n > ctx->fe.fc.max_rows) { set_err(ctx->err, "n=%d outside 1..max_rows=%d", n, ctx->fe.fc.max_rows); return QT_E_CAPACITY; }
  if (!text_ids || !codec_ids || !out) { set_err(ctx->err, "text_ids, codec_ids and out must not be NULL"); return QT_E_INVALID; }
  if (((uintptr_t)out | (uintptr_t)extra) % 16) { set_err(ctx->err, "out and extra must be 16-byte aligned"); return QT_E_INVALID; }
  QTCK(check_ids(ctx, n, text_ids, ctx->fe.fc.text_vocab, "text_ids"));
  QTCK(check_ids(ctx, n, codec_ids, ctx->cfg.talker_vocab, "codec_ids"));
  return fe_embed(ctx, n, text_ids, codec_ids, extra, out);
}

qt_status qt_prefill_ids(qt_ctx* ctx, int32_t B, const int32_t* text_ids, const int32_t* codec_ids,
                         const int32_t* prompt_lens, const int32_t* trailing_ids, const int32_t* trailing_lens,
                         int32_t tts_pad_id, const qt_sampling* talker, const qt_sampling* predictor, uint64_t seed,
                         int32_t max_frames) {
  if (!ctx) { set_err(g_err, "ctx is NULL"); return QT_E_INVALID; }
  if (!ctx->fe.on) { set_err(ctx->err, "no frontend attached (qt_attach_frontend)"); return QT_E_STATE; }
  if (B < 1 || B > ctx->cfg.max_batch) { set_err(ctx->err, "B=%d outside 1..max_batch=%d", B, ctx->cfg.max_batch); return QT_E_CAPACITY; }
  if (!text_ids || !codec_ids || !prompt_lens) { set_err(ctx->err, "text_ids, codec_ids and prompt_lens must not be NULL"); return QT_E_INVALID; }
  long P = 0, Tn = 0;
  for (int r = 0; r < B; ++r) {
    if (prompt_lens[r] < 1) { set_err(ctx->err, "prompt_lens[%d]=%d must be >= 1", r, prompt_lens[r]); return QT_E_RANGE; }
    P += prompt_lens[r];
    if (trailing_lens) {
      if (trailing_lens[r] < 0) { set_err(ctx->err, "trailing_lens[%d] must be >= 0", r); return QT_E_RANGE; }
      Tn += trailing_lens[r];
    }
  }
  if (Tn > 0 && !trailing_ids) { set_err(ctx->err, "trailing_ids is NULL but trailing_lens are positive"); return QT_E_INVALID; }
  const long rows = P + Tn + 1;
  if (rows > ctx->fe.fc.max_rows) {
    set_err(ctx->err, "%ld prompt + trailing + pad rows exceed the frontend's max_rows=%d", rows, ctx->fe.fc.max_rows);
    return QT_E_CAPACITY;
  }
  if (tts_pad_id < 0 || tts_pad_id >= ctx->fe.fc.text_vocab) { set_err(ctx->err, "tts_pad_id out of range"); return QT_E_RANGE; }
  QTCK(check_ids(ctx, (int)P, text_ids, ctx->fe.fc.text_vocab, "text_ids"));
  QTCK(check_ids(ctx, (int)P, codec_ids, ctx->cfg.talker_vocab, "codec_ids"));
  if (Tn > 0) {
    QTCK(check_ids(ctx, (int)Tn, trailing_ids, ctx->fe.fc.text_vocab, "trailing_ids"));
    for (long i = 0; i < Tn; ++i)
      if (trailing_ids[i] < 0) { set_err(ctx->err, "trailing_ids[%ld] must be a text id", i); return QT_E_RANGE; }
  }
  std::vector<int> tid((size_t)rows), cid((size_t)rows, -1);
  memcpy(tid.data(), text_ids, (size_t)P * 4);
  memcpy(cid.data(), codec_ids, (size_t)P * 4);
  if (Tn > 0) memcpy(tid.data() + P, trailing_ids, (size_t)Tn * 4);
  tid[(size_t)rows - 1] = tts_pad_id;
  QTCK(fe_embed(ctx, (int)rows, tid.data(), cid.data(), nullptr, ctx->fe.prompt));
  const int H = ctx->t.H;
  return qt_prefill(ctx, B, ctx->fe.prompt, prompt_lens, Tn > 0 ? ctx->fe.prompt + (size_t)P * H : nullptr,
                    Tn > 0 ? trailing_lens : nullptr, ctx->fe.prompt + (size_t)(P + Tn) * H, talker, predictor, seed,
                    max_frames);
}

qt_status qt_debug_step_forced(qt_ctx* ctx, const int32_t* forced, float* talker_logits, float* pred_logits,
                               int32_t* chosen) {
  if (!ctx) { set_err(g_err, "ctx is NULL"); return QT_E_INVALID; }
  if (!forced) { set_err(ctx->err, "forced must not be NULL"); return QT_E_INVALID; }
  if (!ctx->prefilled || ctx->failed) { set_err(ctx->err, "qt_debug_step_forced needs a successful qt_prefill first"); return QT_E_STATE; }
  if (ctx->frames_done >= ctx->max_frames) { set_err(ctx->err, "max_frames reached"); return QT_E_STATE; }
  const qt_config& c = ctx->cfg;
  const int B = ctx->B, MB = c.max_batch;
  for (int r = 0; r < B; ++r)
    for (int g = 0; g < kGroups; ++g) {
      const int v = forced[r * kGroups + g];
      const int hi = g == 0 ? c.talker_vocab : c.codebook;
      if (v < 0 || v >= hi) { set_err(ctx->err, "forced[%d][%d]=%d out of range", r, g, v); return QT_E_RANGE; }
    }
  hipStream_t s = ctx->stream;
  HIPCK(hipMemcpyAsync(ctx->forced, forced, (size_t)B * kGroups * sizeof(int), hipMemcpyHostToDevice, s));
  qt_status r = frame_common(ctx, ctx->forced);
  if (r != QT_OK) return r;
  if (talker_logits)
    HIPCK(hipMemcpy(talker_logits, ctx->logits_t, (size_t)B * c.talker_vocab * 4, hipMemcpyDeviceToHost));
  if (pred_logits) {
    std::vector<float> tmp((size_t)15 * MB * c.codebook);
    HIPCK(hipMemcpy(tmp.data(), ctx->logits_p, tmp.size() * 4, hipMemcpyDeviceToHost));
    for (int st = 0; st < 15; ++st)
      for (int i = 0; i < B; ++i)
        memcpy(pred_logits + ((size_t)i * 15 + st) * c.codebook, tmp.data() + ((size_t)st * MB + i) * c.codebook,
               (size_t)c.codebook * 4);
  }
  if (chosen) HIPCK(hipMemcpy(chosen, ctx->own, (size_t)B * kGroups * sizeof(int), hipMemcpyDeviceToHost));
  ctx->frames_done++;
  return QT_OK;
}

qt_status qt_debug_talker_logits(qt_ctx* ctx, float* logits) {
  if (!ctx) { set_err(g_err, "ctx is NULL"); return QT_E_INVALID; }
  if (!logits) { set_err(ctx->err, "logits must not be NULL"); return QT_E_INVALID; }
  if (!ctx->prefilled) { set_err(ctx->err, "no prefill yet"); return QT_E_STATE; }
  HIPCK(hipStreamSynchronize(ctx->stream));
  HIPCK(hipMemcpy(logits, ctx->logits_t, (size_t)ctx->B * ctx->cfg.talker_vocab * 4, hipMemcpyDeviceToHost));
  return QT_OK;
}

qt_status qt_debug_select(void* hip_stream, int32_t B, int32_t V, const float* logits, const uint32_t* seen,
                          const float* noise, const float* probs, int32_t processors, int32_t eos,
                          int32_t suppress_begin, int32_t suppress_end, const qt_sampling* samp, uint64_t seed,
                          int32_t stream, int32_t sel_index, int32_t* out_code, float* processed, int32_t* status) {
  if (B < 1 || B > 65535 || V < 2 || V > kMaxVocab) { set_err(g_err, "B or V out of range"); return QT_E_INVALID; }
  if (!logits || !out_code || !status) { set_err(g_err, "logits, out_code and status must not be NULL"); return QT_E_INVALID; }
  if (!sampling_ok(samp, g_err, "select")) return QT_E_INVALID;
  if (processors && (eos < 0 || eos >= V || suppress_begin < 0 || suppress_begin > suppress_end || suppress_end > V)) {
    set_err(g_err, "eos / suppress range out of range");
    return QT_E_INVALID;
  }
  if (sel_index < 0 || stream < 0) { set_err(g_err, "sel_index and stream must be >= 0"); return QT_E_INVALID; }
  SelectArgs a{};
  a.logits = logits; a.ld = V; a.V = V; a.B = B;
  a.processors = processors;
  a.seen = const_cast<uint32_t*>(seen); a.seen_words = (V + 31) / 32;
  a.penalty = seen ? samp->repetition_penalty : 1.0f; a.min_new = samp->min_new_tokens;
  a.eos = eos; a.sup_b = suppress_begin; a.sup_e = suppress_end;
  a.do_sample = samp->do_sample; a.temperature = samp->temperature; a.top_k = samp->top_k; a.top_p = samp->top_p;
  a.seed = seed; a.stream = stream; a.ctr = nullptr; a.ctr_add = sel_index;
  a.noise_in = noise; a.probs_in = probs;
  a.used = out_code; a.used_ld = 1; a.used_col = 0;
  a.processed_out = processed; a.status = status; a.epi = 0;
  hipError_t e = launch_select(a, (hipStream_t)hip_stream);
  if (e != hipSuccess) { set_err(g_err, "select launch failed: %s", hipGetErrorString(e)); return QT_E_HIP; }
  return QT_OK;
}

qt_status qt_debug_exp_noise(void* hip_stream, int32_t mode, const uint64_t* in, int64_t n, uint64_t seed,
                             float* out) {
  if (mode != 0 && mode != 1) { set_err(g_err, "mode must be 0 (counters) or 1 (words)"); return QT_E_INVALID; }
  if (n < 0 || n > (1L << 30)) { set_err(g_err, "n must be in 0..2^30"); return QT_E_INVALID; }
  if (n > 0 && (!in || !out)) { set_err(g_err, "in and out must not be NULL"); return QT_E_INVALID; }
  hipError_t e = launch_noise(in, mode, seed, out, n, (hipStream_t)hip_stream);
  if (e != hipSuccess) { set_err(g_err, "noise launch failed: %s", hipGetErrorString(e)); return QT_E_HIP; }
  return QT_OK;
}

qt_status qt_debug_linear(void* hip_stream, int32_t wdtype, const void* W, int32_t N, int32_t K, const float* X,
                          int32_t M, const float* gain, float eps, int32_t epilogue, float* Y, float* scratch,
                          int64_t scratch_floats, int32_t reps, int32_t w_copies, int64_t w_copy_stride) {
  if (wdtype != QT_DTYPE_F32 && wdtype != QT_DTYPE_BF16) { set_err(g_err, "bad wdtype"); return QT_E_INVALID; }
  if (!W || !X || !Y) { set_err(g_err, "W, X and Y must not be NULL"); return QT_E_INVALID; }
  if (N < 1 || K < 8 || K % 8 || M < 1 || reps < 1 || epilogue < 0 || epilogue > 2 || (epilogue == 2 && N % 2)) {
    set_err(g_err, "bad shape: need N >= 1, K a positive multiple of 8, M >= 1, even N for SwiGLU");
    return QT_E_INVALID;
  }
  if (K > 24576) { set_err(g_err, "K too large for the LDS activation tile"); return QT_E_INVALID; }
  LinearArgs a{};
  a.W = W; a.wdtype = wdtype; a.N = N; a.K = K; a.X = X; a.ldx = K; a.M = M; a.gain = gain; a.eps = eps;
  a.Y = Y; a.ldy = epilogue == 2 ? N / 2 : N; a.epi = epilogue;
  if (scratch && scratch_floats >= M) {
    const long den = ((long)M + 63) / 64 * 64;   // partial sums start 256-byte aligned
    a.row_den = scratch;
    if (scratch_floats > den) {
      a.part = scratch + den; a.part_floats = scratch_floats - den;
      a.xs = a.part; a.xs_floats = a.part_floats;   // the split of > 128 rows needs no partial sums
    }
  }
  if (w_copies < 1 || (w_copies > 1 && w_copy_stride < (int64_t)N * K * (wdtype == QT_DTYPE_BF16 ? 2 : 4))) {
    set_err(g_err, "w_copies must be >= 1 and copies must not overlap");
    return QT_E_INVALID;
  }
  for (int i = 0; i < reps; ++i) {
    a.W = (const char*)W + (long)(i % w_copies) * w_copy_stride;
    hipError_t e = launch_linear(a, (hipStream_t)hip_stream);
    if (e != hipSuccess) { set_err(g_err, "linear launch failed: %s", hipGetErrorString(e)); return QT_E_HIP; }
  }
  return QT_OK;
}

qt_status qt_linear_noalloc(void* hip_stream, int32_t wdtype, const void* W, int32_t N, int32_t K, const float* X,
                            int32_t M, const float* gain, float eps, int32_t epilogue, float* Y) {
  if (wdtype != QT_DTYPE_F32 && wdtype != QT_DTYPE_BF16) { set_err(g_err, "bad wdtype"); return QT_E_INVALID; }
  if (!W || !X || !Y) { set_err(g_err, "W, X and Y must not be NULL"); return QT_E_INVALID; }
  if (N < 1 || K < 8 || K % 8 || M < 1 || epilogue < 0 || epilogue > 2 || (epilogue == 2 && N % 2)) {
    set_err(g_err, "bad shape: need N >= 1, K a positive multiple of 8, M >= 1, even N for SwiGLU");
    return QT_E_INVALID;
  }
  if (K > 24576) { set_err(g_err, "K too large for the LDS activation tile"); return QT_E_INVALID; }
  const long need = linear_scratch_floats(M, N, K);
  if (need > kNoallocScratchFloats) {
    set_err(g_err, "projection needs %ld scratch floats, above the %ld of the static scratch", need,
            kNoallocScratchFloats);
    return QT_E_CAPACITY;
  }
  float* sc = nullptr;
  const qt_status st = noalloc_scratch(&sc);
  if (st != QT_OK) return st;
  LinearArgs a{};
  a.W = W; a.wdtype = wdtype; a.N = N; a.K = K; a.X = X; a.ldx = K; a.M = M; a.gain = gain; a.eps = eps;
  a.Y = Y; a.ldy = epilogue == 2 ? N / 2 : N; a.epi = epilogue;
  const long den = ((long)M + 63) / 64 * 64;
  a.row_den = sc;
  a.part = sc + den; a.part_floats = need - den;
  a.xs = a.part; a.xs_floats = a.part_floats;
  const hipError_t e = launch_linear(a, (hipStream_t)hip_stream);
  if (e != hipSuccess) { set_err(g_err, "linear launch failed: %s", hipGetErrorString(e)); return QT_E_HIP; }
  return QT_OK;
}

qt_status qt_debug_prefill_attention(void* hip_stream, int32_t kv_dtype, int32_t head_dim, int32_t nq, int32_t nkv,
                                     int32_t B, const int32_t* lens, int32_t max_pos, const float* qkv,
                                     const float* q_gain, const float* k_gain, float eps, const float* cos,
                                     const float* sin, void* kc, void* vc, float* out, int32_t tiled,
                                     int32_t* runs, int64_t runs_ints) {
  if (kv_dtype != QT_DTYPE_F32 && kv_dtype != QT_DTYPE_BF16 && kv_dtype != QT_DTYPE_F16) {
    set_err(g_err, "bad kv_dtype");
    return QT_E_INVALID;
  }
  const int G = nkv > 0 ? nq / nkv : 0;
  if (!(head_dim == 16 || head_dim == 32 || head_dim == 64 || head_dim == 128 || head_dim == 256) || nkv < 1 ||
      nq % nkv || !(G == 1 || G == 2 || G == 4 || G == 8) || B < 1 || max_pos < 1 || !(eps > 0.f)) {
    set_err(g_err, "bad shape");
    return QT_E_INVALID;
  }
  if (!lens || !qkv || !q_gain || !k_gain || !cos || !sin || !kc || !vc || !out || !runs) {
    set_err(g_err, "NULL argument");
    return QT_E_INVALID;
  }
  if (tiled && !attn_prefill_tiles(head_dim, nq, nkv, kv_dtype)) {
    set_err(g_err, "no tiled prefill attention for this shape");
    return QT_E_INVALID;
  }
  std::vector<Run> rv;
  long T = 0;
  for (int r = 0; r < B; ++r) {
    if (lens[r] < 1 || lens[r] > max_pos) { set_err(g_err, "lens[%d] out of 1..max_pos", r); return QT_E_INVALID; }
    T += lens[r];
  }
  if (T > (1L << 24) || runs_ints < 4 * (T + T / kAttnTileTokens + B)) {
    set_err(g_err, "run scratch too small or too many tokens");
    return QT_E_INVALID;
  }
  // one run per token (the write pass), then runs of up to kAttnTileTokens
  long t0 = 0;
  for (int r = 0; r < B; ++r) {
    for (int i = 0; i < lens[r]; ++i) rv.push_back(Run{r, (int)(t0 + i), 1, i});
    t0 += lens[r];
  }
  const int ntok = (int)rv.size();
  t0 = 0;
  for (int r = 0; r < B; ++r) {
    for (int i = 0; i < lens[r]; i += kAttnTileTokens)
      rv.push_back(Run{r, (int)(t0 + i), std::min(kAttnTileTokens, lens[r] - i), i});
    t0 += lens[r];
  }
  hipStream_t s = (hipStream_t)hip_stream;
  hipError_t e = hipMemcpyAsync(runs, rv.data(), rv.size() * sizeof(Run), hipMemcpyHostToDevice, s);
  AttnArgs t{};
  t.qkv = qkv; t.ld_qkv = (long)(nq + 2 * nkv) * head_dim; t.out = out; t.ld_out = (long)nq * head_dim;
  t.q_gain = q_gain; t.k_gain = k_gain; t.eps = eps; t.scale = (float)(1.0 / std::sqrt((double)head_dim));
  t.cos = cos; t.sin = sin; t.kc = kc; t.vc = vc; t.kvdtype = kv_dtype;
  t.row_stride = (long)nkv * max_pos * head_dim; t.max_pos = max_pos;
  t.nq = nq; t.nkv = nkv; t.d = head_dim;
  t.runs = (const Run*)runs; t.n_runs = ntok;
  t.mode = ATT_WRITE;
  if (e == hipSuccess) e = launch_attention(t, s);
  t.mode = ATT_ATTEND;
  if (tiled) { t.runs = (const Run*)runs + ntok; t.n_runs = (int)rv.size() - ntok; t.max_ntok = kAttnTileTokens; }
  if (e == hipSuccess) e = launch_attention(t, s);
  const hipError_t e2 = hipStreamSynchronize(s);   // also keeps rv alive until the copy has been made
  if (e == hipSuccess) e = e2;
  if (e != hipSuccess) { set_err(g_err, "prefill attention failed: %s", hipGetErrorString(e)); return QT_E_HIP; }
  return QT_OK;
}

qt_status qt_debug_decode_attention(void* hip_stream, int32_t kv_dtype, int32_t head_dim, int32_t nq, int32_t nkv,
                                    int32_t B, int32_t ntok, const int32_t* pos, int32_t* pos_dev, int32_t max_pos,
                                    const float* qkv, const float* q_gain, const float* k_gain, float eps,
                                    const float* cos, const float* sin, void* kc, void* vc, float* out,
                                    int32_t kv_split, float* split_buf) {
  if (kv_dtype != QT_DTYPE_F32 && kv_dtype != QT_DTYPE_BF16 && kv_dtype != QT_DTYPE_F16) {
    set_err(g_err, "bad kv_dtype");
    return QT_E_INVALID;
  }
  const int G = nkv > 0 ? nq / nkv : 0;
  if (!(head_dim == 16 || head_dim == 32 || head_dim == 64 || head_dim == 128 || head_dim == 256) || nkv < 1 ||
      nq % nkv || !(G == 1 || G == 2 || G == 4 || G == 8) || B < 1 || B > 4096 || max_pos < 1 || !(eps > 0.f)) {
    set_err(g_err, "bad shape");
    return QT_E_INVALID;
  }
  if (!pos || !pos_dev || !qkv || !q_gain || !k_gain || !cos || !sin || !kc || !vc || !out) {
    set_err(g_err, "NULL argument");
    return QT_E_INVALID;
  }
  if (!(kv_split == 1 || ((kv_split == 2 || kv_split == 4 || kv_split == 8 || kv_split == 16) && split_buf &&
                          head_dim == 128 && G <= 4))) {
    set_err(g_err, "kv_split must be 1, or 2, 4, 8 or 16 with split_buf at head_dim 128 and nq / nkv <= 4");
    return QT_E_INVALID;
  }
  if (!(ntok == 1 || (ntok == 2 && kv_split == 1 && head_dim <= 128))) {
    set_err(g_err, "ntok must be 1, or 2 with kv_split 1 and head_dim <= 128");
    return QT_E_INVALID;
  }
  for (int r = 0; r < B; ++r)
    if (pos[r] < 0 || pos[r] > max_pos - ntok) { set_err(g_err, "pos[%d] out of 0..max_pos - ntok", r); return QT_E_INVALID; }
  hipStream_t s = (hipStream_t)hip_stream;
  hipError_t e = hipMemcpyAsync(pos_dev, pos, (size_t)B * sizeof(int32_t), hipMemcpyHostToDevice, s);
  AttnArgs t{};
  t.mode = ATT_WRITE_ATTEND; t.single_token = 1; t.ntok = ntok;
  if (ntok == 2) { t.tok_stride = 2; t.tok_off = 0; }   // activation rows 2 r and 2 r + 1
  t.qkv = qkv; t.ld_qkv = (long)(nq + 2 * nkv) * head_dim; t.out = out; t.ld_out = (long)nq * head_dim;
  t.q_gain = q_gain; t.k_gain = k_gain; t.eps = eps; t.scale = (float)(1.0 / std::sqrt((double)head_dim));
  t.cos = cos; t.sin = sin; t.kc = kc; t.vc = vc; t.kvdtype = kv_dtype;
  t.row_stride = (long)nkv * max_pos * head_dim; t.max_pos = max_pos;
  t.nq = nq; t.nkv = nkv; t.d = head_dim;
  t.n_runs = B; t.row_pos = pos_dev; t.pos_base = 0;
  if (kv_split > 1) { t.kv_split = kv_split; t.split_buf = split_buf; }
  if (e == hipSuccess) e = launch_attention(t, s);
  const hipError_t e2 = hipStreamSynchronize(s);   // also keeps pos alive until the copy has been made
  if (e == hipSuccess) e = e2;
  if (e != hipSuccess) { set_err(g_err, "decode attention failed: %s", hipGetErrorString(e)); return QT_E_HIP; }
  return QT_OK;
}

}  // extern "C"
