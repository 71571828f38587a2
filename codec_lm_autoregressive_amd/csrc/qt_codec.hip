// The 12 Hz codec decoder on gfx950: 16 codes per frame -> hop samples of
// audio (ncnn port discussion 6798, section 1, Codec Decoder bullet; Mizuoto
// page, codec and frame-streaming bullets). Its own context and C ABI
// (include/qt.h, qt_codec_*).
//
// Layout: activations fp32, time-major [rows][channels]. Every linear map and
// every convolution runs through the projection kernels (launch_linear:
// register GEMV .. split-activation MFMA GEMM by row count): a causal
// convolution of kernel k and dilation d is k accumulated GEMMs over the
// input shifted by (k-1-j) d rows, a causal transposed convolution of stride
// s is, per output phase p, the GEMMs of taps p, p + s, ... over the input
// shifted by 0, 1, ... rows, written with row stride s. Buffers that
// convolutions read carry zeroed rows in front of row 0, so the shifted reads
// see the causal zero padding. The small kernels here do the rest: the
// SplitRVQ gather-sums, LayerNorm, GELU, LayerScale residual adds, the
// windowed attention, the depthwise convolution, SnakeBeta and the one-channel
// output convolution with its tanh.
#include "qt.h"
#include "qt_device.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

namespace qt {
namespace {

// ---------------------------------------------------------------- kernels
// SplitRVQ sums of one frame: s0 = book_0[c_0], sa = sum_{j>=1} book_j[c_j] (j in order).
template <typename WT>
__global__ __launch_bounds__(NT) void dequant_kernel(const int* __restrict__ codes, int nq, const WT* __restrict__ books,
                                                     int C, int dim, float* __restrict__ s0, float* __restrict__ sa) {
  const int t = blockIdx.x;
  const int* c = codes + (long)t * nq;
  for (int k = threadIdx.x; k < dim; k += NT) {
    s0[(long)t * dim + k] = ld_elem<WT>(books, (long)c[0] * dim + k);
    float acc = 0.f;
    for (int j = 1; j < nq; ++j) acc += ld_elem<WT>(books, ((long)j * C + c[j]) * dim + k);
    sa[(long)t * dim + k] = acc;
  }
}

// y = (x - mean) / sqrt(var + eps) * g + b over each row of D <= 8 NT floats (in place allowed).
__global__ __launch_bounds__(NT) void layernorm_kernel(const float* x, float* y, const float* __restrict__ g,
                                                       const float* __restrict__ b, int D, float eps) {
  __shared__ float red[NT / 64];
  const float* xr = x + (long)blockIdx.x * D;
  float v[8];
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int k = threadIdx.x + q * NT;
    v[q] = k < D ? xr[k] : 0.f;
    s += v[q];
  }
  const float mean = block_sum(s, red) / (float)D;
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int k = threadIdx.x + q * NT;
    const float d = k < D ? v[q] - mean : 0.f;
    ss += d * d;
  }
  const float rstd = 1.f / sqrtf(block_sum(ss, red) / (float)D + eps);
  float* yr = y + (long)blockIdx.x * D;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int k = threadIdx.x + q * NT;
    if (k < D) yr[k] = (v[q] - mean) * rstd * g[k] + b[k];
  }
}

__global__ void gelu_kernel(float* x, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
    const float v = x[i];
    x[i] = 0.5f * v * (1.f + erff(v * 0.70710678118654752f));
  }
}

// x[r][c] += g[c] * y[r][c]
__global__ void scale_add_kernel(float* x, const float* __restrict__ y, const float* __restrict__ g, int D, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    x[i] += g[i % D] * y[i];
}

// y[t][c] = sum_j w[j][c] x[t - 6 + j][c] (x zero before row 0)
__global__ void dwconv7_kernel(const float* __restrict__ x, float* __restrict__ y, const float* __restrict__ w, long T,
                               int C) {
  const long n = T * C;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
    const long t = i / C;
    const int c = (int)(i % C);
    float acc = 0.f;
    for (int j = 0; j < 7; ++j) {
      const long tt = t - 6 + j;
      if (tt >= 0) acc += w[j * C + c] * x[tt * C + c];
    }
    y[i] = acc;
  }
}

// y = x + sin(alpha x)^2 / bden, per channel
__global__ void snake_kernel(const float* __restrict__ x, float* __restrict__ y, const float* __restrict__ alpha,
                             const float* __restrict__ bden, int C, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
    const int c = (int)(i % C);
    const float v = x[i];
    const float s = sinf(alpha[c] * v);
    y[i] = v + s * s / bden[c];
  }
}

// alpha = exp(a), bden = exp(b) + 1e-9 from the stored log-parameters
template <typename WT>
__global__ void snake_prep_kernel(const WT* __restrict__ a, const WT* __restrict__ b, float* alpha, float* bden, int C) {
  for (int c = blockIdx.x * blockDim.x + threadIdx.x; c < C; c += gridDim.x * blockDim.x) {
    alpha[c] = expf(ld_elem<WT>(a, c));
    bden[c] = expf(ld_elem<WT>(b, c)) + 1e-9f;
  }
}

// out[t - skip] = tanh(sum_j sum_c w[j][c] x[t - 6 + j][c]) for skip <= t < T;
// x has >= 6 zeroed rows before row 0. Four threads per sample, C / 4 channels each.
__global__ __launch_bounds__(NT) void out_conv_kernel(const float* __restrict__ x, const float* __restrict__ w, long T,
                                                      int C, long skip, float* __restrict__ out) {
  const long t = (long)blockIdx.x * (NT / 4) + threadIdx.x / 4;
  const int sub = threadIdx.x & 3;
  float acc = 0.f;
  if (t < T) {
    for (int j = 0; j < 7; ++j) {
      const float* xr = x + (t - 6 + j) * C;
      const float* wr = w + j * C;
      for (int c = sub; c < C; c += 4) acc = fmaf(wr[c], xr[c], acc);
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  if (t < T && t >= skip && sub == 0) out[t - skip] = tanhf(acc);
}

// The same output convolution with the SnakeBeta before it fused in: a block
// takes OC_R samples; rows t0 - 6 .. t0 + OC_R - 1 of x are read once,
// coalesced, passed through SnakeBeta (alpha, bden per channel) and staged in
// LDS with row stride C + 4; two threads per sample then contract half the
// channels of its 7 rows each. C % 8 == 0; x has >= 6 zeroed rows before row
// 0 (SnakeBeta keeps them zero).
constexpr int OC_R = 128;
__global__ __launch_bounds__(NT) void out_conv_snake_kernel(const float* __restrict__ x, const float* __restrict__ w,
                                                            const float* __restrict__ alpha,
                                                            const float* __restrict__ bden, long T, int C, long skip,
                                                            float* __restrict__ out) {
  extern __shared__ float xs[];   // [OC_R + 6][C + 4]
  const long t0 = (long)blockIdx.x * OC_R;
  const int L = C + 4, n4 = (OC_R + 6) * C / 4;
  const float* src = x + (t0 - 6) * C;
  for (int i = threadIdx.x; i < n4; i += NT) {
    const int e = 4 * i, r = e / C, c = e - r * C;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (t0 - 6 + r < T) {
      v = *(const f32x4*)(src + e);
      const f32x4 a = *(const f32x4*)(alpha + c), b = *(const f32x4*)(bden + c);
      v = (f32x4){snake_beta(v.x, a.x, b.x), snake_beta(v.y, a.y, b.y), snake_beta(v.z, a.z, b.z),
                  snake_beta(v.w, a.w, b.w)};
    }
    *(f32x4*)&xs[r * L + c] = v;
  }
  __syncthreads();
  const int sidx = threadIdx.x >> 1, half = C / 2, c0 = (threadIdx.x & 1) * half;
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    const float* xr = xs + (sidx + j) * L;
    const float* wr = w + j * C;
    for (int c = c0; c < c0 + half; c += 4) {
      const f32x4 xv = *(const f32x4*)(xr + c), wv = *(const f32x4*)(wr + c);
      acc = fmaf(wv.x, xv.x, acc);
      acc = fmaf(wv.y, xv.y, acc);
      acc = fmaf(wv.z, xv.z, acc);
      acc = fmaf(wv.w, xv.w, acc);
    }
  }
  acc += __shfl_xor(acc, 1);
  const long t = t0 + sidx;
  if (t < T && t >= skip && !(threadIdx.x & 1)) out[t - skip] = tanhf(acc);
}

// Windowed causal attention of the codec transformer: block = (16 queries, head);
// query t sees keys max(0, t - W + 1) .. t. q and k are rotated (rotate-half
// rope at positions = row index) while staged in LDS; 16 threads per query.
constexpr int CQ = 16;
__global__ __launch_bounds__(NT) void codec_attn_kernel(const float* __restrict__ qkv, int T, int H, int d,
                                                        float* __restrict__ out, const float* __restrict__ cs,
                                                        const float* __restrict__ sn, int W, float scale) {
  extern __shared__ float sm[];
  const int t0 = blockIdx.x * CQ, h = blockIdx.y, tid = threadIdx.x;
  const int k0 = max(0, t0 - W + 1), k1 = min(T - 1, t0 + CQ - 1), nk = k1 - k0 + 1;
  const int half = d / 2, ld = 3 * H * d;
  float* Qs = sm;                 // [CQ][d]
  float* Ks = Qs + CQ * d;        // [nk][d]
  float* Vs = Ks + (long)nk * d;  // [nk][d]
  float* P = Vs + (long)nk * d;   // [CQ][nk]
  for (int i = tid; i < CQ * half; i += NT) {
    const int r = i / half, e = i % half, t = t0 + r;
    float a = 0.f, b = 0.f, c = 1.f, s = 0.f;
    if (t < T) {
      a = qkv[(long)t * ld + h * d + e];
      b = qkv[(long)t * ld + h * d + e + half];
      c = cs[(long)t * half + e];
      s = sn[(long)t * half + e];
    }
    Qs[r * d + e] = a * c - b * s;
    Qs[r * d + e + half] = b * c + a * s;
  }
  for (int i = tid; i < nk * half; i += NT) {
    const int r = i / half, e = i % half, t = k0 + r;
    const float a = qkv[(long)t * ld + H * d + h * d + e], b = qkv[(long)t * ld + H * d + h * d + e + half];
    const float c = cs[(long)t * half + e], s = sn[(long)t * half + e];
    Ks[r * d + e] = a * c - b * s;
    Ks[r * d + e + half] = b * c + a * s;
  }
  for (int i = tid; i < nk * d; i += NT) {
    const int r = i / d, e = i % d;
    Vs[i] = qkv[(long)(k0 + r) * ld + 2 * H * d + h * d + e];
  }
  __syncthreads();
  const int qi = tid / 16, sub = tid % 16, t = t0 + qi;
  float mx = -INFINITY;
  for (int j = sub; j < nk; j += 16) {
    const int kp = k0 + j;
    float s = -INFINITY;
    if (t < T && kp <= t && kp > t - W) {
      float acc = 0.f;
      for (int e = 0; e < d; ++e) acc = fmaf(Qs[qi * d + e], Ks[j * d + e], acc);
      s = acc * scale;
    }
    P[qi * nk + j] = s;
    mx = fmaxf(mx, s);
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 16));
  float sum = 0.f;
  for (int j = sub; j < nk; j += 16) {
    const float p = P[qi * nk + j] == -INFINITY ? 0.f : expf(P[qi * nk + j] - mx);
    P[qi * nk + j] = p;
    sum += p;
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 16);
  __syncthreads();
  if (t < T) {
    const float rs = 1.f / sum;
    for (int e = sub; e < d; e += 16) {
      float acc = 0.f;
      for (int j = 0; j < nk; ++j) acc = fmaf(P[qi * nk + j], Vs[j * d + e], acc);
      out[(long)t * H * d + h * d + e] = acc * rs;
    }
  }
}

static unsigned grid_for(long n) { return (unsigned)std::min<long>((n + NT - 1) / NT, 16384); }

}  // namespace
}  // namespace qt

using namespace qt;

namespace {

thread_local char g_cerr[512] = "";
constexpr int kPadRows = 64;          // zeroed rows in front of padded buffers (>= 6 x the largest dilation)
constexpr long kGemmScratch = 32L << 20;   // floats of GEMM scratch (hi/lo planes of one row piece)

void cset(char* buf, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, 512, fmt, ap);
  va_end(ap);
}

struct CPlan {
  size_t off = 0;
  bool ovf = false;
  size_t take(size_t bytes) {
    const size_t o = off;
    const size_t b = (bytes + 255) & ~(size_t)255;
    if (__builtin_add_overflow(off, b, &off)) ovf = true;
    return o;
  }
  size_t mul(std::initializer_list<size_t> xs) {
    size_t r = 1;
    for (size_t x : xs)
      if (__builtin_mul_overflow(r, x, &r)) ovf = true;
    return r;
  }
};

bool codec_cfg_ok(const qt_codec_config* c, char* err) {
  if (!c) { cset(err, "codec config is NULL"); return false; }
  auto bad = [&](const char* m) { cset(err, "%s", m); return false; };
  if (c->n_q < 2 || c->n_q > 64) return bad("n_q must be in 2..64");
  if (c->codebook < 1 || c->codebook > (1 << 20)) return bad("codebook must be in 1..2^20");
  if (c->codebook_dim < 8 || c->codebook_dim % 8 || c->codebook_dim > 8192) return bad("codebook_dim must be a multiple of 8 in 8..8192");
  if (c->hidden < 64 || c->hidden % 64 || c->hidden > 2048) return bad("hidden must be a multiple of 64 in 64..2048");
  if (c->layers < 0 || c->layers > 64) return bad("layers must be in 0..64");
  if (c->heads < 1 || c->head_dim < 2 || c->head_dim % 2 || c->head_dim > 128 || (c->heads * c->head_dim) % 8)
    return bad("heads >= 1 and an even head_dim <= 128 with heads * head_dim a multiple of 8");
  if (c->ffn < 8 || c->ffn % 8 || c->up_ffn < 8 || c->up_ffn % 8) return bad("ffn and up_ffn must be multiples of 8");
  if (c->window < 1) return bad("window must be >= 1");
  if (!(c->rope_theta > 0.f)) return bad("rope_theta must be positive");
  if (c->n_blocks < 1 || c->n_blocks > QT_CODEC_MAX_BLOCKS) return bad("n_blocks must be in 1..QT_CODEC_MAX_BLOCKS");
  for (int b = 0; b <= c->n_blocks; ++b)
    if (c->channels[b] < 8 || c->channels[b] % 8 || c->channels[b] > 8192) return bad("channels must be multiples of 8 in 8..8192");
  for (int b = 0; b < c->n_blocks; ++b)
    if (c->strides[b] < 1 || c->strides[b] > 64) return bad("strides must be in 1..64");
  for (int u = 0; u < QT_CODEC_UNITS; ++u)
    if (c->dilations[u] < 1 || 6 * c->dilations[u] > kPadRows) return bad("dilations must be in 1..10");
  if (c->chunk < 1 || c->context < 0 || c->chunk + c->context > 65536) return bad("chunk >= 1, context >= 0, chunk + context <= 65536");
  if (c->weight_dtype != QT_DTYPE_F32 && c->weight_dtype != QT_DTYPE_BF16) return bad("weight_dtype must be F32 or BF16");
  return true;
}

struct CLayout {
  // packed weights
  size_t books, proj_sem, proj_ac;
  struct L { size_t ln1_g, ln1_b, wqkv, wo, ls1, ln2_g, ln2_b, fc1, fc2, ls2; };
  std::vector<L> layers;
  size_t ln_f_g, ln_f_b;
  struct U { size_t up, dw, ln_g, ln_b, fc1, fc2, gamma; } up[2];
  size_t voc_in;
  struct Un { size_t alpha1, bden1, conv7, alpha2, bden2, conv1; };
  struct B { size_t alpha, bden, up; Un units[QT_CODEC_UNITS]; } blocks[QT_CODEC_MAX_BLOCKS];
  size_t out_alpha, out_bden, voc_out;
  // buffers
  size_t codes, s0, sa, bx, ba, bt, bm, q, r, s, scratch, cs, sn;
  size_t bxd_elems, vocp_elems;   // elements of the padded buffers after their pad
  long hop, F;
  size_t total;
  bool ovf;
};

CLayout plan_codec(const qt_codec_config& c) {
  CLayout L;
  CPlan p;
  const size_t es = c.weight_dtype == QT_DTYPE_BF16 ? 2 : 4;
  const size_t D = c.hidden, Hd = (size_t)c.heads * c.head_dim, F = (size_t)c.chunk + c.context;
  L.F = (long)F;
  L.books = p.take(p.mul({(size_t)c.n_q, (size_t)c.codebook, (size_t)c.codebook_dim, es}));
  L.proj_sem = p.take(p.mul({D, (size_t)c.codebook_dim, es}));
  L.proj_ac = p.take(p.mul({D, (size_t)c.codebook_dim, es}));
  for (int i = 0; i < c.layers; ++i) {
    CLayout::L l;
    l.ln1_g = p.take(D * 4); l.ln1_b = p.take(D * 4);
    l.wqkv = p.take(p.mul({3 * Hd, D, es})); l.wo = p.take(p.mul({D, Hd, es})); l.ls1 = p.take(D * 4);
    l.ln2_g = p.take(D * 4); l.ln2_b = p.take(D * 4);
    l.fc1 = p.take(p.mul({(size_t)c.ffn, D, es})); l.fc2 = p.take(p.mul({D, (size_t)c.ffn, es})); l.ls2 = p.take(D * 4);
    L.layers.push_back(l);
  }
  L.ln_f_g = p.take(D * 4); L.ln_f_b = p.take(D * 4);
  for (int u = 0; u < 2; ++u) {
    L.up[u].up = p.take(p.mul({2, D, D, es})); L.up[u].dw = p.take(7 * D * 4);
    L.up[u].ln_g = p.take(D * 4); L.up[u].ln_b = p.take(D * 4);
    L.up[u].fc1 = p.take(p.mul({(size_t)c.up_ffn, D, es})); L.up[u].fc2 = p.take(p.mul({D, (size_t)c.up_ffn, es}));
    L.up[u].gamma = p.take(D * 4);
  }
  const size_t* ch = nullptr;
  (void)ch;
  L.voc_in = p.take(p.mul({7, (size_t)c.channels[0], D, es}));
  size_t rows = 4 * F, vmax = rows * c.channels[0];
  for (int b = 0; b < c.n_blocks; ++b) {
    const size_t ci = c.channels[b], co = c.channels[b + 1];
    L.blocks[b].alpha = p.take(ci * 4); L.blocks[b].bden = p.take(ci * 4);
    L.blocks[b].up = p.take(p.mul({2 * (size_t)c.strides[b], co, ci, es}));
    for (int u = 0; u < QT_CODEC_UNITS; ++u) {
      CLayout::Un& un = L.blocks[b].units[u];
      un.alpha1 = p.take(co * 4); un.bden1 = p.take(co * 4); un.conv7 = p.take(p.mul({7, co, co, es}));
      un.alpha2 = p.take(co * 4); un.bden2 = p.take(co * 4); un.conv1 = p.take(p.mul({co, co, es}));
    }
    rows = p.mul({rows, (size_t)c.strides[b]});
    vmax = std::max(vmax, p.mul({rows, co}));
  }
  const size_t cl = c.channels[c.n_blocks];
  L.out_alpha = p.take(cl * 4); L.out_bden = p.take(cl * 4); L.voc_out = p.take(7 * cl * 4);
  L.hop = (long)(rows / F);
  // buffers
  size_t cmax = D;
  for (int b = 0; b <= c.n_blocks; ++b) cmax = std::max(cmax, (size_t)c.channels[b]);
  L.codes = p.take(p.mul({F, (size_t)c.n_q, 4}));
  L.s0 = p.take(p.mul({F, (size_t)c.codebook_dim, 4}));
  L.sa = p.take(p.mul({F, (size_t)c.codebook_dim, 4}));
  L.bxd_elems = p.mul({4 * F, D});
  const size_t pad = (size_t)kPadRows * cmax;
  L.bx = p.take((pad + L.bxd_elems) * 4);
  L.ba = p.take((pad + L.bxd_elems) * 4);
  L.bt = p.take(p.mul({4 * F, D, 4}));
  L.bm = p.take(p.mul({4 * F, std::max({(size_t)c.ffn, (size_t)c.up_ffn, 3 * Hd}), 4}));
  L.vocp_elems = vmax;
  L.q = p.take((pad + vmax) * 4);
  L.r = p.take((pad + vmax) * 4);
  L.s = p.take((pad + vmax) * 4);
  L.scratch = p.take((size_t)kGemmScratch * 4);
  L.cs = p.take(p.mul({F, (size_t)c.head_dim / 2, 4}));
  L.sn = p.take(p.mul({F, (size_t)c.head_dim / 2, 4}));
  L.total = p.off;
  L.ovf = p.ovf;
  return L;
}

}  // namespace

struct qt_codec {
  qt_codec_config cfg;
  CLayout lay;
  hipStream_t stream = nullptr;
  char* ws = nullptr;
  bool own_ws = false;
  char err[512] = "";
  long hop = 0;
  size_t pad_elems = 0;
  template <typename T> T* at(size_t off) const { return (T*)(ws + off); }
};

namespace {

#define CHK(call)                                                                 \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) {                                                       \
      cset(c->err, "%s failed: %s", #call, hipGetErrorString(e_));                \
      return QT_E_HIP;                                                            \
    }                                                                             \
  } while (0)

// Y (op)= W X over M rows, in row pieces whose hi/lo planes fit the scratch.
hipError_t gemm(qt_codec* c, const void* W, int N, int K, const float* X, long ldx, long M, float* Y, long ldy, int epi) {
  float* sc = c->at<float>(c->lay.scratch);
  // a piece of m rows takes m (rounded up to 64) row denominators and m K hi/lo floats
  const long piece = std::max<long>(128, (kGemmScratch - 64) / (K + 1) / 64 * 64);
  for (long m0 = 0; m0 < M; m0 += piece) {
    const long m = std::min(piece, M - m0);
    LinearArgs a{};
    a.W = W; a.wdtype = c->cfg.weight_dtype; a.N = N; a.K = K;
    a.X = X + m0 * ldx; a.ldx = ldx; a.M = (int)m; a.gain = nullptr; a.eps = 1e-6f;
    a.Y = Y + m0 * ldy; a.ldy = ldy; a.epi = epi;
    const long den = (m + 63) / 64 * 64;
    a.row_den = sc; a.part = sc + den; a.part_floats = kGemmScratch - den;
    a.xs = a.part; a.xs_floats = a.part_floats;
    const hipError_t e = launch_linear(a, c->stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

size_t wbytes(const qt_codec* c, size_t n) { return n * (c->cfg.weight_dtype == QT_DTYPE_BF16 ? 2 : 4); }

// A convolution over Cin channels with bf16 weights and Cin % 32 == 0 runs as
// one GEMM of K = taps x Cin whose activation loader reads the shifted rows
// itself (implicit im2col); its weights are stored [Cout][tap][Cin], oldest
// input row first. Otherwise the weights stay tap-major and each tap is its own
// accumulated GEMM.
bool conv_packed(const qt_codec* c, int Cin) { return c->cfg.weight_dtype == QT_DTYPE_BF16 && Cin % 32 == 0; }

// The vocoder runs fused (SnakeBeta in convolution epilogues, the fused output
// convolution) when every convolution in it is packed and the output
// convolution's staged tile fits 64 KiB of LDS.
bool vocoder_fused(const qt_codec* c) {
  const qt_codec_config& g = c->cfg;
  if (!conv_packed(c, g.hidden)) return false;
  for (int b = 0; b <= g.n_blocks; ++b)
    if (!conv_packed(c, g.channels[b])) return false;
  const int cl = g.channels[g.n_blocks];
  return cl % 8 == 0 && (size_t)(OC_R + 6) * (cl + 4) * 4 <= 65536;
}

// Optional SnakeBeta epilogue (per output channel alpha / bden): into Y2 when
// given, else applied to Y itself.
struct Snk { const float* alpha = nullptr; const float* bden = nullptr; float* Y2 = nullptr; long ldy2 = 0; };

hipError_t conv_gemm(qt_codec* c, const void* W, int taps, int d, int Cin, int Cout, const float* X, long T, float* Y,
                     long ldy, int epi = EPI_STORE, Snk sk = {}) {
  LinearArgs a{};
  a.W = W; a.wdtype = DT_BF16; a.N = Cout; a.K = taps * Cin;
  a.X = X; a.ldx = Cin; a.M = (int)T; a.eps = 1e-6f;
  a.Y = Y; a.ldy = ldy; a.epi = epi;
  a.conv_taps = taps; a.conv_cin = Cin; a.conv_dil = d;
  a.snake_alpha = sk.alpha; a.snake_bden = sk.bden; a.Y2 = sk.Y2; a.ldy2 = sk.ldy2;
  return launch_linear(a, c->stream);
}

// causal convolution, kernel k, dilation d: W [Cout][k][Cin] (packed) or
// tap-major [k][Cout][Cin]; X padded
hipError_t conv(qt_codec* c, const void* W, int k, int d, int Cin, int Cout, const float* X, long T, float* Y, int epi0) {
  if (conv_packed(c, Cin)) return conv_gemm(c, W, k, d, Cin, Cout, X, T, Y, Cout, epi0);
  for (int j = 0; j < k; ++j) {
    const long sh = (long)(k - 1 - j) * d;
    const hipError_t e = gemm(c, (const char*)W + wbytes(c, (size_t)j * Cout * Cin), Cout, Cin, X - sh * Cin, Cin, T,
                              Y, Cout, j == 0 ? epi0 : EPI_RESIDUAL);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// causal transposed convolution, K taps, stride s: Y[m s + p] = sum_i W_(p + i s) X[m - i];
// packed (K / s > 1): phase p's weights [Cout][K / s][Cin] at p Cout K Cin,
// tap p + (K / s - 1 - j) s in slot j
hipError_t convT(qt_codec* c, const void* W, int K, int s, int Cin, int Cout, const float* X, long T, float* Y) {
  if (conv_packed(c, Cin) && K / s > 1) {
    for (int p = 0; p < s; ++p) {
      const hipError_t e = conv_gemm(c, (const char*)W + wbytes(c, (size_t)p * Cout * (K / s) * Cin), K / s, 1, Cin,
                                     Cout, X, T, Y + (long)p * Cout, (long)s * Cout);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  for (int p = 0; p < s; ++p)
    for (int i = 0; i * s + p < K; ++i) {
      const hipError_t e = gemm(c, (const char*)W + wbytes(c, (size_t)(p + i * s) * Cout * Cin), Cout, Cin,
                                X - (long)i * Cin, Cin, T, Y + (long)p * Cout, (long)s * Cout,
                                i == 0 ? EPI_STORE : EPI_RESIDUAL);
      if (e != hipSuccess) return e;
    }
  return hipSuccess;
}

hipError_t ln(qt_codec* c, const float* x, float* y, size_t g, size_t b, long rows) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(layernorm_kernel, dim3((unsigned)rows), dim3(NT), 0, c->stream, x, y, c->at<float>(g),
                     c->at<float>(b), c->cfg.hidden, 1e-5f);
  return hipGetLastError();
}

hipError_t gelu(qt_codec* c, float* x, long n) {
  hipLaunchKernelGGL(gelu_kernel, dim3(grid_for(n)), dim3(NT), 0, c->stream, x, n);
  return hipGetLastError();
}

hipError_t scale_add(qt_codec* c, float* x, const float* y, size_t g, long rows, int D) {
  const long n = rows * D;
  hipLaunchKernelGGL(scale_add_kernel, dim3(grid_for(n)), dim3(NT), 0, c->stream, x, y, c->at<float>(g), D, n);
  return hipGetLastError();
}

hipError_t snake(qt_codec* c, const float* x, float* y, size_t alpha, size_t bden, int C, long rows) {
  const long n = rows * C;
  hipLaunchKernelGGL(snake_kernel, dim3(grid_for(n)), dim3(NT), 0, c->stream, x, y, c->at<float>(alpha),
                     c->at<float>(bden), C, n);
  return hipGetLastError();
}

// ConvNeXt block in place on x [rows, D]: y, t, m are work buffers
hipError_t convnext(qt_codec* c, const CLayout::U& u, float* x, float* y, float* t, float* m, long rows) {
  const int D = c->cfg.hidden;
  hipLaunchKernelGGL(dwconv7_kernel, dim3(grid_for(rows * D)), dim3(NT), 0, c->stream, x, y, c->at<float>(u.dw), rows,
                     D);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = ln(c, y, y, u.ln_g, u.ln_b, rows);
  if (e == hipSuccess) e = gemm(c, c->ws + u.fc1, c->cfg.up_ffn, D, y, D, rows, m, c->cfg.up_ffn, EPI_STORE);
  if (e == hipSuccess) e = gelu(c, m, rows * c->cfg.up_ffn);
  if (e == hipSuccess) e = gemm(c, c->ws + u.fc2, D, c->cfg.up_ffn, m, c->cfg.up_ffn, rows, t, D, EPI_STORE);
  if (e == hipSuccess) e = scale_add(c, x, t, u.gamma, rows, D);
  return e;
}

// One causal pass over the T frames already in the device code buffer;
// samples skip .. T hop - 1 go to out[0 ..].
qt_status decode_frames(qt_codec* c, long T, long skip, float* out) {
  const qt_codec_config& g = c->cfg;
  const CLayout& L = c->lay;
  const int D = g.hidden, Hd = g.heads * g.head_dim, dim = g.codebook_dim;
  const hipStream_t s = c->stream;
  float* s0 = c->at<float>(L.s0);
  float* sa = c->at<float>(L.sa);
  float* bx = c->at<float>(L.bx) + c->pad_elems;
  float* ba = c->at<float>(L.ba) + c->pad_elems;
  float* bt = c->at<float>(L.bt);
  float* bm = c->at<float>(L.bm);
  if (g.weight_dtype == QT_DTYPE_BF16)
    hipLaunchKernelGGL(dequant_kernel<uint16_t>, dim3((unsigned)T), dim3(NT), 0, s, c->at<int>(L.codes), g.n_q,
                       c->at<uint16_t>(L.books), g.codebook, dim, s0, sa);
  else
    hipLaunchKernelGGL(dequant_kernel<float>, dim3((unsigned)T), dim3(NT), 0, s, c->at<int>(L.codes), g.n_q,
                       c->at<float>(L.books), g.codebook, dim, s0, sa);
  CHK(hipGetLastError());
  CHK(gemm(c, c->ws + L.proj_sem, D, dim, s0, dim, T, bx, D, EPI_STORE));
  CHK(gemm(c, c->ws + L.proj_ac, D, dim, sa, dim, T, bx, D, EPI_RESIDUAL));
  // transformer
  const size_t lds = (size_t)(CQ * g.head_dim + 2 * (g.window + CQ) * g.head_dim + CQ * (g.window + CQ)) * 4;
  for (const CLayout::L& l : L.layers) {
    CHK(ln(c, bx, ba, l.ln1_g, l.ln1_b, T));
    CHK(gemm(c, c->ws + l.wqkv, 3 * Hd, D, ba, D, T, bm, 3 * Hd, EPI_STORE));
    hipLaunchKernelGGL(codec_attn_kernel, dim3((unsigned)((T + CQ - 1) / CQ), g.heads), dim3(NT), lds, s, bm, (int)T,
                       g.heads, g.head_dim, bt, c->at<float>(L.cs), c->at<float>(L.sn), g.window,
                       (float)(1.0 / std::sqrt((double)g.head_dim)));
    CHK(hipGetLastError());
    CHK(gemm(c, c->ws + l.wo, D, Hd, bt, Hd, T, ba, D, EPI_STORE));
    CHK(scale_add(c, bx, ba, l.ls1, T, D));
    CHK(ln(c, bx, ba, l.ln2_g, l.ln2_b, T));
    CHK(gemm(c, c->ws + l.fc1, g.ffn, D, ba, D, T, bm, g.ffn, EPI_STORE));
    CHK(gelu(c, bm, T * g.ffn));
    CHK(gemm(c, c->ws + l.fc2, D, g.ffn, bm, g.ffn, T, ba, D, EPI_STORE));
    CHK(scale_add(c, bx, ba, l.ls2, T, D));
  }
  CHK(ln(c, bx, ba, L.ln_f_g, L.ln_f_b, T));
  // two upsampling stages: transformer output in ba -> bx (2T) -> ba (4T)
  CHK(convT(c, c->ws + L.up[0].up, 2, 2, D, D, ba, T, bx));
  CHK(convnext(c, L.up[0], bx, ba, bt, bm, 2 * T));
  CHK(convT(c, c->ws + L.up[1].up, 2, 2, D, D, bx, 2 * T, ba));
  CHK(convnext(c, L.up[1], ba, bx, bt, bm, 4 * T));
  // vocoder
  float* q = c->at<float>(L.q) + c->pad_elems;
  float* r = c->at<float>(L.r) + c->pad_elems;
  float* sbuf = c->at<float>(L.s) + c->pad_elems;
  long rows = 4 * T;
  const int cl = g.channels[g.n_blocks];
  if (vocoder_fused(c)) {
    // every SnakeBeta rides on the epilogue of the convolution before it, the
    // last one on the output convolution; each convolution reads the SnakeBeta
    // output in cur and writes the next one to the other of r, sbuf
    auto snk = [&](size_t alpha, size_t bden, float* y2, long ld) {
      Snk k; k.alpha = c->at<float>(alpha); k.bden = c->at<float>(bden); k.Y2 = y2; k.ldy2 = ld; return k;
    };
    float* cur = r;
    float* oth = sbuf;
    CHK(conv_gemm(c, c->ws + L.voc_in, 7, 1, D, g.channels[0], ba, rows, q, g.channels[0], EPI_STORE,
                  snk(L.blocks[0].alpha, L.blocks[0].bden, cur, g.channels[0])));
    for (int b = 0; b < g.n_blocks; ++b) {
      const int ci = g.channels[b], co = g.channels[b + 1], st = g.strides[b];
      const CLayout::B& B = L.blocks[b];
      for (int ph = 0; ph < st; ++ph)
        CHK(conv_gemm(c, c->ws + B.up + wbytes(c, (size_t)ph * co * 2 * ci), 2, 1, ci, co, cur, rows,
                      q + (long)ph * co, (long)st * co, EPI_STORE,
                      snk(B.units[0].alpha1, B.units[0].bden1, oth + (long)ph * co, (long)st * co)));
      std::swap(cur, oth);
      rows *= st;
      for (int u = 0; u < QT_CODEC_UNITS; ++u) {
        const CLayout::Un& un = B.units[u];
        CHK(conv_gemm(c, c->ws + un.conv7, 7, g.dilations[u], co, co, cur, rows, oth, co, EPI_STORE,
                      snk(un.alpha2, un.bden2, nullptr, 0)));
        std::swap(cur, oth);
        Snk next;
        if (u + 1 < QT_CODEC_UNITS) next = snk(B.units[u + 1].alpha1, B.units[u + 1].bden1, oth, co);
        else if (b + 1 < g.n_blocks) next = snk(L.blocks[b + 1].alpha, L.blocks[b + 1].bden, oth, co);
        CHK(conv_gemm(c, c->ws + un.conv1, 1, 1, co, co, cur, rows, q, co, EPI_RESIDUAL, next));
        std::swap(cur, oth);
      }
    }
    hipLaunchKernelGGL(out_conv_snake_kernel, dim3((unsigned)((rows + OC_R - 1) / OC_R)), dim3(NT),
                       (size_t)(OC_R + 6) * (cl + 4) * 4, s, q, c->at<float>(L.voc_out), c->at<float>(L.out_alpha),
                       c->at<float>(L.out_bden), rows, cl, skip, out);
    CHK(hipGetLastError());
    return QT_OK;
  }
  CHK(conv(c, c->ws + L.voc_in, 7, 1, D, g.channels[0], ba, rows, q, EPI_STORE));
  for (int b = 0; b < g.n_blocks; ++b) {
    const int ci = g.channels[b], co = g.channels[b + 1], st = g.strides[b];
    const CLayout::B& B = L.blocks[b];
    CHK(snake(c, q, r, B.alpha, B.bden, ci, rows));
    CHK(convT(c, c->ws + B.up, 2 * st, st, ci, co, r, rows, q));
    rows *= st;
    for (int u = 0; u < QT_CODEC_UNITS; ++u) {
      const CLayout::Un& un = B.units[u];
      CHK(snake(c, q, r, un.alpha1, un.bden1, co, rows));
      CHK(conv(c, c->ws + un.conv7, 7, g.dilations[u], co, co, r, rows, sbuf, EPI_STORE));
      CHK(snake(c, sbuf, r, un.alpha2, un.bden2, co, rows));
      CHK(gemm(c, c->ws + un.conv1, co, co, r, co, rows, q, co, EPI_RESIDUAL));
    }
  }
  CHK(snake(c, q, r, L.out_alpha, L.out_bden, cl, rows));
  hipLaunchKernelGGL(out_conv_kernel, dim3((unsigned)((rows + NT / 4 - 1) / (NT / 4))), dim3(NT), 0, s, r,
                     c->at<float>(L.voc_out), rows, cl, skip, out);
  CHK(hipGetLastError());
  return QT_OK;
}

qt_status check_codes(qt_codec* c, const int32_t* codes, long T) {
  for (long i = 0; i < T * c->cfg.n_q; ++i)
    if (codes[i] < 0 || codes[i] >= c->cfg.codebook) {
      cset(c->err, "codes[%ld][%ld]=%d outside 0..%d", i / c->cfg.n_q, i % c->cfg.n_q, codes[i], c->cfg.codebook - 1);
      return QT_E_RANGE;
    }
  return QT_OK;
}

// frames [f0, f1) of the host codes into the device code buffer, then one
// pass; samples from frame `from` on go to out
qt_status decode_span(qt_codec* c, const int32_t* codes, long f0, long f1, long from, float* out) {
  const long n = f1 - f0;
  CHK(hipMemcpyAsync(c->at<int>(c->lay.codes), codes + f0 * c->cfg.n_q, (size_t)n * c->cfg.n_q * 4,
                     hipMemcpyHostToDevice, c->stream));
  CHK(hipStreamSynchronize(c->stream));   // the pageable host codes are consumed
  return decode_frames(c, n, (from - f0) * c->hop, out);
}

}  // namespace

extern "C" {

qt_status qt_codec_workspace_bytes(const qt_codec_config* cfg, size_t* bytes) {
  if (!codec_cfg_ok(cfg, g_cerr)) return QT_E_INVALID;
  if (!bytes) { cset(g_cerr, "bytes is NULL"); return QT_E_INVALID; }
  CLayout L = plan_codec(*cfg);
  if (L.ovf) { cset(g_cerr, "codec workspace size overflows size_t"); return QT_E_CAPACITY; }
  *bytes = L.total;
  return QT_OK;
}

const char* qt_codec_last_error(const qt_codec* c) { return c ? c->err : g_cerr; }

void qt_codec_destroy(qt_codec* c) {
  if (!c) return;
  if (c->stream) (void)hipStreamSynchronize(c->stream);
  if (c->own_ws && c->ws) (void)hipFree(c->ws);
  delete c;
}

qt_status qt_codec_create(const qt_codec_config* cfg, const qt_codec_weights* w, void* workspace, size_t ws_bytes,
                          void* hip_stream, qt_codec** out) {
  if (!codec_cfg_ok(cfg, g_cerr)) return QT_E_INVALID;
  if (!out) { cset(g_cerr, "out is NULL"); return QT_E_INVALID; }
  *out = nullptr;
  if (!w || !w->codebooks || !w->proj_sem || !w->proj_ac || !w->ln_f_g || !w->ln_f_b || !w->voc_in || !w->voc_out ||
      !w->voc_out_a || !w->voc_out_b || (cfg->layers > 0 && !w->layers)) {
    cset(g_cerr, "a codec weight pointer is NULL");
    return QT_E_INVALID;
  }
  for (int i = 0; i < cfg->layers; ++i) {
    const qt_codec_layer_weights& l = w->layers[i];
    if (!l.ln1_g || !l.ln1_b || !l.wqkv || !l.wo || !l.ls1 || !l.ln2_g || !l.ln2_b || !l.fc1 || !l.fc2 || !l.ls2) {
      cset(g_cerr, "codec layer %d: a weight pointer is NULL", i);
      return QT_E_INVALID;
    }
  }
  for (int u = 0; u < 2; ++u) {
    const qt_codec_up_weights& x = w->up[u];
    if (!x.up || !x.dw || !x.ln_g || !x.ln_b || !x.fc1 || !x.fc2 || !x.gamma) { cset(g_cerr, "codec upsampling stage %d: a weight pointer is NULL", u); return QT_E_INVALID; }
  }
  for (int b = 0; b < cfg->n_blocks; ++b) {
    const qt_codec_block_weights& x = w->blocks[b];
    if (!x.snake_a || !x.snake_b || !x.up) { cset(g_cerr, "codec block %d: a weight pointer is NULL", b); return QT_E_INVALID; }
    for (int u = 0; u < QT_CODEC_UNITS; ++u) {
      const qt_codec_unit_weights& y = x.units[u];
      if (!y.a1 || !y.b1 || !y.conv7 || !y.a2 || !y.b2 || !y.conv1) { cset(g_cerr, "codec block %d unit %d: a weight pointer is NULL", b, u); return QT_E_INVALID; }
    }
  }
  CLayout L = plan_codec(*cfg);
  if (L.ovf) { cset(g_cerr, "codec workspace size overflows size_t"); return QT_E_CAPACITY; }
  if (workspace && ws_bytes < L.total) { cset(g_cerr, "codec workspace too small: %zu < %zu bytes", ws_bytes, L.total); return QT_E_NOMEM; }
  qt_codec* c = new (std::nothrow) qt_codec();
  if (!c) { cset(g_cerr, "out of host memory"); return QT_E_NOMEM; }
  c->cfg = *cfg;
  c->lay = L;
  c->stream = (hipStream_t)hip_stream;
  c->hop = L.hop;
  size_t cmax = cfg->hidden;
  for (int b = 0; b <= cfg->n_blocks; ++b) cmax = std::max(cmax, (size_t)cfg->channels[b]);
  c->pad_elems = (size_t)kPadRows * cmax;
  auto fail = [&](qt_status st) {
    snprintf(g_cerr, sizeof g_cerr, "%s", c->err);
    qt_codec_destroy(c);
    return st;
  };
  if (workspace) {
    c->ws = (char*)workspace;
  } else {
    if (hipMalloc((void**)&c->ws, L.total) != hipSuccess) { cset(c->err, "hipMalloc of %zu bytes failed", L.total); c->ws = nullptr; return fail(QT_E_NOMEM); }
    c->own_ws = true;
  }
  const int wd = cfg->weight_dtype;
  const hipStream_t s = c->stream;
  const long D = cfg->hidden, Hd = (long)cfg->heads * cfg->head_dim;
  bool ok = true;
  auto cp = [&](const void* src, size_t dst, long rows, long n, int ddt) {
    if (ok) ok = launch_convert(src, wd, n, c->ws + dst, ddt, n, rows, (int)n, s) == hipSuccess;
  };
  cp(w->codebooks, L.books, (long)cfg->n_q * cfg->codebook, cfg->codebook_dim, wd);
  cp(w->proj_sem, L.proj_sem, D, cfg->codebook_dim, wd);
  cp(w->proj_ac, L.proj_ac, D, cfg->codebook_dim, wd);
  for (int i = 0; i < cfg->layers; ++i) {
    const qt_codec_layer_weights& l = w->layers[i];
    const CLayout::L& o = L.layers[i];
    cp(l.ln1_g, o.ln1_g, 1, D, DT_F32); cp(l.ln1_b, o.ln1_b, 1, D, DT_F32);
    cp(l.wqkv, o.wqkv, 3 * Hd, D, wd); cp(l.wo, o.wo, D, Hd, wd); cp(l.ls1, o.ls1, 1, D, DT_F32);
    cp(l.ln2_g, o.ln2_g, 1, D, DT_F32); cp(l.ln2_b, o.ln2_b, 1, D, DT_F32);
    cp(l.fc1, o.fc1, cfg->ffn, D, wd); cp(l.fc2, o.fc2, D, cfg->ffn, wd); cp(l.ls2, o.ls2, 1, D, DT_F32);
  }
  cp(w->ln_f_g, L.ln_f_g, 1, D, DT_F32); cp(w->ln_f_b, L.ln_f_b, 1, D, DT_F32);
  for (int u = 0; u < 2; ++u) {
    const qt_codec_up_weights& x = w->up[u];
    cp(x.up, L.up[u].up, 2 * D, D, wd); cp(x.dw, L.up[u].dw, 7, D, DT_F32);
    cp(x.ln_g, L.up[u].ln_g, 1, D, DT_F32); cp(x.ln_b, L.up[u].ln_b, 1, D, DT_F32);
    cp(x.fc1, L.up[u].fc1, cfg->up_ffn, D, wd); cp(x.fc2, L.up[u].fc2, D, cfg->up_ffn, wd);
    cp(x.gamma, L.up[u].gamma, 1, D, DT_F32);
  }
  // tap-major [k][Cout][Cin] source; packed: slot j of output row n at (n k + j) Cin
  auto cp_conv = [&](const void* src, size_t dst, int k, int Cout, int Cin) {
    if (!conv_packed(c, Cin)) { cp(src, dst, (long)k * Cout, Cin, wd); return; }
    for (int j = 0; j < k && ok; ++j)
      ok = launch_convert((const char*)src + (size_t)j * Cout * Cin * (wd == QT_DTYPE_BF16 ? 2 : 4), wd, Cin,
                          c->ws + dst + (size_t)j * Cin * 2, wd, (long)k * Cin, Cout, Cin, s) == hipSuccess;
  };
  // transposed, K = kt taps of stride st: phase p's taps p + i st, slot kt / st - 1 - i
  auto cp_convT = [&](const void* src, size_t dst, int kt, int st, int Cout, int Cin) {
    if (!conv_packed(c, Cin) || kt / st <= 1) { cp(src, dst, (long)kt * Cout, Cin, wd); return; }
    const int n = kt / st;
    for (int p = 0; p < st; ++p)
      for (int i = 0; i < n && ok; ++i)
        ok = launch_convert((const char*)src + (size_t)(p + i * st) * Cout * Cin * 2, wd, Cin,
                            c->ws + dst + ((size_t)p * Cout * n + (n - 1 - i)) * Cin * 2, wd, (long)n * Cin, Cout, Cin,
                            s) == hipSuccess;
  };
  cp_conv(w->voc_in, L.voc_in, 7, cfg->channels[0], D);
  auto prep = [&](const void* a, const void* b, size_t alpha, size_t bden, int C) {
    if (!ok) return;
    if (wd == QT_DTYPE_BF16)
      hipLaunchKernelGGL(snake_prep_kernel<uint16_t>, dim3(1), dim3(NT), 0, s, (const uint16_t*)a, (const uint16_t*)b,
                         c->at<float>(alpha), c->at<float>(bden), C);
    else
      hipLaunchKernelGGL(snake_prep_kernel<float>, dim3(1), dim3(NT), 0, s, (const float*)a, (const float*)b,
                         c->at<float>(alpha), c->at<float>(bden), C);
    ok = hipGetLastError() == hipSuccess;
  };
  for (int b = 0; b < cfg->n_blocks; ++b) {
    const qt_codec_block_weights& x = w->blocks[b];
    const int ci = cfg->channels[b], co = cfg->channels[b + 1];
    prep(x.snake_a, x.snake_b, L.blocks[b].alpha, L.blocks[b].bden, ci);
    cp_convT(x.up, L.blocks[b].up, 2 * cfg->strides[b], cfg->strides[b], co, ci);
    for (int u = 0; u < QT_CODEC_UNITS; ++u) {
      const qt_codec_unit_weights& y = x.units[u];
      const CLayout::Un& un = L.blocks[b].units[u];
      prep(y.a1, y.b1, un.alpha1, un.bden1, co);
      cp_conv(y.conv7, un.conv7, 7, co, co);
      prep(y.a2, y.b2, un.alpha2, un.bden2, co);
      cp(y.conv1, un.conv1, co, co, wd);
    }
  }
  const int cl = cfg->channels[cfg->n_blocks];
  prep(w->voc_out_a, w->voc_out_b, L.out_alpha, L.out_bden, cl);
  cp(w->voc_out, L.voc_out, 7, cl, DT_F32);
  // zeroed pad rows in front of the padded buffers
  for (size_t off : {L.bx, L.ba, L.q, L.r, L.s})
    if (ok) ok = launch_fill_i32((int*)(c->ws + off), 0, (long)c->pad_elems, s) == hipSuccess;
  if (!ok) { cset(c->err, "codec weight repack launch failed"); return fail(QT_E_HIP); }
  // rope tables of the transformer (positions 0 .. chunk + context - 1)
  const int half = cfg->head_dim / 2;
  std::vector<float> inv(half), cs((size_t)L.F * half), sn((size_t)L.F * half);
  for (int i = 0; i < half; ++i) inv[i] = (float)std::pow((double)cfg->rope_theta, -(2.0 * i) / cfg->head_dim);
  for (long p = 0; p < L.F; ++p)
    for (int i = 0; i < half; ++i) {
      const float ang = (float)p * inv[i];
      cs[(size_t)p * half + i] = (float)std::cos((double)ang);
      sn[(size_t)p * half + i] = (float)std::sin((double)ang);
    }
  if (hipMemcpyAsync(c->ws + L.cs, cs.data(), cs.size() * 4, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipMemcpyAsync(c->ws + L.sn, sn.data(), sn.size() * 4, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess) {
    cset(c->err, "codec rope table upload failed");
    return fail(QT_E_HIP);
  }
  const size_t lds = (size_t)(CQ * cfg->head_dim + 2 * (cfg->window + CQ) * cfg->head_dim + CQ * (cfg->window + CQ)) * 4;
  static size_t have = 0;
  if (ensure_lds((const void*)codec_attn_kernel, lds, &have) != hipSuccess || lds > 160 * 1024) {
    cset(c->err, "window %d x head_dim %d needs %zu bytes of LDS", cfg->window, cfg->head_dim, lds);
    return fail(QT_E_INVALID);
  }
  *out = c;
  return QT_OK;
}

qt_status qt_codec_decode(qt_codec* c, const int32_t* codes, int32_t T, float* audio) {
  if (!c) { cset(g_cerr, "codec is NULL"); return QT_E_INVALID; }
  if (!codes || !audio) { cset(c->err, "codes and audio must not be NULL"); return QT_E_INVALID; }
  if (T < 1 || T > c->lay.F) { cset(c->err, "T=%d outside 1..chunk+context=%ld", T, c->lay.F); return QT_E_CAPACITY; }
  const qt_status st = check_codes(c, codes, T);
  if (st != QT_OK) return st;
  return decode_span(c, codes, 0, T, 0, audio);
}

qt_status qt_codec_decode_chunked(qt_codec* c, const int32_t* codes, int32_t T, float* audio) {
  if (!c) { cset(g_cerr, "codec is NULL"); return QT_E_INVALID; }
  if (!codes || !audio) { cset(c->err, "codes and audio must not be NULL"); return QT_E_INVALID; }
  if (T < 1) { cset(c->err, "T must be >= 1"); return QT_E_INVALID; }
  qt_status st = check_codes(c, codes, T);
  if (st != QT_OK) return st;
  const long N = c->cfg.chunk, ctx = c->cfg.context;
  for (long c0 = 0; c0 < T; c0 += N) {
    st = decode_span(c, codes, std::max(0L, c0 - ctx), std::min<long>(T, c0 + N), c0, audio + c0 * c->hop);
    if (st != QT_OK) return st;
  }
  return QT_OK;
}

qt_status qt_codec_stream(qt_codec* c, const int32_t* codes, int32_t T, int64_t sent, float* out) {
  if (!c) { cset(g_cerr, "codec is NULL"); return QT_E_INVALID; }
  if (!codes || !out) { cset(c->err, "codes and out must not be NULL"); return QT_E_INVALID; }
  if (T < 1 || sent < 0 || sent % c->hop || sent >= (int64_t)T * c->hop) {
    cset(c->err, "need T >= 1 and sent a multiple of hop below T * hop");
    return QT_E_INVALID;
  }
  qt_status st = check_codes(c, codes, T);
  if (st != QT_OK) return st;
  const long N = c->cfg.chunk, ctx = c->cfg.context;
  long f = sent / c->hop;
  float* dst = out;
  while (f < T) {
    const long c0 = f / N * N, end = std::min<long>(T, c0 + N);
    st = decode_span(c, codes, std::max(0L, c0 - ctx), end, f, dst);
    if (st != QT_OK) return st;
    dst += (end - f) * c->hop;
    f = end;
  }
  return QT_OK;
}

}  // extern "C"
