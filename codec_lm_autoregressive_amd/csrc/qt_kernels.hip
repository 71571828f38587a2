// gfx950 (CDNA4) kernels of the Qwen3-TTS 12 Hz per-frame generation step.
//
// Every step of the frame runs here: the weight-streaming projections with
// fused RMSNorm prologues and residual / SwiGLU epilogues, the fused
// QK-RMSNorm + rope + KV write + GQA attention, the logits processors and the
// single-sample selection (Philox4x64-10 exponential race), the frame-start
// commit of code 0 and the code-predictor gathers that also build the
// embedding-sum feedback. Activations are fp32, weights fp32 or bf16, the KV
// cache fp32 or bf16; accumulation is fp32 throughout.
#include "qt_internal.h"

#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>
#include <type_traits>

namespace qt {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;  // threads per block for every kernel here
constexpr int MFMA_MIN_ROWS = 16;  // activation rows from which projections use the matrix cores
#ifndef GEMM_SPLIT_SW
#define GEMM_SPLIT_SW 2        // LDS layout of the prefill GEMM tiles (see SplitLds)
#endif
#ifndef GEMV8_MAX_TILES
#define GEMV8_MAX_TILES 3       // 8-row tiles per block of the 8-row matrix-core GEMV (1..3)
#endif
#ifndef ROWS_DIRECT_TILES
#define ROWS_DIRECT_TILES 192      // output tiles from which the row-block GEMM runs without K ranges
#endif

// Weight rows are streamed once per pass. QT_WEIGHT_NT selects nontemporal
// loads (1) or ordinary cached loads (0).
#ifndef QT_WEIGHT_NT
#define QT_WEIGHT_NT 1
#endif
__device__ __forceinline__ u32x4 ld_weight(const void* p) {
#if QT_WEIGHT_NT
  return __builtin_nontemporal_load((const u32x4*)p);
#else
  return *(const u32x4*)p;
#endif
}

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }
// Round to nearest even; inputs are finite activations.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float ld_elem(const T* p, long i);
template <> __device__ __forceinline__ float ld_elem<float>(const float* p, long i) { return p[i]; }
template <> __device__ __forceinline__ float ld_elem<uint16_t>(const uint16_t* p, long i) { return bf16_to_f32(p[i]); }
template <typename T> __device__ __forceinline__ void st_elem(T* p, long i, float v);
template <> __device__ __forceinline__ void st_elem<float>(float* p, long i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void st_elem<uint16_t>(uint16_t* p, long i, float v) { p[i] = f32_to_bf16(v); }
template <> __device__ __forceinline__ void st_elem<_Float16>(_Float16* p, long i, float v) { p[i] = (_Float16)v; }

__device__ __forceinline__ float ld_any(const void* p, int dt, long i) {
  return dt == DT_BF16 ? bf16_to_f32(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}

// Wave-wide reductions with DPP lane moves (no LDS round trips): within each
// row of 16 lanes via quad permutes and mirrors, then row 0 -> 1, 2 -> 3
// (row_bcast:15) and row 1 -> 2, 3 (row_bcast:31); lane 63 then holds the
// result, which readlane broadcasts. Every lane of the wave must be active.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_f(float v, float id) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, id), __builtin_bit_cast(int, v),
                                                               CTRL, ROWS, 0xf, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xb1, 0xf>(v, 0.f);    // quad_perm [1,0,3,2]
  v += dpp_f<0x4e, 0xf>(v, 0.f);    // quad_perm [2,3,0,1]
  v += dpp_f<0x141, 0xf>(v, 0.f);   // row_half_mirror
  v += dpp_f<0x140, 0xf>(v, 0.f);   // row_mirror
  v += dpp_f<0x142, 0xa>(v, 0.f);   // row_bcast:15 into rows 1, 3
  v += dpp_f<0x143, 0xc>(v, 0.f);   // row_bcast:31 into rows 2, 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xb1, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp_f<0x4e, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp_f<0x141, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp_f<0x140, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp_f<0x142, 0xa>(v, -INFINITY));
  v = fmaxf(v, dpp_f<0x143, 0xc>(v, -INFINITY));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Block-wide reductions for NT threads; `red` is LDS scratch of >= NT/64 floats.
// All threads of the block must call them.
__device__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) t += red[i];
  return t;
}
__device__ float block_max(float v, float* red) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) t = fmaxf(t, red[i]);
  return t;
}
__device__ int block_or(int v, int* redi) {
  __syncthreads();
  if (threadIdx.x == 0) redi[0] = 0;
  __syncthreads();
  if (v) atomicOr(&redi[0], 1);
  __syncthreads();
  return redi[0];
}
// argmax with the lowest index on ties; (value, index) pairs, -inf allowed.
__device__ __forceinline__ void better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}
__device__ int block_argmax(float v, int i, float* redf, int* redi) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o);
    int oi = __shfl_xor(i, o);
    better(v, i, ov, oi);
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { redf[threadIdx.x >> 6] = v; redi[threadIdx.x >> 6] = i; }
  __syncthreads();
  float bv = redf[0];
  int bi = redi[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) better(bv, bi, redf[w], redi[w]);
  return bi;
}

// Raise a kernel's dynamic-LDS limit when a launch needs more than the
// default 64 KB (static LDS of the kernel still counts against the 160 KB).
static hipError_t ensure_lds(const void* fn, size_t bytes, size_t* have) {
  if (bytes <= 64 * 1024 || bytes <= *have) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) *have = bytes;
  return e;
}

// ---------------------------------------------------------------- linear
// Weight-streaming projection. Block = 4 waves; a wave owns R consecutive
// output rows (KS waves share one row group and split K). Each lane streams
// 16-byte chunks of its rows with nontemporal loads; the MT activation rows
// (RMSNorm'd when a gain is given) sit in LDS and are reused by all rows.
template <typename WT, int R, int MT>
__device__ __forceinline__ void linear_fma(float (&acc)[R][MT], const u32x4 (&wv)[R], const float* xs, int K, int k0) {
  constexpr int EPC = 16 / sizeof(WT);
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if constexpr (EPC == 8) {
      const f32x4 xa = *(const f32x4*)(xs + m * K + k0);
      const f32x4 xb = *(const f32x4*)(xs + m * K + k0 + 4);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float s = acc[r][m];
        s = fmaf(bf_lo(wv[r].x), xa.x, s); s = fmaf(bf_hi(wv[r].x), xa.y, s);
        s = fmaf(bf_lo(wv[r].y), xa.z, s); s = fmaf(bf_hi(wv[r].y), xa.w, s);
        s = fmaf(bf_lo(wv[r].z), xb.x, s); s = fmaf(bf_hi(wv[r].z), xb.y, s);
        s = fmaf(bf_lo(wv[r].w), xb.z, s); s = fmaf(bf_hi(wv[r].w), xb.w, s);
        acc[r][m] = s;
      }
    } else {
      const f32x4 xa = *(const f32x4*)(xs + m * K + k0);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float s = acc[r][m];
        s = fmaf(__uint_as_float(wv[r].x), xa.x, s); s = fmaf(__uint_as_float(wv[r].y), xa.y, s);
        s = fmaf(__uint_as_float(wv[r].z), xa.z, s); s = fmaf(__uint_as_float(wv[r].w), xa.w, s);
        acc[r][m] = s;
      }
    }
  }
}

template <typename WT, int R, int MT, int KS>
__global__ __launch_bounds__(NT) void linear_kernel(LinearArgs p) {
  extern __shared__ float xs[];  // [MT][K], then reduction scratch
  const int K = p.K, N = p.N;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m0 = blockIdx.y * MT;
  const int mt = min(MT, p.M - m0);
  float* red = xs + (long)MT * K;          // [4]
  float* part = red + 4;                   // [4][R][MT]

  constexpr int EPC = 16 / sizeof(WT);     // weight elements per 16-byte chunk
  constexpr int RG = 4 / KS;               // row groups per block
  constexpr int NPRE = R == 1 ? 4 : 2;     // chunks per row fetched before the prologue
  const int wrow = wave / KS, ks = wave % KS;
  const int row0 = (blockIdx.x * RG + wrow) * R;
  const int kbase = (ks * 64 + lane) * EPC;
  const int kstride = KS * 64 * EPC;
  const WT* W = (const WT*)p.W;
  // The weights do not depend on the activations: put this lane's first
  // chunks in flight before the activation tile is read and normalised.
  u32x4 wpre[NPRE][R];
#pragma unroll
  for (int c = 0; c < NPRE; ++c) {
    const int k0 = kbase + c * kstride;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = row0 + r;
      if (row < N && k0 < K) wpre[c][r] = ld_weight(W + (long)row * K + k0);
      else wpre[c][r] = (u32x4){0u, 0u, 0u, 0u};
    }
  }

  for (int m = 0; m < mt; ++m) {
    const float* xr = p.X + (long)(m0 + m) * p.ldx;
    if (p.gain) {
      float ss = 0.f;
      for (int k = tid; k < K; k += NT) { float v = xr[k]; ss += v * v; }
      ss = block_sum(ss, red);
      const float den = sqrtf(ss / (float)K + p.eps);
      for (int k = tid; k < K; k += NT) xs[m * K + k] = xr[k] / den * p.gain[k];
    } else {
      for (int k = tid; k < K; k += NT) xs[m * K + k] = xr[k];
    }
  }
  for (int m = mt; m < MT; ++m)
    for (int k = tid; k < K; k += NT) xs[m * K + k] = 0.f;
  __syncthreads();
  if (p.norm_out && blockIdx.x == 0)
    for (int m = 0; m < mt; ++m)
      for (int k = tid; k < K; k += NT) p.norm_out[(long)(m0 + m) * p.ld_norm + k] = xs[m * K + k];

  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;
#pragma unroll
  for (int c = 0; c < NPRE; ++c) {
    const int k0 = kbase + c * kstride;
    if (k0 < K) linear_fma<WT, R, MT>(acc, wpre[c], xs, K, k0);
  }
  for (int k0 = kbase + NPRE * kstride; k0 < K; k0 += kstride) {
    u32x4 wv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = row0 + r;
      if (row < N) wv[r] = ld_weight(W + (long)row * K + k0);
      else wv[r] = (u32x4){0u, 0u, 0u, 0u};
    }
    linear_fma<WT, R, MT>(acc, wv, xs, K, k0);
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = wave_sum(acc[r][m]);
  if constexpr (KS > 1) {
    if (lane == 0)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) part[(wave * R + r) * MT + m] = acc[r][m];
    __syncthreads();
    if (ks == 0 && lane == 0)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float s = 0.f;
          for (int j = 0; j < KS; ++j) s += part[((wave + j) * R + r) * MT + m];
          acc[r][m] = s;
        }
  }
  if (ks != 0 || lane != 0) return;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m >= mt) break;
    float* y = p.Y + (long)(m0 + m) * p.ldy;
    if (p.epi == EPI_SWIGLU) {
#pragma unroll
      for (int r = 0; r + 1 < R; r += 2) {
        const int row = row0 + r;
        if (row + 1 < N) {
          const float g = acc[r][m], u = acc[r + 1][m];
          y[row >> 1] = g / (1.f + expf(-g)) * u;
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = row0 + r;
        if (row < N) y[row] = (p.epi == EPI_RESIDUAL) ? y[row] + acc[r][m] : acc[r][m];
      }
    }
  }
}

// Register-only projection for a few activation rows (decode batches). A wave
// owns R output rows and 1/KS of K: its weight chunks and the matching
// activation chunks go out in one batch (addresses clamped, no divergent
// loads), the RMSNorm sum of squares comes from a wave reduction (plus one
// LDS exchange between the KS waves of a row group), and no activation tile
// is staged in LDS.
template <typename WT, int R, int MT, int KS, int NC>
__global__ __launch_bounds__(NT) void gemv_kernel(LinearArgs p) {
  constexpr int EPC = 16 / sizeof(WT);
  constexpr int RG = 4 / KS;
  __shared__ float red[4][MT];
  __shared__ float part[4][R][MT];
  const int K = p.K, N = p.N;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wrow = wave / KS, ks = wave % KS;
  const int row0 = (blockIdx.x * RG + wrow) * R;
  const int m0 = blockIdx.y * MT;
  const int mt = min(MT, p.M - m0);
  const WT* W = (const WT*)p.W;
  u32x4 w[NC][R];
  float x[NC][MT][EPC];
  float g[NC][EPC];
  bool kin[NC];
  // Activations and gains first, weights last: the vector-memory counter
  // drains in issue order, so the RMSNorm below waits only for the small
  // activation loads while the weight rows are still in flight.
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int k0 = ((c * KS + ks) * 64 + lane) * EPC;
    kin[c] = k0 < K;
    const int kc = kin[c] ? k0 : K - EPC;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float* xr = p.X + (long)(m0 + min(m, mt - 1)) * p.ldx + kc;
#pragma unroll
      for (int e = 0; e < EPC; e += 4) {
        const f32x4 v = *(const f32x4*)(xr + e);
        x[c][m][e] = v.x; x[c][m][e + 1] = v.y; x[c][m][e + 2] = v.z; x[c][m][e + 3] = v.w;
      }
    }
    if (p.gain) {
      const float* gp = p.gain + kc;
#pragma unroll
      for (int e = 0; e < EPC; e += 4) {
        const f32x4 v = *(const f32x4*)(gp + e);
        g[c][e] = v.x; g[c][e + 1] = v.y; g[c][e + 2] = v.z; g[c][e + 3] = v.w;
      }
    }
  }
  // residual epilogue: the old output values, loaded now (only this wave writes them)
  float yold[R][MT];
  if (p.epi == EPI_RESIDUAL)
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) yold[r][m] = p.Y[(long)(m0 + min(m, mt - 1)) * p.ldy + min(row0 + r, N - 1)];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int k0 = ((c * KS + ks) * 64 + lane) * EPC;
    const int kc = k0 < K ? k0 : K - EPC;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min(row0 + r, N - 1);
      w[c][r] = ld_weight(W + (long)row * K + kc);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if (p.gain) {
    float ss[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (kin[c])
#pragma unroll
          for (int e = 0; e < EPC; ++e) s += x[c][m][e] * x[c][m][e];
      ss[m] = wave_sum(s);
    }
    if constexpr (KS > 1) {
      if (lane == 0)
#pragma unroll
        for (int m = 0; m < MT; ++m) red[wave][m] = ss[m];
      __syncthreads();
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float s = 0.f;
        for (int j = 0; j < KS; ++j) s += red[wrow * KS + j][m];
        ss[m] = s;
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float rden = 1.f / sqrtf(ss[m] / (float)K + p.eps);   // one division, then products
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < EPC; ++e) x[c][m][e] = x[c][m][e] * rden * g[c][e];
    }
  }
  if (p.norm_out && blockIdx.x == 0 && wrow == 0)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int k0 = ((c * KS + ks) * 64 + lane) * EPC;
      if (kin[c])
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (m < mt)
#pragma unroll
            for (int e = 0; e < EPC; ++e) p.norm_out[(long)(m0 + m) * p.ld_norm + k0 + e] = x[c][m][e];
    }
  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (!kin[c]) continue;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float wf[8];
      if constexpr (EPC == 8) {
        wf[0] = bf_lo(w[c][r].x); wf[1] = bf_hi(w[c][r].x); wf[2] = bf_lo(w[c][r].y); wf[3] = bf_hi(w[c][r].y);
        wf[4] = bf_lo(w[c][r].z); wf[5] = bf_hi(w[c][r].z); wf[6] = bf_lo(w[c][r].w); wf[7] = bf_hi(w[c][r].w);
      } else {
        wf[0] = __uint_as_float(w[c][r].x); wf[1] = __uint_as_float(w[c][r].y);
        wf[2] = __uint_as_float(w[c][r].z); wf[3] = __uint_as_float(w[c][r].w);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float s = acc[r][m];
#pragma unroll
        for (int e = 0; e < EPC; ++e) s = fmaf(wf[e], x[c][m][e], s);
        acc[r][m] = s;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = wave_sum(acc[r][m]);
  if constexpr (KS > 1) {
    if (lane == 0)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) part[wave][r][m] = acc[r][m];
    __syncthreads();
    if (ks == 0 && lane == 0)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float s = 0.f;
          for (int j = 0; j < KS; ++j) s += part[wave + j][r][m];
          acc[r][m] = s;
        }
  }
  if (ks != 0 || lane != 0) return;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m >= mt) break;
    float* y = p.Y + (long)(m0 + m) * p.ldy;
    if (p.epi == EPI_SWIGLU) {
#pragma unroll
      for (int r = 0; r + 1 < R; r += 2) {
        const int row = row0 + r;
        if (row + 1 < N) {
          const float g = acc[r][m], u = acc[r + 1][m];
          y[row >> 1] = g / (1.f + expf(-g)) * u;
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = row0 + r;
        if (row < N) y[row] = (p.epi == EPI_RESIDUAL) ? yold[r][m] + acc[r][m] : acc[r][m];
      }
    }
  }
}

template <typename WT, int R, int MT, int KS, int NC>
static hipError_t launch_gemv_t(const LinearArgs& a, hipStream_t s) {
  constexpr int RG = 4 / KS;
  dim3 grid((a.N + RG * R - 1) / (RG * R), (a.M + MT - 1) / MT);
  hipLaunchKernelGGL((gemv_kernel<WT, R, MT, KS, NC>), grid, dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <typename WT, int R, int MT, int KS>
static hipError_t launch_gemv_nc(const LinearArgs& a, int nc, hipStream_t s) {
  switch (nc) {
    case 1: return launch_gemv_t<WT, R, MT, KS, 1>(a, s);
    case 2: return launch_gemv_t<WT, R, MT, KS, 2>(a, s);
    case 3: return launch_gemv_t<WT, R, MT, KS, 3>(a, s);
    default: return launch_gemv_t<WT, R, MT, KS, 4>(a, s);
  }
}
template <typename WT, int R, int MT>
static hipError_t launch_gemv_ks(const LinearArgs& a, int ks, int nc, hipStream_t s) {
  if (ks == 4) return launch_gemv_nc<WT, R, MT, 4>(a, nc, s);
  if (ks == 2) return launch_gemv_nc<WT, R, MT, 2>(a, nc, s);
  return launch_gemv_nc<WT, R, MT, 1>(a, nc, s);
}

// Register path when the batch is small and K fits in <= 4 chunks per lane.
static bool gemv_fits(const LinearArgs& a) {
  const int epc = a.wdtype == DT_BF16 ? 8 : 4;
  if (a.M > 2 || a.K % epc) return false;
  const bool wide = a.epi == EPI_SWIGLU || a.N >= 2048;
  const int R = wide ? 2 : 1, min_blocks = wide ? 256 : 768;
  int ks = 1;
  while (ks < 4 && a.N / (4 / ks * R) < min_blocks) ks *= 2;
  return (a.K + ks * 64 * epc - 1) / (ks * 64 * epc) <= 4;
}

template <typename WT>
static bool try_gemv(const LinearArgs& a, hipStream_t s, hipError_t* err) {
  constexpr int EPC = 16 / sizeof(WT);
  if (a.M > 2 || a.K % EPC) return false;
  // Wide outputs: two rows per wave and at least 256 blocks; narrow ones
  // (1024 rows): one row per wave and at least 768 blocks (measured with the
  // weights streamed from HBM).
  const bool wide = a.epi == EPI_SWIGLU || a.N >= 2048;
  const int R = wide ? 2 : 1, min_blocks = wide ? 256 : 768;
  int ks = 1;
  while (ks < 4 && a.N / (4 / ks * R) < min_blocks) ks *= 2;
  const int per = ks * 64 * EPC;
  const int nc = (a.K + per - 1) / per;
  if (nc > 4) return false;
  // both activation rows in one block: the weights stream once
  if (a.M == 1) *err = R == 2 ? launch_gemv_ks<WT, 2, 1>(a, ks, nc, s) : launch_gemv_ks<WT, 1, 1>(a, ks, nc, s);
  else *err = R == 2 ? launch_gemv_ks<WT, 2, 2>(a, ks, nc, s) : launch_gemv_ks<WT, 1, 2>(a, ks, nc, s);
  return true;
}

template <typename WT, int R, int MT, int KS>
static hipError_t launch_linear_t(const LinearArgs& a, hipStream_t s) {
  constexpr int RG = 4 / KS;
  dim3 grid((a.N + RG * R - 1) / (RG * R), (a.M + MT - 1) / MT);
  const size_t lds = ((size_t)MT * a.K + 4 + 4 * R * MT) * sizeof(float);
  static size_t have = 0;
  hipError_t e = ensure_lds((const void*)linear_kernel<WT, R, MT, KS>, lds, &have);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((linear_kernel<WT, R, MT, KS>), grid, dim3(NT), lds, s, a);
  return hipGetLastError();
}

template <typename WT, int R, int KS>
static hipError_t launch_linear_mt(const LinearArgs& a, int mt, hipStream_t s) {
  switch (mt) {
    case 1: return launch_linear_t<WT, R, 1, KS>(a, s);
    case 2: return launch_linear_t<WT, R, 2, KS>(a, s);
    case 4: return launch_linear_t<WT, R, 4, KS>(a, s);
    default: return launch_linear_t<WT, R, 8, KS>(a, s);
  }
}

template <typename WT>
static hipError_t launch_linear_w(const LinearArgs& a, int mt, int R, int KS, hipStream_t s) {
  if (R == 2) return KS == 4 ? launch_linear_mt<WT, 2, 4>(a, mt, s) : launch_linear_mt<WT, 2, 1>(a, mt, s);
  return KS == 4 ? launch_linear_mt<WT, 1, 4>(a, mt, s) : launch_linear_mt<WT, 1, 1>(a, mt, s);
}

// ---------------------------------------------------------------- MFMA GEMM
// Y[M, N] (op)= norm(X)[M, K] · W[N, K]^T for many activation rows (prompt
// prefill, large batches) on the bf16 matrix cores. The fp32 activations are
// split into bf16 hi + lo parts (hi = rne(x), lo = rne(x - hi)); W is exactly
// bf16, so each product is exact and two v_mfma_f32_32x32x16_bf16 per step
// with fp32 accumulation keep the result within ~2^-17 of an fp32 GEMM.
// Block: 4 waves in a 2x2 grid, tile BM x BN, K staged 32 at a time in LDS
// (rows padded to 40 elements). RMSNorm uses per-row denominators from
// row_norm_kernel and is applied while the activation tile is staged.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int GK = 32;        // K per LDS stage
constexpr int GLD = GK + 8;   // padded LDS row (bf16 elements)

__device__ __forceinline__ uint32_t pack_bf16x2(uint16_t lo, uint16_t hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

// Two fp32 -> two bf16 (round to nearest even) with one v_cvt_pk_bf16_f32; a in the low half.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  const bf16x2_t h = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, h);
}
// Split (a, b) into bf16 hi = rne(x) and lo = rne(x - hi), packed in pairs.
__device__ __forceinline__ void split_pk(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = cvt_pk_bf16(a, b);
  lo = cvt_pk_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

template <int BM, int BN>
__global__ __launch_bounds__(NT) void mfma_gemm_kernel(LinearArgs p, const float* __restrict__ den) {
  constexpr int TM = BM / 64, TN = BN / 64;      // 32x32 MFMA tiles per wave
  __shared__ __attribute__((aligned(16))) uint16_t sah[BM * GLD];
  __shared__ __attribute__((aligned(16))) uint16_t sal[BM * GLD];
  __shared__ __attribute__((aligned(16))) uint16_t sb[BN * GLD];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int M = p.M, N = p.N, K = p.K;
  const uint16_t* W = (const uint16_t*)p.W;
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  constexpr int AV = BM * GK / 4 / NT;   // float4 of X per thread per stage
  constexpr int BV = BN * GK / 8 / NT;   // 16-byte W chunks per thread per stage
  for (int k0 = 0; k0 < K; k0 += GK) {
    f32x4 xa[AV];
    u32x4 wb[BV];
#pragma unroll
    for (int q = 0; q < AV; ++q) {
      const int idx = tid + q * NT, r = idx / (GK / 4), c = (idx % (GK / 4)) * 4;
      const int row = m0 + r;
      xa[q] = row < M ? *(const f32x4*)(p.X + (long)row * p.ldx + k0 + c) : (f32x4){0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int q = 0; q < BV; ++q) {
      const int idx = tid + q * NT, r = idx / (GK / 8), c = (idx % (GK / 8)) * 8;
      const int n = n0 + r;
      wb[q] = n < N ? ld_weight(W + (long)n * K + k0 + c) : (u32x4){0u, 0u, 0u, 0u};
    }
    __syncthreads();   // the previous stage's MFMAs are done with the LDS tiles
#pragma unroll
    for (int q = 0; q < AV; ++q) {
      const int idx = tid + q * NT, r = idx / (GK / 4), c = (idx % (GK / 4)) * 4;
      const int row = m0 + r;
      float x[4] = {xa[q].x, xa[q].y, xa[q].z, xa[q].w};
      if (p.gain && row < M) {
        const float rd = 1.f / den[row];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = x[e] * rd * p.gain[k0 + c + e];
      }
      uint32_t h0, l0, h1, l1;
      split_pk(x[0], x[1], h0, l0);
      split_pk(x[2], x[3], h1, l1);
      *(uint2*)&sah[r * GLD + c] = make_uint2(h0, h1);
      *(uint2*)&sal[r * GLD + c] = make_uint2(l0, l1);
    }
#pragma unroll
    for (int q = 0; q < BV; ++q) {
      const int idx = tid + q * NT, r = idx / (GK / 8), c = (idx % (GK / 8)) * 8;
      *(u32x4*)&sb[r * GLD + c] = wb[q];
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < GK; ks += 16) {
      bf16x8 ah[TM], al[TM], bv[TN];
      const int kk = ks + (lane >> 5) * 8;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * (BM / 2) + i * 32 + (lane & 31);
        ah[i] = *(const bf16x8*)&sah[r * GLD + kk];
        al[i] = *(const bf16x8*)&sal[r * GLD + kk];
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * (BN / 2) + j * 32 + (lane & 31);
        bv[j] = *(const bf16x8*)&sb[r * GLD + kk];
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bv[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bv[j], acc[i][j], 0, 0, 0);
        }
    }
  }
  // D(i, j) of a 32x32 tile: lane j + 32 * ((i / 4) % 2), register (i / 8) * 4 + i % 4
#pragma unroll
  for (int ti = 0; ti < TM; ++ti)
#pragma unroll
    for (int tj = 0; tj < TN; ++tj)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int row = m0 + wm * (BM / 2) + ti * 32 + i;
        const int col = n0 + wn * (BN / 2) + tj * 32 + (lane & 31);
        const float v = acc[ti][tj][r];
        if (p.epi == EPI_SWIGLU) {
          const float u = __shfl_xor(v, 1);   // the (gate, up) pair sits in lanes 2c, 2c+1
          if (!(lane & 1) && row < M && col + 1 < N) p.Y[(long)row * p.ldy + (col >> 1)] = v / (1.f + expf(-v)) * u;
        } else if (row < M && col < N) {
          float* y = p.Y + (long)row * p.ldy + col;
          *y = p.epi == EPI_RESIDUAL ? *y + v : v;
        }
      }
}

// den[m] = sqrt(mean(X[m]^2) + eps); optionally the normalised rows.
__global__ __launch_bounds__(NT) void row_norm_kernel(LinearArgs p, float* den) {
  __shared__ float red[8];
  const int m = blockIdx.x;
  const float* x = p.X + (long)m * p.ldx;
  float ss = 0.f;
  for (int k = threadIdx.x; k < p.K; k += NT) ss += x[k] * x[k];
  ss = block_sum(ss, red);
  const float d = sqrtf(ss / (float)p.K + p.eps);
  if (threadIdx.x == 0) den[m] = d;
  if (p.norm_out)
    for (int k = threadIdx.x; k < p.K; k += NT) p.norm_out[(long)m * p.ld_norm + k] = x[k] / d * p.gain[k];
}

// ---------------------------------------------------------------- prefill GEMM
// Projection of many activation rows (prompt prefill chunks). A prologue
// kernel normalises each row once (RMSNorm and gain when a gain is given) and
// splits it into bf16 hi + lo planes, xs = [2][M][K]; the GEMM then reads
// plain bf16 tiles of both planes and of W. Block = 4 waves in a 2 x 2 grid on
// a (64 TM) x (64 TN) tile, each wave a TM x TN grid of 32 x 32
// v_mfma_f32_32x32x16_bf16 tiles (hi and lo products into one accumulator).
// K runs in stages of 32 through two LDS buffers: the global loads of stage
// s + 1 are in flight while stage s is contracted, then stored to the other
// buffer, so one barrier per stage keeps every buffer's readers and writers
// apart (a buffer is rewritten only after the barrier that ends its reads).
__global__ __launch_bounds__(NT) void split_rows_kernel(LinearArgs p, uint16_t* __restrict__ xs) {
  __shared__ float red[8];
  const int m = blockIdx.x, K = p.K;
  const float* x = p.X + (long)m * p.ldx;
  float rs = 1.f;
  if (p.gain) {
    float ss = 0.f;
    for (int k = 4 * threadIdx.x; k < K; k += 4 * NT) {
      const f32x4 v = *(const f32x4*)(x + k);
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = block_sum(ss, red);
    rs = 1.f / sqrtf(ss / (float)K + p.eps);
  }
  uint16_t* hi = xs + (long)m * K;
  uint16_t* lo = xs + ((long)p.M + m) * K;
  for (int k = 4 * threadIdx.x; k < K; k += 4 * NT) {
    f32x4 v = *(const f32x4*)(x + k);
    if (p.gain) {
      const f32x4 g = *(const f32x4*)(p.gain + k);
      v = (f32x4){v.x * rs * g.x, v.y * rs * g.y, v.z * rs * g.z, v.w * rs * g.w};
      if (p.norm_out) *(f32x4*)(p.norm_out + (long)m * p.ld_norm + k) = v;
    }
    uint32_t h0, l0, h1, l1;
    split_pk(v.x, v.y, h0, l0);
    split_pk(v.z, v.w, h1, l1);
    *(uint2*)(hi + k) = make_uint2(h0, h1);
    *(uint2*)(lo + k) = make_uint2(l0, l1);
  }
}

// LDS tile addressing: SW = 0 pads rows to GLD elements; SW = 1 / 2 keep
// 32-element rows and place 16-byte chunk c of row r at c ^ ((r >> 2) & 3)
// (1) or c ^ ((r >> 1) & 3) (2), so the lanes of one access fall on distinct
// banks without padding.
template <int SW> struct SplitLds {
  static constexpr int LD = SW == 0 ? GLD : GK;
  __device__ static int at(int r, int c) {   // c: element offset, a multiple of 8
    if constexpr (SW == 0) return r * LD + c;
    else if constexpr (SW == 1) return r * LD + (((c >> 3) ^ ((r >> 2) & 3)) << 3);
    else return r * LD + (((c >> 3) ^ ((r >> 1) & 3)) << 3);
  }
};

// FA (no gain: the o and down projections): the activations are read as
// fp32 rows instead and split into the hi + lo LDS planes on the way in, so
// no prologue writes the planes.
template <int TM, int TN, int SW, bool FA = false>
__global__ __launch_bounds__(NT) void gemm_split_kernel(LinearArgs p, const uint16_t* __restrict__ xs) {
  using LT = SplitLds<SW>;
  constexpr int GLD_ = LT::LD;
  constexpr int BM = 64 * TM, BN = 64 * TN;
  constexpr int AF = FA ? BM * GK / 4 / NT : 1;  // fp32 16-byte chunks per thread per stage (FA)
  constexpr int AV = FA ? 1 : BM * GK / 8 / NT;  // 16-byte chunks per thread per stage, each A plane
  constexpr int BV = BN * GK / 8 / NT;            // and of W
  constexpr int BUF = (2 * BM + BN) * GLD_;        // bf16 elements of one stage: A hi, A lo, W
  __shared__ __attribute__((aligned(16))) uint16_t sm[2 * BUF];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int M = p.M, N = p.N, K = p.K;
  // staging slots: A rows idx / 4 (4 chunks of 8 per 32-k row), W rows likewise
  const uint16_t* ah_src[AV];
  const uint16_t* al_src[AV];
  const uint16_t* w_src[BV];
  int a_off[AV], w_off[BV];
  if constexpr (!FA)
#pragma unroll
  for (int q = 0; q < AV; ++q) {
    const int idx = tid + q * NT, r = idx >> 2, c = (idx & 3) * 8;
    const long row = min(m0 + r, M - 1);
    ah_src[q] = xs + row * K + c;
    al_src[q] = xs + ((long)M + row) * K + c;
    a_off[q] = LT::at(r, c);
  }
  // FA staging slots: A rows idx / 8 (8 chunks of 4 floats per 32-k row);
  // chunk c lands in half c & 4 of the 8-element LDS chunk c & ~7
  const float* af_src[AF];
  int af_off[AF];
  if constexpr (FA)
#pragma unroll
  for (int q = 0; q < AF; ++q) {
    const int idx = tid + q * NT, r = idx >> 3, c = (idx & 7) * 4;
    const long row = min(m0 + r, M - 1);
    af_src[q] = p.X + row * p.ldx + c;
    af_off[q] = LT::at(r, c & ~7) + (c & 4);
  }
  u32x4 raf[AF];
#pragma unroll
  for (int q = 0; q < BV; ++q) {
    const int idx = tid + q * NT, r = idx >> 2, c = (idx & 3) * 8;
    w_src[q] = (const uint16_t*)p.W + (long)min(n0 + r, N - 1) * K + c;
    w_off[q] = LT::at(r, c);
  }
  u32x4 ra_h[AV], ra_l[AV], rw[BV];
  auto load = [&](int k0) __attribute__((always_inline)) {
    if constexpr (FA) {
#pragma unroll
      for (int q = 0; q < AF; ++q) raf[q] = *(const u32x4*)(af_src[q] + k0);
    } else {
#pragma unroll
      for (int q = 0; q < AV; ++q) { ra_h[q] = *(const u32x4*)(ah_src[q] + k0); ra_l[q] = *(const u32x4*)(al_src[q] + k0); }
    }
#pragma unroll
    for (int q = 0; q < BV; ++q) rw[q] = *(const u32x4*)(w_src[q] + k0);
  };
  auto store = [&](int b) __attribute__((always_inline)) {
    uint16_t* base = sm + b * BUF;
    if constexpr (FA) {
#pragma unroll
      for (int q = 0; q < AF; ++q) {
        const f32x4 v = __builtin_bit_cast(f32x4, raf[q]);
        uint32_t h0, l0, h1, l1;
        split_pk(v.x, v.y, h0, l0);
        split_pk(v.z, v.w, h1, l1);
        *(uint2*)&base[af_off[q]] = make_uint2(h0, h1);
        *(uint2*)&base[BM * GLD_ + af_off[q]] = make_uint2(l0, l1);
      }
    } else {
#pragma unroll
      for (int q = 0; q < AV; ++q) {
        *(u32x4*)&base[a_off[q]] = ra_h[q];
        *(u32x4*)&base[BM * GLD_ + a_off[q]] = ra_l[q];
      }
    }
#pragma unroll
    for (int q = 0; q < BV; ++q) *(u32x4*)&base[2 * BM * GLD_ + w_off[q]] = rw[q];
  };
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int S = K / GK;
  load(0);
  store(0);
  __syncthreads();
  for (int st = 0; st < S; ++st) {
    if (st + 1 < S) load((st + 1) * GK);
    const uint16_t* base = sm + (st & 1) * BUF;
#pragma unroll
    for (int ks = 0; ks < GK; ks += 16) {
      const int kk = ks + (lane >> 5) * 8;
      bf16x8 ah[TM], al[TM], bv[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * (BM / 2) + i * 32 + (lane & 31);
        ah[i] = *(const bf16x8*)&base[LT::at(r, kk)];
        al[i] = *(const bf16x8*)&base[BM * GLD_ + LT::at(r, kk)];
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * (BN / 2) + j * 32 + (lane & 31);
        bv[j] = *(const bf16x8*)&base[2 * BM * GLD_ + LT::at(r, kk)];
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bv[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bv[j], acc[i][j], 0, 0, 0);
        }
    }
    if (st + 1 < S) store((st + 1) & 1);
    __syncthreads();
  }
  // D(i, j) of a 32x32 tile: lane j + 32 * ((i / 4) % 2), register (i / 8) * 4 + i % 4
#pragma unroll
  for (int ti = 0; ti < TM; ++ti)
#pragma unroll
    for (int tj = 0; tj < TN; ++tj)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int row = m0 + wm * (BM / 2) + ti * 32 + i;
        const int col = n0 + wn * (BN / 2) + tj * 32 + (lane & 31);
        const float v = acc[ti][tj][r];
        if (p.epi == EPI_SWIGLU) {
          const float u = __shfl_xor(v, 1);   // the (gate, up) pair sits in lanes 2c, 2c+1
          if (!(lane & 1) && row < M && col + 1 < N) p.Y[(long)row * p.ldy + (col >> 1)] = v / (1.f + expf(-v)) * u;
        } else if (row < M && col < N) {
          float* y = p.Y + (long)row * p.ldy + col;
          *y = p.epi == EPI_RESIDUAL ? *y + v : v;
        }
      }
}

// The split GEMM needs K % 32 == 0, rows of 16-byte aligned activations and
// the split scratch; 128 x 128 tiles while they give at least 512 blocks (two
// per compute unit at a time), else 64 x 128.
static bool gemm_split_fits(const LinearArgs& a) {
  return a.wdtype == DT_BF16 && a.K % GK == 0 && a.ldx % 4 == 0 && a.xs && a.xs_floats >= (long)a.M * a.K;
}

// Without a gain and from 2048 rows the GEMM splits fp32 activation tiles
// itself (FA): 4096 rows, o 64 us and down 88 us against 74 and 108 with the
// prologue; with a gain (an extra gain load per chunk, fewer waves) and at
// 1051 rows the prologue path measured as fast or faster.
static hipError_t launch_gemm_split(const LinearArgs& a, hipStream_t s) {
  uint16_t* xs = (uint16_t*)a.xs;
  const bool fa = !a.gain && !a.norm_out && a.M >= 2048;
  if (!fa) hipLaunchKernelGGL(split_rows_kernel, dim3(a.M), dim3(NT), 0, s, a, xs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long big = (long)((a.M + 127) / 128) * ((a.N + 127) / 128);
  if (big >= 512) {
    dim3 grid((a.N + 127) / 128, (a.M + 127) / 128);
    if (fa) hipLaunchKernelGGL((gemm_split_kernel<2, 2, GEMM_SPLIT_SW, true>), grid, dim3(NT), 0, s, a, xs);
    else hipLaunchKernelGGL((gemm_split_kernel<2, 2, GEMM_SPLIT_SW>), grid, dim3(NT), 0, s, a, xs);
  } else {
    dim3 grid((a.N + 127) / 128, (a.M + 63) / 64);
    if (fa) hipLaunchKernelGGL((gemm_split_kernel<1, 2, GEMM_SPLIT_SW, true>), grid, dim3(NT), 0, s, a, xs);
    else hipLaunchKernelGGL((gemm_split_kernel<1, 2, GEMM_SPLIT_SW>), grid, dim3(NT), 0, s, a, xs);
  }
  return hipGetLastError();
}

static hipError_t launch_mfma(const LinearArgs& a, float* den, hipStream_t s) {
  if (a.gain) {
    hipLaunchKernelGGL(row_norm_kernel, dim3(a.M), dim3(NT), 0, s, a, den);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.M > 64) {
    dim3 grid((a.N + 127) / 128, (a.M + 127) / 128);
    hipLaunchKernelGGL((mfma_gemm_kernel<128, 128>), grid, dim3(NT), 0, s, a, den);
  } else {
    dim3 grid((a.N + 63) / 64, (a.M + 63) / 64);
    hipLaunchKernelGGL((mfma_gemm_kernel<64, 64>), grid, dim3(NT), 0, s, a, den);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- skinny MFMA
// Projection for 3..16 activation rows with bf16 weights: the weights stream
// once, with coalesced loads, and the products run on the matrix cores
// (v_mfma_f32_16x16x32_bf16).
// Block = 4 waves on one tile of 16 weight rows; K is cut into slices of 256
// and wave w takes slices w, w + 4, ... (S per wave). Per slice a wave loads
// its 16 x 256 weight tile (each half-wave reads 512 contiguous bytes of one
// row) and the M activation rows (a full wave per row), writes them to its own
// LDS region (activations RMSNorm'd and split into bf16 hi + lo on the way)
// and reads back MFMA fragments: step u contracts k in [32u, 32u + 32).
// The hi and lo parts both multiply the exact bf16 weights with fp32
// accumulation; the four waves' 16 x 16 tiles are summed in LDS in a fixed
// order. Weight loads run PF slices ahead, activation loads two.
constexpr int SK_SLICE = 256;
constexpr int SK_LD = SK_SLICE + 8;      // LDS row stride (bf16 elements): 528 bytes
constexpr int SK_NW = 4;                 // waves per block
constexpr int SK_MAXM = 16;

static size_t skinny_lds_bytes(int M) {
  return (size_t)SK_NW * (16 * SK_LD * 2 + 2 * M * SK_LD * 2) + SK_NW * 4 * 64 * 4 + SK_NW * 16 * 4;
}

template <int S, bool NORM>
__global__ __launch_bounds__(SK_NW * 64) void skinny_kernel(LinearArgs p) {
  static_assert(!NORM || S <= 2, "the norm prologue keeps every slice of a row in registers");
  constexpr int PF = S < 3 ? S : 3;      // weight slices in flight
  constexpr int XB = S < 2 ? S : 2;      // activation slices in flight
  extern __shared__ __attribute__((aligned(16))) unsigned char sk_smem[];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int j = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int K = p.K, N = p.N, M = p.M;
  uint16_t* Wl = (uint16_t*)sk_smem + w * 16 * SK_LD;
  uint16_t* Xh = (uint16_t*)sk_smem + SK_NW * 16 * SK_LD + w * 2 * M * SK_LD;
  uint16_t* Xl = Xh + M * SK_LD;
  float* red = (float*)(sk_smem + SK_NW * (16 * SK_LD * 2 + 2 * M * SK_LD * 2));
  float* rss = red + SK_NW * 4 * 64;
  const uint16_t* W = (const uint16_t*)p.W;
  // weight tile load: instruction q reads row 2q + lane / 32, elements 8 (lane % 32) .. + 8
  const uint16_t* wrow[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) wrow[q] = W + (long)min(n0 + 2 * q + (lane >> 5), N - 1) * K + 8 * (lane & 31);
  u32x4 wv[PF][8];
  f32x4 xv[XB][SK_MAXM];
  auto load_w = [&](int si, int slot) __attribute__((always_inline)) {
    const int k0 = (si * SK_NW + w) * SK_SLICE;
    if (k0 < K)
#pragma unroll
      for (int q = 0; q < 8; ++q) wv[slot][q] = ld_weight(wrow[q] + k0);
  };
  auto load_x = [&](int si, int slot) __attribute__((always_inline)) {
    const int k0 = (si * SK_NW + w) * SK_SLICE;
    if (k0 < K)
#pragma unroll
      for (int m = 0; m < SK_MAXM; ++m)
        if (m < M) xv[slot][m] = *(const f32x4*)(p.X + (long)m * p.ldx + k0 + 4 * lane);
  };
  // activations, gains and the residual inputs first, weights last: the
  // vector-memory counter drains in issue order, so the norm below waits
  // only for the activations while the weight slices are in flight
#pragma unroll
  for (int si = 0; si < XB; ++si) load_x(si, si);
  f32x4 gvs[NORM ? S : 1];
  if constexpr (NORM)
#pragma unroll
    for (int si = 0; si < S; ++si) gvs[si] = *(const f32x4*)(p.gain + min((si * SK_NW + w) * SK_SLICE, K - SK_SLICE) + 4 * lane);
  const int orow = 4 * g + w, ocol = n0 + j;   // this lane's output element
  float yold = 0.f;
  if (p.epi == EPI_RESIDUAL) yold = p.Y[(long)min(orow, M - 1) * p.ldy + min(ocol, N - 1)];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int si = 0; si < PF; ++si) load_w(si, si);
  __builtin_amdgcn_sched_barrier(0);
  float inv[SK_MAXM];   // per row 1 / sqrt(mean(x^2) + eps)
  const float rk = 1.f / (float)K;
  if constexpr (NORM) {
    // row sums of squares over all of K: lanes, then the waves
#pragma unroll
    for (int m = 0; m < SK_MAXM; ++m) {
      float ss = 0.f;
#pragma unroll
      for (int si = 0; si < S; ++si)
        if ((si * SK_NW + w) * SK_SLICE < K && m < M) {
          const f32x4 v = xv[si][m];
          ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        }
      ss = wave_sum(ss);
      if (lane == 0 && m < M) rss[w * 16 + m] = ss;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < SK_MAXM; ++m) {
      float tot = 0.f;
      if (m < M)
#pragma unroll
        for (int q = 0; q < SK_NW; ++q) tot += rss[q * 16 + m];
      inv[m] = 1.f / sqrtf(tot * rk + p.eps);   // reciprocal of the row's RMS denominator
    }
  }
  f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int jr = min(j, M - 1);   // padding rows of the tile repeat the last row; their results are dropped
#pragma unroll
  for (int si = 0; si < S; ++si) {
    const int k0 = (si * SK_NW + w) * SK_SLICE;
    const bool live = k0 < K;
    if (live) {
#pragma unroll
      for (int q = 0; q < 8; ++q) *(u32x4*)&Wl[(2 * q + (lane >> 5)) * SK_LD + 8 * (lane & 31)] = wv[si % PF][q];
      f32x4 gv = (f32x4){1.f, 1.f, 1.f, 1.f};
      if constexpr (NORM) gv = gvs[si];
#pragma unroll
      for (int m = 0; m < SK_MAXM; ++m) {
        if (m < M) {
        float x[4] = {xv[si % 2][m].x, xv[si % 2][m].y, xv[si % 2][m].z, xv[si % 2][m].w};
        if constexpr (NORM) {
          x[0] = x[0] * inv[m] * gv.x; x[1] = x[1] * inv[m] * gv.y;
          x[2] = x[2] * inv[m] * gv.z; x[3] = x[3] * inv[m] * gv.w;
          if (p.norm_out && blockIdx.x == 0)
            *(f32x4*)(p.norm_out + (long)m * p.ld_norm + k0 + 4 * lane) = (f32x4){x[0], x[1], x[2], x[3]};
        }
        uint32_t h0, l0, h1, l1;
        split_pk(x[0], x[1], h0, l0);
        split_pk(x[2], x[3], h1, l1);
        *(uint2*)&Xh[m * SK_LD + 4 * lane] = make_uint2(h0, h1);
        *(uint2*)&Xl[m * SK_LD + 4 * lane] = make_uint2(l0, l1);
        }
      }
    }
    // refill the register slots just drained
    if (si + PF < S) load_w(si + PF, si % PF);
    if (si + 2 < S) load_x(si + 2, si % 2);
    __syncthreads();
    if (live)
#pragma unroll
      for (int u = 0; u < SK_SLICE / 32; ++u) {
        const int kk = 32 * u + 8 * g;
        const bf16x8 bw = *(const bf16x8*)&Wl[j * SK_LD + kk];
        const bf16x8 ah = *(const bf16x8*)&Xh[jr * SK_LD + kk];
        const bf16x8 al = *(const bf16x8*)&Xl[jr * SK_LD + kk];
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bw, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bw, acc, 0, 0, 0);
      }
    __syncthreads();
  }
  // D(i, j) of the 16x16 tile: lane j + 16 * (i / 4), register i % 4; wave r sums register r
#pragma unroll
  for (int r = 0; r < 4; ++r) red[(w * 4 + r) * 64 + lane] = acc[r];
  __syncthreads();
  const int r = w;
  float v = 0.f;
#pragma unroll
  for (int q = 0; q < SK_NW; ++q) v += red[(q * 4 + r) * 64 + lane];
  const int row = 4 * g + r, col = n0 + j;
  if (p.epi == EPI_SWIGLU) {
    const float up = __shfl_xor(v, 1);   // (gate, up) rows 2c, 2c + 1 sit in lanes j, j ^ 1
    if (!(j & 1) && row < M && col + 1 < N) p.Y[(long)row * p.ldy + (col >> 1)] = v / (1.f + expf(-v)) * up;
  } else if (row < M && col < N) {
    p.Y[(long)row * p.ldy + col] = p.epi == EPI_RESIDUAL ? yold + v : v;
  }
}

template <int S, bool NORM>
static hipError_t launch_skinny_k(const LinearArgs& a, hipStream_t s) {
  static size_t have = 0;
  hipError_t e = ensure_lds((const void*)skinny_kernel<S, NORM>, skinny_lds_bytes(SK_MAXM), &have);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((skinny_kernel<S, NORM>), dim3((a.N + 15) / 16), dim3(SK_NW * 64), skinny_lds_bytes(a.M), s, a);
  return hipGetLastError();
}

static bool skinny_fits(const LinearArgs& a) {
  if (a.wdtype != DT_BF16 || a.M < 3 || a.M > SK_MAXM || a.K % SK_SLICE != 0) return false;
  const int S = (a.K / SK_SLICE + SK_NW - 1) / SK_NW;
  return a.gain ? S <= 2 : S <= 6;
}

static hipError_t launch_skinny(const LinearArgs& a, hipStream_t s) {
  const int S = (a.K / SK_SLICE + SK_NW - 1) / SK_NW;
  if (a.gain) return S == 1 ? launch_skinny_k<1, true>(a, s) : launch_skinny_k<2, true>(a, s);
  switch (S) {
    case 1: return launch_skinny_k<1, false>(a, s);
    case 2: return launch_skinny_k<2, false>(a, s);
    case 3: return launch_skinny_k<3, false>(a, s);
    case 4: return launch_skinny_k<4, false>(a, s);
    case 5: return launch_skinny_k<5, false>(a, s);
    default: return launch_skinny_k<6, false>(a, s);
  }
}

// ---------------------------------------------------------------- row-block MFMA GEMM
// Projection for 17..128 activation rows (batched decode, short prompts).
// Block = 4 waves (2 x 2) on a 64 x 64 output tile and a K range of kz
// (gridDim.z ranges split K). The range is read in chunks of 256 with
// coalesced loads, the next chunk's loads in flight while the current one is
// staged 64 k at a time through LDS (activations split into bf16 hi + lo) and
// contracted with v_mfma_f32_32x32x16_bf16, each wave owning a 32 x 32 tile.
// RMSNorm is applied after the contraction: norm(x) W^T = (x * g) W^T / rms(x)
// row by row, so the blocks contract x * g and accumulate the row sums of
// squares while staging. With one K range the block finishes the rows itself;
// otherwise it writes its partial tile (and partial sums of squares) and
// rows_reduce_kernel adds the ranges in a fixed order, scales and applies the
// epilogue, so results do not depend on timing.
constexpr int SG_T = 64;          // output tile edge (rows and columns)
constexpr int SG_GK = 64;         // k per LDS stage
constexpr int SG_LD = SG_GK + 8;  // LDS row stride (bf16): 144 bytes
constexpr int SG_CH = 256;        // k per register chunk

// sum over the 16 lanes of a DPP row; every lane of the row gets the result
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xb1, 0xf>(v, 0.f);
  v += dpp_f<0x4e, 0xf>(v, 0.f);
  v += dpp_f<0x141, 0xf>(v, 0.f);
  v += dpp_f<0x140, 0xf>(v, 0.f);
  return v;
}

// KW groups of 4 waves split the block's K range (group w takes NCH chunks
// from kb + w * NCH * 256); their 64 x 64 tiles and row sums of squares are
// added through LDS in group order before the block finishes or writes its
// partial tile.
template <bool NORM, int NCH, int KW>
__global__ __launch_bounds__(NT * KW) void rows_gemm_kernel(LinearArgs p) {
  constexpr int kz = NCH * SG_CH * KW;   // k per block; each group's NCH register chunks are straight-line
                                         // code, so the prefetch of chunk c + 1 stays in flight during chunk c
  constexpr int XV = SG_T * SG_GK / 4 / NT;   // float4 of X per thread per stage (4)
  constexpr int WV = SG_T * SG_GK / 8 / NT;   // 16-byte W chunks per thread per stage (2)
  constexpr int NS = SG_CH / SG_GK;           // stages per chunk (4)
  constexpr int STAGE = 3 * SG_T * SG_LD;     // bf16 elements of one group's LDS stage
  static_assert(KW == 1 || (KW - 1) * SG_T * SG_T * 4 <= KW * STAGE * 2, "reduction fits in the stages");
  __shared__ __attribute__((aligned(16))) uint16_t smem[KW * STAGE];
  __shared__ float rs_lds[SG_T];
  __shared__ float ss_lds[KW][SG_T];
  const int gtid = threadIdx.x, grp = gtid >> 8, tid = gtid & (NT - 1), wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  uint16_t* xh = smem + grp * STAGE;
  uint16_t* xl = xh + SG_T * SG_LD;
  uint16_t* wl = xl + SG_T * SG_LD;
  const int n0 = blockIdx.x * SG_T, m0 = blockIdx.y * SG_T, kb = blockIdx.z * kz + grp * NCH * SG_CH;
  const int M = p.M, N = p.N, K = p.K;
  const uint16_t* W = (const uint16_t*)p.W;
  // this thread's staging slots: W rows tid / 8 + 32 q, X rows tid / 16 + 16 q
  const int wc = (tid & 7) * 8, xc = (tid & 15) * 4;
  const uint16_t* wrow[WV];
  const float* xrow[XV];
#pragma unroll
  for (int q = 0; q < WV; ++q) wrow[q] = W + (long)min(n0 + (tid >> 3) + 32 * q, N - 1) * K + wc;
#pragma unroll
  for (int q = 0; q < XV; ++q) xrow[q] = p.X + (long)min(m0 + (tid >> 4) + 16 * q, M - 1) * p.ldx + xc;
  u32x4 wa[NS][WV], wb[NS][WV];
  f32x4 xa[NS][XV], xb[NS][XV];
  float ss[XV];
#pragma unroll
  for (int q = 0; q < XV; ++q) ss[q] = 0.f;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  // a group's barrier: the 4 waves of the group (all groups run in lock step)
  auto load = [&](int k0, u32x4 (&wv)[NS][WV], f32x4 (&xv)[NS][XV]) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < NS; ++st) {
#pragma unroll
      for (int q = 0; q < WV; ++q) wv[st][q] = ld_weight(wrow[q] + k0 + st * SG_GK);
#pragma unroll
      for (int q = 0; q < XV; ++q) xv[st][q] = *(const f32x4*)(xrow[q] + k0 + st * SG_GK);
    }
  };
  auto process = [&](int k0, const u32x4 (&wv)[NS][WV], const f32x4 (&xv)[NS][XV]) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      __syncthreads();   // the previous stage's fragments have been read
#pragma unroll
      for (int q = 0; q < WV; ++q) *(u32x4*)&wl[((tid >> 3) + 32 * q) * SG_LD + wc] = wv[st][q];
      f32x4 g = (f32x4){1.f, 1.f, 1.f, 1.f};
      if constexpr (NORM) g = *(const f32x4*)(p.gain + k0 + st * SG_GK + xc);
#pragma unroll
      for (int q = 0; q < XV; ++q) {
        const f32x4 v = xv[st][q];
        if constexpr (NORM) ss[q] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        uint32_t h0, l0, h1, l1;
        split_pk(v.x * g.x, v.y * g.y, h0, l0);
        split_pk(v.z * g.z, v.w * g.w, h1, l1);
        const int r = (tid >> 4) + 16 * q;
        *(uint2*)&xh[r * SG_LD + xc] = make_uint2(h0, h1);
        *(uint2*)&xl[r * SG_LD + xc] = make_uint2(l0, l1);
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < SG_GK; kk += 16) {
        const int k = kk + 8 * (lane >> 5);
        const bf16x8 ah = *(const bf16x8*)&xh[(wm * 32 + (lane & 31)) * SG_LD + k];
        const bf16x8 al = *(const bf16x8*)&xl[(wm * 32 + (lane & 31)) * SG_LD + k];
        const bf16x8 bw = *(const bf16x8*)&wl[(wn * 32 + (lane & 31)) * SG_LD + k];
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bw, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bw, acc, 0, 0, 0);
      }
    }
  };
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (c == 0) load(kb, wa, xa);
    if (c + 1 < NCH) {
      if (c % 2 == 0) load(kb + (c + 1) * SG_CH, wb, xb);
      else load(kb + (c + 1) * SG_CH, wa, xa);
    }
    if (c % 2 == 0) process(kb + c * SG_CH, wa, xa);
    else process(kb + c * SG_CH, wb, xb);
  }
  if constexpr (NORM) {
#pragma unroll
    for (int q = 0; q < XV; ++q) ss[q] = row16_sum(ss[q]);   // the 16 lanes of a row hold its k slices
    if ((tid & 15) == 0)
#pragma unroll
      for (int q = 0; q < XV; ++q) ss_lds[grp][(tid >> 4) + 16 * q] = ss[q];
  }
  __syncthreads();
  if constexpr (KW > 1) {
    // groups 1.. park their tiles in the (now idle) stage buffers; group 0 adds them in order
    float* red = (float*)smem;
    if (grp > 0)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[((grp - 1) * 16 + r) * NT + tid] = acc[r];
    __syncthreads();
    if (grp == 0)
#pragma unroll
      for (int g2 = 1; g2 < KW; ++g2)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] += red[((g2 - 1) * 16 + r) * NT + tid];
  }
  const bool direct = gridDim.z == 1;
  if constexpr (NORM) {
    if (gtid < SG_T) {
      float t = ss_lds[0][gtid];
#pragma unroll
      for (int g2 = 1; g2 < KW; ++g2) t += ss_lds[g2][gtid];
      const int row = m0 + gtid;
      if (direct) rs_lds[gtid] = 1.f / sqrtf(t / (float)K + p.eps);
      else if (blockIdx.x == 0 && row < M) p.part[(long)gridDim.z * M * N + (long)blockIdx.z * M + row] = t;
    }
    __syncthreads();
    if (grp == 0 && direct && p.norm_out && blockIdx.x == 0)
      for (int k = xc; k < K; k += SG_GK)
#pragma unroll
        for (int q = 0; q < XV; ++q) {
          const int r = (tid >> 4) + 16 * q, row = m0 + r;
          if (row < M) {
            const f32x4 v = *(const f32x4*)(p.X + (long)row * p.ldx + k), g = *(const f32x4*)(p.gain + k);
            const float rs = rs_lds[r];
            *(f32x4*)(p.norm_out + (long)row * p.ld_norm + k) =
                (f32x4){v.x * g.x * rs, v.y * g.y * rs, v.z * g.z * rs, v.w * g.w * rs};
          }
        }
  }
  if (grp > 0) return;   // no barrier follows
  // D(i, j) of the 32x32 tile: lane j + 32 * ((i / 4) % 2), register (i / 8) * 4 + i % 4
  const int col = n0 + wn * 32 + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int lr = wm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3), row = m0 + lr;
    float v = acc[r];
    if (!direct) {
      if (row < M && col < N) p.part[((long)blockIdx.z * M + row) * N + col] = v;
      continue;
    }
    if constexpr (NORM) v *= rs_lds[lr];
    if (p.epi == EPI_SWIGLU) {
      const float up = __shfl_xor(v, 1);   // (gate, up) rows 2c, 2c + 1 sit in lanes 2c, 2c + 1
      if (!(lane & 1) && row < M && col + 1 < N) p.Y[(long)row * p.ldy + (col >> 1)] = v / (1.f + expf(-v)) * up;
    } else if (row < M && col < N) {
      float* y = p.Y + (long)row * p.ldy + col;
      *y = p.epi == EPI_RESIDUAL ? *y + v : v;
    }
  }
}

// One 256-wide K range per block (the plan with one 4-wave group and one
// register chunk): every load of the range (activations, then weights, then
// the gains) leaves before the first use, and each 64-k stage is staged into
// its own LDS buffer (NB buffers, stage st in buffer st % NB), so one barrier
// per stage suffices: a wave that writes stage st has passed barrier st - 1,
// which every wave reaches only after its MFMAs on stage st - 2. With four
// buffers the stores of a stage never wait on another wave's MFMAs; two
// buffers halve the LDS so two blocks share a compute unit when the grid has
// more blocks than there are units. Partial tiles go out with nontemporal
// stores (the reduce or the attention kernel reads them once).
template <bool NORM, int NB>
__global__ __launch_bounds__(NT) void rows_gemm1_kernel(LinearArgs p) {
  constexpr int XV = SG_T * SG_GK / 4 / NT;   // float4 of X per thread per stage (4)
  constexpr int WV = SG_T * SG_GK / 8 / NT;   // 16-byte W chunks per thread per stage (2)
  constexpr int NS = SG_CH / SG_GK;           // stages (4)
  constexpr int STAGE = 3 * SG_T * SG_LD;     // bf16 elements of one stage: X hi, X lo, W
  extern __shared__ __attribute__((aligned(16))) uint16_t dsm[];
  __shared__ float rs_lds[SG_T];
  __shared__ float ss_lds[SG_T];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * SG_T, m0 = blockIdx.y * SG_T, kb = blockIdx.z * SG_CH;
  const int M = p.M, N = p.N, K = p.K;
  const int wc = (tid & 7) * 8, xc = (tid & 15) * 4;
  f32x4 xv[NS][XV];
  u32x4 wv[NS][WV];
  f32x4 gv[NS];
#pragma unroll
  for (int q = 0; q < XV; ++q) {
    const float* xr = p.X + (long)min(m0 + (tid >> 4) + 16 * q, M - 1) * p.ldx + kb + xc;
#pragma unroll
    for (int st = 0; st < NS; ++st) xv[st][q] = *(const f32x4*)(xr + st * SG_GK);
  }
#pragma unroll
  for (int q = 0; q < WV; ++q) {
    const uint16_t* wr = (const uint16_t*)p.W + (long)min(n0 + (tid >> 3) + 32 * q, N - 1) * K + kb + wc;
#pragma unroll
    for (int st = 0; st < NS; ++st) wv[st][q] = ld_weight(wr + st * SG_GK);
  }
  if constexpr (NORM)
#pragma unroll
    for (int st = 0; st < NS; ++st) gv[st] = *(const f32x4*)(p.gain + kb + st * SG_GK + xc);
  float ss[XV];
#pragma unroll
  for (int q = 0; q < XV; ++q) ss[q] = 0.f;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    uint16_t* xh = dsm + (st % NB) * STAGE;
    uint16_t* xl = xh + SG_T * SG_LD;
    uint16_t* wl = xl + SG_T * SG_LD;
#pragma unroll
    for (int q = 0; q < WV; ++q) *(u32x4*)&wl[((tid >> 3) + 32 * q) * SG_LD + wc] = wv[st][q];
    f32x4 g = (f32x4){1.f, 1.f, 1.f, 1.f};
    if constexpr (NORM) g = gv[st];
#pragma unroll
    for (int q = 0; q < XV; ++q) {
      const f32x4 v = xv[st][q];
      if constexpr (NORM) ss[q] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      uint32_t h0, l0, h1, l1;
      split_pk(v.x * g.x, v.y * g.y, h0, l0);
      split_pk(v.z * g.z, v.w * g.w, h1, l1);
      const int r = (tid >> 4) + 16 * q;
      *(uint2*)&xh[r * SG_LD + xc] = make_uint2(h0, h1);
      *(uint2*)&xl[r * SG_LD + xc] = make_uint2(l0, l1);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < SG_GK; kk += 16) {
      const int k = kk + 8 * (lane >> 5);
      const bf16x8 ah = *(const bf16x8*)&xh[(wm * 32 + (lane & 31)) * SG_LD + k];
      const bf16x8 al = *(const bf16x8*)&xl[(wm * 32 + (lane & 31)) * SG_LD + k];
      const bf16x8 bw = *(const bf16x8*)&wl[(wn * 32 + (lane & 31)) * SG_LD + k];
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bw, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bw, acc, 0, 0, 0);
    }
  }
  const bool direct = gridDim.z == 1;
  if constexpr (NORM) {
#pragma unroll
    for (int q = 0; q < XV; ++q) ss[q] = row16_sum(ss[q]);   // the 16 lanes of a row hold its k slices
    if ((tid & 15) == 0)
#pragma unroll
      for (int q = 0; q < XV; ++q) ss_lds[(tid >> 4) + 16 * q] = ss[q];
    __syncthreads();
    if (tid < SG_T) {
      const int row = m0 + tid;
      if (direct) rs_lds[tid] = 1.f / sqrtf(ss_lds[tid] / (float)K + p.eps);
      else if (blockIdx.x == 0 && row < M) p.part[(long)gridDim.z * M * N + (long)blockIdx.z * M + row] = ss_lds[tid];
    }
    if (direct) {
      __syncthreads();
      if (p.norm_out && blockIdx.x == 0)
        for (int k = xc; k < K; k += SG_GK)
#pragma unroll
          for (int q = 0; q < XV; ++q) {
            const int r = (tid >> 4) + 16 * q, row = m0 + r;
            if (row < M) {
              const f32x4 v = *(const f32x4*)(p.X + (long)row * p.ldx + k), g = *(const f32x4*)(p.gain + k);
              const float rs = rs_lds[r];
              *(f32x4*)(p.norm_out + (long)row * p.ld_norm + k) =
                  (f32x4){v.x * g.x * rs, v.y * g.y * rs, v.z * g.z * rs, v.w * g.w * rs};
            }
          }
    }
  }
  // D(i, j) of the 32x32 tile: lane j + 32 * ((i / 4) % 2), register (i / 8) * 4 + i % 4
  const int col = n0 + wn * 32 + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int lr = wm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3), row = m0 + lr;
    float v = acc[r];
    if (!direct) {
      if (row < M && col < N) __builtin_nontemporal_store(v, p.part + ((long)blockIdx.z * M + row) * N + col);
      continue;
    }
    if constexpr (NORM) v *= rs_lds[lr];
    if (p.epi == EPI_SWIGLU) {
      const float up = __shfl_xor(v, 1);   // (gate, up) rows 2c, 2c + 1 sit in lanes 2c, 2c + 1
      if (!(lane & 1) && row < M && col + 1 < N) p.Y[(long)row * p.ldy + (col >> 1)] = v / (1.f + expf(-v)) * up;
    } else if (row < M && col < N) {
      float* y = p.Y + (long)row * p.ldy + col;
      *y = p.epi == EPI_RESIDUAL ? *y + v : v;
    }
  }
}

// Adds the Z partial tiles of each output in order z = 0..Z-1, applies the
// row's RMS scale (sums of squares added in the same order) and the epilogue;
// one thread per 2 consecutive columns (N % 2 == 0: twice the threads of 4
// columns each, measured 0.2-0.4 us faster per launch at 64 rows). Also
// writes norm_out. ZT > 0: exactly ZT ranges, every partial load issued
// before the first add (a loop would wait for each load in turn); ZT == 0:
// any Z.
template <int ZT>
__global__ __launch_bounds__(NT) void rows_reduce_kernel(LinearArgs p, int Z) {
  const int n2 = p.N / 2;
  const long t = (long)blockIdx.x * NT + threadIdx.x;
  if (t >= (long)p.M * n2) return;
  const int row = (int)(t / n2), c = (int)(t % n2) * 2;
  const float* pss = p.part + (long)Z * p.M * p.N;
  // the residual's old values go out with the partial loads
  float2 yold = make_float2(0.f, 0.f);
  if (p.epi == EPI_RESIDUAL) yold = *(const float2*)(p.Y + (long)row * p.ldy + c);
  float2 s;
  float ssum = 0.f;
  if constexpr (ZT > 0) {
    float2 v[ZT];
    float q[ZT];
#pragma unroll
    for (int z = 0; z < ZT; ++z) v[z] = *(const float2*)(p.part + ((long)z * p.M + row) * p.N + c);
    if (p.gain)
#pragma unroll
      for (int z = 0; z < ZT; ++z) q[z] = pss[(long)z * p.M + row];
    s = v[0];
#pragma unroll
    for (int z = 1; z < ZT; ++z) { s.x += v[z].x; s.y += v[z].y; }
    if (p.gain) {
      ssum = q[0];
#pragma unroll
      for (int z = 1; z < ZT; ++z) ssum += q[z];
    }
  } else {
    s = *(const float2*)(p.part + (long)row * p.N + c);
    for (int z = 1; z < Z; ++z) {
      const float2 v = *(const float2*)(p.part + ((long)z * p.M + row) * p.N + c);
      s.x += v.x; s.y += v.y;
    }
    if (p.gain) {
      ssum = pss[row];
      for (int z = 1; z < Z; ++z) ssum += pss[(long)z * p.M + row];
    }
  }
  if (p.gain) {
    const float rs = 1.f / sqrtf(ssum / (float)p.K + p.eps);
    s.x *= rs; s.y *= rs;
    if (p.norm_out)
      for (int k = c; k < p.K; k += p.N) {
        const float2 v = *(const float2*)(p.X + (long)row * p.ldx + k), g = *(const float2*)(p.gain + k);
        *(float2*)(p.norm_out + (long)row * p.ld_norm + k) = make_float2(v.x * g.x * rs, v.y * g.y * rs);
      }
  }
  float* y = p.Y + (long)row * p.ldy;
  if (p.epi == EPI_SWIGLU) {
    y[c / 2] = s.x / (1.f + expf(-s.x)) * s.y;
  } else if (p.epi == EPI_RESIDUAL) {
    *(float2*)(y + c) = make_float2(yold.x + s.x, yold.y + s.y);
  } else {
    *(float2*)(y + c) = s;
  }
}

// Shapes of the row-block GEMM: Z K ranges (blocks along z), KW 4-wave groups
// per block and NCH 256-wide register chunks per group, Z * KW * NCH * 256 = K.
struct RowsPlan { int Z, KW, NCH; };

// (KW, NCH) pairs with an instantiation of rows_gemm_kernel: four groups hold
// one chunk each (128 registers per lane at 16 waves per CU), two groups up
// to 4, one group up to 12.
static bool rows_inst(int kw, int nch) {
  if (kw == 4) return nch == 1;
  if (kw == 2) return nch == 1 || nch == 2 || nch == 3 || nch == 4;
  return kw == 1 && (nch == 1 || nch == 2 || nch == 3 || nch == 4 || nch == 6 || nch == 8 || nch == 12);
}

// One K range (no reduce launch, the K groups of a block share the work) when
// the output tiles alone give ROWS_DIRECT_TILES blocks; else single-group
// blocks over the fewest K ranges that give about 256 blocks, limited by the
// partial-sum space.
static bool rows_plan(const LinearArgs& a, RowsPlan* pl) {
  if (a.wdtype != DT_BF16 || a.M < 17 || a.M > 128 || a.K % SG_CH || a.N % 4 || a.ldx % 4 || a.ldy % 2 ||
      (a.norm_out && a.ld_norm % 2))
    return false;
  const long tiles = (long)((a.N + SG_T - 1) / SG_T) * ((a.M + SG_T - 1) / SG_T);
  const int chunks = a.K / SG_CH;
  if (tiles >= ROWS_DIRECT_TILES)
    for (int kw = 4; kw >= 1; kw /= 2)
      if (chunks % kw == 0 && rows_inst(kw, chunks / kw)) { *pl = {1, kw, chunks / kw}; return true; }
  auto fits = [&](int z) {
    return chunks % z == 0 && rows_inst(1, chunks / z) &&
           (z == 1 || (a.part && (long)z * a.M * a.N + (long)z * a.M <= a.part_floats));
  };
  int z = 0;
  for (int c = 1; !z && c <= chunks; ++c)
    if (fits(c) && (tiles * c >= 256 || c == chunks)) z = c;
  for (int c = chunks; !z && c >= 1; --c)
    if (fits(c)) z = c;
  if (!z) return false;
  *pl = {z, 1, chunks / z};
  return true;
}

template <bool NORM, int KW>
static hipError_t launch_rows_n(const LinearArgs& a, int nch, dim3 grid, hipStream_t s) {
  const dim3 block(NT * KW);
  switch (nch) {
    case 1: hipLaunchKernelGGL((rows_gemm_kernel<NORM, 1, KW>), grid, block, 0, s, a); break;
    case 2: if constexpr (KW <= 2) { hipLaunchKernelGGL((rows_gemm_kernel<NORM, 2, KW>), grid, block, 0, s, a); break; }
            return hipErrorInvalidValue;
    case 3: if constexpr (KW <= 2) { hipLaunchKernelGGL((rows_gemm_kernel<NORM, 3, KW>), grid, block, 0, s, a); break; }
            return hipErrorInvalidValue;
    case 4: if constexpr (KW <= 2) { hipLaunchKernelGGL((rows_gemm_kernel<NORM, 4, KW>), grid, block, 0, s, a); break; }
            return hipErrorInvalidValue;
    case 6: if constexpr (KW == 1) { hipLaunchKernelGGL((rows_gemm_kernel<NORM, 6, KW>), grid, block, 0, s, a); break; }
            return hipErrorInvalidValue;
    case 8: if constexpr (KW == 1) { hipLaunchKernelGGL((rows_gemm_kernel<NORM, 8, KW>), grid, block, 0, s, a); break; }
            return hipErrorInvalidValue;
    case 12: if constexpr (KW == 1) { hipLaunchKernelGGL((rows_gemm_kernel<NORM, 12, KW>), grid, block, 0, s, a); break; }
             return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool NORM>
static hipError_t launch_rows_g(const LinearArgs& a, const RowsPlan& pl, dim3 grid, hipStream_t s) {
  if (pl.KW == 4) return launch_rows_n<NORM, 4>(a, pl.NCH, grid, s);
  if (pl.KW == 2) return launch_rows_n<NORM, 2>(a, pl.NCH, grid, s);
  return launch_rows_n<NORM, 1>(a, pl.NCH, grid, s);
}

template <bool NORM, int NB>
static hipError_t launch_rows1(const LinearArgs& a, dim3 grid, hipStream_t s) {
  static size_t have = 0;
  const size_t lds = (size_t)NB * 3 * SG_T * SG_LD * sizeof(uint16_t);
  hipError_t e = ensure_lds((const void*)rows_gemm1_kernel<NORM, NB>, lds, &have);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((rows_gemm1_kernel<NORM, NB>), grid, dim3(NT), lds, s, a);
  return hipGetLastError();
}

static hipError_t launch_rows(const LinearArgs& a, const RowsPlan& pl, hipStream_t s) {
  dim3 grid((a.N + SG_T - 1) / SG_T, (a.M + SG_T - 1) / SG_T, pl.Z);
  hipError_t e;
  if (pl.KW == 1 && pl.NCH == 1) {
    // four stage buffers (110 KB of LDS, one block per compute unit) while the grid fits the
    // 256 units, else two (55 KB, two blocks per unit)
    const bool wide = (long)grid.x * grid.y * grid.z > 256;
    e = a.gain ? (wide ? launch_rows1<true, 2>(a, grid, s) : launch_rows1<true, 4>(a, grid, s))
               : (wide ? launch_rows1<false, 2>(a, grid, s) : launch_rows1<false, 4>(a, grid, s));
  } else {
    e = a.gain ? launch_rows_g<true>(a, pl, grid, s) : launch_rows_g<false>(a, pl, grid, s);
  }
  if (e != hipSuccess || pl.Z == 1 || a.defer) return e;
  const long threads = (long)a.M * (a.N / 2);
  const dim3 grid_r((unsigned)((threads + NT - 1) / NT));
  switch (pl.Z) {
    case 2: hipLaunchKernelGGL(rows_reduce_kernel<2>, grid_r, dim3(NT), 0, s, a, pl.Z); break;
    case 3: hipLaunchKernelGGL(rows_reduce_kernel<3>, grid_r, dim3(NT), 0, s, a, pl.Z); break;
    case 4: hipLaunchKernelGGL(rows_reduce_kernel<4>, grid_r, dim3(NT), 0, s, a, pl.Z); break;
    case 6: hipLaunchKernelGGL(rows_reduce_kernel<6>, grid_r, dim3(NT), 0, s, a, pl.Z); break;
    case 8: hipLaunchKernelGGL(rows_reduce_kernel<8>, grid_r, dim3(NT), 0, s, a, pl.Z); break;
    case 12: hipLaunchKernelGGL(rows_reduce_kernel<12>, grid_r, dim3(NT), 0, s, a, pl.Z); break;
    case 16: hipLaunchKernelGGL(rows_reduce_kernel<16>, grid_r, dim3(NT), 0, s, a, pl.Z); break;
    default: hipLaunchKernelGGL(rows_reduce_kernel<0>, grid_r, dim3(NT), 0, s, a, pl.Z); break;
  }
  return hipGetLastError();
}

static bool mfma_gemv_plan(const LinearArgs& a, int* ksw, int* ng);
static bool mfma_gemv8_plan(const LinearArgs& a, int* ksw, int* ns, int* tiles);
int linear_split_ranges(const LinearArgs& a) {
  int ksw, ng, t8;
  if (a.M <= 0 || gemv_fits(a) || skinny_fits(a) || mfma_gemv_plan(a, &ksw, &ng) || mfma_gemv8_plan(a, &ksw, &ng, &t8)) return 1;
  RowsPlan pl;
  return rows_plan(a, &pl) ? pl.Z : 1;
}

// ---------------------------------------------------------------- matrix-core GEMV
// Projection of up to 16 MT activation rows (MT 16-row tiles) on the matrix
// cores with no LDS staging of either operand: v_mfma_f32_16x16x32_bf16 takes B = W^T straight
// from a 16-byte load of a weight row (lane l: row n0 + l % 16, k offset
// 8 (l / 16)), and A = the activations, which each lane loads as fp32 for its
// row l % 16 (rows past M repeat row M - 1 and are dropped), scales by the
// RMSNorm gain and splits into bf16 hi + lo (two MFMAs, fp32-accurate).
// Block = KSW waves (KSW >= MT), one 16-row output tile; wave w covers K
// range w with NG groups of 8 / MT k-steps of 32, the next group's loads in
// flight while a group is processed. The waves' tiles and the row sums of
// squares are added in LDS in wave order (wave t finishes m-tile t); RMSNorm
// is applied after the contraction as a per-row scale.
template <int KSW, int NG, bool NORM, int MT>
__global__ __launch_bounds__(KSW * 64) void mfma_gemv_kernel(LinearArgs p) {
  constexpr int GS = 8 / MT;                   // k-steps of 32 per group
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lk = lane >> 4;    // operand row, k sub-block
  const int n0 = blockIdx.x * 16;
  const int M = p.M, N = p.N, K = p.K;
  const int kw0 = w * (K / KSW);               // this wave's K range
  __shared__ __align__(16) float red[KSW][MT][64][4];
  __shared__ float ssr[KSW][16 * MT];
  __shared__ float inv_s[16 * MT];
  const uint16_t* wrow = (const uint16_t*)p.W + (long)min(n0 + li, N - 1) * K + kw0 + 8 * lk;
  const float* xrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) xrow[t] = p.X + (long)min(16 * t + li, M - 1) * p.ldx + kw0 + 8 * lk;
  const float* grow = NORM ? p.gain + kw0 + 8 * lk : nullptr;
  // the residual's old values of this lane's outputs (rows 4 lk + r, column n0 + li)
  float yold[MT][4] = {};
  if (p.epi == EPI_RESIDUAL)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) yold[t][r] = p.Y[(long)min(16 * t + 4 * lk + r, M - 1) * p.ldy + min(n0 + li, N - 1)];
  u32x4 wa[GS], wb[GS];
  f32x4 xa[GS][MT][2], xb[GS][MT][2], ga[GS][2], gb[GS][2];
  auto load_x = [&](int gi, f32x4 (&xv)[GS][MT][2], f32x4 (&gv)[GS][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < GS; ++st) {
      const int k = (gi * GS + st) * 32;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        xv[st][t][0] = *(const f32x4*)(xrow[t] + k);
        xv[st][t][1] = *(const f32x4*)(xrow[t] + k + 4);
      }
      if constexpr (NORM) {
        gv[st][0] = *(const f32x4*)(grow + k);
        gv[st][1] = *(const f32x4*)(grow + k + 4);
      }
    }
  };
  auto load_w = [&](int gi, u32x4 (&wv)[GS]) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < GS; ++st) wv[st] = ld_weight(wrow + (gi * GS + st) * 32);
  };
  f32x4 acc[MT];
  float ss[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) { acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f}; ss[t] = 0.f; }
  auto process = [&](const u32x4 (&wv)[GS], const f32x4 (&xv)[GS][MT][2], const f32x4 (&gv)[GS][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < GS; ++st) {
      const bf16x8 bw = __builtin_bit_cast(bf16x8, wv[st]);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        float x[8] = {xv[st][t][0].x, xv[st][t][0].y, xv[st][t][0].z, xv[st][t][0].w,
                      xv[st][t][1].x, xv[st][t][1].y, xv[st][t][1].z, xv[st][t][1].w};
        if constexpr (NORM) {
          const float g[8] = {gv[st][0].x, gv[st][0].y, gv[st][0].z, gv[st][0].w, gv[st][1].x, gv[st][1].y, gv[st][1].z, gv[st][1].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) { ss[t] = fmaf(x[e], x[e], ss[t]); x[e] *= g[e]; }
        }
        uint32_t h[4], l[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) split_pk(x[2 * e], x[2 * e + 1], h[e], l[e]);
        const bf16x8 ah = __builtin_bit_cast(bf16x8, (u32x4){h[0], h[1], h[2], h[3]});
        const bf16x8 al = __builtin_bit_cast(bf16x8, (u32x4){l[0], l[1], l[2], l[3]});
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bw, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bw, acc[t], 0, 0, 0);
      }
    }
  };
  // activations (and gains) first, weights last: the norm sums below wait
  // only for the activations
  load_x(0, xa, ga);
  __builtin_amdgcn_sched_barrier(0);
  load_w(0, wa);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    if (gi + 1 < NG) {
      if (gi % 2 == 0) { load_x(gi + 1, xb, gb); load_w(gi + 1, wb); }
      else { load_x(gi + 1, xa, ga); load_w(gi + 1, wa); }
    }
    if (gi % 2 == 0) process(wa, xa, ga);
    else process(wb, xb, gb);
  }
  // D(i, j) of a tile: lane j + 16 (i / 4), register i % 4
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    *(f32x4*)red[w][t][lane] = acc[t];
    if constexpr (NORM) {
      float q = ss[t];
      q += __shfl_xor(q, 16);
      q += __shfl_xor(q, 32);
      if (lk == 0) ssr[w][16 * t + li] = q;
    }
  }
  __syncthreads();
  if constexpr (NORM) {
    if (threadIdx.x < 16 * MT) {
      float t = ssr[0][threadIdx.x];
#pragma unroll
      for (int q = 1; q < KSW; ++q) t += ssr[q][threadIdx.x];
      inv_s[threadIdx.x] = 1.f / sqrtf(t / (float)K + p.eps);
    }
    __syncthreads();
  }
  // wave w < MT finishes m-tile w
  if (w >= MT) return;
  const int t = w;
  f32x4 v = *(const f32x4*)red[0][t][lane];
#pragma unroll
  for (int q = 1; q < KSW; ++q) v += *(const f32x4*)red[q][t][lane];
  float rs[4] = {1.f, 1.f, 1.f, 1.f};
  if constexpr (NORM) {
#pragma unroll
    for (int r = 0; r < 4; ++r) rs[r] = inv_s[16 * t + 4 * lk + r];
    if (p.norm_out && blockIdx.x == 0 && t == 0)
      for (int e = lane; e < M * (K / 4); e += 64) {
        const int row = e / (K / 4), k = (e % (K / 4)) * 4;
        if (row < M) {
          const f32x4 xv = *(const f32x4*)(p.X + (long)row * p.ldx + k), gv = *(const f32x4*)(p.gain + k);
          const float s = inv_s[row];
          *(f32x4*)(p.norm_out + (long)row * p.ld_norm + k) = (f32x4){xv.x * gv.x * s, xv.y * gv.y * s, xv.z * gv.z * s, xv.w * gv.w * s};
        }
      }
  }
  const int col = n0 + li;
  const float vv[4] = {v.x * rs[0], v.y * rs[1], v.z * rs[2], v.w * rs[3]};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 16 * t + 4 * lk + r;
    if (p.epi == EPI_SWIGLU) {
      const float up = __shfl_xor(vv[r], 1);   // (gate, up) rows 2c, 2c + 1 sit in lanes li, li ^ 1
      if (!(li & 1) && row < M && col + 1 < N) p.Y[(long)row * p.ldy + (col >> 1)] = vv[r] / (1.f + expf(-vv[r])) * up;
    } else if (row < M && col < N) {
      p.Y[(long)row * p.ldy + col] = p.epi == EPI_RESIDUAL ? yold[t][r] + vv[r] : vv[r];
    }
  }
}

template <int KSW, bool NORM, int MT>
static hipError_t launch_mfma_gemv_k(const LinearArgs& a, int ng, hipStream_t s) {
  const dim3 grid((a.N + 15) / 16), block(KSW * 64);
  switch (ng) {
    case 1: hipLaunchKernelGGL((mfma_gemv_kernel<KSW, 1, NORM, MT>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((mfma_gemv_kernel<KSW, 2, NORM, MT>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((mfma_gemv_kernel<KSW, 3, NORM, MT>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((mfma_gemv_kernel<KSW, 4, NORM, MT>), grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL((mfma_gemv_kernel<KSW, 6, NORM, MT>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// 3..32 activation rows of bf16 weights with K a multiple of 256 and at
// least 128 output tiles (narrower outputs stream better through the
// row-block kernel): 4 waves (2 or 1 for short K; at least MT).
static bool mfma_gemv_plan(const LinearArgs& a, int* ksw, int* ng) {
  if (a.wdtype != DT_BF16 || a.M < 3 || a.M > 32 || a.N < 2048 || a.K % 256 || a.ldx % 4 || a.defer)
    return false;
  const int mt = a.M <= 16 ? 1 : 2;
  const int groups = a.K / (256 / mt);          // groups of 8 / mt k-steps
  for (int k = 4; k >= mt; k /= 2)
    if (groups % k == 0) {
      const int g = groups / k;
      if (g == 1 || g == 2 || g == 3 || g == 4 || g == 6) { *ksw = k; *ng = g; return true; }
    }
  return false;
}

template <int MT>
static hipError_t launch_mfma_gemv_mt(const LinearArgs& a, int ksw, int ng, hipStream_t s) {
  if (ksw == 4) return a.gain ? launch_mfma_gemv_k<4, true, MT>(a, ng, s) : launch_mfma_gemv_k<4, false, MT>(a, ng, s);
  if constexpr (MT <= 2)
    if (ksw == 2) return a.gain ? launch_mfma_gemv_k<2, true, MT>(a, ng, s) : launch_mfma_gemv_k<2, false, MT>(a, ng, s);
  if constexpr (MT == 1) return a.gain ? launch_mfma_gemv_k<1, true, MT>(a, ng, s) : launch_mfma_gemv_k<1, false, MT>(a, ng, s);
  return hipErrorInvalidValue;
}

static hipError_t launch_mfma_gemv(const LinearArgs& a, int ksw, int ng, hipStream_t s) {
  if (a.M <= 16) return launch_mfma_gemv_mt<1>(a, ksw, ng, s);
  if (a.M <= 32) return launch_mfma_gemv_mt<2>(a, ksw, ng, s);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- 8-row matrix-core GEMV
// Projection of 3..8 activation rows on tiles of 8 weight rows. One
// v_mfma_f32_16x16x32_bf16 covers 64 k of the tile: A rows 0-7 are the
// activation rows on the first 32 k, rows 8-15 the same activation rows on the
// next 32 k, and B columns 0-7 / 8-15 the 8 weight rows on the same two k
// halves, so the two diagonal 8 x 8 blocks of the product are the tile's
// partial sums over the two halves (the off-diagonal blocks are discarded)
// and lane l's 16-byte weight load is row l % 8 at k offset 32 ((l / 8) % 2)
// + 8 (l / 16): eight lanes read 128 contiguous bytes of a row. Half-height
// tiles give twice the blocks of the 16-row GEMV, so wide outputs fill every
// compute unit evenly. Block = KSW waves over K, NS steps of 64 k per wave,
// every load issued before the first use (activations and gains, then
// weights); the waves' tiles and row sums of squares are added in LDS in wave
// order and RMSNorm is applied as a per-row scale after the contraction.
template <int KSW, int NS, bool NORM, int T>
__global__ __launch_bounds__(KSW * 64) void mfma_gemv8_kernel(LinearArgs p) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r8 = lane & 7, koff = 32 * ((lane >> 3) & 1) + 8 * (lane >> 4);
  const int nb = blockIdx.x * 8 * T;   // T tiles of 8 weight rows share the activation fragments
  const int M = p.M, N = p.N, K = p.K;
  const int kw0 = w * NS * 64 + koff;
  __shared__ __align__(16) float red[KSW][T][64][4];
  __shared__ float ssr[KSW][8];
  __shared__ float inv_s[8];
  const float* xr = p.X + (long)min(r8, M - 1) * p.ldx + kw0;
  const uint16_t* wr[T];
#pragma unroll
  for (int t = 0; t < T; ++t) wr[t] = (const uint16_t*)p.W + (long)min(nb + 8 * t + r8, N - 1) * K + kw0;
  f32x4 xv[NS][2], gv[NS][2];
  u32x4 wv[NS][T];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    xv[s][0] = *(const f32x4*)(xr + 64 * s);
    xv[s][1] = *(const f32x4*)(xr + 64 * s + 4);
  }
  if constexpr (NORM)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      gv[s][0] = *(const f32x4*)(p.gain + kw0 + 64 * s);
      gv[s][1] = *(const f32x4*)(p.gain + kw0 + 64 * s + 4);
    }
  // output (i, j) of this lane after the half combine: activation row 4 (lane / 16) + r, weight row lane % 16
  const bool owner = (lane & 15) < 8 && lane < 32;
  float yold[T][4] = {};
  if (p.epi == EPI_RESIDUAL && owner && w == 0)
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) yold[t][r] = p.Y[(long)min(4 * (lane >> 4) + r, M - 1) * p.ldy + min(nb + 8 * t + (lane & 15), N - 1)];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int t = 0; t < T; ++t) wv[s][t] = ld_weight(wr[t] + 64 * s);
  __builtin_amdgcn_sched_barrier(0);
  f32x4 acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    float x[8] = {xv[s][0].x, xv[s][0].y, xv[s][0].z, xv[s][0].w, xv[s][1].x, xv[s][1].y, xv[s][1].z, xv[s][1].w};
    if constexpr (NORM) {
      const float g[8] = {gv[s][0].x, gv[s][0].y, gv[s][0].z, gv[s][0].w, gv[s][1].x, gv[s][1].y, gv[s][1].z, gv[s][1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) { ss = fmaf(x[e], x[e], ss); x[e] *= g[e]; }
    }
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split_pk(x[2 * e], x[2 * e + 1], h[e], l[e]);
    const bf16x8 ah = __builtin_bit_cast(bf16x8, (u32x4){h[0], h[1], h[2], h[3]});
    const bf16x8 al = __builtin_bit_cast(bf16x8, (u32x4){l[0], l[1], l[2], l[3]});
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const bf16x8 bw = __builtin_bit_cast(bf16x8, wv[s][t]);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bw, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bw, acc[t], 0, 0, 0);
    }
  }
  // D(i, j): lane j + 16 (i / 4), register i % 4; block (i + 8, j + 8) sits 40 lanes up
#pragma unroll
  for (int t = 0; t < T; ++t) {
    f32x4 hi;
    hi.x = __shfl(acc[t].x, (lane + 40) & 63); hi.y = __shfl(acc[t].y, (lane + 40) & 63);
    hi.z = __shfl(acc[t].z, (lane + 40) & 63); hi.w = __shfl(acc[t].w, (lane + 40) & 63);
    *(f32x4*)red[w][t][lane] = acc[t] + hi;
  }
  if constexpr (NORM) {
    ss += __shfl_xor(ss, 8);
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    if (lane < 8) ssr[w][lane] = ss;
  }
  __syncthreads();
  if constexpr (NORM) {
    if (threadIdx.x < 8) {
      float t = ssr[0][threadIdx.x];
#pragma unroll
      for (int q = 1; q < KSW; ++q) t += ssr[q][threadIdx.x];
      inv_s[threadIdx.x] = 1.f / sqrtf(t / (float)K + p.eps);
    }
    __syncthreads();
  }
  if (w != 0) return;
  if constexpr (NORM)
    if (p.norm_out && blockIdx.x == 0)
      for (int e = lane; e < M * (K / 4); e += 64) {
        const int row = e / (K / 4), k = (e % (K / 4)) * 4;
        const f32x4 xx = *(const f32x4*)(p.X + (long)row * p.ldx + k), gg = *(const f32x4*)(p.gain + k);
        const float sc = inv_s[row];
        *(f32x4*)(p.norm_out + (long)row * p.ld_norm + k) = (f32x4){xx.x * gg.x * sc, xx.y * gg.y * sc, xx.z * gg.z * sc, xx.w * gg.w * sc};
      }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    f32x4 v = *(const f32x4*)red[0][t][lane];
#pragma unroll
    for (int q = 1; q < KSW; ++q) v += *(const f32x4*)red[q][t][lane];
    const int col = nb + 8 * t + (lane & 15);
    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * (lane >> 4) + r;
      float o = vv[r];
      if constexpr (NORM) o *= inv_s[row & 7];
      if (p.epi == EPI_SWIGLU) {
        const float up = __shfl_xor(o, 1);   // (gate, up) rows 2c, 2c + 1 sit in lanes 2c, 2c + 1
        if (owner && !(lane & 1) && row < M && col + 1 < N) p.Y[(long)row * p.ldy + (col >> 1)] = o / (1.f + expf(-o)) * up;
      } else if (owner && row < M && col < N) {
        p.Y[(long)row * p.ldy + col] = p.epi == EPI_RESIDUAL ? yold[t][r] + o : o;
      }
    }
  }
}

// 3..8 rows of bf16 weights, K a multiple of 64 KSW with at most 6 steps per
// wave: 4 waves per block, 8 when the grid has fewer than 256 blocks or K is
// long.
static bool mfma_gemv8_plan(const LinearArgs& a, int* ksw, int* ns, int* tiles) {
  if (a.wdtype != DT_BF16 || a.M < 3 || a.M > 8 || a.ldx % 4 || a.defer) return false;
  // tiles per block: as many as keep at least 256 blocks (1..3), sharing the activation fragments
  int T = 1;
  for (int t : {3, 2})
    if (t <= GEMV8_MAX_TILES && a.N % (8 * t) == 0 && a.N / (8 * t) >= 256) { T = t; break; }
  if (T == 1) {
    // a 16-row GEMV grid that is already a multiple of the 256 compute units stays (measured equal or better)
    int k16, g16;
    if (mfma_gemv_plan(a, &k16, &g16) && ((a.N + 15) / 16) % 256 == 0) return false;
  }
  for (int k : {4, 8}) {
    if (k == 4 && (a.N + 8 * T - 1) / (8 * T) < 256) continue;
    if (a.K % (64 * k)) continue;
    const int n = a.K / (64 * k);
    if (n >= 1 && n <= 6) { *ksw = k; *ns = n; *tiles = T; return true; }
  }
  return false;
}

template <int KSW, bool NORM, int T>
static hipError_t launch_mfma_gemv8_k(const LinearArgs& a, int ns, hipStream_t s) {
  const dim3 grid((a.N + 8 * T - 1) / (8 * T)), block(KSW * 64);
  switch (ns) {
    case 1: hipLaunchKernelGGL((mfma_gemv8_kernel<KSW, 1, NORM, T>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((mfma_gemv8_kernel<KSW, 2, NORM, T>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((mfma_gemv8_kernel<KSW, 3, NORM, T>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((mfma_gemv8_kernel<KSW, 4, NORM, T>), grid, block, 0, s, a); break;
    case 5: hipLaunchKernelGGL((mfma_gemv8_kernel<KSW, 5, NORM, T>), grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL((mfma_gemv8_kernel<KSW, 6, NORM, T>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int T>
static hipError_t launch_mfma_gemv8_t(const LinearArgs& a, int ksw, int ns, hipStream_t s) {
  if (ksw == 4) return a.gain ? launch_mfma_gemv8_k<4, true, T>(a, ns, s) : launch_mfma_gemv8_k<4, false, T>(a, ns, s);
  return a.gain ? launch_mfma_gemv8_k<8, true, T>(a, ns, s) : launch_mfma_gemv8_k<8, false, T>(a, ns, s);
}

static hipError_t launch_mfma_gemv8(const LinearArgs& a, int ksw, int ns, int tiles, hipStream_t s) {
  if (tiles == 3) return launch_mfma_gemv8_t<3>(a, ksw, ns, s);
  if (tiles == 2) return launch_mfma_gemv8_t<2>(a, ksw, ns, s);
  return launch_mfma_gemv8_t<1>(a, ksw, ns, s);
}

hipError_t launch_linear(const LinearArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  // one or two rows: register GEMV, the weights streamed once with fp32 FMA
  {
    hipError_t e = hipSuccess;
    if (a.wdtype == DT_BF16 ? try_gemv<uint16_t>(a, s, &e) : try_gemv<float>(a, s, &e)) return e;
  }
  // a few more rows of bf16 weights: matrix-core GEMV (wide outputs), else
  // the row-block weight-streaming MFMA kernel
  {
    int ksw, ng;
    int t8;
    if (mfma_gemv8_plan(a, &ksw, &ng, &t8)) return launch_mfma_gemv8(a, ksw, ng, t8, s);
    if (mfma_gemv_plan(a, &ksw, &ng)) return launch_mfma_gemv(a, ksw, ng, s);
  }
  if (skinny_fits(a)) return launch_skinny(a, s);
  // up to 128 rows: row-block MFMA GEMM
  {
    RowsPlan pl;
    if (rows_plan(a, &pl)) return launch_rows(a, pl, s);
  }
  // many rows of bf16 weights: matrix-core GEMM (needs K % 32 == 0 and row scratch)
  if (a.M >= MFMA_MIN_ROWS && gemm_split_fits(a)) return launch_gemm_split(a, s);
  if (a.wdtype == DT_BF16 && a.M >= MFMA_MIN_ROWS && a.K % GK == 0 && a.row_den)
    return launch_mfma(a, a.row_den, s);
  // activation tile: as many rows as fit in 96 KB of LDS, up to 8
  int mtmax = 8;
  while (mtmax > 1 && (size_t)mtmax * a.K * 4 > 96 * 1024) mtmax >>= 1;
  int mt = 1;
  while (mt < a.M && mt < mtmax) mt <<= 1;
  const int R = (a.epi == EPI_SWIGLU || a.N >= 4096) ? 2 : 1;
  const int KS = (a.N / (4 * R) < 512 && a.K >= 1024) ? 4 : 1;
  if (a.wdtype == DT_BF16) return launch_linear_w<uint16_t>(a, mt, R, KS, s);
  return launch_linear_w<float>(a, mt, R, KS, s);
}

// ---------------------------------------------------------------- attention
// One block per (kv head g, run of tokens of one row); D = head_dim and
// G = q heads per kv head are compile-time, so every per-head array lives in
// registers. For each token: RMSNorm of k and of the G q heads over head_dim,
// rotate-half rope at the token's position, K/V row write into the cache,
// then causal attention of the G q heads over positions 0..pos in chunks of NT
// keys with an online softmax. Scores: one key per thread, its row read with
// 16-byte loads, q broadcast from LDS. P·V: one wave per 64-key slice, each
// lane owning D/64 adjacent elements of every V row (one vector load per row),
// partial outputs combined across the 4 waves in LDS.
// Modes: ATT_WRITE_ATTEND (decode / predictor: per token write, then attend),
// ATT_WRITE (prefill pass 1: K/V rows only), ATT_ATTEND (prefill pass 2: the
// cache already holds every key).
template <int G>
__device__ __forceinline__ void block_reduce_g(float (&v)[G], float* red, bool is_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int hh = 0; hh < G; ++hh) v[hh] = is_max ? wave_max(v[hh]) : wave_sum(v[hh]);
  __syncthreads();
  if (lane == 0)
#pragma unroll
    for (int hh = 0; hh < G; ++hh) red[wave * G + hh] = v[hh];
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float t = red[hh];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) t = is_max ? fmaxf(t, red[w * G + hh]) : t + red[w * G + hh];
    v[hh] = t;
  }
}

// the value a cache element holds after being stored
template <typename KVT> __device__ __forceinline__ float kv_round(float x);
template <> __device__ __forceinline__ float kv_round<float>(float x) { return x; }
template <> __device__ __forceinline__ float kv_round<uint16_t>(float x) { return bf16_to_f32(f32_to_bf16(x)); }
template <> __device__ __forceinline__ float kv_round<_Float16>(float x) { return (float)(_Float16)x; }

// 16-byte chunk of a cache row -> floats
template <typename KVT>
__device__ __forceinline__ void unpack_chunk(const u32x4& w, float* x) {
  if constexpr (std::is_same<KVT, _Float16>::value) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const h8 h = __builtin_bit_cast(h8, w);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)h[e];
  } else if constexpr (sizeof(KVT) == 2) {
    x[0] = bf_lo(w.x); x[1] = bf_hi(w.x); x[2] = bf_lo(w.y); x[3] = bf_hi(w.y);
    x[4] = bf_lo(w.z); x[5] = bf_hi(w.z); x[6] = bf_lo(w.w); x[7] = bf_hi(w.w);
  } else {
    x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
  }
}

template <typename KVT, int D, int G>
__global__ __launch_bounds__(NT) void attn_kernel(AttnArgs p) {
  constexpr int HALF = D / 2;
  constexpr int EPN = (D + 63) / 64;       // elements per lane in the RMSNorm step (strided by 64)
  constexpr int EPC = 16 / sizeof(KVT);    // cache elements per 16-byte chunk
  constexpr int CPK = D / EPC;             // chunks per cache row
  constexpr int TPK = CPK < 4 ? CPK : 4;   // threads per key in the score step
  constexpr int CPT = CPK / TPK;           // chunks per thread in the score step
  constexpr int KCH = NT / TPK;            // keys per chunk of the online softmax
  constexpr int KPP = NT / CPK;            // keys per pass of the P·V product
  constexpr int NPV = KCH / KPP;           // P·V passes per chunk (V chunks per thread)
  static_assert(CPK <= 64 && 64 % CPK == 0 && KCH % KPP == 0, "cache row layout");
  const int g = blockIdx.x;
  const Run rn = p.runs[blockIdx.y];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pos0 = rn.pos0 + p.pos_base + (p.row_pos ? p.row_pos[rn.row] : 0);
  const bool write = p.mode != ATT_ATTEND, attend = p.mode != ATT_WRITE;
  extern __shared__ float sm[];
  float* raw = sm;                      // [G + 1][D] normalised q heads, then k
  float* qs = raw + (G + 1) * D;        // [G][D] rotated q heads
  float* pl = qs + G * D;               // [G][KCH] probabilities of the chunk
  float* part = pl + G * KCH;           // [4][G][D] per-wave partial outputs
  float* red = part + 4 * G * D;        // [2][4][G]
  KVT* kc = (KVT*)p.kc + (long)rn.row * p.row_stride + (long)g * p.max_pos * D;
  KVT* vc = (KVT*)p.vc + (long)rn.row * p.row_stride + (long)g * p.max_pos * D;
  const int ksub = tid % TPK, kkey = tid / TPK;       // score role: (key of the chunk, row part)
  const int vchunk = tid % CPK, vslot = tid / CPK;    // P·V role: (key slot, 16-byte chunk)

  for (int i = 0; i < rn.ntok; ++i) {
    const long t = rn.tok0 + i;
    const int pos = pos0 + i;
    const float* src = p.qkv + t * p.ld_qkv;
    // (a) RMSNorm over head_dim: vector v (< G: q head, == G: k) on wave v % 4
    for (int v = wave; v <= G; v += NT / 64) {
      if ((v < G && !attend) || (v == G && !write)) continue;
      const float* x = src + (v < G ? (long)(g * G + v) * D : (long)p.nq * D + (long)g * D);
      const float* gain = v < G ? p.q_gain : p.k_gain;
      float vals[EPN], gv[EPN];
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < EPN; ++c) {
        const int e = lane + 64 * c;
        vals[c] = e < D ? x[e] : 0.f;
        gv[c] = e < D ? gain[e] : 0.f;
        ss += vals[c] * vals[c];
      }
      ss = wave_sum(ss);
      const float den = sqrtf(ss / (float)D + p.eps);
#pragma unroll
      for (int c = 0; c < EPN; ++c) {
        const int e = lane + 64 * c;
        if (e < D) raw[v * D + e] = vals[c] / den * gv[c];
      }
    }
    if (write)
      for (int e = tid; e < D; e += NT)
        st_elem<KVT>(vc, (long)pos * D + e, src[(long)(p.nq + p.nkv) * D + (long)g * D + e]);
    __syncthreads();
    // (b) rope of the q heads and of k; the k row goes to the cache
    for (int e = tid; e < (G + 1) * HALF; e += NT) {
      const int v = e / HALF, j = e % HALF;
      if ((v < G && !attend) || (v == G && !write)) continue;
      const float c = p.cos[(long)pos * HALF + j], s = p.sin[(long)pos * HALF + j];
      const float x1 = raw[v * D + j], x2 = raw[v * D + j + HALF];
      const float o1 = x1 * c - x2 * s, o2 = x2 * c + x1 * s;
      if (v < G) {
        qs[v * D + j] = o1;
        qs[v * D + j + HALF] = o2;
      } else {
        st_elem<KVT>(kc, (long)pos * D + j, o1);
        st_elem<KVT>(kc, (long)pos * D + j + HALF, o2);
      }
    }
    // Rows written above are read back below by other threads of this block.
    // Their cache lines were not read earlier in this kernel, except by the
    // earlier tokens of a multi-token run, which the fence covers.
    if (write && attend && rn.ntok > 1) __threadfence();
    __syncthreads();
    if (!attend) continue;

    // (c) attention over positions 0..pos in chunks of KCH keys. Loads are
    // unconditional (rows past the end are clamped to the last valid one and
    // weighted 0) so each thread's K and V chunks go out in one batch.
    const int L = pos + 1;
    float m[G], l[G], acc[G][EPC];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      m[hh] = -INFINITY;
      l[hh] = 0.f;
#pragma unroll
      for (int c = 0; c < EPC; ++c) acc[hh][c] = 0.f;
    }
    u32x4 kv[CPT], vv[NPV];
    auto load_chunk = [&](int c0, u32x4 (&kd)[CPT], u32x4 (&vd)[NPV]) {
      const int cn = min(KCH, L - c0);
      const int jk = c0 + min(kkey, cn - 1);
#pragma unroll
      for (int c = 0; c < CPT; ++c) kd[c] = *(const u32x4*)(kc + (long)jk * D + (ksub * CPT + c) * EPC);
#pragma unroll
      for (int b = 0; b < NPV; ++b) {
        const int jv = c0 + min(vslot + b * KPP, cn - 1);
        vd[b] = *(const u32x4*)(vc + (long)jv * D + vchunk * EPC);
      }
    };
    load_chunk(0, kv, vv);
    for (int c0 = 0; c0 < L; c0 += KCH) {
      const int cn = min(KCH, L - c0);
      float sc[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) sc[hh] = 0.f;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        float x[EPC];
        unpack_chunk<KVT>(kv[c], x);
        const int e0 = (ksub * CPT + c) * EPC;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const f32x4* q4 = (const f32x4*)(qs + hh * D + e0);
#pragma unroll
          for (int e = 0; e < EPC; e += 4) {
            const f32x4 q = q4[e / 4];
            sc[hh] = fmaf(q.x, x[e], sc[hh]);
            sc[hh] = fmaf(q.y, x[e + 1], sc[hh]);
            sc[hh] = fmaf(q.z, x[e + 2], sc[hh]);
            sc[hh] = fmaf(q.w, x[e + 3], sc[hh]);
          }
        }
      }
      const bool kvalid = kkey < cn;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
#pragma unroll
        for (int o = 1; o < TPK; o <<= 1) sc[hh] += __shfl_xor(sc[hh], o);
        sc[hh] = kvalid ? sc[hh] * p.scale : -INFINITY;
      }
      // the next chunk's rows go in flight behind this chunk's softmax and P·V
      u32x4 vn[NPV];
      const bool more = c0 + KCH < L;
      if (more) load_chunk(c0 + KCH, kv, vn);
      float mx[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) mx[hh] = sc[hh];
      block_reduce_g<G>(mx, red, true);
      float ps[G], corr[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float mnew = fmaxf(m[hh], mx[hh]);
        corr[hh] = expf(m[hh] - mnew);
        m[hh] = mnew;
        const float e = kvalid ? expf(sc[hh] - mnew) : 0.f;
        if (ksub == 0) pl[hh * KCH + kkey] = e;
        ps[hh] = ksub == 0 ? e : 0.f;
      }
      block_reduce_g<G>(ps, red + 4 * G, false);   // its barriers also publish pl
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        l[hh] = l[hh] * corr[hh] + ps[hh];
#pragma unroll
        for (int c = 0; c < EPC; ++c) acc[hh][c] *= corr[hh];
      }
#pragma unroll
      for (int b = 0; b < NPV; ++b) {
        const int jl = vslot + b * KPP;          // pl is 0 for jl >= cn
        float x[EPC];
        unpack_chunk<KVT>(vv[b], x);
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float pw = pl[hh * KCH + jl];
#pragma unroll
          for (int c = 0; c < EPC; ++c) acc[hh][c] = fmaf(pw, x[c], acc[hh][c]);
        }
      }
      if (more)
#pragma unroll
        for (int b = 0; b < NPV; ++b) vv[b] = vn[b];
      __syncthreads();   // pl is rewritten by the next chunk
    }
    // sum the key slots: lanes CPK apart inside a wave, then the 4 waves in LDS
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int c = 0; c < EPC; ++c) {
        float s = acc[hh][c];
        for (int o = CPK; o < 64; o <<= 1) s += __shfl_xor(s, o);
        acc[hh][c] = s;
      }
    if (lane < CPK)
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int c = 0; c < EPC; ++c) part[(wave * G + hh) * D + vchunk * EPC + c] = acc[hh][c];
    __syncthreads();
    for (int e = tid; e < G * D; e += NT) {
      const int hh = e / D, dim = e % D;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NT / 64; ++w) s += part[(w * G + hh) * D + dim];
      p.out[t * p.ld_out + (long)(g * G + hh) * D + dim] = s / l[hh];
    }
    __syncthreads();
  }
}

// Single-token decode (the talker step and predictor steps 1..14): every
// load is issued at kernel start (this token's q/k/v, gains, cos/sin, and the
// first chunk of older K/V rows), and this token's own K/V stay in LDS instead
// of being read back from the cache. Older rows come only from positions
// < pos, which earlier kernels wrote.
template <typename KVT, int D, int G>
__global__ __launch_bounds__(NT) void attn_decode_kernel(AttnArgs p) {
  constexpr int HALF = D / 2;
  constexpr int EPN = (D + 63) / 64;
  constexpr int EPC = 16 / sizeof(KVT);
  constexpr int CPK = D / EPC;
  constexpr int TPK = CPK < 4 ? CPK : 4;
  constexpr int CPT = CPK / TPK;
  constexpr int KCH = NT / TPK;
  constexpr int KPP = NT / CPK;
  constexpr int NPV = KCH / KPP;
  static_assert(CPK <= 64 && 64 % CPK == 0 && KCH % KPP == 0, "cache row layout");
  const int g = blockIdx.x;
  const int row = blockIdx.y;          // batch row (cache row)
  // activation row of its token: the row itself, or row * tok_stride + tok_off
  const long arow = p.tok_stride > 0 ? (long)row * p.tok_stride + p.tok_off : row;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pos = p.pos_base + (p.row_pos ? p.row_pos[row] : 0);
  const int L = pos + 1;
  extern __shared__ float sm[];
  float* raw = sm;                      // [G + 1][D]
  float* qs = raw + (G + 1) * D;        // [G][D]
  float* kcur = qs + G * D;             // [D] this token's key, as stored
  float* vcur = kcur + D;               // [D] this token's value, as stored
  float* pl = vcur + D;                 // [G][KCH]
  float* part = pl + G * KCH;           // [4][G][D]
  float* red = part + 4 * G * D;        // [2][4][G]
  KVT* kc = (KVT*)p.kc + (long)row * p.row_stride + (long)g * p.max_pos * D;
  KVT* vc = (KVT*)p.vc + (long)row * p.row_stride + (long)g * p.max_pos * D;
  const int ksub = tid % TPK, kkey = tid / TPK;
  const int vchunk = tid % CPK, vslot = tid / CPK;
  const float* src = p.qkv + arow * p.ld_qkv;
  const int lastrow = p.max_pos - 1;
  // q/k/v value at column col of this token's projection row: the stored row,
  // or the sum of the split-K partials (ranges in order) times 1 / rms
  float prs = 1.f;
  if (p.part_z > 0) {
    const float* pss = p.part + (long)p.part_z * p.part_rows * p.ld_qkv;
    float ssum = pss[arow];
    for (int z = 1; z < p.part_z; ++z) ssum += pss[(long)z * p.part_rows + arow];
    prs = 1.f / sqrtf(ssum / (float)p.part_k + p.part_eps);
  }
  auto qkv_at = [&](long col) -> float {
    if (p.part_z <= 0) return src[col];
    float v = p.part[arow * p.ld_qkv + col];
    for (int z = 1; z < p.part_z; ++z) v += p.part[((long)z * p.part_rows + arow) * p.ld_qkv + col];
    return v * prs;
  };

  // Row addresses do not depend on pos (only clamped to the cache), so these
  // loads leave together with this token's loads; rows >= pos may hold
  // anything and are kept out of the sums by the key guards below.
  u32x4 kv[CPT], vv[NPV];
  auto load_chunk = [&](int c0, u32x4 (&kd)[CPT], u32x4 (&vd)[NPV]) {
    const int jk = min(c0 + kkey, lastrow);
#pragma unroll
    for (int c = 0; c < CPT; ++c) kd[c] = *(const u32x4*)(kc + (long)jk * D + (ksub * CPT + c) * EPC);
#pragma unroll
    for (int b = 0; b < NPV; ++b) {
      const int jv = min(c0 + vslot + b * KPP, lastrow);
      vd[b] = *(const u32x4*)(vc + (long)jv * D + vchunk * EPC);
    }
  };
  load_chunk(0, kv, vv);
  // cos/sin of this thread's rope pairs: from the per-row rows prepared for
  // this step (no dependence on pos) or from the table
  constexpr int RPT = ((G + 1) * HALF + NT - 1) / NT;
  float cs_t[RPT], sn_t[RPT];
#pragma unroll
  for (int q = 0; q < RPT; ++q) {
    const int e = tid + q * NT;
    const int j = e % HALF;
    if (p.rope_rows) {
      cs_t[q] = p.rope_rows[(long)row * D + j];
      sn_t[q] = p.rope_rows[(long)row * D + HALF + j];
    } else {
      cs_t[q] = p.cos[(long)pos * HALF + j];
      sn_t[q] = p.sin[(long)pos * HALF + j];
    }
  }

  // this token: RMSNorm of the q heads and k (vector v on wave v % 4), v as stored
  for (int v = wave; v <= G; v += NT / 64) {
    const float* x = src + (v < G ? (long)(g * G + v) * D : (long)p.nq * D + (long)g * D);
    const float* gain = v < G ? p.q_gain : p.k_gain;
    float vals[EPN], gv[EPN];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < EPN; ++c) {
      const int e = lane + 64 * c;
      vals[c] = e < D ? qkv_at((x - src) + e) : 0.f;
      gv[c] = e < D ? gain[e] : 0.f;
      ss += vals[c] * vals[c];
    }
    ss = wave_sum(ss);
    const float den = sqrtf(ss / (float)D + p.eps);
#pragma unroll
    for (int c = 0; c < EPN; ++c) {
      const int e = lane + 64 * c;
      if (e < D) raw[v * D + e] = vals[c] / den * gv[c];
    }
  }
  for (int e = tid; e < D; e += NT) {
    const float vvv = qkv_at((long)(p.nq + p.nkv) * D + (long)g * D + e);
    st_elem<KVT>(vc, (long)pos * D + e, vvv);
    vcur[e] = kv_round<KVT>(vvv);
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < RPT; ++q) {
    const int e = tid + q * NT;
    if (e >= (G + 1) * HALF) break;
    const int v = e / HALF, j = e % HALF;
    const float c = cs_t[q], s = sn_t[q];
    const float x1 = raw[v * D + j], x2 = raw[v * D + j + HALF];
    const float o1 = x1 * c - x2 * s, o2 = x2 * c + x1 * s;
    if (v < G) {
      qs[v * D + j] = o1;
      qs[v * D + j + HALF] = o2;
    } else {
      st_elem<KVT>(kc, (long)pos * D + j, o1);
      st_elem<KVT>(kc, (long)pos * D + j + HALF, o2);
      kcur[j] = kv_round<KVT>(o1);
      kcur[j + HALF] = kv_round<KVT>(o2);
    }
  }
  __syncthreads();

  float m[G], l[G], acc[G][EPC];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int c = 0; c < EPC; ++c) acc[hh][c] = 0.f;
  }
  for (int c0 = 0; c0 < L; c0 += KCH) {
    const int cn = min(KCH, L - c0);
    const int j = c0 + kkey;
    float sc[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) sc[hh] = 0.f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      float x[EPC];
      const int e0 = (ksub * CPT + c) * EPC;
      if (j == pos) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) x[e] = kcur[e0 + e];
      } else {
        unpack_chunk<KVT>(kv[c], x);
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const f32x4* q4 = (const f32x4*)(qs + hh * D + e0);
#pragma unroll
        for (int e = 0; e < EPC; e += 4) {
          const f32x4 q = q4[e / 4];
          sc[hh] = fmaf(q.x, x[e], sc[hh]);
          sc[hh] = fmaf(q.y, x[e + 1], sc[hh]);
          sc[hh] = fmaf(q.z, x[e + 2], sc[hh]);
          sc[hh] = fmaf(q.w, x[e + 3], sc[hh]);
        }
      }
    }
    const bool kvalid = kkey < cn;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
#pragma unroll
      for (int o = 1; o < TPK; o <<= 1) sc[hh] += __shfl_xor(sc[hh], o);
      sc[hh] = kvalid ? sc[hh] * p.scale : -INFINITY;
    }
    u32x4 vn[NPV];
    const bool more = c0 + KCH < L;
    if (more) load_chunk(c0 + KCH, kv, vn);
    float mx[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) mx[hh] = sc[hh];
    block_reduce_g<G>(mx, red, true);
    float ps[G], corr[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float mnew = fmaxf(m[hh], mx[hh]);
      corr[hh] = expf(m[hh] - mnew);
      m[hh] = mnew;
      const float e = kvalid ? expf(sc[hh] - mnew) : 0.f;
      if (ksub == 0) pl[hh * KCH + kkey] = e;
      ps[hh] = ksub == 0 ? e : 0.f;
    }
    block_reduce_g<G>(ps, red + 4 * G, false);
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      l[hh] = l[hh] * corr[hh] + ps[hh];
#pragma unroll
      for (int c = 0; c < EPC; ++c) acc[hh][c] *= corr[hh];
    }
#pragma unroll
    for (int b = 0; b < NPV; ++b) {
      const int jl = vslot + b * KPP;
      if (jl < cn) {                 // rows past pos are never multiplied in
        float x[EPC];
        if (c0 + jl == pos) {
#pragma unroll
          for (int e = 0; e < EPC; ++e) x[e] = vcur[vchunk * EPC + e];
        } else {
          unpack_chunk<KVT>(vv[b], x);
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float pw = pl[hh * KCH + jl];
#pragma unroll
          for (int c = 0; c < EPC; ++c) acc[hh][c] = fmaf(pw, x[c], acc[hh][c]);
        }
      }
    }
    if (more)
#pragma unroll
      for (int b = 0; b < NPV; ++b) vv[b] = vn[b];
    __syncthreads();
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int c = 0; c < EPC; ++c) {
      float s = acc[hh][c];
      for (int o = CPK; o < 64; o <<= 1) s += __shfl_xor(s, o);
      acc[hh][c] = s;
    }
  if (lane < CPK)
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int c = 0; c < EPC; ++c) part[(wave * G + hh) * D + vchunk * EPC + c] = acc[hh][c];
  __syncthreads();
  for (int e = tid; e < G * D; e += NT) {
    const int hh = e / D, dim = e % D;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) s += part[(w * G + hh) * D + dim];
    p.out[arow * p.ld_out + (long)(g * G + hh) * D + dim] = s / l[hh];
  }
}

// Decode attention for head_dim 128, one kernel launch for the NTOK new
// tokens of every row (NTOK = 1: a talker or predictor step; NTOK = 2: the
// predictor's two-token pass at positions 0 and 1). Block = (kv head, row).
// Keys older than the first new token come from the cache in chunks of KCH
// rows (large chunks when the grid is a single wave of blocks, small ones,
// with fewer registers, when several blocks share a compute unit) whose
// loads all leave at once (4 threads per key for the scores,
// (16-byte column, key slot) threads for P·V); the new tokens' own keys and
// values stay in LDS. Each thread keeps its own running softmax sums, so a
// chunk costs one block-wide max exchange; slots, waves and the sums are
// combined once at the end.
template <typename KVT, int G, int NTOK, int KCH, bool SPLIT = false>
__global__ __launch_bounds__(NT) void attn_step_kernel(AttnArgs p) {
  constexpr int D = 128, HALF = 64;
  constexpr int EPC = 16 / sizeof(KVT);      // cache elements per 16-byte chunk
  constexpr int CPK = D / EPC;               // chunks per cache row
  constexpr int TPK = 4;                     // threads per key (scores)
  constexpr int CPT = CPK / TPK;             // chunks per thread (scores)
  constexpr int KPR = NT / TPK;              // keys per score row
  constexpr int SR = KCH / KPR;              // keys per thread (scores)
  constexpr int VS = NT / CPK;               // key slots (P·V)
  constexpr int NV = KCH / VS;               // keys per thread (P·V)
  static_assert(KCH % KPR == 0 && KCH % VS == 0 && CPK <= 64, "layout");
  const int g = blockIdx.x;
  const int row = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ksub = tid % TPK, kkey = tid / TPK;
  const int vchunk = tid % CPK, vslot = tid / CPK;
  __shared__ __align__(16) float qs[NTOK][G][D];   // normalised, rotated q heads
  __shared__ float knew[NTOK][D], vnew[NTOK][D];   // the new rows, as stored
  __shared__ float pl[G][KCH];               // probabilities of the chunk
  __shared__ float part[NT / 64][G][D];
  __shared__ float red[2][NT / 64][G];
  KVT* kc = (KVT*)p.kc + (long)row * p.row_stride + (long)g * p.max_pos * D;
  KVT* vc = (KVT*)p.vc + (long)row * p.row_stride + (long)g * p.max_pos * D;

  // Only keys older than the new tokens come from the cache (rows < pos0);
  // groups of keys past them are neither loaded nor computed (the group
  // tests are uniform across the block).
  const int pos0 = p.pos_base + (p.row_pos ? p.row_pos[row] : 0);
  // SPLIT: this block's keys are [kb, ke) of the cached keys, the last range
  // also the new ones (a range is a whole number of chunks; ranges past the
  // cached keys are empty)
  int kb = 0, ke_cached = pos0;
  bool owns_new = true;
  if constexpr (SPLIT) {
    static_assert(NTOK == 1, "split ranges serve single-token decode");
    const int S = gridDim.z, sp = blockIdx.z;
    const int per = ((pos0 + S - 1) / S + KCH - 1) / KCH * KCH;
    kb = min(sp * per, pos0);
    ke_cached = min(kb + per, pos0);
    owns_new = sp == S - 1;
  }
  u32x4 kr[SR][CPT], vr[NV];
  auto load_k = [&](int c0) {
#pragma unroll
    for (int r = 0; r < SR; ++r) {
      if (c0 + r * KPR >= ke_cached) break;
      const int j = min(c0 + kkey + r * KPR, pos0 - 1);
#pragma unroll
      for (int c = 0; c < CPT; ++c) kr[r][c] = *(const u32x4*)(kc + (long)j * D + (ksub * CPT + c) * EPC);
    }
  };
  auto load_v = [&](int c0) {
#pragma unroll
    for (int b = 0; b < NV; ++b) {
      if (c0 + b * VS >= ke_cached) break;
      const int j = min(c0 + vslot + b * VS, pos0 - 1);
      vr[b] = *(const u32x4*)(vc + (long)j * D + vchunk * EPC);
    }
  };
  load_k(kb);
  load_v(kb);

  // the new tokens: QK-RMSNorm + rope of q heads and k (one wave per vector;
  // lane owns the rope pair (lane, lane + 64)), K/V rows to the cache and LDS
  float prs[NTOK];
  const long arow0 = p.tok_stride > 0 ? (long)row * p.tok_stride + p.tok_off : row;
  // split-K partial sums: up to PZ ranges with every load issued before the
  // first add (clamped ranges past part_z are loaded but not added)
  constexpr int PZ = 8;
  const bool pz_fast = p.part_z <= PZ;
#pragma unroll
  for (int t = 0; t < NTOK; ++t) {
    prs[t] = 1.f;
    if (p.part_z > 0) {
      const float* pss = p.part + (long)p.part_z * p.part_rows * p.ld_qkv;
      float ssum = 0.f;
      if (pz_fast) {
        float q[PZ];
#pragma unroll
        for (int z = 0; z < PZ; ++z) q[z] = pss[(long)min(z, p.part_z - 1) * p.part_rows + arow0 + t];
#pragma unroll
        for (int z = 0; z < PZ; ++z) if (z < p.part_z) ssum += q[z];
      } else {
        for (int z = 0; z < p.part_z; ++z) ssum += pss[(long)z * p.part_rows + arow0 + t];
      }
      prs[t] = 1.f / sqrtf(ssum / (float)p.part_k + p.part_eps);
    }
  }
  auto qkv_at = [&](int t, long col) -> float {
    const long ar = arow0 + t;
    if (p.part_z <= 0) return p.qkv[ar * p.ld_qkv + col];
    float v;
    if (pz_fast) {
      float q[PZ];
#pragma unroll
      for (int z = 0; z < PZ; ++z) q[z] = p.part[((long)min(z, p.part_z - 1) * p.part_rows + ar) * p.ld_qkv + col];
      v = q[0];
#pragma unroll
      for (int z = 1; z < PZ; ++z) if (z < p.part_z) v += q[z];
    } else {
      v = p.part[ar * p.ld_qkv + col];
      for (int z = 1; z < p.part_z; ++z) v += p.part[((long)z * p.part_rows + ar) * p.ld_qkv + col];
    }
    return v * prs[t];
  };
#pragma unroll
  for (int t = 0; t < NTOK; ++t) {
    const int pos = pos0 + t;
    float cs, sn;
    if (p.rope_rows) {
      cs = p.rope_rows[(long)row * D + lane];
      sn = p.rope_rows[(long)row * D + HALF + lane];
    } else {
      cs = p.cos[(long)pos * HALF + lane];
      sn = p.sin[(long)pos * HALF + lane];
    }
    if (!owns_new)   // masked keys past this range may index the new rows: keep them finite (0 x NaN is NaN)
      for (int i = tid; i < D; i += NT) { knew[t][i] = 0.f; vnew[t][i] = 0.f; }
    for (int v = wave; v <= (owns_new ? G + 1 : G - 1); v += NT / 64) {
      if (v == G + 1) {                       // value row, stored as is
        const long col = (long)(p.nq + p.nkv) * D + (long)g * D;
        const float x1 = qkv_at(t, col + lane), x2 = qkv_at(t, col + lane + HALF);
        st_elem<KVT>(vc, (long)pos * D + lane, x1);
        st_elem<KVT>(vc, (long)pos * D + lane + HALF, x2);
        vnew[t][lane] = kv_round<KVT>(x1);
        vnew[t][lane + HALF] = kv_round<KVT>(x2);
        continue;
      }
      const long col = v < G ? (long)(g * G + v) * D : (long)p.nq * D + (long)g * D;
      const float* gain = v < G ? p.q_gain : p.k_gain;
      const float x1 = qkv_at(t, col + lane), x2 = qkv_at(t, col + lane + HALF);
      const float g1 = gain[lane], g2 = gain[lane + HALF];
      const float ss = wave_sum(x1 * x1 + x2 * x2);
      const float rden = 1.f / sqrtf(ss / (float)D + p.eps);
      const float y1 = x1 * rden * g1, y2 = x2 * rden * g2;
      const float o1 = y1 * cs - y2 * sn, o2 = y2 * cs + y1 * sn;
      if (v < G) {
        qs[t][v][lane] = o1;
        qs[t][v][lane + HALF] = o2;
      } else {
        st_elem<KVT>(kc, (long)pos * D + lane, o1);
        st_elem<KVT>(kc, (long)pos * D + lane + HALF, o2);
        knew[t][lane] = kv_round<KVT>(o1);
        knew[t][lane + HALF] = kv_round<KVT>(o2);
      }
    }
  }
  __syncthreads();

#pragma unroll
  for (int t = 0; t < NTOK; ++t) {
    const int L = owns_new ? pos0 + t + 1 : ke_cached;   // keys kb .. L - 1 (0 .. pos0 + t unsplit)
    float m[G], l[G], acc[G][EPC];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      m[hh] = -INFINITY;
      l[hh] = 0.f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[hh][e] = 0.f;
    }
    if (t > 0 && pos0 > KCH) { load_k(0); load_v(0); }   // the registers hold the previous token's last chunk
    for (int c0 = kb; c0 < L; c0 += KCH) {
      float s[SR][G];
#pragma unroll
      for (int r = 0; r < SR; ++r) {
        const int j = c0 + kkey + r * KPR;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) s[r][hh] = -INFINITY;
        if (c0 + r * KPR >= L) continue;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) s[r][hh] = 0.f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          const int e0 = (ksub * CPT + c) * EPC;
          float x[EPC];
          if (j >= pos0) {
            const int jn = min(j - pos0, NTOK - 1);
#pragma unroll
            for (int e = 0; e < EPC; ++e) x[e] = knew[jn][e0 + e];
          } else {
            unpack_chunk<KVT>(kr[r][c], x);
          }
#pragma unroll
          for (int hh = 0; hh < G; ++hh) {
            const f32x4* q4 = (const f32x4*)(&qs[t][hh][e0]);
#pragma unroll
            for (int e = 0; e < EPC; e += 4) {
              const f32x4 q = q4[e / 4];
              s[r][hh] = fmaf(q.x, x[e], s[r][hh]);
              s[r][hh] = fmaf(q.y, x[e + 1], s[r][hh]);
              s[r][hh] = fmaf(q.z, x[e + 2], s[r][hh]);
              s[r][hh] = fmaf(q.w, x[e + 3], s[r][hh]);
            }
          }
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          s[r][hh] += __shfl_xor(s[r][hh], 1);
          s[r][hh] += __shfl_xor(s[r][hh], 2);
          s[r][hh] = j < L ? s[r][hh] * p.scale : -INFINITY;
        }
      }
      const bool more = c0 + KCH < L;
      if (more) load_k(c0 + KCH);              // next chunk's keys, behind this chunk's softmax
      float mx[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float v = s[0][hh];
#pragma unroll
        for (int r = 1; r < SR; ++r) v = fmaxf(v, s[r][hh]);
        mx[hh] = wave_max(v);
      }
      if (lane == 0)
#pragma unroll
        for (int hh = 0; hh < G; ++hh) red[0][wave][hh] = mx[hh];
      __syncthreads();
      float corr[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float v = red[0][0][hh];
#pragma unroll
        for (int w = 1; w < NT / 64; ++w) v = fmaxf(v, red[0][w][hh]);
        const float mnew = fmaxf(m[hh], v);
        corr[hh] = expf(m[hh] - mnew);
        m[hh] = mnew;
        float lsum = 0.f;
#pragma unroll
        for (int r = 0; r < SR; ++r) {
          const float e = expf(s[r][hh] - mnew);
          if (ksub == 0) pl[hh][kkey + r * KPR] = e;
          lsum += e;
        }
        l[hh] = l[hh] * corr[hh] + (ksub == 0 ? lsum : 0.f);
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[hh][e] *= corr[hh];
      }
      __syncthreads();
#pragma unroll
      for (int b = 0; b < NV; ++b) {
        const int jl = vslot + b * VS, j = c0 + jl;
        if (c0 + b * VS >= L) break;
        float x[EPC];
        if (j >= pos0) {
          const int jn = min(j - pos0, NTOK - 1);
#pragma unroll
          for (int e = 0; e < EPC; ++e) x[e] = vnew[jn][vchunk * EPC + e];
        } else {
          unpack_chunk<KVT>(vr[b], x);
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float pw = pl[hh][jl];         // 0 past the last key
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[hh][e] = fmaf(pw, x[e], acc[hh][e]);
        }
      }
      if (more) load_v(c0 + KCH);
      __syncthreads();                         // pl and red are rewritten next
    }
    // combine: key slots (lanes CPK apart), then waves; the softmax sums too
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        float v = acc[hh][e];
#pragma unroll
        for (int o = CPK; o < 64; o <<= 1) v += __shfl_xor(v, o);
        acc[hh][e] = v;
      }
      l[hh] = wave_sum(l[hh]);
    }
    if (lane < CPK)
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int e = 0; e < EPC; ++e) part[wave][hh][vchunk * EPC + e] = acc[hh][e];
    if (lane == 0)
#pragma unroll
      for (int hh = 0; hh < G; ++hh) red[1][wave][hh] = l[hh];
    __syncthreads();
    for (int e = tid; e < G * D; e += NT) {
      const int hh = e / D, dim = e % D;
      float v = 0.f, ls = 0.f;
#pragma unroll
      for (int w = 0; w < NT / 64; ++w) { v += part[w][hh][dim]; ls += red[1][w][hh]; }
      if constexpr (SPLIT) {
        float* sb = p.split_buf + ((((long)row * p.nkv + g) * gridDim.z + blockIdx.z) * G + hh) * (D + 2);
        sb[dim] = v;
        if (dim == 0) { sb[D] = m[hh]; sb[D + 1] = ls; }
      } else {
        p.out[(arow0 + t) * p.ld_out + (long)(g * G + hh) * D + dim] = v / ls;
      }
    }
    if (t + 1 < NTOK) __syncthreads();
  }
}

// Adds the key ranges of a split decode step in range order: with M the
// largest running max, out = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s.
// Thread = (row, q head, dim); every partial load of the S ranges is issued
// before the first use. Empty ranges hold m = -inf, l = 0.
template <int G, int S>
__global__ __launch_bounds__(NT) void attn_split_combine_kernel(AttnArgs p) {
  constexpr int D = 128;
  const long e = (long)blockIdx.x * NT + threadIdx.x;
  const int per_row = p.nq * D;
  if (e >= (long)p.n_runs * per_row) return;
  const int row = (int)(e / per_row), c = (int)(e % per_row);
  const int h = c / D, dim = c % D, g = h / G, hh = h % G;
  const long arow = p.tok_stride > 0 ? (long)row * p.tok_stride + p.tok_off : row;
  const float* sb = p.split_buf + (((long)row * p.nkv + g) * S * G + hh) * (D + 2);
  float m[S], o[S], l[S];
#pragma unroll
  for (int sp = 0; sp < S; ++sp) {
    const float* q = sb + (long)sp * G * (D + 2);
    m[sp] = q[D];
    o[sp] = q[dim];
    l[sp] = q[D + 1];
  }
  float mx = m[0];
#pragma unroll
  for (int sp = 1; sp < S; ++sp) mx = fmaxf(mx, m[sp]);
  float num = 0.f, den = 0.f;
#pragma unroll
  for (int sp = 0; sp < S; ++sp) {
    const float w = m[sp] == -INFINITY ? 0.f : expf(m[sp] - mx);
    num = fmaf(w, o[sp], num);
    den = fmaf(w, l[sp], den);
  }
  p.out[arow * p.ld_out + (long)h * D + dim] = num / den;
}

template <int G>
static hipError_t launch_split_combine(const AttnArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(((long)a.n_runs * a.nq * 128 + NT - 1) / NT));
  switch (a.kv_split) {
    case 2: hipLaunchKernelGGL((attn_split_combine_kernel<G, 2>), grid, dim3(NT), 0, s, a); break;
    case 4: hipLaunchKernelGGL((attn_split_combine_kernel<G, 4>), grid, dim3(NT), 0, s, a); break;
    case 8: hipLaunchKernelGGL((attn_split_combine_kernel<G, 8>), grid, dim3(NT), 0, s, a); break;
    case 16: hipLaunchKernelGGL((attn_split_combine_kernel<G, 16>), grid, dim3(NT), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Single-token decode attention over at most 16 positions (the code
// predictor's steps at batch rows > 1), head_dim 128, 16-bit cache.
// Block = (kv head, row): waves 0..G-1 take the q heads of the group, wave G
// the new key, wave G + 1 the new value (QK-RMSNorm + rope as in
// attn_step_kernel, the K/V rows to the cache and LDS); after the one
// barrier each q-head wave finishes alone. Scores: lane = (key l % 16,
// quarter l / 16 of the dims), the quarters added with two shuffles; the
// softmax over the 16 keys stays in 16-lane groups; P.V: lane = 2 dims, the
// key weights broadcast by shuffles. Every cache load leaves before the
// prologue (clamped to the cached keys).
template <typename KVT, int G>
__global__ __launch_bounds__((G + 2) * 64) void attn_short_kernel(AttnArgs p) {
  constexpr int D = 128, HALF = 64;
  const int g = blockIdx.x, row = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ __align__(16) float qs[G][D];
  __shared__ __align__(16) float knew[D];
  __shared__ __align__(16) float vnew[D];
  KVT* kc = (KVT*)p.kc + (long)row * p.row_stride + (long)g * p.max_pos * D;
  KVT* vc = (KVT*)p.vc + (long)row * p.row_stride + (long)g * p.max_pos * D;
  const int pos0 = p.pos_base + (p.row_pos ? p.row_pos[row] : 0);
  const int jk = lane & 15, qd = lane >> 4;
  const int last = max(pos0 - 1, 0);
  u32x4 kr[4];
  uint32_t vr[16];
  if (wave < G) {
    const KVT* kp = kc + (long)min(jk, last) * D + 32 * qd;
#pragma unroll
    for (int c = 0; c < 4; ++c) kr[c] = *(const u32x4*)(kp + 8 * c);
#pragma unroll
    for (int j = 0; j < 16; ++j) vr[j] = *(const uint32_t*)(vc + (long)min(j, last) * D + 2 * lane);
  }
  // q/k/v of the new token: the projection's rows, or its split-K partial sums
  const long ar = p.tok_stride > 0 ? (long)row * p.tok_stride + p.tok_off : row;
  // up to PZ ranges with every load issued before the first add (ranges past
  // part_z are clamped loads that are not added); more ranges: a loop
  constexpr int PZ = 8;
  const bool pz_fast = p.part_z <= PZ;
  float prs = 1.f;
  if (p.part_z > 0) {
    const float* pss = p.part + (long)p.part_z * p.part_rows * p.ld_qkv;
    float ssum = 0.f;
    if (pz_fast) {
      float q[PZ];
#pragma unroll
      for (int z = 0; z < PZ; ++z) q[z] = pss[(long)min(z, p.part_z - 1) * p.part_rows + ar];
#pragma unroll
      for (int z = 0; z < PZ; ++z) if (z < p.part_z) ssum += q[z];
    } else {
      for (int z = 0; z < p.part_z; ++z) ssum += pss[(long)z * p.part_rows + ar];
    }
    prs = 1.f / sqrtf(ssum / (float)p.part_k + p.part_eps);
  }
  auto qkv_at = [&](long col) -> float {
    if (p.part_z <= 0) return p.qkv[ar * p.ld_qkv + col];
    float v;
    if (pz_fast) {
      float q[PZ];
#pragma unroll
      for (int z = 0; z < PZ; ++z) q[z] = p.part[((long)min(z, p.part_z - 1) * p.part_rows + ar) * p.ld_qkv + col];
      v = q[0];
#pragma unroll
      for (int z = 1; z < PZ; ++z) if (z < p.part_z) v += q[z];
    } else {
      v = p.part[ar * p.ld_qkv + col];
      for (int z = 1; z < p.part_z; ++z) v += p.part[((long)z * p.part_rows + ar) * p.ld_qkv + col];
    }
    return v * prs;
  };
  {
    float cs, sn;
    if (p.rope_rows) {
      cs = p.rope_rows[(long)row * D + lane];
      sn = p.rope_rows[(long)row * D + HALF + lane];
    } else {
      cs = p.cos[(long)pos0 * HALF + lane];
      sn = p.sin[(long)pos0 * HALF + lane];
    }
    const int v = wave;
    if (v == G + 1) {                       // value row, stored as is
      const long col = (long)(p.nq + p.nkv) * D + (long)g * D;
      const float x1 = qkv_at(col + lane), x2 = qkv_at(col + lane + HALF);
      st_elem<KVT>(vc, (long)pos0 * D + lane, x1);
      st_elem<KVT>(vc, (long)pos0 * D + lane + HALF, x2);
      vnew[lane] = kv_round<KVT>(x1);
      vnew[lane + HALF] = kv_round<KVT>(x2);
    } else {
      const long col = v < G ? (long)(g * G + v) * D : (long)p.nq * D + (long)g * D;
      const float* gain = v < G ? p.q_gain : p.k_gain;
      const float x1 = qkv_at(col + lane), x2 = qkv_at(col + lane + HALF);
      const float g1 = gain[lane], g2 = gain[lane + HALF];
      const float ss = wave_sum(x1 * x1 + x2 * x2);
      const float rden = 1.f / sqrtf(ss / (float)D + p.eps);
      const float y1 = x1 * rden * g1, y2 = x2 * rden * g2;
      const float o1 = y1 * cs - y2 * sn, o2 = y2 * cs + y1 * sn;
      if (v < G) {
        qs[v][lane] = o1;
        qs[v][lane + HALF] = o2;
      } else {
        st_elem<KVT>(kc, (long)pos0 * D + lane, o1);
        st_elem<KVT>(kc, (long)pos0 * D + lane + HALF, o2);
        knew[lane] = kv_round<KVT>(o1);
        knew[lane + HALF] = kv_round<KVT>(o2);
      }
    }
  }
  __syncthreads();
  if (wave >= G) return;
  const int hh = wave, L = pos0 + 1;
  float x[32];
  if (jk < pos0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) unpack_chunk<KVT>(kr[c], x + 8 * c);
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] = jk == pos0 ? knew[32 * qd + e] : 0.f;
  }
  const f32x4* q4 = (const f32x4*)&qs[hh][32 * qd];
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const f32x4 qa = q4[e], qb = q4[e + 1];
    s0 = fmaf(qa.x, x[4 * e], s0); s0 = fmaf(qa.y, x[4 * e + 1], s0); s0 = fmaf(qa.z, x[4 * e + 2], s0); s0 = fmaf(qa.w, x[4 * e + 3], s0);
    s1 = fmaf(qb.x, x[4 * e + 4], s1); s1 = fmaf(qb.y, x[4 * e + 5], s1); s1 = fmaf(qb.z, x[4 * e + 6], s1); s1 = fmaf(qb.w, x[4 * e + 7], s1);
  }
  float sc = s0 + s1;
  sc += __shfl_xor(sc, 16);
  sc += __shfl_xor(sc, 32);
  sc = jk < L ? sc * p.scale : -INFINITY;
  float mx = sc;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const float ew = jk < L ? expf(sc - mx) : 0.f;
  float lsum = ew;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) lsum += __shfl_xor(lsum, o);
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float pj = __shfl(ew, j);        // lanes 0..15 hold the key weights
    float v0, v1;
    if (j < pos0) {
      if constexpr (std::is_same<KVT, _Float16>::value) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        const h2 h = __builtin_bit_cast(h2, vr[j]);
        v0 = (float)h[0]; v1 = (float)h[1];
      } else {
        v0 = bf_lo(vr[j]); v1 = bf_hi(vr[j]);
      }
    } else if (j == pos0) {
      v0 = vnew[2 * lane]; v1 = vnew[2 * lane + 1];
    } else {
      v0 = 0.f; v1 = 0.f;
    }
    a0 = fmaf(pj, v0, a0);
    a1 = fmaf(pj, v1, a1);
  }
  const float rl = 1.f / lsum;
  float* o = p.out + ar * p.ld_out + (long)(g * G + hh) * D + 2 * lane;
  *(float2*)o = make_float2(a0 * rl, a1 * rl);
}

// ---------------------------------------------------------------- prefill attention on the matrix cores
// Causal attention of the prompt prefill for head_dim 128 and a 16-bit cache
// (attend pass: the cache already holds every key). Block = (kv head, run of
// up to FA_TOK consecutive tokens of one row); wave w takes q head w % G and
// tokens 16 (w / G) .. 16 (w / G) + 15. Keys 0 .. (last token's position) go
// through LDS in blocks of FA_KB, double-buffered: K as rows, V transposed.
// Scores are formed transposed, S^T = K Q^T, so a lane holds one query's
// scores for 16 keys; that is the B-operand layout of P^T in O^T = V^T P^T
// (the contraction may visit the keys in any order as long as the V^T rows
// follow the same order), so the running max and sum stay per query lane
// and no shuffle moves them. q and P are split into 16-bit hi + lo parts,
// two products each, which keeps fp32-level accuracy against the cache's
// exact 16-bit keys and values.
#define FA_TOK kAttnTileTokens
#define FA_KB 64
#define FA_KP 136   // K rows in LDS: pitch in 16-bit elements (128 + 8)
#define FA_VP 68    // V^T rows in LDS: pitch in 16-bit elements (64 + 4)

template <typename KVT>
__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  if constexpr (std::is_same<KVT, _Float16>::value) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
  }
}

// (a, b) -> packed 16-bit hi = round(x) and lo = round(x - hi)
template <typename KVT>
__device__ __forceinline__ void split16_pk(float a, float b, uint32_t& hi, uint32_t& lo) {
  if constexpr (std::is_same<KVT, _Float16>::value) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 h = {(_Float16)a, (_Float16)b};
    const h2 l = {(_Float16)(a - (float)h[0]), (_Float16)(b - (float)h[1])};
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, l);
  } else {
    split_pk(a, b, hi, lo);
  }
}

template <typename KVT, int G>
__global__ __launch_bounds__(2 * G * 64) void attn_prefill_mfma_kernel(AttnArgs p) {
  constexpr int D = 128, HALF = 64, NTH = 2 * G * 64;
  static_assert(NTH == 256, "one (key quad, 16-byte column) load item per thread");
  const int g = blockIdx.x;
  const Run rn = p.runs[blockIdx.y];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, quad = lane >> 4;
  const int hh = wave % G, tw0 = 16 * (wave / G);
  extern __shared__ __align__(16) uint16_t fsm[];
  constexpr int STAGE = FA_KB * FA_KP + D * FA_VP;   // K rows, then V^T rows, per buffer
  const KVT* kc = (const KVT*)p.kc + (long)rn.row * p.row_stride + (long)g * p.max_pos * D;
  const KVT* vc = (const KVT*)p.vc + (long)rn.row * p.row_stride + (long)g * p.max_pos * D;
  const int L = rn.pos0 + rn.ntok;                  // keys of the block: positions 0 .. L - 1
  const int nkb = (L + FA_KB - 1) / FA_KB;

  // load role: keys 4 m .. 4 m + 3 of a key block, 16-byte column c
  const int lm = tid >> 4, lcol = tid & 15;
  u32x4 kr[4], vr[4];
  auto load_block = [&](int kb) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int key = min(kb * FA_KB + 4 * lm + u, L - 1);   // rows past L: clamped, weighted 0
      kr[u] = *(const u32x4*)(kc + (long)key * D + 8 * lcol);
      vr[u] = *(const u32x4*)(vc + (long)key * D + 8 * lcol);
    }
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u) *(u32x4*)(fsm + buf * STAGE + (4 * lm + u) * FA_KP + 8 * lcol) = kr[u];
    // V^T: dims 8 c .. 8 c + 7, keys 4 m .. 4 m + 3 (one 8-byte row piece per dim)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = 16 * (e & 1);
      uint32_t x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const u32x4 v = vr[u];
        const uint32_t word = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
        x[u] = (word >> sh) & 0xffffu;
      }
      *(uint2*)(fsm + buf * STAGE + FA_KB * FA_KP + (8 * lcol + e) * FA_VP + 4 * lm) = make_uint2(x[0] | (x[1] << 16), x[2] | (x[3] << 16));
    }
  };
  load_block(0);

  // this lane's query: token tw0 + col of the run (padding lanes repeat the
  // last token and store nothing)
  const int tok = tw0 + col;
  const bool tok_ok = tok < rn.ntok;
  const int tk = min(tok, rn.ntok - 1);
  const int qpos = rn.pos0 + tk;
  const int wlast = rn.pos0 + min(tw0 + 15, rn.ntok - 1);   // the wave's last query position
  const bool wave_live = tw0 < rn.ntok;
  // q: dims 32 s + 8 quad .. + 7 for s = 0..3, RMSNorm with the q gain, rope
  // pairs (j, j + 64) = (s, s + 2) in the same lane
  u32x4 qh[4], ql[4];
  {
    const float* src = p.qkv + ((long)rn.tok0 + tk) * p.ld_qkv + (long)(g * G + hh) * D;
    float x[4][8], gn[4][8], cs[2][8], sn[2][8];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int d0 = 32 * s + 8 * quad;
      const f32x4 a0 = *(const f32x4*)(src + d0), a1 = *(const f32x4*)(src + d0 + 4);
      const f32x4 g0 = *(const f32x4*)(p.q_gain + d0), g1 = *(const f32x4*)(p.q_gain + d0 + 4);
      x[s][0] = a0.x; x[s][1] = a0.y; x[s][2] = a0.z; x[s][3] = a0.w;
      x[s][4] = a1.x; x[s][5] = a1.y; x[s][6] = a1.z; x[s][7] = a1.w;
      gn[s][0] = g0.x; gn[s][1] = g0.y; gn[s][2] = g0.z; gn[s][3] = g0.w;
      gn[s][4] = g1.x; gn[s][5] = g1.y; gn[s][6] = g1.z; gn[s][7] = g1.w;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const long j0 = (long)qpos * HALF + 32 * s + 8 * quad;
      const f32x4 c0 = *(const f32x4*)(p.cos + j0), c1 = *(const f32x4*)(p.cos + j0 + 4);
      const f32x4 s0 = *(const f32x4*)(p.sin + j0), s1 = *(const f32x4*)(p.sin + j0 + 4);
      cs[s][0] = c0.x; cs[s][1] = c0.y; cs[s][2] = c0.z; cs[s][3] = c0.w;
      cs[s][4] = c1.x; cs[s][5] = c1.y; cs[s][6] = c1.z; cs[s][7] = c1.w;
      sn[s][0] = s0.x; sn[s][1] = s0.y; sn[s][2] = s0.z; sn[s][3] = s0.w;
      sn[s][4] = s1.x; sn[s][5] = s1.y; sn[s][6] = s1.z; sn[s][7] = s1.w;
    }
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(x[s][e], x[s][e], ss);
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    const float den = sqrtf(ss / (float)D + p.eps);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[s][e] = x[s][e] / den * gn[s][e];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x1 = x[s][e], x2 = x[s + 2][e];
        x[s][e] = x1 * cs[s][e] - x2 * sn[s][e];
        x[s + 2][e] = x2 * cs[s][e] + x1 * sn[s][e];
      }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t h[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) split16_pk<KVT>(x[s][2 * e], x[s][2 * e + 1], h[e], l[e]);
      qh[s] = (u32x4){h[0], h[1], h[2], h[3]};
      ql[s] = (u32x4){l[0], l[1], l[2], l[3]};
    }
  }

  float m = -INFINITY, lsum = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  store_block(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    const bool more = kb + 1 < nkb;
    if (more) load_block(kb + 1);
    const int k0 = kb * FA_KB;
    if (wave_live && k0 <= wlast) {
      const uint16_t* Kl = fsm + cur * STAGE;
      const uint16_t* Vl = Kl + FA_KB * FA_KP;
      // S^T tiles: keys 16 kt + (4 quad + r), query col. Tiles whose keys all
      // lie past the wave's last query (the causal edge) are skipped: their
      // scores are masked below and their P rows are 0.
      const int ktn = min(4, (wlast - k0) / 16 + 1);
      f32x4 sc[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        f32x4 c = (f32x4){0.f, 0.f, 0.f, 0.f};
        if (kt < ktn)
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const u32x4 a = *(const u32x4*)(Kl + (16 * kt + col) * FA_KP + 32 * s + 8 * quad);
            c = mfma16x16x32<KVT>(a, qh[s], c);
            c = mfma16x16x32<KVT>(a, ql[s], c);
          }
        sc[kt] = c;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + 16 * kt + 4 * quad + r;
          const float v = key <= qpos ? sc[kt][r] * p.scale : -INFINITY;
          sc[kt][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m, mx);     // finite: key 0 is in every query's range
      const float corr = expf(m - mnew);
      m = mnew;
      float ps = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + 16 * kt + 4 * quad + r;
          const float e = key <= qpos ? expf(sc[kt][r] - mnew) : 0.f;
          sc[kt][r] = e;
          ps += e;
        }
      lsum = lsum * corr + ps;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc[dt] *= corr;
      // O^T += V^T P^T over two 32-key steps; slot 8 quad + e is key
      // 32 ks + 4 quad + e (e < 4) or 32 ks + 16 + 4 quad + e - 4
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (2 * ks >= ktn) break;   // both key tiles past the edge: P is 0
        uint32_t h[4], l[4];
        split16_pk<KVT>(sc[2 * ks][0], sc[2 * ks][1], h[0], l[0]);
        split16_pk<KVT>(sc[2 * ks][2], sc[2 * ks][3], h[1], l[1]);
        split16_pk<KVT>(sc[2 * ks + 1][0], sc[2 * ks + 1][1], h[2], l[2]);
        split16_pk<KVT>(sc[2 * ks + 1][2], sc[2 * ks + 1][3], h[3], l[3]);
        const u32x4 ph = (u32x4){h[0], h[1], h[2], h[3]}, pl = (u32x4){l[0], l[1], l[2], l[3]};
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const uint16_t* vrow = Vl + (16 * dt + col) * FA_VP + 32 * ks + 4 * quad;
          const uint2 v0 = *(const uint2*)vrow, v1 = *(const uint2*)(vrow + 16);
          const u32x4 a = (u32x4){v0.x, v0.y, v1.x, v1.y};
          acc[dt] = mfma16x16x32<KVT>(a, ph, acc[dt]);
          acc[dt] = mfma16x16x32<KVT>(a, pl, acc[dt]);
        }
      }
    }
    if (more) store_block(cur ^ 1);
    __syncthreads();
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (!wave_live || !tok_ok) return;
  float* o = p.out + ((long)rn.tok0 + tok) * p.ld_out + (long)(g * G + hh) * D + 4 * quad;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) *(f32x4*)(o + 16 * dt) = acc[dt] / lsum;
}

template <typename KVT, int G>
static hipError_t launch_attn_prefill_mfma(const AttnArgs& a, hipStream_t s) {
  constexpr size_t lds = (size_t)2 * (FA_KB * FA_KP + 128 * FA_VP) * sizeof(uint16_t);
  static size_t have = 0;
  hipError_t e = ensure_lds((const void*)attn_prefill_mfma_kernel<KVT, G>, lds, &have);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_prefill_mfma_kernel<KVT, G>), dim3(a.nkv, a.n_runs), dim3(2 * G * 64), lds, s, a);
  return hipGetLastError();
}

bool attn_prefill_tiles(int d, int nq, int nkv, int kvdtype) {
  return d == 128 && nkv > 0 && nq == 2 * nkv && (kvdtype == DT_F16 || kvdtype == DT_BF16);
}


// Prefill write pass for head_dim 128: one wave per (token, kv head). Lane j
// holds the rope pair (j, j + 64) of k and of v: RMSNorm of k with its gain
// (one wave sum), rope, and both rows to the cache; a wave's 2- or 4-byte
// stores cover whole row segments.
template <typename KVT>
__global__ __launch_bounds__(256) void kv_write_kernel(AttnArgs p) {
  constexpr int D = 128, HALF = 64;
  const int lane = threadIdx.x & 63;
  const long w = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (long)p.n_runs * p.nkv) return;   // whole waves
  const int g = (int)(w % p.nkv);
  const Run rn = p.runs[w / p.nkv];
  const int pos0 = rn.pos0 + p.pos_base + (p.row_pos ? p.row_pos[rn.row] : 0);
  KVT* kc = (KVT*)p.kc + (long)rn.row * p.row_stride + (long)g * p.max_pos * D;
  KVT* vc = (KVT*)p.vc + (long)rn.row * p.row_stride + (long)g * p.max_pos * D;
  const float g1 = p.k_gain[lane], g2 = p.k_gain[lane + HALF];
  for (int i = 0; i < rn.ntok; ++i) {
    const float* src = p.qkv + ((long)rn.tok0 + i) * p.ld_qkv + (long)p.nq * D + (long)g * D;
    const float* vsrc = src + (long)p.nkv * D;
    const int pos = pos0 + i;
    const float x1 = src[lane], x2 = src[lane + HALF], v1 = vsrc[lane], v2 = vsrc[lane + HALF];
    const float c = p.cos[(long)pos * HALF + lane], sn = p.sin[(long)pos * HALF + lane];
    const float ss = wave_sum(x1 * x1 + x2 * x2);
    const float den = sqrtf(ss / (float)D + p.eps);
    const float y1 = x1 / den * g1, y2 = x2 / den * g2;
    st_elem<KVT>(kc, (long)pos * D + lane, y1 * c - y2 * sn);
    st_elem<KVT>(kc, (long)pos * D + lane + HALF, y2 * c + y1 * sn);
    st_elem<KVT>(vc, (long)pos * D + lane, v1);
    st_elem<KVT>(vc, (long)pos * D + lane + HALF, v2);
  }
}

template <typename KVT, int D, int G>
static hipError_t launch_attention_dg(const AttnArgs& a, hipStream_t s) {
  constexpr int EPC = 16 / sizeof(KVT), CPK = D / EPC, TPK = CPK < 4 ? CPK : 4, KCH = NT / TPK;
  const size_t lds = ((size_t)(2 * G + 1) * D + 2 * D + (size_t)G * KCH + 4 * (size_t)G * D + 8 * G) * sizeof(float);
  if constexpr (D == 128) {
    if (a.mode == ATT_WRITE && !a.single_token) {
      const long waves = (long)a.n_runs * a.nkv;
      hipLaunchKernelGGL((kv_write_kernel<KVT>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a);
      return hipGetLastError();
    }
  }
  if constexpr (D == 128 && G == 2 && sizeof(KVT) == 2) {
    // prompt prefill, attend pass over runs of up to FA_TOK tokens
    if (a.mode == ATT_ATTEND && !a.single_token && a.max_ntok > 0) {
      if (a.max_ntok > FA_TOK) return hipErrorInvalidValue;
      return launch_attn_prefill_mfma<KVT, G>(a, s);
    }
    if (a.single_token && a.mode == ATT_WRITE_ATTEND && (a.ntok <= 1) && a.max_pos <= 16 && a.n_runs > 1 &&
        a.ld_out % 2 == 0) {
      hipLaunchKernelGGL((attn_short_kernel<KVT, G>), dim3(a.nkv, a.n_runs), dim3((G + 2) * 64), 0, s, a);
      return hipGetLastError();
    }
  }
  if constexpr (D == 128 && G <= 4) {
    const int nt = a.ntok > 0 ? a.ntok : 1;
    if (a.single_token && a.mode == ATT_WRITE_ATTEND && (nt == 1 || (nt == 2 && a.tok_stride == 2 && a.tok_off == 0))) {
      constexpr int big = 512 / sizeof(KVT), small = 64;
      const dim3 grid(a.nkv, a.n_runs);
      // large chunks when the grid is at most one block per compute unit and
      // contexts can be long (not the code predictor's 16 positions: 64-key
      // chunks measured 5.1 against 5.7 us there)
      const bool one_wave = (long)a.nkv * a.n_runs <= 256 && a.max_pos > small;
      if (nt == 1 && a.split_buf && (a.kv_split == 2 || a.kv_split == 4 || a.kv_split == 8 || a.kv_split == 16)) {
        hipLaunchKernelGGL((attn_step_kernel<KVT, G, 1, small, true>), dim3(a.nkv, a.n_runs, a.kv_split), dim3(NT), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_split_combine<G>(a, s);
      }
      if (nt == 2) hipLaunchKernelGGL((attn_step_kernel<KVT, G, 2, small>), grid, dim3(NT), 0, s, a);
      else if (one_wave) hipLaunchKernelGGL((attn_step_kernel<KVT, G, 1, big>), grid, dim3(NT), 0, s, a);
      else hipLaunchKernelGGL((attn_step_kernel<KVT, G, 1, small>), grid, dim3(NT), 0, s, a);
      return hipGetLastError();
    }
  }
  if constexpr (D <= 128) {   // wider heads use the general kernel (register budget)
    if (a.single_token && a.mode == ATT_WRITE_ATTEND && a.ntok == 2) {
      // two tokens per row (activation rows 2 r and 2 r + 1): token 0, then
      // token 1, which attends to the key and value the first launch wrote
      AttnArgs b = a;
      b.ntok = 1;
      b.tok_stride = 2;
      for (int t = 0; t < 2; ++t) {
        b.tok_off = t;
        b.pos_base = a.pos_base + t;
        hipError_t e = launch_attention_dg<KVT, D, G>(b, s);
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    }
    if (a.single_token && a.mode == ATT_WRITE_ATTEND) {
      static size_t have1 = 0;
      hipError_t e = ensure_lds((const void*)attn_decode_kernel<KVT, D, G>, lds, &have1);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((attn_decode_kernel<KVT, D, G>), dim3(a.nkv, a.n_runs), dim3(NT), lds, s, a);
      return hipGetLastError();
    }
  }
  static size_t have = 0;
  hipError_t e = ensure_lds((const void*)attn_kernel<KVT, D, G>, lds, &have);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_kernel<KVT, D, G>), dim3(a.nkv, a.n_runs), dim3(NT), lds, s, a);
  return hipGetLastError();
}

template <typename KVT, int D>
static hipError_t launch_attention_d(const AttnArgs& a, hipStream_t s) {
  switch (a.nq / a.nkv) {
    case 1: return launch_attention_dg<KVT, D, 1>(a, s);
    case 2: return launch_attention_dg<KVT, D, 2>(a, s);
    case 4: return launch_attention_dg<KVT, D, 4>(a, s);
    case 8: return launch_attention_dg<KVT, D, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename KVT>
static hipError_t launch_attention_t(const AttnArgs& a, hipStream_t s) {
  switch (a.d) {
    case 16: return launch_attention_d<KVT, 16>(a, s);
    case 32: return launch_attention_d<KVT, 32>(a, s);
    case 64: return launch_attention_d<KVT, 64>(a, s);
    case 128: return launch_attention_d<KVT, 128>(a, s);
    case 256: return launch_attention_d<KVT, 256>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.n_runs <= 0) return hipSuccess;
  if (a.kvdtype == DT_BF16) return launch_attention_t<uint16_t>(a, s);
  if (a.kvdtype == DT_F16) return launch_attention_t<_Float16>(a, s);
  return launch_attention_t<float>(a, s);
}

// ---------------------------------------------------------------- predictor attention + o-projection
// The code predictor at batch 1 attends over at most 16 positions, so every
// block of the o-projection recomputes the whole attention (one wave per kv
// head) while its rows of W_o are in flight, then applies them: one launch
// instead of two. NTOK new tokens (1: a step, 2: the two-token pass at
// positions 0 and 1) sit in activation rows 0 .. NTOK-1. Block b owns output
// rows [b RO, (b + 1) RO); block 0 also writes the new K/V rows.
// Scores: lane = (key j, quarter of the head dims); P·V: lane = (8-dim
// column chunk, key slot j mod 4).
template <typename KVT, int NKV, int G, int RO, int NTOK>
__global__ __launch_bounds__(NKV * 64) void pred_attn_o_kernel(AttnArgs p, LinearArgs o) {
  constexpr int D = 128, HALF = 64, NQ = NKV * G, KO = NQ * D;
  constexpr int EPC = 8;                       // 16-bit cache elements per 16-byte chunk
  constexpr int RW = RO / NKV;                 // o rows per wave
  constexpr int KC = KO / 512;                 // 16-byte weight chunks per lane and row
  static_assert(sizeof(KVT) == 2 && RO % NKV == 0 && KO % 512 == 0, "layout");
  const int g = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = blockIdx.x * RO + g * RW;
  __shared__ __align__(16) float qs[NKV][NTOK][G][D];
  __shared__ __align__(16) float knew[NKV][NTOK][D];
  __shared__ __align__(16) float vnew[NKV][NTOK][D];
  __shared__ __align__(16) float att[NTOK][KO];

  // Loads leave in the order they are needed (the vector-memory counter
  // drains in issue order): this wave's q/k/v values, gains and rope rows,
  // then the cached K/V rows (unconditional, clamped rows; rows past the
  // context are never used), then this wave's rows of W_o, which stream in
  // behind the attention.
  const int pos0 = p.pos_base;                 // keys 0 .. pos0 - 1 are cached
  KVT* kc = (KVT*)p.kc + (long)g * p.max_pos * D;
  KVT* vc = (KVT*)p.vc + (long)g * p.max_pos * D;
  const int sj = lane >> 2, sq = lane & 3;     // score role: key, quarter
  const int vch = lane & 15, vsl = lane >> 4;  // P·V role: column chunk, key slot
  float xin[NTOK][G + 2][2], cs[NTOK], sn[NTOK];
#pragma unroll
  for (int t = 0; t < NTOK; ++t) {
    const float* src = p.qkv + (long)t * p.ld_qkv;
#pragma unroll
    for (int v = 0; v < G + 2; ++v) {
      const float* x = src + (v < G ? (long)(g * G + v) * D : (long)(NQ + (v - G) * NKV) * D + (long)g * D);
      xin[t][v][0] = x[lane];
      xin[t][v][1] = x[lane + HALF];
    }
    cs[t] = p.cos[(long)(pos0 + t) * HALF + lane];
    sn[t] = p.sin[(long)(pos0 + t) * HALF + lane];
  }
  const float gq1 = p.q_gain[lane], gq2 = p.q_gain[lane + HALF];
  const float gk1 = p.k_gain[lane], gk2 = p.k_gain[lane + HALF];
  const int jmax = max(pos0 - 1, 0);
  u32x4 kr[4], vr[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) kr[c] = *(const u32x4*)(kc + (long)min(sj, jmax) * D + sq * 32 + c * EPC);
#pragma unroll
  for (int i = 0; i < 4; ++i) vr[i] = *(const u32x4*)(vc + (long)min(vsl + 4 * i, jmax) * D + vch * EPC);
  __builtin_amdgcn_sched_barrier(0);
  const uint16_t* W = (const uint16_t*)o.W;
  u32x4 w[RW][KC];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int c = 0; c < KC; ++c) w[r][c] = ld_weight(W + (long)(n0 + r) * KO + c * 512 + lane * 8);
  __builtin_amdgcn_sched_barrier(0);

  // new tokens: QK-RMSNorm and rope (lane owns the pair (lane, lane + 64))
#pragma unroll
  for (int t = 0; t < NTOK; ++t) {
    const int pos = pos0 + t;
#pragma unroll
    for (int v = 0; v <= G; ++v) {
      const float x1 = xin[t][v][0], x2 = xin[t][v][1];
      const float ss = wave_sum(x1 * x1 + x2 * x2);
      const float rden = 1.f / sqrtf(ss / (float)D + p.eps);
      const float y1 = x1 * rden * (v < G ? gq1 : gk1), y2 = x2 * rden * (v < G ? gq2 : gk2);
      const float o1 = y1 * cs[t] - y2 * sn[t], o2 = y2 * cs[t] + y1 * sn[t];
      if (v < G) {
        qs[g][t][v][lane] = o1;
        qs[g][t][v][lane + HALF] = o2;
      } else {
        knew[g][t][lane] = kv_round<KVT>(o1);
        knew[g][t][lane + HALF] = kv_round<KVT>(o2);
        if (blockIdx.x == 0) {
          st_elem<KVT>(kc, (long)pos * D + lane, o1);
          st_elem<KVT>(kc, (long)pos * D + lane + HALF, o2);
        }
      }
    }
    const float v1 = xin[t][G + 1][0], v2 = xin[t][G + 1][1];
    vnew[g][t][lane] = kv_round<KVT>(v1);
    vnew[g][t][lane + HALF] = kv_round<KVT>(v2);
    if (blockIdx.x == 0) {
      st_elem<KVT>(vc, (long)pos * D + lane, v1);
      st_elem<KVT>(vc, (long)pos * D + lane + HALF, v2);
    }
  }
  // the attention below reads only this wave's own LDS rows
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

#pragma unroll
  for (int t = 0; t < NTOK; ++t) {
    const int L = pos0 + t + 1;
    float s[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) s[hh] = 0.f;
    if (sj < L) {
      float sp[G][4];                          // one partial sum per chunk: short dependence chains
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e0 = sq * 32 + c * EPC;
        float x[EPC];
        if (sj >= pos0) {
#pragma unroll
          for (int e = 0; e < EPC; ++e) x[e] = knew[g][sj - pos0][e0 + e];
        } else {
          unpack_chunk<KVT>(kr[c], x);
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const f32x4* q4 = (const f32x4*)(&qs[g][t][hh][e0]);
          float a = 0.f;
#pragma unroll
          for (int e = 0; e < EPC; e += 4) {
            const f32x4 q = q4[e / 4];
            a = fmaf(q.x, x[e], a);
            a = fmaf(q.y, x[e + 1], a);
            a = fmaf(q.z, x[e + 2], a);
            a = fmaf(q.w, x[e + 3], a);
          }
          sp[hh][c] = a;
        }
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) s[hh] = (sp[hh][0] + sp[hh][1]) + (sp[hh][2] + sp[hh][3]);
    }
    float pr[G], l[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      s[hh] += dpp_f<0xb1, 0xf>(s[hh], 0.f);   // quad_perm [1,0,3,2]
      s[hh] += dpp_f<0x4e, 0xf>(s[hh], 0.f);   // quad_perm [2,3,0,1]
      s[hh] = sj < L ? s[hh] * p.scale : -INFINITY;
      const float mx = wave_max(s[hh]);
      pr[hh] = expf(s[hh] - mx);
      l[hh] = wave_sum(sq == 0 ? pr[hh] : 0.f);
    }
    float acc[G][EPC];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[hh][e] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = vsl + 4 * i;
      float pw[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) pw[hh] = __shfl(pr[hh], (j & 15) * 4);
      if (j < L) {
        float x[EPC];
        if (j >= pos0) {
#pragma unroll
          for (int e = 0; e < EPC; ++e) x[e] = vnew[g][j - pos0][vch * EPC + e];
        } else {
          unpack_chunk<KVT>(vr[i], x);
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[hh][e] = fmaf(pw[hh], x[e], acc[hh][e]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        float v = acc[hh][e];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        acc[hh][e] = v;
      }
    if (vsl == 0)
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float rl = 1.f / l[hh];
#pragma unroll
        for (int e = 0; e < EPC; ++e) att[t][(g * G + hh) * D + vch * EPC + e] = acc[hh][e] * rl;
      }
  }
  __syncthreads();

  // o-projection rows of this wave, residual added in place
#pragma unroll
  for (int t = 0; t < NTOK; ++t) {
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      float ap[KC];                            // one partial sum per chunk: short dependence chains
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const f32x4* x4 = (const f32x4*)(&att[t][c * 512 + lane * 8]);
        const f32x4 xa = x4[0], xb = x4[1];
        const u32x4 q = w[r][c];
        float b = bf_lo(q.x) * xa.x;
        b = fmaf(bf_hi(q.x), xa.y, b);
        b = fmaf(bf_lo(q.y), xa.z, b); b = fmaf(bf_hi(q.y), xa.w, b);
        b = fmaf(bf_lo(q.z), xb.x, b); b = fmaf(bf_hi(q.z), xb.y, b);
        b = fmaf(bf_lo(q.w), xb.z, b); b = fmaf(bf_hi(q.w), xb.w, b);
        ap[c] = b;
      }
      float a = ap[0];
#pragma unroll
      for (int c = 1; c < KC; ++c) a += ap[c];
      a = wave_sum(a);
      if (lane == 0) {
        float* y = o.Y + (long)t * o.ldy + n0 + r;
        *y = *y + a;
      }
    }
  }
}

template <typename KVT>
static hipError_t launch_pred_attn_o_t(const AttnArgs& a, const LinearArgs& o, hipStream_t s) {
  constexpr int RO = 16;
  hipLaunchKernelGGL((pred_attn_o_kernel<KVT, 8, 2, RO, 1>), dim3(o.N / RO), dim3(512), 0, s, a, o);
  return hipGetLastError();
}

hipError_t launch_attention_oproj(const AttnArgs& a, const LinearArgs& o, hipStream_t s) {
  // one new token per launch: for the two-token pass the separate kernels are as fast
  const int nt = a.ntok > 0 ? a.ntok : 1;
  const bool ok = nt == 1 && a.single_token && a.mode == ATT_WRITE_ATTEND && a.n_runs == 1 && a.d == 128 && a.nkv == 8 &&
                  a.nq == 16 && a.ld_qkv >= (long)(a.nq + 2 * a.nkv) * a.d && a.part_z <= 0 && !a.row_pos && !a.rope_rows && a.max_pos <= 16 &&
                  a.pos_base >= 0 && a.pos_base + nt <= a.max_pos &&
                  (nt == 1 || (nt == 2 && a.tok_stride == 2 && a.tok_off == 0)) && (nt == 2 || a.tok_stride == 0) &&
                  (a.kvdtype == DT_F16 || a.kvdtype == DT_BF16) &&
                  o.wdtype == DT_BF16 && o.K == a.nq * a.d && o.N % 16 == 0 && o.M == nt && o.epi == EPI_RESIDUAL &&
                  !o.gain && o.ldx == o.K && o.X == a.out && a.ld_out == o.K;
  if (!ok) return hipErrorNotSupported;
  if (a.kvdtype == DT_F16) return launch_pred_attn_o_t<_Float16>(a, o, s);
  return launch_pred_attn_o_t<uint16_t>(a, o, s);
}

// ---------------------------------------------------------------- Philox
// Philox4x64-10 (Salmon et al., SC'11): 10 rounds of two 64x64->128-bit
// multiplies of counter words 0 and 2, halves mixed with words 1 and 3 and
// the key; the key is bumped by two Weyl constants between rounds.
__device__ __forceinline__ uint64_t philox_word0(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                                 uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) { k0 += W0; k1 += W1; }
    const uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
    const uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
  return c0;
}
// E ~ Exp(1): u = ((x >> 12) + 1/2) 2^-52 in (0,1), E = -ln u in double, rounded to float.
__device__ __forceinline__ float exp_noise(uint64_t seed, int row, int stream, int index, int id) {
  const uint64_t x = philox_word0((uint64_t)id, (uint64_t)stream, (uint64_t)(int64_t)index, (uint64_t)row, seed, 0ull);
  const double u = ((double)(x >> 12) + 0.5) * 0x1p-52;
  return (float)(-log(u));
}

// ---------------------------------------------------------------- selection
__device__ __forceinline__ uint32_t ord_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// MPT logits per thread (V <= MPT * NT). Every global load of a phase is
// issued before its first use (the row's logits and seen bits, the feedback
// row; then the chosen table row), so a selection costs two memory round
// trips whatever V is.
template <int MPT>
__global__ __launch_bounds__(NT) void select_kernel(SelectArgs a) {
  const int r = blockIdx.x, tid = threadIdx.x, V = a.V;
  extern __shared__ float sm[];
  int P2 = 1;                            // V rounded up to a power of two
  while (P2 < V) P2 <<= 1;
  float* v = sm;                         // [V] logits -> processed -> tempered -> p
  float* cp = v + V;                     // [P2] compacted survivor p (top-k candidates before that)
  int* cid = (int*)(cp + P2);            // [P2] compacted survivor ids
  float* sp = (float*)(cid + P2);        // [V] survivors in (p desc, id asc) order
  int* sid = (int*)(sp + V);             // [V]
  __shared__ float redf[8];
  __shared__ int redi[8];
  __shared__ __align__(16) int hist[NT / 64 * 256];
  __shared__ int scan[NT];
  __shared__ int sh_int[4];
  __shared__ float sh_f[2];

  // this row's logits (element tid + q NT), the seen bits they need and, for
  // the code-predictor epilogue, the feedback row: one batch of loads
  const float* lg = a.logits + (long)r * a.ld;
  float lv[MPT];
  uint32_t sw[MPT];
#pragma unroll
  for (int q = 0; q < MPT; ++q) lv[q] = lg[min(tid + q * NT, V - 1)];
  // (no seen bits without a seen array: the penalty is then off)
  const bool has_seen = a.processors && a.seen != nullptr;
  if (has_seen) {
    const uint32_t* seen = a.seen + (long)r * a.seen_words;
#pragma unroll
    for (int q = 0; q < MPT; ++q) sw[q] = seen[min((tid + q * NT) >> 5, a.seen_words - 1)];
  }
  constexpr int EPT = 8;                 // feedback elements per thread (tab_dim <= EPT * NT)
  float fbv[EPT];
  const bool epi_fast = a.epi == 1 && a.tab_dim <= EPT * NT;
  if (epi_fast)
#pragma unroll
    for (int q = 0; q < EPT; ++q) fbv[q] = a.fb[(long)r * a.fb_ld + min(tid + q * NT, a.tab_dim - 1)];
  const int kf0 = a.frame_k ? *a.frame_k : 0, kf = kf0;
  const int forced_v = a.forced ? a.forced[(long)r * a.forced_ld + a.forced_col] : 0;
  const int fin = a.epi == 2 ? a.finished[r] : 0;

  // settings: from the request block when given
  int do_sample = a.do_sample, top_k = a.top_k, min_new = a.min_new, max_frames = a.max_frames;
  float temperature = a.temperature, top_p = a.top_p, penalty = a.penalty;
  uint64_t seed = a.seed;
  const float* text = a.text;
  const float* pad = a.pad;
  int has_text = a.text_len != nullptr;
  if (a.req) {
    const SampParams sp = a.req->samp[a.which];
    do_sample = sp.do_sample; top_k = sp.top_k; min_new = sp.min_new; temperature = sp.temperature;
    top_p = sp.top_p; penalty = sp.penalty; seed = a.req->seed; max_frames = a.req->max_frames;
    text = a.req->text; pad = a.req->pad; has_text = a.req->has_text;
  }
  const int jsel = (a.ctr ? *a.ctr : 0) + a.ctr_add;
  float padv[EPT] = {};
  if (epi_fast && a.add_text)
#pragma unroll
    for (int q = 0; q < EPT; ++q) padv[q] = pad[min(tid + q * NT, a.tab_dim - 1)];
  int choice = 0;
  if (!do_sample && !a.processed_out) {
    // greedy: the non-finite check, the processors and the argmax (lowest
    // id on ties) in one pass over the logits, one exchange between waves
    const bool pen = has_seen && penalty != 1.0f;
    float bv = -INFINITY;
    int bi = 0x7fffffff, badl = 0;
#pragma unroll
    for (int q = 0; q < MPT; ++q) {
      const int i = tid + q * NT;
      if (i >= V) break;
      float x = lv[q];
      badl |= isnan(x) || x == INFINITY;
      if (a.processors) {
        if (pen && ((sw[q] >> (i & 31)) & 1u)) x = x < 0.f ? x * penalty : x / penalty;
        if (i == a.eos && jsel < min_new) x = -INFINITY;
        if (i >= a.sup_b && i < a.sup_e && i != a.eos) x = -INFINITY;
      }
      better(bv, bi, x, i);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) better(bv, bi, __shfl_xor(bv, o), __shfl_xor(bi, o));
    const int wbad = __any(badl);
    const int lane = tid & 63, wv = tid >> 6;
    if (lane == 0) { redf[wv] = bv; redi[wv] = bi; redi[4 + wv] = wbad; }
    __syncthreads();
    bv = redf[0]; bi = redi[0];
    int bad = redi[4];
#pragma unroll
    for (int q = 1; q < NT / 64; ++q) { better(bv, bi, redf[q], redi[q]); bad |= redi[4 + q]; }
    if (bad) {
      if (tid == 0) atomicOr(a.status, ST_NONFINITE);
    } else {
      choice = bi < V ? bi : 0;   // every logit -inf cannot happen: EOS or codes survive
    }
  } else {
  int bad = 0;
  const bool pen = has_seen && penalty != 1.0f;
#pragma unroll
  for (int q = 0; q < MPT; ++q) {
    const int i = tid + q * NT;
    if (i >= V) break;
    float x = lv[q];
    if (isnan(x) || x == INFINITY) bad = 1;
    if (a.processors) {
      if (pen && ((sw[q] >> (i & 31)) & 1u)) x = x < 0.f ? x * penalty : x / penalty;
      if (i == a.eos && jsel < min_new) x = -INFINITY;
      if (i >= a.sup_b && i < a.sup_e && i != a.eos) x = -INFINITY;
    }
    lv[q] = x;
    v[i] = x;
  }
  bad = block_or(bad, redi);
  if (a.processed_out)
    for (int i = tid; i < V; i += NT) a.processed_out[(long)r * V + i] = v[i];

  if (bad) {
    if (tid == 0) atomicOr(a.status, ST_NONFINITE);
  } else if (!do_sample) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int i = tid; i < V; i += NT) better(bv, bi, v[i], i);
    choice = block_argmax(bv, bi, redf, redi);
    if (choice >= V) choice = 0;   // every logit -inf (cannot happen: EOS or codes survive)
  } else {
    // probabilities in registers, element tid + q NT (every pass over the row
    // is register arithmetic plus a block reduction; no LDS round trips)
    float pv[MPT];
    if (a.probs_in) {
#pragma unroll
      for (int q = 0; q < MPT; ++q) pv[q] = a.probs_in[(long)r * V + min(tid + q * NT, V - 1)];
#pragma unroll
      for (int q = 0; q < MPT; ++q) if (tid + q * NT >= V) pv[q] = 0.f;
    } else {
#pragma unroll
      for (int q = 0; q < MPT; ++q) pv[q] = tid + q * NT < V ? lv[q] / temperature : -INFINITY;
      if (top_k > 0 && top_k < V) {
        // radix select of the k-th largest value, 8 bits at a time from the top;
        // per-wave histograms, then a parallel suffix count finds the digit
        uint32_t prefix = 0, mask = 0;
        int kk = top_k;
        const int lane = tid & 63, wv = tid >> 6;
        for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
          for (int q = 0; q < NT / 64; ++q) hist[q * 256 + tid] = 0;
          __syncthreads();
#pragma unroll
          for (int q = 0; q < MPT; ++q) {
            const uint32_t key = ord_key(pv[q]);
            if (tid + q * NT < V && (key & mask) == prefix) atomicAdd(&hist[wv * 256 + ((key >> shift) & 255u)], 1);
          }
          __syncthreads();
          int h = 0;   // count of digit tid
#pragma unroll
          for (int q = 0; q < NT / 64; ++q) h += hist[q * 256 + tid];
          int sfx = h;   // inclusive suffix count over digits >= tid, within the wave
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_down(sfx, o);
            if (lane + o < 64) sfx += t;
          }
          if (lane == 0) scan[wv] = sfx;
          __syncthreads();
          for (int q = wv + 1; q < NT / 64; ++q) sfx += scan[q];
          const int above = sfx - h;   // count of digits > tid
          if (sfx >= kk && above < kk) {   // exactly one digit: the k-th largest lies in it
            sh_int[0] = tid;
            sh_int[1] = kk - above;
          }
          __syncthreads();
          prefix |= ((uint32_t)sh_int[0]) << shift;
          mask |= 255u << shift;
          kk = sh_int[1];
          __syncthreads();
        }
        const float tau = key_float(prefix);
#pragma unroll
        for (int q = 0; q < MPT; ++q) if (pv[q] < tau) pv[q] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int q = 0; q < MPT; ++q) mx = fmaxf(mx, pv[q]);
      mx = block_max(mx, redf);
      float sum = 0.f;
#pragma unroll
      for (int q = 0; q < MPT; ++q) {
        const float e = expf(pv[q] - mx);
        pv[q] = e;
        sum += e;
      }
      sum = block_sum(sum, redf);
#pragma unroll
      for (int q = 0; q < MPT; ++q) pv[q] = pv[q] / sum;
    }
    // Few survivors (p > 0): they are gathered (in any order: the ranks below
    // make the result independent of it) and one wave ranks them by (p desc,
    // id asc), runs the sequential top-p sum in rank order and the race.
    if (tid == 0) sh_int[2] = 0;
    __syncthreads();
    int* tid_list = (int*)cid;
    float* tp_list = cp;
#pragma unroll
    for (int q = 0; q < MPT; ++q) {
      const int i = tid + q * NT;
      if (i < V && pv[q] > 0.f) {
        const int slot = atomicAdd(&sh_int[2], 1);
        tp_list[slot] = pv[q];
        tid_list[slot] = i;
      }
    }
    __syncthreads();
    const int nsv = sh_int[2];
    if (nsv <= 64) {
      if (tid < 64) {
        const int lane = tid;
        const float pp = lane < nsv ? tp_list[lane] : -1.f;
        const int id = lane < nsv ? tid_list[lane] : 0x7fffffff;
        // rank in (p desc, id asc) order: every lane against every survivor,
        // broadcast with lane reads, 4 survivors per step (padding lanes hold
        // p = -1 and never rank above a survivor)
        int rank = 0;
        for (int j0 = 0; j0 < nsv; j0 += 4) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int j = min(j0 + u, 63);
            const float pj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pp), j));
            const int ij = __builtin_amdgcn_readlane(id, j);
            // bitwise, not short-circuit: no branch per compare
            rank += (int)((j0 + u < nsv) & ((pj > pp) | ((pj == pp) & (ij < id))));
          }
        }
        // sequential fp32 running sum in that order, 4 ranks per step: the
        // survivor of rank r is the lane whose rank is r
        int keep = nsv;
        if (top_p < 1.0f) {
          float cs = 0.f;
          bool found = false;
          for (int r0 = 0; r0 < nsv && !found; r0 += 4) {
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const unsigned long long bm = __ballot(rank == r0 + u);
              const int src = bm ? __ffsll(bm) - 1 : 0;
              v[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pp), src));
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const bool act = !found & (r0 + u < nsv);
              cs = act ? cs + v[u] : cs;
              const bool hit = act & (cs >= top_p);
              keep = hit ? r0 + u + 1 : keep;
              found = found | hit;
            }
          }
        }
        float sc = -INFINITY;
        int bi = 0x7fffffff;
        if (lane < nsv && rank < keep) {
          const float e = a.noise_in ? a.noise_in[(long)r * V + id] : exp_noise(seed, r, a.stream, jsel, id);
          sc = pp / e;
          bi = id;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) better(sc, bi, __shfl_xor(sc, o), __shfl_xor(bi, o));
        if (lane == 0) sh_int[2] = bi < V ? bi : 0;
      }
      __syncthreads();
      choice = sh_int[2];
    } else {
#pragma unroll
    for (int q = 0; q < MPT; ++q) if (tid + q * NT < V) v[tid + q * NT] = pv[q];
    __syncthreads();
    // compact survivors (p > 0) in index order: contiguous chunk per thread + scan
    const int chunk = (V + NT - 1) / NT;
    const int b0 = tid * chunk, b1 = min(V, b0 + chunk);
    int cnt = 0;
    for (int i = b0; i < b1; ++i) cnt += v[i] > 0.f;
    // exclusive prefix of the counts in thread order: within the wave, then
    // across the waves' totals
    const int lane = tid & 63, wv = tid >> 6;
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    if (lane == 63) scan[wv] = incl;
    __syncthreads();
    int ns = 0, o = incl - cnt;
#pragma unroll
    for (int q = 0; q < NT / 64; ++q) {
      if (q < wv) o += scan[q];
      ns += scan[q];
    }
    for (int i = b0; i < b1; ++i)
      if (v[i] > 0.f) { cp[o] = v[i]; cid[o] = i; ++o; }
    __syncthreads();
    // Order by (p desc, id asc), which only top-p needs (the race is order
    // free): ranks for a few survivors, a bitonic sort of the padded list in
    // place for many.
    const float* spo = sp;
    const int* sido = sid;
    if (top_p >= 1.0f) {
      spo = cp;
      sido = cid;
    } else if (ns <= 2 * NT) {
      for (int c = tid; c < ns; c += NT) {
        const float pc = cp[c];
        const int ic = cid[c];
        int rank = 0;
        for (int j = 0; j < ns; ++j) {
          const float pj = cp[j];
          rank += (pj > pc) || (pj == pc && cid[j] < ic);
        }
        sp[rank] = pc;
        sid[rank] = ic;
      }
      __syncthreads();
    } else {
      for (int i = ns + tid; i < P2; i += NT) { cp[i] = -1.f; cid[i] = 0x7fffffff; }   // padding sorts last
      __syncthreads();
      for (int k = 2; k <= P2; k <<= 1)
        for (int j = k >> 1; j > 0; j >>= 1) {
          for (int i = tid; i < P2; i += NT) {
            const int l = i ^ j;
            if (l > i) {
              const float pa = cp[i], pb = cp[l];
              const int ia = cid[i], ib = cid[l];
              const bool b_first = pb > pa || (pb == pa && ib < ia);
              const bool a_first = pa > pb || (pa == pb && ia < ib);
              if ((i & k) == 0 ? b_first : a_first) {
                cp[i] = pb; cp[l] = pa; cid[i] = ib; cid[l] = ia;
              }
            }
          }
          __syncthreads();
        }
      spo = cp;
      sido = cid;
    }
    if (tid == 0) {
      // sequential fp32 cumulative sum in (p desc, id asc) order; reads batched by 8
      int keep = ns;
      if (top_p < 1.0f) {
        float cs = 0.f;
        for (int j0 = 0; j0 < ns && keep == ns; j0 += 8) {
          float t[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) t[e] = j0 + e < ns ? spo[j0 + e] : 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (keep == ns && j0 + e < ns) {
              cs += t[e];
              if (cs >= top_p) keep = j0 + e + 1;
            }
        }
      }
      sh_int[2] = keep;
    }
    __syncthreads();
    const int keep = sh_int[2];
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int j = tid; j < keep; j += NT) {
      const int id = sido[j];
      const float e = a.noise_in ? a.noise_in[(long)r * V + id]
                                 : exp_noise(seed, r, a.stream, jsel, id);
      better(bv, bi, spo[j] / e, id);
    }
    choice = block_argmax(bv, bi, redf, redi);
    if (choice >= V) choice = 0;
    }
  }
  }

  // commit
  if (tid == 0) {
    int used = choice;
    if (a.forced) used = forced_v;
    a.used[(long)r * a.used_ld + a.used_col] = used;
    if (a.own) a.own[(long)r * a.own_ld + a.own_col] = choice;
    sh_int[3] = used;
    if (a.epi == 2) {
      const int kf = a.frame_k ? kf0 : -1;
      if (fin) {
        a.state[r] = 3;
      } else if (used == a.eos) {
        a.state[r] = 1;
        a.finished[r] = 1;
      } else if (kf >= 0 && kf + 1 >= max_frames) {
        a.state[r] = 2;
        a.finished[r] = 1;
      } else {
        a.state[r] = 0;
      }
    }
  }
  __syncthreads();
  if (epi_fast) {
    const int used = sh_int[3];
    const long base = (a.tab_off + used) * (long)a.tab_dim;
    const bool txt = a.add_text && has_text && kf < a.text_len[r];
    float tv[EPT], xt[EPT];
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const int k = min(tid + q * NT, a.tab_dim - 1);
      tv[q] = ld_any(a.tab, a.tab_dtype, base + k);
      xt[q] = txt ? text[((long)a.text_off[r] + kf) * a.tab_dim + k] : padv[q];
    }
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const int k = tid + q * NT;
      if (k >= a.tab_dim) break;
      if (a.next_in) a.next_in[(long)r * a.next_ld + k] = tv[q];
      float f = fbv[q] + tv[q];
      if (a.add_text) f = f + xt[q];
      a.fb[(long)r * a.fb_ld + k] = f;
    }
  } else if (a.epi == 1) {
    const int used = sh_int[3];
    const long base = (a.tab_off + used) * (long)a.tab_dim;
    const bool txt = a.add_text && has_text && kf < a.text_len[r];
    for (int k = tid; k < a.tab_dim; k += NT) {
      const float val = ld_any(a.tab, a.tab_dtype, base + k);
      if (a.next_in) a.next_in[(long)r * a.next_ld + k] = val;
      float f = a.fb[(long)r * a.fb_ld + k] + val;
      if (a.add_text) f = f + (txt ? text[((long)a.text_off[r] + kf) * a.tab_dim + k] : pad[k]);
      a.fb[(long)r * a.fb_ld + k] = f;
    }
  }
}

template <int MPT>
static hipError_t launch_select_t(const SelectArgs& a, hipStream_t s) {
  size_t p2 = 1;
  while (p2 < (size_t)a.V) p2 <<= 1;
  const size_t lds = ((size_t)a.V * 3 + 2 * p2) * sizeof(float);
  static size_t have = 0;
  hipError_t e = ensure_lds((const void*)select_kernel<MPT>, lds, &have);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_kernel<MPT>, dim3(a.B), dim3(NT), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  if (a.V < 1 || a.V > 24 * NT) return hipErrorInvalidValue;
  if (a.V <= 4 * NT) return launch_select_t<4>(a, s);
  if (a.V <= 8 * NT) return launch_select_t<8>(a, s);
  if (a.V <= 12 * NT) return launch_select_t<12>(a, s);
  if (a.V <= 16 * NT) return launch_select_t<16>(a, s);
  return launch_select_t<24>(a, s);
}

// ---------------------------------------------------------------- frame control
__global__ __launch_bounds__(NT) void frame_start_kernel(FrameStartArgs a) {
  const int r = blockIdx.x, tid = threadIdx.x;
  __shared__ int sh;
  if (tid == 0) {
    int c = a.finished[r] ? a.eos : (a.forced ? a.forced[(long)r * a.forced_ld] : a.code0_next[r]);
    if (c < 0 || c >= a.V) { atomicOr(a.status, ST_RANGE); c = 0; }
    if (!a.finished[r]) a.seen[(long)r * a.seen_words + (c >> 5)] |= 1u << (c & 31);
    a.codes[(long)r * 16] = c;
    sh = c;
  }
  __syncthreads();
  const int c = sh;
  if (a.rope_rows) {
    const long pr = (long)a.pos[r] * a.half;
    for (int j = tid; j < a.half; j += NT) {
      a.rope_rows[(long)r * 2 * a.half + j] = a.cos[pr + j];
      a.rope_rows[(long)r * 2 * a.half + a.half + j] = a.sin[pr + j];
    }
  }
  const long tb = (long)c * a.H;
  for (int k = tid; k < a.H; k += NT) {
    const float t = ld_any(a.temb, a.tdtype, tb + k);
    a.pass0[(long)(2 * r) * a.pass0_ld + k] = a.h[(long)r * a.H + k];
    a.pass0[(long)(2 * r + 1) * a.pass0_ld + k] = t;
    a.fb[(long)r * a.fb_ld + k] = t;
  }
}

hipError_t launch_frame_start(const FrameStartArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(frame_start_kernel, dim3(a.B), dim3(NT), 0, s, a);
  return hipGetLastError();
}

__global__ void frame_advance_kernel(int* frame_k, int* pos, int B) {
  const int t = threadIdx.x;
  for (int r = t; r < B; r += blockDim.x) pos[r] += 1;
  if (t == 0) *frame_k += 1;
}

hipError_t launch_frame_advance(int* frame_k, int* pos, int B, hipStream_t s) {
  hipLaunchKernelGGL(frame_advance_kernel, dim3(1), dim3(NT), 0, s, frame_k, pos, B);
  return hipGetLastError();
}

__global__ void copy_rows_kernel(const float* src, long ld_src, const int* idx, float* dst, long ld_dst, int n) {
  const int i = blockIdx.x;
  const float* s = src + (long)idx[i] * ld_src;
  float* d = dst + (long)i * ld_dst;
  for (int k = threadIdx.x; k < n; k += blockDim.x) d[k] = s[k];
}

hipError_t launch_copy_rows(const float* src, long ld_src, const int* idx, int count, float* dst, long ld_dst,
                            int n, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_rows_kernel, dim3(count), dim3(NT), 0, s, src, ld_src, idx, dst, ld_dst, n);
  return hipGetLastError();
}

__global__ void convert_kernel(const void* src, int sdt, long ld_src, void* dst, int ddt, long ld_dst,
                               long rows, int n) {
  const long total = rows * n;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < total; i += (long)gridDim.x * blockDim.x) {
    const long rr = i / n, c = i % n;
    if (sdt == ddt && sdt == DT_BF16) {
      ((uint16_t*)dst)[rr * ld_dst + c] = ((const uint16_t*)src)[rr * ld_src + c];
    } else {
      const float x = ld_any(src, sdt, rr * ld_src + c);
      if (ddt == DT_BF16) ((uint16_t*)dst)[rr * ld_dst + c] = f32_to_bf16(x);
      else ((float*)dst)[rr * ld_dst + c] = x;
    }
  }
}

hipError_t launch_convert(const void* src, int sdtype, long ld_src, void* dst, int ddtype, long ld_dst, long rows,
                          int n, hipStream_t s) {
  const long total = rows * n;
  if (total <= 0) return hipSuccess;
  long blocks = (total + NT - 1) / NT;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(convert_kernel, dim3((unsigned)blocks), dim3(NT), 0, s, src, sdtype, ld_src, dst, ddtype, ld_dst,
                     rows, n);
  return hipGetLastError();
}

__global__ void fill_i32_kernel(int* p, int v, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) p[i] = v;
}

hipError_t launch_fill_i32(int* p, int v, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  long blocks = (n + NT - 1) / NT;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)blocks), dim3(NT), 0, s, p, v, n);
  return hipGetLastError();
}

}  // namespace qt
