// gfx950 projection kernels of the Qwen3-TTS 12 Hz frame step: the
// weight-streaming GEMVs with fused RMSNorm prologues and residual / SwiGLU
// epilogues, the matrix-core GEMVs and row-block GEMMs of small batches, and
// the prompt prefill's tiled MFMA GEMM. Activations fp32, weights fp32 or
// bf16, fp32 accumulation.
#include "qt_device.h"

namespace qt {

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

constexpr int GK = 32;        // K per LDS stage
constexpr int GLD = GK + 8;   // padded LDS row (bf16 elements)


template <int BM, int BN>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(BM == 128 ? 3 : 8)))
void mfma_gemm_kernel(LinearArgs p, const float* __restrict__ den) {
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
  // D(i, j) of a 32x32 tile: lane j + 32 * ((i / 4) % 2), register (i / 8) * 4 + i % 4;
  // a tile's residual values are all loaded before its first store
#pragma unroll
  for (int ti = 0; ti < TM; ++ti)
#pragma unroll
    for (int tj = 0; tj < TN; ++tj) {
      float yo[16];
      if (p.epi == EPI_RESIDUAL)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const int row = min(m0 + wm * (BM / 2) + ti * 32 + i, M - 1);
          const int col = min(n0 + wn * (BN / 2) + tj * 32 + (lane & 31), N - 1);
          yo[r] = p.Y[(long)row * p.ldy + col];
        }
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
          p.Y[(long)row * p.ldy + col] = p.epi == EPI_RESIDUAL ? yo[r] + v : v;
        }
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

// LDS tile addressing: 32-element (64-byte) rows, 16-byte chunk c of row r
// stored at chunk c ^ ((r >> 2) & 3). The MFMA operand reads (rows r .. r + 31,
// one chunk each, two chunks per row across the wave halves) then fall on
// distinct banks: measured on gfx950, this layout and 80-byte padded rows read
// without bank conflicts, c ^ ((r >> 1) & 3) is 2-way conflicted.
struct SplitLds {
  static constexpr int LD = GK;
  __device__ static int at(int r, int c) {   // c: element offset, a multiple of 8
    return r * LD + (((c >> 3) ^ ((r >> 2) & 3)) << 3);
  }
};

// FA (no gain: the o and down projections): the activations are read as
// fp32 rows instead and split into the hi + lo LDS planes on the way in, so
// no prologue writes the planes.
// SNK: the SnakeBeta epilogue of a convolution. WN: waves along N (2 or 4;
// 4 gives a 512-thread block on a 64 TM x 128 TN tile). RES: the residual
// epilogue (its old values take registers only in this variant).
template <int TM, int TN, bool FA = false, bool SNK = false, int WN = 2, bool RES = false>
__global__ __launch_bounds__(128 * WN) __attribute__((amdgpu_waves_per_eu(WN == 4 ? 4 : SNK && RES ? 2 : 3)))
void gemm_split_kernel(LinearArgs p, const uint16_t* __restrict__ xs) {
  using LT = SplitLds;
  constexpr int GLD_ = LT::LD;
  constexpr int NT = 128 * WN;                    // threads: 2 x WN waves
  constexpr int BM = 64 * TM, BN = 32 * WN * TN;
  constexpr int AF = FA ? BM * GK / 4 / NT : 1;  // fp32 16-byte chunks per thread per stage (FA)
  constexpr int AV = FA ? 1 : BM * GK / 8 / NT;  // 16-byte chunks per thread per stage, each A plane
  constexpr int BV = BN * GK / 8 / NT;            // and of W
  constexpr int BUF = (2 * BM + BN) * GLD_;        // bf16 elements of one stage: A hi, A lo, W
  __shared__ __attribute__((aligned(16))) uint16_t sm[2 * BUF];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
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
      // a convolution's K slice k0 lies in one tap j: its rows are shifted back
      long a_k = k0;
      if (p.conv_taps > 0) {
        const int j = k0 / p.conv_cin;
        a_k = (long)(k0 - j * p.conv_cin) - (long)(p.conv_taps - 1 - j) * p.conv_dil * p.ldx;
      }
#pragma unroll
      for (int q = 0; q < AF; ++q) raf[q] = *(const u32x4*)(af_src[q] + a_k);
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
        const int r = wn * (BN / WN) + j * 32 + (lane & 31);
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
  // D(i, j) of a 32x32 tile: lane j + 32 * ((i / 4) % 2), register (i / 8) * 4 + i % 4.
  // A tile's residual values (and the lane's SnakeBeta parameters) are all
  // loaded before its first store, so the tile costs one memory round trip
  // rather than one per element.
  float sa[TN], sb[TN];
  if constexpr (SNK)
#pragma unroll
    for (int tj = 0; tj < TN; ++tj) {
      const int col = min(n0 + wn * (BN / WN) + tj * 32 + (lane & 31), N - 1);
      sa[tj] = p.snake_alpha[col];
      sb[tj] = p.snake_bden[col];
    }
#pragma unroll
  for (int ti = 0; ti < TM; ++ti)
#pragma unroll
    for (int tj = 0; tj < TN; ++tj) {
      float yo[16];
      if constexpr (RES)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const int row = min(m0 + wm * (BM / 2) + ti * 32 + i, M - 1);
          const int col = min(n0 + wn * (BN / WN) + tj * 32 + (lane & 31), N - 1);
          yo[r] = p.Y[(long)row * p.ldy + col];
        }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int row = m0 + wm * (BM / 2) + ti * 32 + i;
        const int col = n0 + wn * (BN / WN) + tj * 32 + (lane & 31);
        const float v = acc[ti][tj][r];
        if (!RES && p.epi == EPI_SWIGLU) {
          // the (gate, up) pair sits in lanes 2c, 2c+1; hardware exp2 and reciprocal
          // (gate/up 3.8 % faster per 8192-row chunk than expf and a division)
          const float u = __shfl_xor(v, 1);
          if (!(lane & 1) && row < M && col + 1 < N) p.Y[(long)row * p.ldy + (col >> 1)] = v * __frcp_rn(1.f + __expf(-v)) * u;
        } else if (row < M && col < N) {
          float* y = p.Y + (long)row * p.ldy + col;
          float o = v;
          if constexpr (RES) o += yo[r];
          if constexpr (SNK) {
            const float so = snake_beta(o, sa[tj], sb[tj]);
            if (p.Y2) {
              *y = o;
              p.Y2[(long)row * p.ldy2 + col] = so;
            } else {
              *y = so;
            }
          } else {
            *y = o;
          }
        }
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
template <bool RES>
static hipError_t launch_gemm_split_t(const LinearArgs& a, hipStream_t s) {
  uint16_t* xs = (uint16_t*)a.xs;
  const bool fa = a.conv_taps > 0 || (!a.gain && !a.norm_out && a.M >= 2048);
  if (!fa) hipLaunchKernelGGL(split_rows_kernel, dim3(a.M), dim3(NT), 0, s, a, xs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long big = (long)((a.M + 127) / 128) * ((a.N + 127) / 128);
  if (!RES && a.N >= 4096 && a.M >= 2048 && !a.snake_alpha) {
    // wide projections (q/k/v, gate/up): 8 waves on 128 x 256 tiles, measured
    // 5-18 % faster than 4 waves on 128 x 128 at 8192 rows
    dim3 grid((a.N + 255) / 256, (a.M + 127) / 128);
    if constexpr (!RES) {
      if (fa) hipLaunchKernelGGL((gemm_split_kernel<2, 2, true, false, 4>), grid, dim3(512), 0, s, a, xs);
      else hipLaunchKernelGGL((gemm_split_kernel<2, 2, false, false, 4>), grid, dim3(512), 0, s, a, xs);
    }
  } else if (big >= 512) {
    dim3 grid((a.N + 127) / 128, (a.M + 127) / 128);
    if (a.snake_alpha) hipLaunchKernelGGL((gemm_split_kernel<2, 2, true, true, 2, RES>), grid, dim3(NT), 0, s, a, xs);
    else if (fa) hipLaunchKernelGGL((gemm_split_kernel<2, 2, true, false, 2, RES>), grid, dim3(NT), 0, s, a, xs);
    else hipLaunchKernelGGL((gemm_split_kernel<2, 2, false, false, 2, RES>), grid, dim3(NT), 0, s, a, xs);
  } else {
    dim3 grid((a.N + 127) / 128, (a.M + 63) / 64);
    if (a.snake_alpha) hipLaunchKernelGGL((gemm_split_kernel<1, 2, true, true, 2, RES>), grid, dim3(NT), 0, s, a, xs);
    else if (fa) hipLaunchKernelGGL((gemm_split_kernel<1, 2, true, false, 2, RES>), grid, dim3(NT), 0, s, a, xs);
    else hipLaunchKernelGGL((gemm_split_kernel<1, 2, false, false, 2, RES>), grid, dim3(NT), 0, s, a, xs);
  }
  return hipGetLastError();
}

static hipError_t launch_gemm_split(const LinearArgs& a, hipStream_t s) {
  if (a.epi == EPI_RESIDUAL) return launch_gemm_split_t<true>(a, s);
  return launch_gemm_split_t<false>(a, s);
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
      for (int q = 0; q < WV; ++q) wv[st][q] = ld_weight_cached(wrow[q] + k0 + st * SG_GK);
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
  // D(i, j) of the 32x32 tile: lane j + 32 * ((i / 4) % 2), register (i / 8) * 4 + i % 4;
  // the residual's old values are all loaded before the first store
  const int col = n0 + wn * 32 + (lane & 31);
  float yo[16];
  if (direct && p.epi == EPI_RESIDUAL)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = min(m0 + wm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3), M - 1);
      yo[r] = p.Y[(long)row * p.ldy + min(col, N - 1)];
    }
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
      p.Y[(long)row * p.ldy + col] = p.epi == EPI_RESIDUAL ? yo[r] + v : v;
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
    for (int st = 0; st < NS; ++st) wv[st][q] = ld_weight_cached(wr + st * SG_GK);
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
  // D(i, j) of the 32x32 tile: lane j + 32 * ((i / 4) % 2), register (i / 8) * 4 + i % 4;
  // the residual's old values are all loaded before the first store
  const int col = n0 + wn * 32 + (lane & 31);
  float yo[16];
  if (direct && p.epi == EPI_RESIDUAL)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = min(m0 + wm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3), M - 1);
      yo[r] = p.Y[(long)row * p.ldy + min(col, N - 1)];
    }
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
      p.Y[(long)row * p.ldy + col] = p.epi == EPI_RESIDUAL ? yo[r] + v : v;
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
// the output tiles alone give kRowsDirectTiles blocks; else single-group
// blocks over the fewest K ranges that give about 256 blocks, limited by the
// partial-sum space.
constexpr int kRowsDirectTiles = 192;
static bool rows_plan(const LinearArgs& a, RowsPlan* pl) {
  if (a.wdtype != DT_BF16 || a.M < 17 || a.M > 128 || a.K % SG_CH || a.N % 4 || a.ldx % 4 || a.ldy % 2 ||
      (a.norm_out && a.ld_norm % 2))
    return false;
  const long tiles = (long)((a.N + SG_T - 1) / SG_T) * ((a.M + SG_T - 1) / SG_T);
  const int chunks = a.K / SG_CH;
  if (tiles >= kRowsDirectTiles)
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
      q = add_xor<16>(q);
      q = add_xor<32>(q);
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
    ss += dpp_f<0x128, 0xf>(ss, 0.f);   // row_ror:8, lane l ^ 8 within its row of 16
    ss = add_xor<16>(ss);
    ss = add_xor<32>(ss);
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
    if (a.N % (8 * t) == 0 && a.N / (8 * t) >= 256) { T = t; break; }
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
  // a causal convolution as one GEMM: only the split GEMM's fp32 loader
  // reads shifted rows
  if (a.conv_taps > 0) {
    if (a.wdtype != DT_BF16 || a.gain || a.norm_out || a.epi == EPI_SWIGLU || a.conv_cin % GK ||
        a.K != a.conv_taps * a.conv_cin || a.ldx % 4 || a.conv_dil < 1 || (a.snake_alpha && !a.snake_bden))
      return hipErrorInvalidValue;
    return launch_gemm_split(a, s);
  }
  if (a.snake_alpha) return hipErrorInvalidValue;
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

}  // namespace qt
