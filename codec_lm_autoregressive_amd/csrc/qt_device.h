// Shared device helpers of the gfx950 kernels (types, bf16 conversions,
// DPP wave reductions, block reductions). Included by every kernel source.
#pragma once
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

// Weight rows are streamed once per pass, with nontemporal loads.
__device__ __forceinline__ u32x4 ld_weight(const void* p) { return __builtin_nontemporal_load((const u32x4*)p); }
// Ordinary cached loads of weight rows, for kernels whose blocks share a row
// group (the 17..128-row GEMMs: measured faster there, slower in the GEMVs).
__device__ __forceinline__ u32x4 ld_weight_cached(const void* p) { return *(const u32x4*)p; }

// ---------------------------------------------------------------- helpers
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

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

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }
// Round to nearest even; inputs are finite activations.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// SnakeBeta x + sin(alpha x)^2 / bden with the hardware sine: the argument is
// taken to revolutions, reduced to [-1/2, 1/2] (rounding to nearest), then
// v_sin_f32; the reciprocal is v_rcp_f32. Within float32 rounding of the
// argument's product for |alpha x| up to a few hundred, which covers the
// decoder's activations.
__device__ __forceinline__ float snake_beta(float x, float alpha, float bden) {
  float rev = alpha * x * 0.15915494309189535f;
  rev -= rintf(rev);
  const float s = __builtin_amdgcn_sinf(rev);
  return x + s * s * __builtin_amdgcn_rcpf(bden);
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

// v combined with its value in lane l ^ O: O = 16 and 32 on the VALU with the
// gfx950 lane-swap instructions (a swap of v with itself leaves lane l's and
// lane l ^ O's values in the two results), other O through a shuffle. The
// same value in either lane order: add and max are commutative.
template <int O>
__device__ __forceinline__ float add_xor(float v) {
  if constexpr (O == 32 || O == 16) {
    const auto r = O == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false)
                           : __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    return v + __shfl_xor(v, O);
  }
}
template <int O>
__device__ __forceinline__ float max_xor(float v) {
  if constexpr (O == 32 || O == 16) {
    const auto r = O == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false)
                           : __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else {
    return fmaxf(v, __shfl_xor(v, O));
  }
}

template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_i(int v, int id) {
  return __builtin_amdgcn_update_dpp(id, v, CTRL, ROWS, 0xf, false);
}
__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, dpp_i<0xb1, 0xf>(v, 0x7fffffff));
  v = min(v, dpp_i<0x4e, 0xf>(v, 0x7fffffff));
  v = min(v, dpp_i<0x141, 0xf>(v, 0x7fffffff));
  v = min(v, dpp_i<0x140, 0xf>(v, 0x7fffffff));
  v = min(v, dpp_i<0x142, 0xa>(v, 0x7fffffff));
  v = min(v, dpp_i<0x143, 0xc>(v, 0x7fffffff));
  return __builtin_amdgcn_readlane(v, 63);
}

// Block-wide reductions for NT threads; `red` is LDS scratch of >= NT/64 floats.
// All threads of the block must call them.
__device__ inline float block_sum(float v, float* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) t += red[i];
  return t;
}
__device__ inline float block_max(float v, float* red) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) t = fmaxf(t, red[i]);
  return t;
}
__device__ inline int block_or(int v, int* redi) {
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
__device__ inline int block_argmax(float v, int i, float* redf, int* redi) {
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

}  // namespace qt
