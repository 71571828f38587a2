// gfx950 kernels of the token-id frontend of the Qwen3-TTS talker: the text
// embedding gather, the ResizeMLP's bias + SiLU between its two projections
// (the projections themselves run through launch_linear), and the dual-track
// assembly of prompt rows (text track + codec track + optional extra rows).
// HBM-bound elementwise work: rows are read and written with 16-byte
// vector accesses, one block per row.
#include "qt_device.h"

namespace qt {

// X[i, :] = float(embed[ids[i], :]) for ids[i] >= 0, zeros otherwise.
// One block per row; a thread moves 8 elements (16 bytes of bf16).
template <typename WT>
__global__ __launch_bounds__(NT) void gather_rows_kernel(const WT* __restrict__ embed, int width,
                                                         const int* __restrict__ ids, float* __restrict__ X) {
  const int i = blockIdx.x;
  const int id = ids[i];
  float* x = X + (long)i * width;
  for (int c = threadIdx.x * 8; c < width; c += NT * 8) {
    float v[8];
    if (id >= 0) {
      const WT* e = embed + (long)id * width + c;
      if constexpr (sizeof(WT) == 2) {
        const u32x4 w = *(const u32x4*)e;
        v[0] = bf_lo(w.x); v[1] = bf_hi(w.x); v[2] = bf_lo(w.y); v[3] = bf_hi(w.y);
        v[4] = bf_lo(w.z); v[5] = bf_hi(w.z); v[6] = bf_lo(w.w); v[7] = bf_hi(w.w);
      } else {
        const f32x4 a = *(const f32x4*)e, b = *(const f32x4*)(e + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    *(f32x4*)(x + c) = (f32x4){v[0], v[1], v[2], v[3]};
    *(f32x4*)(x + c + 4) = (f32x4){v[4], v[5], v[6], v[7]};
  }
}

// Hd[i, :] = silu(Hd[i, :] + b) (b may be null: zero bias).
__global__ __launch_bounds__(NT) void bias_silu_kernel(float* __restrict__ Hd, int width, const float* __restrict__ b) {
  float* h = Hd + (long)blockIdx.x * width;
  for (int c = threadIdx.x * 4; c < width; c += NT * 4) {
    f32x4 v = *(f32x4*)(h + c);
    if (b) {
      const f32x4 bb = *(const f32x4*)(b + c);
      v.x += bb.x; v.y += bb.y; v.z += bb.z; v.w += bb.w;
    }
    v.x = v.x / (1.f + expf(-v.x));
    v.y = v.y / (1.f + expf(-v.y));
    v.z = v.z / (1.f + expf(-v.z));
    v.w = v.w / (1.f + expf(-v.w));
    *(f32x4*)(h + c) = v;
  }
}

// out[i, :] = (tid >= 0 ? Y[i, :] + b2 : 0) + (cid >= 0 ? codec[cid, :] : 0) + (extra ? extra[i, :] : 0)
template <typename WT>
__global__ __launch_bounds__(NT) void assemble_rows_kernel(const float* __restrict__ Y, const float* __restrict__ b2,
                                                           const int* __restrict__ tids, const int* __restrict__ cids,
                                                           const WT* __restrict__ codec, const float* __restrict__ extra,
                                                           float* __restrict__ out, int width) {
  const int i = blockIdx.x;
  const int tid = tids[i], cid = cids[i];
  for (int c = threadIdx.x * 4; c < width; c += NT * 4) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (tid >= 0) {
      v = *(const f32x4*)(Y + (long)i * width + c);
      if (b2) {
        const f32x4 bb = *(const f32x4*)(b2 + c);
        v.x += bb.x; v.y += bb.y; v.z += bb.z; v.w += bb.w;
      }
    }
    if (cid >= 0) {
      const WT* e = codec + (long)cid * width + c;
      v.x += ld_elem<WT>(e, 0); v.y += ld_elem<WT>(e, 1); v.z += ld_elem<WT>(e, 2); v.w += ld_elem<WT>(e, 3);
    }
    if (extra) {
      const f32x4 x = *(const f32x4*)(extra + (long)i * width + c);
      v.x += x.x; v.y += x.y; v.z += x.z; v.w += x.w;
    }
    *(f32x4*)(out + (long)i * width + c) = v;
  }
}

hipError_t launch_gather_rows(const void* embed, int wdtype, int width, const int* ids, int n, float* X, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (width % 8) return hipErrorInvalidValue;
  if (wdtype == DT_BF16)
    hipLaunchKernelGGL(gather_rows_kernel<uint16_t>, dim3(n), dim3(NT), 0, s, (const uint16_t*)embed, width, ids, X);
  else
    hipLaunchKernelGGL(gather_rows_kernel<float>, dim3(n), dim3(NT), 0, s, (const float*)embed, width, ids, X);
  return hipGetLastError();
}

hipError_t launch_bias_silu(float* Hd, int n, int width, const float* b, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (width % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bias_silu_kernel, dim3(n), dim3(NT), 0, s, Hd, width, b);
  return hipGetLastError();
}

hipError_t launch_assemble_rows(const float* Y, const float* b2, const int* tids, const int* cids, const void* codec,
                                int wdtype, const float* extra, float* out, int n, int width, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (width % 4) return hipErrorInvalidValue;
  if (wdtype == DT_BF16)
    hipLaunchKernelGGL(assemble_rows_kernel<uint16_t>, dim3(n), dim3(NT), 0, s, Y, b2, tids, cids,
                       (const uint16_t*)codec, extra, out, width);
  else
    hipLaunchKernelGGL(assemble_rows_kernel<float>, dim3(n), dim3(NT), 0, s, Y, b2, tids, cids, (const float*)codec,
                       extra, out, width);
  return hipGetLastError();
}

}  // namespace qt
