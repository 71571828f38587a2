// gfx950 attention kernels of the Qwen3-TTS 12 Hz frame step: fused
// QK-RMSNorm + rope + KV write + GQA attention for decode steps and the
// prompt prefill (per token and tiled on the matrix cores), the split-range
// combine, and the code predictor's attention fused with its o-projection.
#include "qt_device.h"

namespace qt {

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

// The new tokens of a decode step: the q heads and k through QK-RMSNorm and
// rope (one wave per vector, waves wave, wave + nthreads / 64, ...; lane owns
// the rope pair (lane, lane + 64)), the K and V rows to the cache (as stored)
// and to LDS. Without owns_new only the q heads are formed and knew / vnew are
// zeroed (masked keys past a key range may index them: 0 x NaN is NaN).
template <typename KVT, int G, int NTOK>
__device__ __forceinline__ void decode_new_rows(const AttnArgs& p, int g, int row, int pos0, bool owns_new, int nthreads,
                                                float (*qs)[G][128], float (*knew)[128], float (*vnew)[128],
                                                KVT* kc, KVT* vc) {
  constexpr int D = 128, HALF = 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float prs[NTOK];
  const long arow0 = p.tok_stride > 0 ? (long)row * p.tok_stride + p.tok_off : row;
  // split-K partial sums: up to PZ ranges with every load issued before the
  // first add (clamped ranges past part_z are loaded but not added); 4 is
  // the K = 1024 projections' split (8 clamped loads measured 1 % slower per
  // batch-64 frame), more ranges take a loop
  constexpr int PZ = 4;
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
    if (!owns_new)
      for (int i = tid; i < D; i += nthreads) { knew[t][i] = 0.f; vnew[t][i] = 0.f; }
    for (int v = wave; v <= (owns_new ? G + 1 : G - 1); v += nthreads / 64) {
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
}

// Decode attention for head_dim 128, one kernel launch for the NTOK new
// tokens of every row (NTOK = 2: the predictor's two-token pass at positions
// 0 and 1; NTOK = 1: single steps with fp32 caches or 1 or 4 q heads per kv
// head, the others take attn_stream_kernel). Block = (kv head, row).
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

  // the new tokens: QK-RMSNorm + rope of q heads and k, K/V rows to the cache and LDS
  decode_new_rows<KVT, G, NTOK>(p, g, row, pos0, owns_new, NT, qs, knew, vnew, kc, vc);
  const long arow0 = p.tok_stride > 0 ? (long)row * p.tok_stride + p.tok_off : row;
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
          s[r][hh] += dpp_f<0xb1, 0xf>(s[r][hh], 0.f);   // quad_perm [1,0,3,2]: lane l ^ 1
          s[r][hh] += dpp_f<0x4e, 0xf>(s[r][hh], 0.f);   // quad_perm [2,3,0,1]: lane l ^ 2
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
        static_assert(CPK == 16 || CPK == 32, "key slots 16 or 32 lanes apart");
        if constexpr (CPK == 16) v = add_xor<16>(v);
        v = add_xor<32>(v);
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

// Single-token decode attention for head_dim 128, G = 2 and a 16-bit cache,
// streamed by independent waves. Block = (kv head, row[, key range]) of NW
// waves. After the new token's prologue wave w takes the 16-key chunks w,
// w + NW, ... of the block's cached keys with no block-wide synchronisation:
// lane l holds 16 bytes (dims 8 (l % 16) .. + 7) of key 4 i + l / 16 (i =
// 0..3) of a chunk, for K and for V, so every load instruction reads 1 KB
// contiguous, and NB chunks per wave are in flight (a register set reloads
// with the wave's chunk NB steps ahead as soon as it has been used). A
// lane's 8 partial dot products (4 keys x 2 heads) are added over the 16
// lanes of its row by a reduce-scatter (lane distance 8, 2, 1, then a full
// add at distance 4), which leaves key i = 2 b3 + b1 and head b0 in lane l
// (b: the bits of l, lanes l and l ^ 4 alike). Each wave keeps its own running max and sums; the last
// wave (the one with the fewest chunks) adds the new key from LDS, and the
// waves are combined once at the end. SPLIT: the block's keys are one range
// of kv_split, left as a partial for attn_split_combine_kernel.
template <typename KVT, int NW, int NB, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void attn_stream_kernel(AttnArgs p) {
  constexpr int G = 2, D = 128, CH = 16, NTH = NW * 64;
  static_assert(sizeof(KVT) == 2 && NTH >= G * D, "16-bit cache, one thread per output");
  const int g = blockIdx.x, row = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int dsl = lane & 15, ksl = lane >> 4;       // dims slot, key slot
  const bool b0 = lane & 1, b1 = lane & 2, b2 = lane & 4, b3 = lane & 8;
  __shared__ __align__(16) float qs[1][G][D];
  __shared__ __align__(16) float knew[1][D], vnew[1][D];
  __shared__ __align__(16) float wacc[NW][G][D];
  __shared__ float wm[NW][G], wl[NW][G];
  KVT* kc = (KVT*)p.kc + (long)row * p.row_stride + (long)g * p.max_pos * D;
  KVT* vc = (KVT*)p.vc + (long)row * p.row_stride + (long)g * p.max_pos * D;
  const int pos0 = p.pos_base + (p.row_pos ? p.row_pos[row] : 0);
  int kb = 0, ke = pos0;                            // cached keys kb .. ke - 1
  bool owns_new = true;
  if constexpr (SPLIT) {
    const int S = gridDim.z, sp = blockIdx.z;
    const int per = ((pos0 + S - 1) / S + CH * NW - 1) / (CH * NW) * (CH * NW);
    kb = min(sp * per, pos0);
    ke = min(kb + per, pos0);
    owns_new = sp == S - 1;
  }
  const int nch = (ke - kb + CH - 1) / CH;
  u32x4 kbuf[NB][4], vbuf[NB][4];
  auto load = [&](u32x4 (&kd)[4], u32x4 (&vd)[4], int n) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const long j = min(kb + n * CH + 4 * i + ksl, ke - 1);
      kd[i] = *(const u32x4*)(kc + j * D + dsl * 8);
      vd[i] = *(const u32x4*)(vc + j * D + dsl * 8);
    }
  };
#pragma unroll
  for (int b = 0; b < NB; ++b)
    if (wave + b * NW < nch) load(kbuf[b], vbuf[b], wave + b * NW);

  decode_new_rows<KVT, G, 1>(p, g, row, pos0, owns_new, NTH, qs, knew, vnew, kc, vc);
  __syncthreads();

  // lane l ^ 4 of the row: quad_perm [3,2,1,0] (l ^ 3), then row_half_mirror
  // (l ^ 7), both over the whole wave (a select between two row shifts would
  // become a branch, and a lane move from disabled lanes reads nothing)
  auto xor4 = [](float v) __attribute__((always_inline)) { return dpp_f<0x141, 0xf>(dpp_f<0x1b, 0xf>(v, 0.f), 0.f); };
  float q[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) q[h][e] = qs[0][h][dsl * 8 + e];
  float m[G] = {-INFINITY, -INFINITY}, acc[G][8], lsum = 0.f;
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  // (exponentials as __expf, one hardware exp2 of x log2 e: 3.50 -> 3.45 ms
  // per batch-8 frame against expf here and in the short kernel)
  // one step of the online softmax: s is this lane's score (head b0; -inf if
  // masked; lanes l and l ^ 4 alike), counted in the lane's sum if cnt;
  // add_pv gets the lane's weight once the maxima and sums are rescaled
  auto update = [&](float s, bool cnt, auto&& add_pv) __attribute__((always_inline)) {
    float mx = fmaxf(s, dpp_f<0x4e, 0xf>(s, -INFINITY));
    mx = fmaxf(mx, dpp_f<0x128, 0xf>(mx, -INFINITY));
    mx = max_xor<16>(mx);
    mx = max_xor<32>(mx);
    const float other = dpp_f<0xb1, 0xf>(mx, -INFINITY);
    float corr[G];
    const float mc0 = fmaxf(m[0], b0 ? other : mx), mc1 = fmaxf(m[1], b0 ? mx : other);
    corr[0] = __expf(m[0] - mc0);
    corr[1] = __expf(m[1] - mc1);
    m[0] = mc0;
    m[1] = mc1;
    const float pw = s == -INFINITY ? 0.f : __expf(s - (b0 ? mc1 : mc0));
    lsum = lsum * (b0 ? corr[1] : corr[0]) + (cnt ? pw : 0.f);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= corr[h];
    add_pv(pw);
  };
  auto chunk = [&](const u32x4 (&kd)[4], const u32x4 (&vd)[4], int n) __attribute__((always_inline)) {
    float sc[4][G];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x[8];
      unpack_chunk<KVT>(kd[i], x);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaf(q[h][e], x[e], a);
        sc[i][h] = a;
      }
    }
    // reduce-scatter over the 16 lanes of the row: index t = 2 i + h
    float v4[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float lo = sc[t >> 1][t & 1], hi = sc[2 + (t >> 1)][t & 1];
      v4[t] = (b3 ? hi : lo) + dpp_f<0x128, 0xf>(b3 ? lo : hi, 0.f);     // row_ror:8: lane l ^ 8
    }
    float v2[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) v2[u] = (b1 ? v4[2 + u] : v4[u]) + dpp_f<0x4e, 0xf>(b1 ? v4[u] : v4[2 + u], 0.f);
    float v1 = (b0 ? v2[1] : v2[0]) + dpp_f<0xb1, 0xf>(b0 ? v2[0] : v2[1], 0.f);
    v1 += xor4(v1);
    const int key = kb + n * CH + 4 * ((b3 ? 2 : 0) + (b1 ? 1 : 0)) + ksl;
    update(key < ke ? v1 * p.scale : -INFINITY, !b2, [&](float pw) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x[8];
        unpack_chunk<KVT>(vd[i], x);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float w = __shfl(pw, (lane & 0x30) | ((i >> 1) << 3) | ((i & 1) << 1) | h);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(w, x[e], acc[h][e]);
        }
      }
    });
  };
  for (int n0 = wave; n0 < nch; n0 += NB * NW) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int n = n0 + b * NW;
      if (n >= nch) break;
      chunk(kbuf[b], vbuf[b], n);
      if (n + NB * NW < nch) load(kbuf[b], vbuf[b], n + NB * NW);   // the buffer's next chunk
    }
  }
  if (owns_new && wave == NW - 1) {
    // the new key (every row of the wave forms its score; row 0 adds its value)
    float a[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) t = fmaf(q[h][e], knew[0][dsl * 8 + e], t);
      t += dpp_f<0xb1, 0xf>(t, 0.f);
      t += dpp_f<0x4e, 0xf>(t, 0.f);
      t += dpp_f<0x141, 0xf>(t, 0.f);
      t += dpp_f<0x140, 0xf>(t, 0.f);
      a[h] = t * p.scale;
    }
    // every lane holds both scores; lanes 0 and 1 count head b0 in the sums
    update(b0 ? a[1] : a[0], (lane & ~1) == 0, [&](float) __attribute__((always_inline)) {
      if (ksl == 0)
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float w = __expf(a[h] - m[h]);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(w, vnew[0][dsl * 8 + e], acc[h][e]);
        }
    });
  }
  // the wave's totals: rows of keys, then the softmax sums of each head
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = add_xor<32>(add_xor<16>(acc[h][e]));
  float lt = lsum + dpp_f<0x4e, 0xf>(lsum, 0.f);
  lt += xor4(lt);
  lt += dpp_f<0x128, 0xf>(lt, 0.f);
  lt = add_xor<32>(add_xor<16>(lt));
  if (ksl == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      *(f32x4*)&wacc[wave][h][dsl * 8] = (f32x4){acc[h][0], acc[h][1], acc[h][2], acc[h][3]};
      *(f32x4*)&wacc[wave][h][dsl * 8 + 4] = (f32x4){acc[h][4], acc[h][5], acc[h][6], acc[h][7]};
    }
  }
  if (lane < G) { wm[wave][lane] = m[lane]; wl[wave][lane] = lt; }
  __syncthreads();
  if (tid < G * D) {
    const int hh = tid / D, dim = tid % D;
    float M = wm[0][hh];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, wm[w][hh]);
    float v = 0.f, ls = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = wm[w][hh] == -INFINITY ? 0.f : __expf(wm[w][hh] - M);
      v = fmaf(f, wacc[w][hh][dim], v);
      ls = fmaf(f, wl[w][hh], ls);
    }
    if constexpr (SPLIT) {
      float* sb = p.split_buf + ((((long)row * p.nkv + g) * gridDim.z + blockIdx.z) * G + hh) * (D + 2);
      sb[dim] = v;
      if (dim == 0) { sb[D] = M; sb[D + 1] = ls; }
    } else {
      const long arow = p.tok_stride > 0 ? (long)row * p.tok_stride + p.tok_off : row;
      p.out[arow * p.ld_out + (long)(g * G + hh) * D + dim] = v / ls;
    }
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
    const float w = m[sp] == -INFINITY ? 0.f : __expf(m[sp] - mx);
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

// Decode attention over at most 16 positions (the code predictor's steps at
// batch rows > 1, NTOK = 1, and its two-token pass at positions 0 and 1,
// NTOK = 2, activation rows 2 r and 2 r + 1), head_dim 128, 16-bit cache.
// Block = (kv head, row), G + 2 waves per new token: waves 0..G-1 take the q
// heads of the group, wave G the new key, wave G + 1 the new value
// (QK-RMSNorm + rope as in attn_step_kernel, the K/V rows to the cache and
// LDS); after the one barrier each q-head wave finishes alone (token t
// attends to the cached keys and the new keys 0..t). Scores: lane = (key l % 16,
// quarter l / 16 of the dims), the quarters added with two shuffles; the
// softmax over the 16 keys stays in 16-lane groups; P.V: lane = 2 dims, the
// key weights broadcast by shuffles. Every cache load leaves before the
// prologue (clamped to the cached keys).
template <typename KVT, int G, int NTOK = 1>
__global__ __launch_bounds__(NTOK * (G + 2) * 64) void attn_short_kernel(AttnArgs p) {
  constexpr int D = 128, HALF = 64;
  const int g = blockIdx.x, row = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = wave / (G + 2), role = wave % (G + 2);   // new token, vector of it
  __shared__ __align__(16) float qs[NTOK][G][D];
  __shared__ __align__(16) float knew[NTOK][D];
  __shared__ __align__(16) float vnew[NTOK][D];
  KVT* kc = (KVT*)p.kc + (long)row * p.row_stride + (long)g * p.max_pos * D;
  KVT* vc = (KVT*)p.vc + (long)row * p.row_stride + (long)g * p.max_pos * D;
  const int pos0 = p.pos_base + (p.row_pos ? p.row_pos[row] : 0);
  const int jk = lane & 15, qd = lane >> 4;
  const int last = max(pos0 - 1, 0);
  u32x4 kr[4];
  uint32_t vr[16];
  if (role < G) {
    const KVT* kp = kc + (long)min(jk, last) * D + 32 * qd;
#pragma unroll
    for (int c = 0; c < 4; ++c) kr[c] = *(const u32x4*)(kp + 8 * c);
#pragma unroll
    for (int j = 0; j < 16; ++j) vr[j] = *(const uint32_t*)(vc + (long)min(j, last) * D + 2 * lane);
  }
  // q/k/v of the new token: the projection's rows, its split-K partial sums,
  // or the row of the code-indexed table that the row's code selects
  const long ar = p.tok_stride > 0 ? (long)row * p.tok_stride + p.tok_off + t : row;
  const float* qrow = p.qkv + ar * p.ld_qkv;
  if (p.lut_codes) qrow = p.lut + (long)min(max(p.lut_codes[(long)row * p.lut_code_ld], 0), p.lut_rows - 1) * p.lut_ld;
  // up to PZ ranges with every load issued before the first add (ranges past
  // part_z are clamped loads that are not added); more ranges: a loop
  constexpr int PZ = 4;
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
    if (p.part_z <= 0) return qrow[col];
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
    const int pos = pos0 + t;
    float cs, sn;
    if (p.rope_rows) {
      cs = p.rope_rows[(long)row * D + lane];
      sn = p.rope_rows[(long)row * D + HALF + lane];
    } else {
      cs = p.cos[(long)pos * HALF + lane];
      sn = p.sin[(long)pos * HALF + lane];
    }
    const int v = role;
    if (v == G + 1) {                       // value row, stored as is
      const long col = (long)(p.nq + p.nkv) * D + (long)g * D;
      const float x1 = qkv_at(col + lane), x2 = qkv_at(col + lane + HALF);
      st_elem<KVT>(vc, (long)pos * D + lane, x1);
      st_elem<KVT>(vc, (long)pos * D + lane + HALF, x2);
      vnew[t][lane] = kv_round<KVT>(x1);
      vnew[t][lane + HALF] = kv_round<KVT>(x2);
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
  if (role >= G) return;
  const int hh = role, L = pos0 + t + 1;   // keys 0 .. pos0 + t
  float x[32];
  if (jk < pos0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) unpack_chunk<KVT>(kr[c], x + 8 * c);
  } else {
    const int jn = min(jk - pos0, NTOK - 1);
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] = jk < L ? knew[jn][32 * qd + e] : 0.f;
  }
  const f32x4* q4 = (const f32x4*)&qs[t][hh][32 * qd];
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const f32x4 qa = q4[e], qb = q4[e + 1];
    s0 = fmaf(qa.x, x[4 * e], s0); s0 = fmaf(qa.y, x[4 * e + 1], s0); s0 = fmaf(qa.z, x[4 * e + 2], s0); s0 = fmaf(qa.w, x[4 * e + 3], s0);
    s1 = fmaf(qb.x, x[4 * e + 4], s1); s1 = fmaf(qb.y, x[4 * e + 5], s1); s1 = fmaf(qb.z, x[4 * e + 6], s1); s1 = fmaf(qb.w, x[4 * e + 7], s1);
  }
  float sc = s0 + s1;
  sc = add_xor<16>(sc);
  sc = add_xor<32>(sc);
  sc = jk < L ? sc * p.scale : -INFINITY;
  // max and sum over the 16 keys of a row of 16 lanes: DPP quad permutes, then the half-row and row mirrors
  float mx = sc;
  mx = fmaxf(mx, dpp_f<0xb1, 0xf>(mx, -INFINITY));
  mx = fmaxf(mx, dpp_f<0x4e, 0xf>(mx, -INFINITY));
  mx = fmaxf(mx, dpp_f<0x141, 0xf>(mx, -INFINITY));
  mx = fmaxf(mx, dpp_f<0x140, 0xf>(mx, -INFINITY));
  const float ew = jk < L ? __expf(sc - mx) : 0.f;
  float lsum = ew;
  lsum += dpp_f<0xb1, 0xf>(lsum, 0.f);
  lsum += dpp_f<0x4e, 0xf>(lsum, 0.f);
  lsum += dpp_f<0x141, 0xf>(lsum, 0.f);
  lsum += dpp_f<0x140, 0xf>(lsum, 0.f);
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float pj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ew), j));   // lanes 0..15 hold the key weights
    float v0, v1;
    if (j < pos0) {
      if constexpr (std::is_same<KVT, _Float16>::value) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        const h2 h = __builtin_bit_cast(h2, vr[j]);
        v0 = (float)h[0]; v1 = (float)h[1];
      } else {
        v0 = bf_lo(vr[j]); v1 = bf_hi(vr[j]);
      }
    } else if (j < L) {
      const int jn = min(j - pos0, NTOK - 1);
      v0 = vnew[jn][2 * lane]; v1 = vnew[jn][2 * lane + 1];
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
    ss = add_xor<16>(ss);
    ss = add_xor<32>(ss);
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

  // scores in base-2 units (times scale log2 e): each weight is then one
  // hardware exp2 (81 -> 74.5 us per chunk and layer at batch 64 against expf)
  float m = -INFINITY, lsum = 0.f;
  const float sl2 = p.scale * 1.4426950408889634f;
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
          const float v = key <= qpos ? sc[kt][r] * sl2 : -INFINITY;   // masked: -inf, whose exp2 is 0
          sc[kt][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = max_xor<16>(mx);
      mx = max_xor<32>(mx);
      const float mnew = fmaxf(m, mx);     // finite: key 0 is in every query's range
      const float corr = __builtin_amdgcn_exp2f(m - mnew);
      m = mnew;
      float ps = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __builtin_amdgcn_exp2f(sc[kt][r] - mnew);
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
  lsum = add_xor<16>(lsum);
  lsum = add_xor<32>(lsum);
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
    if (attention_reads_lut(a)) {
      hipLaunchKernelGGL((attn_short_kernel<KVT, G>), dim3(a.nkv, a.n_runs), dim3((G + 2) * 64), 0, s, a);
      return hipGetLastError();
    }
    // the predictor's two-token pass at batch rows > 1 (activation rows 2 r, 2 r + 1)
    if (a.single_token && a.mode == ATT_WRITE_ATTEND && a.ntok == 2 && a.tok_stride == 2 && a.tok_off == 0 &&
        a.max_pos >= 2 && a.max_pos <= 16 && a.n_runs > 1 && !a.lut_codes && !a.rope_rows && a.ld_out % 2 == 0) {
      hipLaunchKernelGGL((attn_short_kernel<KVT, G, 2>), dim3(a.nkv, a.n_runs), dim3(2 * (G + 2) * 64), 0, s, a);
      return hipGetLastError();
    }
  }
  if constexpr (D == 128 && G <= 4) {
    const int nt = a.ntok > 0 ? a.ntok : 1;
    if (a.single_token && a.mode == ATT_WRITE_ATTEND && (nt == 1 || (nt == 2 && a.tok_stride == 2 && a.tok_off == 0))) {
      constexpr int big = 512 / sizeof(KVT), small = 64;
      const dim3 grid(a.nkv, a.n_runs);
      const bool split = nt == 1 && a.split_buf && (a.kv_split == 2 || a.kv_split == 4 || a.kv_split == 8 || a.kv_split == 16);
      if constexpr (G == 2 && sizeof(KVT) == 2) {
        // one token per row: the wave-streaming kernel (4 waves, 3 chunks in
        // flight per wave), measured 4.3 against 5.2 us at 41 keys and batch 1,
        // 9.5 against 10.6 us at batch 8 (4 key ranges) and 23.4 against
        // 25.6 us at batch 64 (128..512-key prompts)
        if (nt == 1) {
          if (split) {
            hipLaunchKernelGGL((attn_stream_kernel<KVT, 4, 3, true>), dim3(a.nkv, a.n_runs, a.kv_split), dim3(256), 0, s, a);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            return launch_split_combine<G>(a, s);
          }
          hipLaunchKernelGGL((attn_stream_kernel<KVT, 4, 3, false>), grid, dim3(256), 0, s, a);
          return hipGetLastError();
        }
      }
      // (the two-token pass; other caches and groupings) large chunks when
      // the grid is at most one block per compute unit and contexts can be
      // long (not the code predictor's 16 positions: 64-key chunks measured
      // 5.1 against 5.7 us there)
      const bool one_wave = (long)a.nkv * a.n_runs <= 256 && a.max_pos > small;
      if (split) {
        hipLaunchKernelGGL((attn_step_kernel<KVT, G, 1, small, true>), dim3(a.nkv, a.n_runs, a.kv_split), dim3(NT), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_split_combine<G>(a, s);
      }
      // several blocks per compute unit and long contexts: 128-key chunks
      // (measured at the batch-64 talker before the wave-streaming kernel:
      // 6.17 against 6.20 ms per frame with 64 and 6.60 with 256)
      if (nt == 2) hipLaunchKernelGGL((attn_step_kernel<KVT, G, 2, small>), grid, dim3(NT), 0, s, a);
      else if (one_wave) hipLaunchKernelGGL((attn_step_kernel<KVT, G, 1, big>), grid, dim3(NT), 0, s, a);
      else if (a.max_pos > small) hipLaunchKernelGGL((attn_step_kernel<KVT, G, 1, 2 * small>), grid, dim3(NT), 0, s, a);
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
// rows [b RO, (b + 1) RO) (with RO < NKV, NKV / RO waves share a row, each
// taking a K part, and the parts are added in order through LDS); block 0
// also writes the new K/V rows.
// Scores: lane = (key j, quarter of the head dims); P·V: lane = (8-dim
// column chunk, key slot j mod 4).
// SEL (steps 1..14, one token): the step's code is the greedy selection over
// the previous head's logits (AttnArgs::sel; each wave takes the argmax of
// its 256 logits, one LDS exchange combines them), the q/k/v values are that
// code's row of the first layer's code-indexed table and the residual row
// that code's input row; block 0 commits the code and the feedback sum.
template <typename KVT, int NKV, int G, int RO, int NTOK, bool SEL = false>
__global__ __launch_bounds__(NKV * 64) void pred_attn_o_kernel(AttnArgs p, LinearArgs o) {
  constexpr int D = 128, HALF = 64, NQ = NKV * G, KO = NQ * D;
  constexpr int EPC = 8;                       // 16-bit cache elements per 16-byte chunk
  constexpr int RW = RO >= NKV ? RO / NKV : 1; // o rows per wave
  constexpr int KS = RO >= NKV ? 1 : NKV / RO; // waves sharing one o row (K split, RO < NKV)
  constexpr int KC = KO / 512 / KS;            // 16-byte weight chunks per lane and row
  static_assert(sizeof(KVT) == 2 && (RO % NKV == 0 || NKV % RO == 0) && KO % (512 * KS) == 0, "layout");
  static_assert(!SEL || NTOK == 1, "a folded selection feeds one token");
  constexpr int FPT = SEL ? 2048 / (NKV * 64) : 1;   // feedback elements per thread (tab_dim <= 2048)
  const int g = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ks = KS > 1 ? g / RO : 0;          // this wave's K part of its row
  const int n0 = KS > 1 ? blockIdx.x * RO + g % RO : blockIdx.x * RO + g * RW;
  const int kc0 = ks * KC;                     // first weight chunk of the K part
  __shared__ float opart[KS > 1 ? NKV : 1][NTOK];
  __shared__ __align__(16) float qs[NKV][NTOK][G][D];
  __shared__ __align__(16) float knew[NKV][NTOK][D];
  __shared__ __align__(16) float vnew[NKV][NTOK][D];
  __shared__ __align__(16) float att[NTOK][KO];
  __shared__ float selv[SEL ? NKV : 1];
  __shared__ int seli[SEL ? NKV : 1], selb[SEL ? NKV : 1];

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
  auto load_xin = [&](const float* base, long ld) {
#pragma unroll
    for (int t = 0; t < NTOK; ++t) {
      const float* src = base + (long)t * ld;
#pragma unroll
      for (int v = 0; v < G + 2; ++v) {
        const float* x = src + (v < G ? (long)(g * G + v) * D : (long)(NQ + (v - G) * NKV) * D + (long)g * D);
        xin[t][v][0] = x[lane];
        xin[t][v][1] = x[lane + HALF];
      }
    }
  };
  // SEL: this wave's 256 logits and (block 0) the feedback row's old values
  // go first; the q/k/v row waits for the code
  f32x4 lgv = {};
  float fbo[FPT];
  if constexpr (SEL) {
    lgv = *(const f32x4*)(p.sel.logits + min((g * 64 + lane) * 4, p.sel.V - 4));
    if (blockIdx.x == 0)
#pragma unroll
      for (int e = 0; e < FPT; ++e) fbo[e] = p.sel.fb[min((int)threadIdx.x + e * NKV * 64, p.sel.tab_dim - 1)];
  } else {
    load_xin(p.qkv, p.ld_qkv);
  }
#pragma unroll
  for (int t = 0; t < NTOK; ++t) {
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
    for (int c = 0; c < KC; ++c) w[r][c] = ld_weight(W + (long)(n0 + r) * KO + (kc0 + c) * 512 + lane * 8);
  // the residual's old values, so that the epilogue has no dependent load
  float yold[NTOK][RW];
  if constexpr (!SEL)
#pragma unroll
    for (int t = 0; t < NTOK; ++t)
#pragma unroll
      for (int r = 0; r < RW; ++r) yold[t][r] = o.Y[(long)t * o.ldy + n0 + r];
  __builtin_amdgcn_sched_barrier(0);
  float tabv[FPT];
  int code = 0;
  if constexpr (SEL) {
    // argmax, lowest id on ties: per wave the largest value (NaN ignored,
    // flagged) and the lowest id holding it, then the waves in order
    const int V = p.sel.V;
    const float lq[4] = {lgv.x, lgv.y, lgv.z, lgv.w};
    float lv[4];
    int badl = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool in = (g * 64 + lane) * 4 + e < V;
      badl |= in && (isnan(lq[e]) || lq[e] == INFINITY);
      lv[e] = in ? lq[e] : -INFINITY;
    }
    const float wmax = wave_max(fmaxf(fmaxf(lv[0], lv[1]), fmaxf(lv[2], lv[3])));
    int ci = 0x7fffffff;
#pragma unroll
    for (int e = 3; e >= 0; --e) ci = lv[e] == wmax ? (g * 64 + lane) * 4 + e : ci;
    const int wi = wave_min_i(ci);
    const int wbad = __any(badl);
    if (lane == 0) { selv[g] = wmax; seli[g] = wi; selb[g] = wbad; }
    __syncthreads();
    float bv = selv[0];
    int bi = seli[0], bad = selb[0];
#pragma unroll
    for (int w = 1; w < NKV; ++w) { better(bv, bi, selv[w], seli[w]); bad |= selb[w]; }
    code = bad || bi >= V ? 0 : bi;
    // the code's q/k/v row, residual values and (block 0) table row
    load_xin(p.lut + (long)code * p.lut_ld, 0);
    const uint16_t* trow = (const uint16_t*)p.sel.tab + (p.sel.tab_off + code) * (long)p.sel.tab_dim;
#pragma unroll
    for (int r = 0; r < RW; ++r)
      yold[0][r] = p.xlut ? p.xlut[(long)code * o.N + n0 + r] : bf16_to_f32(trow[n0 + r]);
    if (blockIdx.x == 0) {
#pragma unroll
      for (int e = 0; e < FPT; ++e) tabv[e] = bf16_to_f32(trow[min((int)threadIdx.x + e * NKV * 64, p.sel.tab_dim - 1)]);
      if (threadIdx.x == 0) {
        p.sel.used[p.sel.col] = code;
        if (p.sel.own) p.sel.own[p.sel.col] = code;
        if (bad) atomicOr(p.sel.status, ST_NONFINITE);
      }
    }
  }

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
      pr[hh] = __expf(s[hh] - mx);
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
        v = add_xor<16>(v);
        v = add_xor<32>(v);
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
        const f32x4* x4 = (const f32x4*)(&att[t][(kc0 + c) * 512 + lane * 8]);
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
      if constexpr (KS == 1) {
        if (lane == 0) o.Y[(long)t * o.ldy + n0 + r] = yold[t][r] + a;
      } else if (lane == 0) {
        opart[g][t] = a;
      }
    }
  }
  if constexpr (KS > 1) {
    // the K parts of each row, added in part order
    __syncthreads();
    if (ks == 0 && lane == 0)
#pragma unroll
      for (int t = 0; t < NTOK; ++t) {
        float a = opart[g][t];
#pragma unroll
        for (int q = 1; q < KS; ++q) a += opart[g + q * RO][t];
        o.Y[(long)t * o.ldy + n0] = yold[t][0] + a;
      }
  }
  if constexpr (SEL) {
    if (blockIdx.x == 0)
#pragma unroll
      for (int e = 0; e < FPT; ++e) {
        const int k = threadIdx.x + e * NKV * 64;
        if (k < p.sel.tab_dim) p.sel.fb[k] = fbo[e] + tabv[e];
      }
  }
}

template <typename KVT>
static hipError_t launch_pred_attn_o_t(const AttnArgs& a, const LinearArgs& o, hipStream_t s) {
  // 4 output rows per block, each row's dot product split over two waves:
  // 256 blocks at the 0.6B shape. Per batch-1 frame (70 launches) this
  // measured 2.081 ms against 2.085 with 8 rows per block (128 blocks); 16
  // rows per block (64 blocks) measured 0.6 us slower per launch than 8.
  constexpr int RO = 4;
  if (a.ntok == 2) hipLaunchKernelGGL((pred_attn_o_kernel<KVT, 8, 2, RO, 2>), dim3(o.N / RO), dim3(512), 0, s, a, o);
  else if (a.sel.logits) hipLaunchKernelGGL((pred_attn_o_kernel<KVT, 8, 2, RO, 1, true>), dim3(o.N / RO), dim3(512), 0, s, a, o);
  else hipLaunchKernelGGL((pred_attn_o_kernel<KVT, 8, 2, RO, 1>), dim3(o.N / RO), dim3(512), 0, s, a, o);
  return hipGetLastError();
}

bool attention_reads_lut(const AttnArgs& a) {
  return a.d == 128 && a.nq == 2 * a.nkv && (a.kvdtype == DT_F16 || a.kvdtype == DT_BF16) && a.single_token &&
         a.mode == ATT_WRITE_ATTEND && a.ntok <= 1 && a.max_pos <= 16 && a.n_runs > 1 && a.ld_out % 2 == 0;
}

bool attention_oproj_sel_ok(int nq, int nkv, int d, int kvdtype, int wdtype, int V, int tab_dim) {
  return nq == 16 && nkv == 8 && d == 128 && (kvdtype == DT_F16 || kvdtype == DT_BF16) && wdtype == DT_BF16 &&
         V >= 4 && V <= 2048 && V % 4 == 0 && tab_dim >= 1 && tab_dim <= 2048;
}

hipError_t launch_attention_oproj(const AttnArgs& a, const LinearArgs& o, hipStream_t s) {
  // one new token per launch, or the two-token pass (positions 0 and 1: 1.943
  // against 1.962 ms per batch-1 frame with the separate attention and o-projection)
  const int nt = a.ntok > 0 ? a.ntok : 1;
  const bool ok = a.single_token && a.mode == ATT_WRITE_ATTEND && a.n_runs == 1 && a.d == 128 && a.nkv == 8 &&
                  a.nq == 16 && a.ld_qkv >= (long)(a.nq + 2 * a.nkv) * a.d && a.part_z <= 0 && !a.row_pos && !a.rope_rows && a.max_pos <= 16 &&
                  a.pos_base >= 0 && a.pos_base + nt <= a.max_pos &&
                  (nt == 1 || (nt == 2 && a.tok_stride == 2 && a.tok_off == 0)) && (nt == 2 || a.tok_stride == 0) &&
                  (a.kvdtype == DT_F16 || a.kvdtype == DT_BF16) &&
                  o.wdtype == DT_BF16 && o.K == a.nq * a.d && o.N % 8 == 0 && o.M == nt && o.epi == EPI_RESIDUAL &&
                  !o.gain && o.ldx == o.K && o.X == a.out && a.ld_out == o.K;
  if (!ok) return hipErrorNotSupported;
  if (a.sel.logits) {
    // a folded selection must run here: every pointer set, the table rows
    // within the weight layout, the residual rows the o-projection's width
    const SelFold& f = a.sel;
    if (nt != 1 || !a.lut || a.lut_ld < (long)(a.nq + 2 * a.nkv) * a.d || !f.tab || !f.used || !f.fb || !f.status ||
        f.tab_off < 0 || !attention_oproj_sel_ok(a.nq, a.nkv, a.d, a.kvdtype, o.wdtype, f.V, f.tab_dim) ||
        (!a.xlut && f.tab_dim != o.N))
      return hipErrorInvalidValue;
  }
  if (a.kvdtype == DT_F16) return launch_pred_attn_o_t<_Float16>(a, o, s);
  return launch_pred_attn_o_t<uint16_t>(a, o, s);
}

}  // namespace qt
