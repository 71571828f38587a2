// gfx950 selection and frame-control kernels of the Qwen3-TTS 12 Hz frame
// step: the logits processors and the single-sample selection (Philox4x64-10
// exponential race), the frame-start commit of code 0, the code-predictor
// gathers that also build the embedding-sum feedback, and small utilities.
#include "qt_device.h"

namespace qt {

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
// E ~ Exp(1) from one 64-bit word x: u = ((x >> 12) + 1/2) 2^-52 in (0,1),
// E = -ln u in double, rounded to float.
__device__ __forceinline__ float noise_from_word(uint64_t x) {
  const double u = ((double)(x >> 12) + 0.5) * 0x1p-52;
  return (float)(-log(u));
}
__device__ __forceinline__ float exp_noise(uint64_t seed, int row, int stream, int index, int id) {
  return noise_from_word(
      philox_word0((uint64_t)id, (uint64_t)stream, (uint64_t)(int64_t)index, (uint64_t)row, seed, 0ull));
}

// The selection kernel's noise for n counters or words (test entry point):
// mode 0: in[4 i .. 4 i + 3] = (vocab id, stream, selection index, row) under
// key (seed, 0); mode 1: in[i] is the 64-bit word itself.
__global__ __launch_bounds__(NT) void noise_kernel(const uint64_t* in, int mode, uint64_t seed, float* out, long n) {
  const long i = (long)blockIdx.x * NT + threadIdx.x;
  if (i >= n) return;
  if (mode == 0) {
    const uint64_t* c = in + 4 * i;
    out[i] = exp_noise(seed, (int)c[3], (int)c[1], (int)(int64_t)c[2], (int)c[0]);
  } else {
    out[i] = noise_from_word(in[i]);
  }
}
hipError_t launch_noise(const uint64_t* in, int mode, uint64_t seed, float* out, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(noise_kernel, dim3((unsigned)((n + NT - 1) / NT)), dim3(NT), 0, s, in, mode, seed, out, n);
  return hipGetLastError();
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
  const int r = blockIdx.x + a.row0, tid = threadIdx.x, V = a.V;
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
  __shared__ __align__(16) int hist[2][NT / 64 * 256];
  __shared__ __align__(16) float nzs[64];
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
  const int kf0 = a.frame_k ? a.frame_k[r] : 0, kf = kf0;
  const int forced_v = a.forced ? a.forced[(long)r * a.forced_ld + a.forced_col] : 0;
  const int fin = a.epi == 2 ? a.finished[r] : 0;

  // settings: from the request block when given
  int do_sample = a.do_sample, top_k = a.top_k, min_new = a.min_new;
  float temperature = a.temperature, top_p = a.top_p, penalty = a.penalty;
  const uint64_t seed = a.row_seed ? a.row_seed[r] : a.seed;
  const int nrow = a.noise_row ? a.noise_row[r] : r;
  const int max_frames = a.row_max ? a.row_max[r] : a.max_frames;
  const float* text = a.text_ptr ? a.text_ptr[r] : nullptr;
  const float* pad = a.pad;
  const int has_text = text != nullptr && a.text_len != nullptr;
  if (a.req) {
    const SampParams sp = a.req->samp[a.which];
    do_sample = sp.do_sample; top_k = sp.top_k; min_new = sp.min_new; temperature = sp.temperature;
    top_p = sp.top_p; penalty = sp.penalty; pad = a.req->pad;
  }
  const int jsel = (a.ctr ? a.ctr[r] : 0) + a.ctr_add;
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
      float rmax = -INFINITY;                // the row's largest value, once the top-k branch has run
      if (top_k > 0 && top_k < V) {
        // tau = the top_k-th largest value (values equal to it are kept). One
        // histogram of each finite value's distance below the row's largest,
        // in HB linear buckets between the largest and smallest: the bucket
        // index never increases with the value, so the k-th largest lies in
        // the bucket where the count from the top first reaches k, and that
        // bucket's values (at most 64) are ranked exactly by one wave. A
        // fuller bucket falls back to a radix select of the k-th largest.
        constexpr int HB = 2 * (NT / 64) * 256;   // both radix histograms
        int* hb = &hist[0][0];
        const int lane = tid & 63, wv = tid >> 6;
#pragma unroll
        for (int q = 0; q < HB / NT; ++q) hb[q * NT + tid] = 0;
        float lmax = -INFINITY, lmin = INFINITY;
#pragma unroll
        for (int q = 0; q < MPT; ++q)
          if (pv[q] > -INFINITY) { lmax = fmaxf(lmax, pv[q]); lmin = fminf(lmin, pv[q]); }
        lmax = wave_max(lmax);
        lmin = -wave_max(-lmin);
        if (lane == 0) { redf[wv] = lmax; redf[NT / 64 + wv] = lmin; }
        if (tid == 0) { sh_int[0] = -1; sh_int[3] = 0; }
        __syncthreads();
        rmax = redf[0];
        float rmin = redf[NT / 64];
#pragma unroll
        for (int w = 1; w < NT / 64; ++w) { rmax = fmaxf(rmax, redf[w]); rmin = fminf(rmin, redf[NT / 64 + w]); }
        float bsc = (float)HB / (rmax - rmin);
        if (!(bsc < INFINITY) || !(bsc > 0.f)) bsc = 0.f;   // one distinct finite value, or none: bucket 0
        auto bucket = [&](float x) { return (int)fminf((rmax - x) * bsc, (float)(HB - 1)); };
#pragma unroll
        for (int q = 0; q < MPT; ++q)
          if (pv[q] > -INFINITY) atomicAdd(&hb[bucket(pv[q])], 1);
        __syncthreads();
        // counts of this thread's HB / NT buckets, then its place in the
        // count from the top: inclusive prefix within the wave, then the waves
        constexpr int BPT = HB / NT;
        int cb[BPT], sown = 0;
#pragma unroll
        for (int u = 0; u < BPT; ++u) { cb[u] = hb[tid * BPT + u]; sown += cb[u]; }
        int incl = sown;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int t = __shfl_up(incl, o);
          if (lane >= o) incl += t;
        }
        if (lane == 63) scan[wv] = incl;
        __syncthreads();
        int c0 = incl - sown;
        for (int w = 0; w < wv; ++w) c0 += scan[w];
        if (c0 < top_k && top_k <= c0 + sown) {   // exactly one thread: the k-th largest is in its buckets
#pragma unroll
          for (int u = 0; u < BPT; ++u) {
            if (c0 < top_k && top_k <= c0 + cb[u]) { sh_int[0] = tid * BPT + u; sh_int[1] = top_k - c0; sh_int[2] = cb[u]; }
            c0 += cb[u];
          }
        }
        __syncthreads();
        const int bstar = sh_int[0];
        float tau = -INFINITY;                   // fewer finite values than top_k: nothing is cut
        if (bstar >= 0 && sh_int[2] <= 64) {
          const int kk = sh_int[1], cnt = sh_int[2];
#pragma unroll
          for (int q = 0; q < MPT; ++q)
            if (pv[q] > -INFINITY && bucket(pv[q]) == bstar) cp[atomicAdd(&sh_int[3], 1)] = pv[q];
          __syncthreads();
          if (tid < 64) {
            // the kk-th largest of the bucket: more than kk - 1 values above it
            // is impossible, at least kk at or above it
            const float v = lane < cnt ? cp[lane] : -INFINITY;
            int gt = 0, ge = 0;
            for (int j = 0; j < cnt; ++j) {
              const float u = cp[j];
              gt += u > v;
              ge += u >= v;
            }
            if (lane < cnt && gt < kk && kk <= ge) sh_f[0] = v;   // lanes that hold equal values write the same
          }
          __syncthreads();
          tau = sh_f[0];
        } else if (bstar >= 0) {
          // radix select of the k-th largest value, 8 bits at a time from
          // the top; per-wave histograms, then a parallel suffix count finds
          // the digit. Two histogram buffers: a pass clears the next pass's
          // one, so a pass costs three barriers.
          uint32_t prefix = 0, mask = 0;
          int kk = top_k;
#pragma unroll
          for (int q = 0; q < NT / 64; ++q) hist[0][q * 256 + tid] = 0;
          __syncthreads();
          for (int shift = 24, pass = 0; shift >= 0; shift -= 8, ++pass) {
            int* hb = hist[pass & 1];
#pragma unroll
            for (int q = 0; q < MPT; ++q) {
              const uint32_t key = ord_key(pv[q]);
              if (tid + q * NT < V && (key & mask) == prefix) atomicAdd(&hb[wv * 256 + ((key >> shift) & 255u)], 1);
            }
#pragma unroll
            for (int q = 0; q < NT / 64; ++q) hist[(pass + 1) & 1][q * 256 + tid] = 0;
            __syncthreads();
            int h = 0;   // count of digit tid
#pragma unroll
            for (int q = 0; q < NT / 64; ++q) h += hb[q * 256 + tid];
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
            // (sh_int and scan are rewritten only after the next pass's first barrier)
            prefix |= ((uint32_t)sh_int[0]) << shift;
            mask |= 255u << shift;
            kk = sh_int[1];
          }
          tau = key_float(prefix);
        }
#pragma unroll
        for (int q = 0; q < MPT; ++q) if (pv[q] < tau) pv[q] = -INFINITY;
      }
      float mx = rmax;                       // the largest value survives the cut
      if (!(top_k > 0 && top_k < V)) {
#pragma unroll
        for (int q = 0; q < MPT; ++q) mx = fmaxf(mx, pv[q]);
        mx = block_max(mx, redf);
      }
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
      // wave 0 ranks the survivors and finds the top-p cut while wave 1 draws
      // their noise; then wave 0 runs the race
      int rank = 0, keep = nsv;
      const int lane = tid & 63;
      const float pp = lane < nsv ? tp_list[lane] : -1.f;
      const int id = lane < nsv ? tid_list[lane] : 0x7fffffff;
      if (tid < 64) {
        // rank in (p desc, id asc) order against every survivor, read as LDS
        // broadcasts (padding lanes hold p = -1 and rank after every survivor)
#pragma unroll 8
        for (int j = 0; j < nsv; ++j) {
          const float pj = tp_list[j];
          const int ij = tid_list[j];
          rank += (int)((pj > pp) | ((pj == pp) & (ij < id)));
        }
        // the sequential fp32 running sum in rank order, the same in every lane
        if (top_p < 1.0f) {
          float* srt = sp;                    // p in rank order
          if (lane < nsv) srt[rank] = pp;
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          float v[64];
#pragma unroll
          for (int c = 0; c < 64; ++c) v[c] = c < nsv ? srt[c] : 0.f;
          float cs = 0.f;
          bool found = false;
#pragma unroll
          for (int r0 = 0; r0 < 64; ++r0) {
            const bool act = !found & (r0 < nsv);
            cs = act ? cs + v[r0] : cs;
            const bool hit = act & (cs >= top_p);
            keep = hit ? r0 + 1 : keep;
            found = found | hit;
          }
        }
      } else if (tid < 128 && lane < nsv) {
        nzs[lane] = a.noise_in ? a.noise_in[(long)r * V + id] : exp_noise(seed, nrow, a.stream, jsel, id);
      }
      __syncthreads();
      if (tid < 64) {
        // the race: largest p / E over the kept survivors, lowest id on ties
        const bool kept = lane < nsv && rank < keep;
        const float sc = kept ? pp / nzs[lane] : -INFINITY;
        const float smax = wave_max(sc);
        const int bi = wave_min_i(kept && sc == smax ? id : 0x7fffffff);
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
                                 : exp_noise(seed, nrow, a.stream, jsel, id);
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
      xt[q] = txt ? text[(long)kf * a.tab_dim + k] : padv[q];
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
      if (a.add_text) f = f + (txt ? text[(long)kf * a.tab_dim + k] : pad[k]);
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

__global__ void frame_advance_kernel(int* frame_k, int* pos, const int* finished, int B) {
  for (int r = threadIdx.x; r < B; r += blockDim.x) {
    if (finished[r]) continue;   // a finished row stays where it ended (fed EOS until refilled)
    pos[r] += 1;
    frame_k[r] += 1;
  }
}

hipError_t launch_frame_advance(int* frame_k, int* pos, const int* finished, int B, hipStream_t s) {
  hipLaunchKernelGGL(frame_advance_kernel, dim3(1), dim3(NT), 0, s, frame_k, pos, finished, B);
  return hipGetLastError();
}

// One block per batch row: the row's first-layer q/k/v (and projected
// input) rows from the code-indexed tables, 16-byte copies.
__global__ __launch_bounds__(NT) void lut_rows_kernel(const int* codes, int code_ld, int C, const float* lut, int n,
                                                      float* qkv, long ld_qkv, const float* xlut, int nx, float* x,
                                                      long ldx) {
  const int r = blockIdx.x;
  const int code = min(max(codes[(long)r * code_ld], 0), C - 1);
  const f32x4* src = (const f32x4*)(lut + (long)code * n);
  f32x4* dst = (f32x4*)(qkv + (long)r * ld_qkv);
  for (int i = threadIdx.x; i < n / 4; i += NT) dst[i] = src[i];
  if (xlut) {
    const f32x4* xs = (const f32x4*)(xlut + (long)code * nx);
    f32x4* xd = (f32x4*)(x + (long)r * ldx);
    for (int i = threadIdx.x; i < nx / 4; i += NT) xd[i] = xs[i];
  }
}
hipError_t launch_lut_rows(const int* codes, int code_ld, int B, int C, const float* lut, int n, float* qkv,
                           long ld_qkv, const float* xlut, int nx, float* x, long ldx, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (C < 1 || n % 4 || ld_qkv % 4 || (xlut && (nx % 4 || ldx % 4))) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lut_rows_kernel, dim3(B), dim3(NT), 0, s, codes, code_ld, C, lut, n, qkv, ld_qkv, xlut, nx, x, ldx);
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
