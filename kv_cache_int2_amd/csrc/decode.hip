// Decode attention over the mixed-precision paged cache: rotate q by the key
// transform, attend the INT2 history in the rotated domain (split over the
// context), merge the splits, un-rotate by the value transform and fold in the
// bf16 recent window.  Method: P1 (gen-hub.ru, "Together AI открывает OSCAR…")
// «Что придумали в Together AI»; P2 (encorp.ai) «OSCAR има значение…» and P4
// (aiforradalom.hu) «OSCAR: figyelem-tudatos…» (bf16 recent tokens, INT2
// history, paged attention).
//
// Kernels (one call = three launches on the caller's stream):
//   rotate_q      grid (B, Hkv):            q' = R_K q for the G heads of a KV head
//   int2_split    grid (splits, Hkv, B):    online softmax over one history range,
//                                           partial (m, l, acc'[128]) per q head
//   merge_window  grid (B, Hkv):            log-sum-exp merge of the splits,
//                                           R_V^T acc', bf16 window, normalise
// Scores are kept in the log2 domain: logit * log2(e) / sqrt(d).
//
// The score of a history token factorises over its group: with dequantised
// k'_c = zero + code_c * scale,  q'.k' = zero * sum_c q'_c + scale * sum_c q'_c code_c.
// The value sum is split around the group midpoint mid = zero + 1.5 scale:
// sum_t p_t v'_t = sum_t p_t mid_t + sum_t (p_t scale_t)(code_t - 1.5).  Both
// parts then stay of the size of the result; the plain split (p zero and
// p scale code) makes two terms ~2.5 sigma sum p that cancel to a long-context
// output ~sigma sum p / sqrt(n), and fp32 rounding of the big terms would be
// amplified by that ratio (~300x at 100K tokens).
#include "common.h"

namespace oscar {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------------------
// q' = R_K[h] q for the G query heads of KV head h
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(128) void rotate_q_kernel(const uint16_t* __restrict__ r_k,
                                                       const uint16_t* __restrict__ q, float* __restrict__ qrot,
                                                       int hq, int hkv) {
  __shared__ float qs[G][kD];
  __shared__ uint32_t rrow[kD][65];
  const int b = blockIdx.x, h = blockIdx.y, c = threadIdx.x;
#pragma unroll
  for (int j = 0; j < G; ++j) qs[j][c] = bf16_to_f32(q[((int64_t)b * hq + h * G + j) * kD + c]);
  const uint32_t* r32 = reinterpret_cast<const uint32_t*>(r_k + (int64_t)h * kD * kD);
  for (int i = c; i < kD * 64; i += 128) rrow[i >> 6][i & 63] = r32[i];
  __syncthreads();
  float acc[G];
#pragma unroll
  for (int j = 0; j < G; ++j) acc[j] = 0.f;
  for (int k = 0; k < 64; ++k) {
    uint32_t w = rrow[c][k];
    float lo = bf16lo(w), hi = bf16hi(w);
#pragma unroll
    for (int j = 0; j < G; ++j) acc[j] = fmaf(lo, qs[j][2 * k], fmaf(hi, qs[j][2 * k + 1], acc[j]));
  }
#pragma unroll
  for (int j = 0; j < G; ++j) qrot[((int64_t)b * hq + h * G + j) * kD + c] = acc[j];
}

struct SplitParams {
  const float* qrot;          // [B][Hq][128] (INT2) -- unused by bf16
  const uint16_t* q;          // [B][Hq][128] bf16 (bf16 comparator)
  const int32_t* seq_lens;
  const int32_t* block_table;
  const uint8_t* pool;        // INT2 pool
  const uint16_t* kv_pool;    // bf16 pool
  float* part;                // [B][Hq][n_splits][130]
  int64_t n_pages;
  int hq, hkv, max_pages, window, split, n_splits;
  float scale_log2;           // log2(e) / sqrt(d)
};

// Combine the 4 waves' (m, l, acc) into the workgroup partial and store it.
template <int G>
__device__ __forceinline__ void combine_and_store(const SplitParams& p, float (*cm)[G], float (*cl)[G],
                                                  float (*cacc)[G][kD], int b, int h, int sp) {
  __syncthreads();
  const int tid = threadIdx.x;
  for (int e = tid; e < G * kD; e += 256) {
    const int g = e / kD, c = e % kD;
    float M = fmaxf(fmaxf(cm[0][g], cm[1][g]), fmaxf(cm[2][g], cm[3][g]));
    float acc = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float f = M == kNegInf ? 0.f : exp2f(cm[w][g] - M);
      acc += f * cacc[w][g][c];
      L += f * cl[w][g];
    }
    float* dst = p.part + (((int64_t)b * p.hq + h * G + g) * p.n_splits + sp) * kPartStride;
    dst[2 + c] = acc;
    if (c == 0) {
      dst[0] = M;
      dst[1] = L;
    }
  }
}

// ---------------------------------------------------------------------------
// INT2 history split (VALU): lane = (token of the page, channel quarter) for
// the scores, lane = 2 channels for the value accumulation.
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void int2_split_kernel(SplitParams p) {
  const int b = blockIdx.z, h = blockIdx.y, sp = blockIdx.x;
  const int n = p.seq_lens[b];
  const int w = n < p.window ? n : p.window;
  const int hist = n - w;
  const int t_begin = sp * p.split;
  if (t_begin >= hist) return;
  const int t_end = min(t_begin + p.split, hist);

  __shared__ float qs[G][kD];
  __shared__ float qsum[G];
  __shared__ float pb[4][16][G];
  __shared__ float vsz[4][16][2];
  __shared__ float cm[4][G], cl[4][G];
  __shared__ float cacc[4][G][kD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < G * kD; e += 256)
    qs[e / kD][e % kD] = p.qrot[((int64_t)b * p.hq + h * G) * kD + e];
  __syncthreads();
  if (wave == 0) {
    for (int g = 0; g < G; ++g) {
      float s = qs[g][lane] + qs[g][lane + 64];
      for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
      if (lane == 0) qsum[g] = s;
    }
  }
  __syncthreads();

  const int tq = lane & 15, quarter = lane >> 4;
  float m_run[G], l_run[G], az[G], acc0[G], acc1[G], qsr[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = kNegInf;
    l_run[g] = 0.f;
    az[g] = 0.f;
    acc0[g] = 0.f;
    acc1[g] = 0.f;
    qsr[g] = qsum[g];
  }
  const int first_page = t_begin >> 4, last_page = (t_end - 1) >> 4;
  for (int pg = first_page + wave; pg <= last_page; pg += 4) {
    const int page = p.block_table[(int64_t)b * p.max_pages + pg];
    if (page < 0 || page >= p.n_pages) continue;
    const uint8_t* blk = p.pool + ((int64_t)page * p.hkv + h) * kBlock;
    const int tok = pg * 16 + tq;
    const bool valid = tok >= t_begin && tok < t_end;
    // ---- scores ----
    const uint2 kw = *reinterpret_cast<const uint2*>(blk + kKCodes + 32 * tq + 8 * quarter);
    float dot[G];
#pragma unroll
    for (int g = 0; g < G; ++g) dot[g] = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float c0 = (float)((kw.x >> (2 * j)) & 3u), c1 = (float)((kw.y >> (2 * j)) & 3u);
#pragma unroll
      for (int g = 0; g < G; ++g)
        dot[g] = fmaf(qs[g][32 * quarter + j], c0, fmaf(qs[g][32 * quarter + 16 + j], c1, dot[g]));
    }
    const float ks = h2f(*reinterpret_cast<const uint16_t*>(blk + kKScale + 2 * tq));
    const float kz = h2f(*reinterpret_cast<const uint16_t*>(blk + kKZero + 2 * tq));
    float alpha[G], pv[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float d = dot[g] + __shfl_xor(dot[g], 16);
      d += __shfl_xor(d, 32);
      float lg = valid ? (kz * qsr[g] + ks * d) * p.scale_log2 : kNegInf;
      float mx = lg;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float m_new = fmaxf(m_run[g], mx);
      alpha[g] = exp2f(m_run[g] - m_new);
      pv[g] = valid ? exp2f(lg - m_new) : 0.f;
      float ps = pv[g];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) ps += __shfl_xor(ps, o);
      l_run[g] = l_run[g] * alpha[g] + ps;
      m_run[g] = m_new;
    }
    if (quarter == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) pb[wave][tq][g] = pv[g];
      const float vsc = h2f(*reinterpret_cast<const uint16_t*>(blk + kVScale + 2 * tq));
      const float vzr = h2f(*reinterpret_cast<const uint16_t*>(blk + kVZero + 2 * tq));
      vsz[wave][tq][0] = valid ? vsc : 0.f;
      vsz[wave][tq][1] = valid ? fmaf(1.5f, vsc, vzr) : 0.f;  // group midpoint
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- values: this lane owns channels 2*lane, 2*lane+1 ----
    const uint2 vw = *reinterpret_cast<const uint2*>(blk + kVCodes + 8 * lane);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      acc0[g] *= alpha[g];
      acc1[g] *= alpha[g];
      az[g] *= alpha[g];
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const float c0 = (float)((vw.x >> (2 * t)) & 3u) - 1.5f, c1 = (float)((vw.y >> (2 * t)) & 3u) - 1.5f;
      const float vs = vsz[wave][t][0], vz = vsz[wave][t][1];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float pt = pb[wave][t][g];
        const float wt = pt * vs;
        acc0[g] = fmaf(wt, c0, acc0[g]);
        acc1[g] = fmaf(wt, c1, acc1[g]);
        az[g] = fmaf(pt, vz, az[g]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    cacc[wave][g][2 * lane] = acc0[g] + az[g];
    cacc[wave][g][2 * lane + 1] = acc1[g] + az[g];
    if (lane == 0) {
      cm[wave][g] = m_run[g];
      cl[wave][g] = l_run[g];
    }
  }
  combine_and_store<G>(p, cm, cl, cacc, b, h, sp);
}

// ---------------------------------------------------------------------------
// bf16 comparator split: plain attention over bf16 pages, all n positions.
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void bf16_split_kernel(SplitParams p) {
  const int b = blockIdx.z, h = blockIdx.y, sp = blockIdx.x;
  const int n = p.seq_lens[b];
  const int t_begin = sp * p.split;
  if (t_begin >= n) return;
  const int t_end = min(t_begin + p.split, n);

  __shared__ float qs[G][kD];
  __shared__ float pb[4][16][G];
  __shared__ float cm[4][G], cl[4][G];
  __shared__ float cacc[4][G][kD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < G * kD; e += 256)
    qs[e / kD][e % kD] = bf16_to_f32(p.q[((int64_t)b * p.hq + h * G) * kD + e]);
  __syncthreads();

  const int tq = lane & 15, quarter = lane >> 4;
  float m_run[G], l_run[G], acc0[G], acc1[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = kNegInf;
    l_run[g] = 0.f;
    acc0[g] = 0.f;
    acc1[g] = 0.f;
  }
  const int first_page = t_begin >> 4, last_page = (t_end - 1) >> 4;
  for (int pg = first_page + wave; pg <= last_page; pg += 4) {
    const int page = p.block_table[(int64_t)b * p.max_pages + pg];
    if (page < 0 || page >= p.n_pages) continue;
    const uint16_t* kb = p.kv_pool + ((int64_t)page * p.hkv + h) * (2 * kPage * kD);
    const uint16_t* vb = kb + kPage * kD;
    const int tok = pg * 16 + tq;
    const bool valid = tok >= t_begin && tok < t_end;
    const uint4* kr = reinterpret_cast<const uint4*>(kb + tq * kD + 32 * quarter);
    uint4 k4[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) k4[s] = kr[s];
    float dot[G];
#pragma unroll
    for (int g = 0; g < G; ++g) dot[g] = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t wv[4] = {k4[s].x, k4[s].y, k4[s].z, k4[s].w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float lo = bf16lo(wv[u]), hi = bf16hi(wv[u]);
        const int c = 32 * quarter + 8 * s + 2 * u;
#pragma unroll
        for (int g = 0; g < G; ++g) dot[g] = fmaf(lo, qs[g][c], fmaf(hi, qs[g][c + 1], dot[g]));
      }
    }
    float alpha[G], pv[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float d = dot[g] + __shfl_xor(dot[g], 16);
      d += __shfl_xor(d, 32);
      float lg = valid ? d * p.scale_log2 : kNegInf;
      float mx = lg;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float m_new = fmaxf(m_run[g], mx);
      alpha[g] = exp2f(m_run[g] - m_new);
      pv[g] = valid ? exp2f(lg - m_new) : 0.f;
      float ps = pv[g];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) ps += __shfl_xor(ps, o);
      l_run[g] = l_run[g] * alpha[g] + ps;
      m_run[g] = m_new;
    }
    if (quarter == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) pb[wave][tq][g] = pv[g];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int g = 0; g < G; ++g) {
      acc0[g] *= alpha[g];
      acc1[g] *= alpha[g];
    }
    const int tcount = min(16, t_end - pg * 16);
    for (int t = 0; t < tcount; ++t) {
      if (pg * 16 + t < t_begin) continue;
      const uint32_t v2 = reinterpret_cast<const uint32_t*>(vb + t * kD)[lane];
      const float v0 = bf16lo(v2), v1 = bf16hi(v2);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float pt = pb[wave][t][g];
        acc0[g] = fmaf(pt, v0, acc0[g]);
        acc1[g] = fmaf(pt, v1, acc1[g]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    cacc[wave][g][2 * lane] = acc0[g];
    cacc[wave][g][2 * lane + 1] = acc1[g];
    if (lane == 0) {
      cm[wave][g] = m_run[g];
      cl[wave][g] = l_run[g];
    }
  }
  combine_and_store<G>(p, cm, cl, cacc, b, h, sp);
}

// ---------------------------------------------------------------------------
// merge: LSE over splits; for the INT2 path also un-rotate with R_V^T and fold
// in the bf16 window (positions [n - w, n) at ring slots pos % W).
// ---------------------------------------------------------------------------
struct MergeParams {
  const float* part;
  const uint16_t* r_v;       // nullptr: no un-rotation, no window (bf16 comparator)
  const uint16_t* q;         // bf16 [B][Hq][128] (window scores)
  const uint16_t* win_k;
  const uint16_t* win_v;
  const int32_t* seq_lens;
  float* out;
  int hq, hkv, window, split, n_splits;
  float scale_log2;
};

constexpr int kWinChunk = 32;

template <int G>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  const int b = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int n = p.seq_lens[b];
  const bool int2 = p.r_v != nullptr;
  const int w = int2 ? (n < p.window ? n : p.window) : 0;
  const int hist = n - w;
  const int ns = (hist + p.split - 1) / p.split;

  __shared__ float a1[G][kD];   // merged split accumulator (rotated domain for INT2)
  __shared__ float o2[G][kD];   // window accumulator
  __shared__ float qs[G][kD];
  __shared__ float M1[G], L1[G], M2[G], L2[G], al[G], mn[G];
  __shared__ uint32_t kw[kWinChunk][65];
  __shared__ uint32_t vw[kWinChunk][65];
  __shared__ float sc[G][kWinChunk];

  for (int e = tid; e < G * kD; e += 256) {
    const int g = e / kD, c = e % kD;
    const float* base = p.part + ((int64_t)b * p.hq + h * G + g) * p.n_splits * kPartStride;
    float M = kNegInf;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, base[s * kPartStride]);
    float acc = 0.f, L = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float f = exp2f(base[s * kPartStride] - M);
      acc += f * base[s * kPartStride + 2 + c];
      L += f * base[s * kPartStride + 1];
    }
    a1[g][c] = acc;
    o2[g][c] = 0.f;
    qs[g][c] = bf16_to_f32(p.q[((int64_t)b * p.hq + h * G + g) * kD + c]);
    if (c == 0) {
      M1[g] = M;
      L1[g] = L;
      M2[g] = kNegInf;
      L2[g] = 0.f;
    }
  }
  __syncthreads();

  float o1[(G * kD + 255) / 256];
  if (int2) {
    const uint16_t* rv = p.r_v + (int64_t)h * kD * kD;
    int k = 0;
    for (int e = tid; e < G * kD; e += 256, ++k) {
      const int g = e / kD, i = e % kD;
      float acc = 0.f;
      for (int j = 0; j < kD; ++j) acc = fmaf(bf16_to_f32(rv[j * kD + i]), a1[g][j], acc);
      o1[k] = acc;
    }
    for (int cs = hist; cs < n; cs += kWinChunk) {
      const int nt = min(kWinChunk, n - cs);
      __syncthreads();
      for (int e = tid; e < nt * 64; e += 256) {
        const int t = e >> 6, u = e & 63;
        const int64_t row = (((int64_t)b * p.window + (cs + t) % p.window) * p.hkv + h) * kD;
        kw[t][u] = reinterpret_cast<const uint32_t*>(p.win_k + row)[u];
        vw[t][u] = reinterpret_cast<const uint32_t*>(p.win_v + row)[u];
      }
      __syncthreads();
      for (int e = tid; e < G * kWinChunk; e += 256) {
        const int g = e / kWinChunk, t = e % kWinChunk;
        float s = kNegInf;
        if (t < nt) {
          s = 0.f;
          for (int u = 0; u < 64; ++u) {
            const uint32_t x = kw[t][u];
            s = fmaf(bf16lo(x), qs[g][2 * u], fmaf(bf16hi(x), qs[g][2 * u + 1], s));
          }
          s *= p.scale_log2;
        }
        sc[g][t] = s;
      }
      __syncthreads();
      if (tid < G) {
        float cmx = kNegInf;
        for (int t = 0; t < nt; ++t) cmx = fmaxf(cmx, sc[tid][t]);
        const float m_new = fmaxf(M2[tid], cmx);
        al[tid] = exp2f(M2[tid] - m_new);
        mn[tid] = m_new;
      }
      __syncthreads();
      for (int e = tid; e < G * kWinChunk; e += 256) {
        const int g = e / kWinChunk, t = e % kWinChunk;
        sc[g][t] = t < nt ? exp2f(sc[g][t] - mn[g]) : 0.f;
      }
      __syncthreads();
      if (tid < G) {
        float s = 0.f;
        for (int t = 0; t < nt; ++t) s += sc[tid][t];
        L2[tid] = L2[tid] * al[tid] + s;
        M2[tid] = mn[tid];
      }
      for (int e = tid; e < G * kD; e += 256) {
        const int g = e / kD, c = e % kD;
        float acc = o2[g][c] * al[g];
        for (int t = 0; t < nt; ++t) {
          const uint32_t x = vw[t][c >> 1];
          acc = fmaf(sc[g][t], (c & 1) ? bf16hi(x) : bf16lo(x), acc);
        }
        o2[g][c] = acc;
      }
    }
    __syncthreads();
  }
  int k = 0;
  for (int e = tid; e < G * kD; e += 256, ++k) {
    const int g = e / kD, c = e % kD;
    const float v1 = int2 ? o1[k] : a1[g][c];
    const float M = fmaxf(M1[g], M2[g]);
    const float f1 = M1[g] == kNegInf ? 0.f : exp2f(M1[g] - M);
    const float f2 = M2[g] == kNegInf ? 0.f : exp2f(M2[g] - M);
    p.out[((int64_t)b * p.hq + h * G + g) * kD + c] = (f1 * v1 + f2 * o2[g][c]) / (f1 * L1[g] + f2 * L2[g]);
  }
}

template <int G>
int launch_decode(bool int2, const SplitParams& sp, const MergeParams& mp, const uint16_t* r_k,
                  const uint16_t* q, int batch, hipStream_t s) {
  if (int2) {
    rotate_q_kernel<G><<<dim3(batch, sp.hkv), 128, 0, s>>>(r_k, q, const_cast<float*>(sp.qrot), sp.hq, sp.hkv);
    if (hipGetLastError() != hipSuccess) return OSCAR_EHIP;
  }
  int slot = -1;
  timing_record_begin(s, int2 ? 1 : 2, &slot);
  dim3 grid(sp.n_splits, sp.hkv, batch);
  if (int2)
    int2_split_kernel<G><<<grid, 256, 0, s>>>(sp);
  else
    bf16_split_kernel<G><<<grid, 256, 0, s>>>(sp);
  if (hipGetLastError() != hipSuccess) return OSCAR_EHIP;
  timing_record_end(s, slot);
  merge_kernel<G><<<dim3(batch, sp.hkv), 256, 0, s>>>(mp);
  return hipGetLastError() == hipSuccess ? OSCAR_OK : OSCAR_EHIP;
}

int decode_common(bool int2, const oscar_shape* shape, const uint16_t* r_k, const uint16_t* r_v,
                  const uint16_t* q, int32_t batch, const int32_t* seq_lens, int32_t max_seq_len,
                  const int32_t* block_table, int32_t max_pages_per_seq, const uint8_t* pool,
                  const uint16_t* kv_pool, int64_t n_pages, const uint16_t* win_k, const uint16_t* win_v,
                  float* out, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != OSCAR_OK) return st;
  if (batch < 1 || max_seq_len < 1 || max_pages_per_seq < 1 || n_pages < 1) return OSCAR_EINVAL;
  if (!q || !seq_lens || !block_table || !out || !workspace) return OSCAR_EINVAL;
  if (int2 && (!r_k || !r_v || !pool)) return OSCAR_EINVAL;
  if (int2 && shape->window > 0 && (!win_k || !win_v)) return OSCAR_EINVAL;
  if (!int2 && !kv_pool) return OSCAR_EINVAL;
  if ((int64_t)max_seq_len > (int64_t)max_pages_per_seq * kPage) return OSCAR_ENOSPACE;
  const SplitPlan plan = plan_splits(batch, shape->n_kv_heads, max_seq_len);
  if (workspace_bytes < oscar::workspace_bytes(batch, shape->n_q_heads, plan)) return OSCAR_ENOSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return OSCAR_EINVAL;

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  SplitParams sp{};
  sp.qrot = reinterpret_cast<float*>(ws);
  sp.q = q;
  sp.seq_lens = seq_lens;
  sp.block_table = block_table;
  sp.pool = pool;
  sp.kv_pool = kv_pool;
  sp.part = reinterpret_cast<float*>(ws + qrot_bytes(batch, shape->n_q_heads));
  sp.n_pages = n_pages;
  sp.hq = shape->n_q_heads;
  sp.hkv = shape->n_kv_heads;
  sp.max_pages = max_pages_per_seq;
  sp.window = int2 ? shape->window : 0;
  sp.split = plan.split;
  sp.n_splits = plan.n_splits;
  sp.scale_log2 = kLog2e / sqrtf((float)kD);
  MergeParams mp{};
  mp.part = sp.part;
  mp.r_v = int2 ? r_v : nullptr;
  mp.q = q;
  mp.win_k = win_k;
  mp.win_v = win_v;
  mp.seq_lens = seq_lens;
  mp.out = out;
  mp.hq = sp.hq;
  mp.hkv = sp.hkv;
  mp.window = sp.window;
  mp.split = sp.split;
  mp.n_splits = sp.n_splits;
  mp.scale_log2 = sp.scale_log2;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (shape->n_q_heads / shape->n_kv_heads) {
    case 1: return launch_decode<1>(int2, sp, mp, r_k, q, batch, s);
    case 2: return launch_decode<2>(int2, sp, mp, r_k, q, batch, s);
    case 4: return launch_decode<4>(int2, sp, mp, r_k, q, batch, s);
    case 8: return launch_decode<8>(int2, sp, mp, r_k, q, batch, s);
    case 16: return launch_decode<16>(int2, sp, mp, r_k, q, batch, s);
  }
  return OSCAR_EUNSUPPORTED;
}

// bf16 comparator append: scatter rows into [page][Hkv][2][16][128]
__global__ __launch_bounds__(256) void bf16_append_kernel(const uint16_t* __restrict__ k_new,
                                                          const uint16_t* __restrict__ v_new, int64_t n_tokens,
                                                          const int32_t* seq_idx, const int32_t* pos, int batch,
                                                          const int32_t* block_table, int max_pages,
                                                          uint16_t* kv_pool, int64_t n_pages, int hkv) {
  // one thread per (token, head, 16-byte chunk of K or V row)
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = n_tokens * hkv * 2 * 16;
  if (i >= total) return;
  const int chunk = i & 15;
  const int kv = (i >> 4) & 1;
  const int64_t th = i >> 5;
  const int h = th % hkv;
  const int64_t t = th / hkv;
  const int b = seq_idx[t], ps = pos[t];
  if (b < 0 || b >= batch || ps < 0 || (ps >> 4) >= max_pages) return;
  const int page = block_table[(int64_t)b * max_pages + (ps >> 4)];
  if (page < 0 || page >= n_pages) return;
  const uint4* src = reinterpret_cast<const uint4*>((kv ? v_new : k_new) + (t * hkv + h) * kD);
  uint4* dst = reinterpret_cast<uint4*>(kv_pool + ((((int64_t)page * hkv + h) * 2 + kv) * kPage + (ps & 15)) * kD);
  dst[chunk] = src[chunk];
}

}  // namespace
}  // namespace oscar

extern "C" size_t oscar_decode_workspace_bytes(const oscar_shape* shape, int32_t batch, int32_t max_seq_len) {
  using namespace oscar;
  if (check_shape(shape) != OSCAR_OK || batch < 1 || max_seq_len < 1) return 0;
  return workspace_bytes(batch, shape->n_q_heads, plan_splits(batch, shape->n_kv_heads, max_seq_len));
}

extern "C" int oscar_decode_attn(const oscar_shape* shape, const uint16_t* r_k, const uint16_t* r_v,
                                 const uint16_t* q, int32_t batch, const int32_t* seq_lens, int32_t max_seq_len,
                                 const int32_t* block_table, int32_t max_pages_per_seq, const uint8_t* pool,
                                 int64_t n_pages, const uint16_t* win_k, const uint16_t* win_v, float* out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return oscar::decode_common(true, shape, r_k, r_v, q, batch, seq_lens, max_seq_len, block_table,
                              max_pages_per_seq, pool, nullptr, n_pages, win_k, win_v, out, workspace,
                              workspace_bytes, stream);
}

extern "C" int oscar_bf16_decode_attn(const oscar_shape* shape, const uint16_t* q, int32_t batch,
                                      const int32_t* seq_lens, int32_t max_seq_len, const int32_t* block_table,
                                      int32_t max_pages_per_seq, const uint16_t* kv_pool, int64_t n_pages,
                                      float* out, void* workspace, size_t workspace_bytes, void* stream) {
  return oscar::decode_common(false, shape, nullptr, nullptr, q, batch, seq_lens, max_seq_len, block_table,
                              max_pages_per_seq, nullptr, kv_pool, n_pages, nullptr, nullptr, out, workspace,
                              workspace_bytes, stream);
}

extern "C" int oscar_bf16_append(const oscar_shape* shape, const uint16_t* k_new, const uint16_t* v_new,
                                 int64_t n_tokens, const int32_t* seq_idx, const int32_t* pos, int32_t batch,
                                 const int32_t* block_table, int32_t max_pages_per_seq, uint16_t* kv_pool,
                                 int64_t n_pages, void* stream) {
  using namespace oscar;
  int st = check_shape(shape);
  if (st != OSCAR_OK) return st;
  if (n_tokens < 0 || batch < 1 || max_pages_per_seq < 1 || n_pages < 1) return OSCAR_EINVAL;
  if (n_tokens == 0) return OSCAR_OK;
  if (!k_new || !v_new || !seq_idx || !pos || !block_table || !kv_pool) return OSCAR_EINVAL;
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new) |
       reinterpret_cast<uintptr_t>(kv_pool)) & 15)
    return OSCAR_EINVAL;
  const int64_t total = n_tokens * shape->n_kv_heads * 32;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  bf16_append_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(
      k_new, v_new, n_tokens, seq_idx, pos, batch, block_table, max_pages_per_seq, kv_pool, n_pages,
      shape->n_kv_heads);
  return hipGetLastError() == hipSuccess ? OSCAR_OK : OSCAR_EHIP;
}
