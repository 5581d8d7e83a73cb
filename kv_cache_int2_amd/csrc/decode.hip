// Decode attention over the mixed-precision paged cache: rotate q by the key
// transform, attend the INT2 history in the rotated domain (split over the
// context), merge the splits, un-rotate by the value transform and fold in the
// bf16 recent window.  Method: P1 (gen-hub.ru, "Together AI открывает OSCAR…")
// «Что придумали в Together AI»; P2 (encorp.ai) «OSCAR има значение…» and P4
// (aiforradalom.hu) «OSCAR: figyelem-tudatos…» (bf16 recent tokens, INT2
// history, paged attention).
//
// Kernels (one call = three launches on the caller's stream):
//   prep_q        grid (B, Hkv):          q' = R_K q for the G heads of a KV head,
//                                         its channel sums and fp8 score operands
//   int2_split    grid (splits, Hkv, B):  online softmax over one history range,
//                                         partial (m, l, acc'[128]) per q head
//   merge         grid (B, Hkv):          log-sum-exp merge of the splits,
//                                         R_V^T acc', bf16 window, normalise
// Scores are kept in the log2 domain: logit * log2(e) / sqrt(d).
//
// INT2 split kernel.  Both contractions of a 128-token tile (8 pages) run on the
// matrix cores as v_mfma_scale_f32_16x16x128_f8f6f4 with the packed 2-bit codes
// as the fp4 (e2m1) operand: a code c zero-extended to a nibble is exactly the
// e2m1 value c/2, so (w & 0x33333333) and ((w >> 2) & 0x33333333) turn 16 packed
// codes into two ready operand dwords.  The other operand (q' for the scores,
// softmax weights for the values) is carried as four fp8 (e4m3) terms
// x = t0 + t1/16 + t2/256 + t3/4096 (each the RNE of the remaining residual),
// one term per MFMA row, with the power-of-two factors in the E8M0 operand
// scales: about 16 significant bits.  Rows are (head, term): 4 heads per MFMA.
//   scores: A = q' terms [(head, term) x 128 channels], B = K codes [128 x 16 tokens]
//   values: A = w terms  [(head, term) x 128 tokens],  B = V codes [128 x 16 channels]
// The score output leaves one (head, token) per lane after an in-lane sum of
// the four term rows, so the softmax runs on full lanes.  The w terms go to a
// per-wave LDS tile to reach the A-operand layout.
//
// gfx950 operand layout of this instruction (16 x 16 output, lane l: column
// l % 16, rows 4 (l / 16) + i): an 8-bit operand lane in group g holds k in
// [16g, 16g + 16) then [64 + 16g, 64 + 16g + 16); a 4-bit operand lane holds k in
// [32g, 32g + 32), low nibble first; the E8M0 scale of k-block b of row / column
// r comes from lane 16b + r.
//
// Value accumulation is split around each group's midpoint mid = zero + 1.5 scale:
//   sum_t p_t v'_t = sum_t p_t mid_t + sum_t (p_t scale_t)(code_t - 1.5),
// the -1.5 sum_t w_t being folded into the accumulator once per tile.  The plain
// split (p zero + p scale code) makes two terms ~2.5 sigma sum p that cancel to a
// long-context output ~ sigma sum p / sqrt(n); their fp32 rounding would be
// amplified by that ratio (~300x at 100K tokens).
#include "common.h"

namespace oscar {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kScaleOne = 127;   // E8M0 1.0
constexpr int kScaleCode = 128;  // E8M0 2.0: an fp4 code nibble c reads as c / 2

__device__ __forceinline__ f32x4 mfma_f8_f4(const i32x8& a, const i32x8& b, f32x4 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0 /*A e4m3*/, 4 /*B e2m1*/, 0, sa, 0, sb);
}

// k index of byte e (0..31) of an 8-bit operand lane in lane group g
__device__ __forceinline__ int k_of_fp8(int g, int e) { return e < 16 ? 16 * g + e : 48 + 16 * g + e; }

// channel of element k of the K-code operand.  Lane group g = k / 32 holds the
// row bytes 8g .. 8g + 7 (row segment g: byte m holds channels 16m + 4g + i at
// bits 2i) as dwords w0, w1 and presents lo(w0), hi(w0), lo(w1), hi(w1), where
// lo keeps bits 2i of each nibble (i even) and hi the bits above (i odd).
__device__ __forceinline__ int k_channel(int k) {
  const int g = k >> 5, e = k & 31, d = e >> 3, nib = e & 7;
  const int m = 4 * (d >> 1) + (nib >> 1), i = 2 * (nib & 1) + (d & 1);
  return 16 * m + 4 * g + i;
}

// A sequence length is clamped to what its block-table row can hold.
__device__ __forceinline__ int clamp_len(int n, int max_pages) {
  return n < 0 ? 0 : (n > max_pages * kPage ? max_pages * kPage : n);
}

__device__ __forceinline__ int clamp_scale(int s) { return s < 1 ? 1 : (s > 254 ? 254 : s); }

// Four e4m3 terms of a pair of values (|x| < 128): term j of a in byte 0 and of
// b in byte 1 of out[j].
__device__ __forceinline__ void split4(float a, float b, uint32_t out[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    out[j] = (uint32_t)pk & 0xffffu;
    if (j < 3) {
      a = (a - __builtin_amdgcn_cvt_f32_fp8(pk, 0)) * 16.f;
      b = (b - __builtin_amdgcn_cvt_f32_fp8(pk, 1)) * 16.f;
    }
  }
}

__device__ __forceinline__ int exponent_above(float x) {  // E with |x| < 2^E (0 for x == 0)
  int e = 0;
  frexpf(x, &e);
  return e;
}

// ---------------------------------------------------------------------------
// Query preparation, once per (sequence, KV head):
//   q' = R_K[h] q for its G query heads (thread pair (c, half): 64 inputs of
//   output channel c from 8 x 16-byte loads of R's row);
//   qsum[head] = sum_c q'_c;
//   the fp8 score operand of every 4-head group: lane (lg, lr) holds term lr%4 of
//   q'_(head lr/4) at the 32 channels its k-slots map to, plus the row's E8M0
//   scale (2^(E - 7 - 4 term), |q'| < 2^E), exactly as the split kernel's MFMA
//   consumes it.
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void prep_q_kernel(const uint16_t* __restrict__ r_k,
                                                     const uint16_t* __restrict__ q, float* __restrict__ qsum_out,
                                                     int* __restrict__ qop, int hq, int hkv) {
  constexpr int NCB = (G + 3) / 4;  // 4-head operand groups
  __shared__ float qs[G][kD];
  __shared__ int qexp[G];
  const int b = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  {
    const int c = tid >> 1, half = tid & 1;
    const uint4* rrow = reinterpret_cast<const uint4*>(r_k + ((int64_t)h * kD + c) * kD + 64 * half);
    uint4 rv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) rv[i] = rrow[i];
    __shared__ float qraw[G][kD];
    for (int e = tid; e < G * kD; e += 256) qraw[e / kD][e % kD] = bf16_to_f32(q[((int64_t)b * hq + h * G) * kD + e]);
    __syncthreads();
#pragma unroll 1
    for (int j = 0; j < G; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t w[4] = {rv[i].x, rv[i].y, rv[i].z, rv[i].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float2 qv = *reinterpret_cast<const float2*>(&qraw[j][64 * half + 8 * i + 2 * u]);
          acc = fmaf(bf16lo(w[u]), qv.x, fmaf(bf16hi(w[u]), qv.y, acc));
        }
      }
      acc += __shfl_xor(acc, 1);
      if (half == 0) qs[j][c] = acc;
    }
  }
  __syncthreads();
  if (tid < G * 16) {  // 16 threads per head: sum and max |q'|
    const int g = tid >> 4, j = tid & 15;
    float s = 0.f, mx = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      s += qs[g][8 * j + c];
      mx = fmaxf(mx, fabsf(qs[g][8 * j + c]));
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      s += __shfl_xor(s, o);
      mx = fmaxf(mx, __shfl_xor(mx, o));
    }
    if (j == 0) {
      qsum_out[(int64_t)b * hq + h * G + g] = s;
      qexp[g] = exponent_above(mx);
    }
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  for (int cb = wave; cb < NCB; cb += 4) {
    const int head = 4 * cb + (lr >> 2), term = lr & 3;
    int op[9];
#pragma unroll
    for (int i = 0; i < 8; ++i) op[i] = 0;
    op[8] = kScaleOne;
    if (head < G) {
      const int E = qexp[head];
      op[8] = clamp_scale(kScaleOne + E - 7 - 4 * term);
#pragma unroll
      for (int e = 0; e < 32; e += 2) {
        const float a = ldexpf(qs[head][k_channel(k_of_fp8(lg, e))], 7 - E);
        const float c = ldexpf(qs[head][k_channel(k_of_fp8(lg, e + 1))], 7 - E);
        uint32_t t[4];
        split4(a, c, t);
        op[e >> 2] |= (int)(t[term] << (8 * (e & 3)));
      }
    }
    int* dst = qop + ((((int64_t)b * hkv + h) * NCB + cb) * 64 + lane) * 9;
#pragma unroll
    for (int i = 0; i < 9; ++i) dst[i] = op[i];
  }
}

struct SplitParams {
  const float* qsum;          // [B][Hq]      (INT2 path)
  const int* qop;             // [B][Hkv][ceil(G/4)][64][9] (INT2 path)
  const uint16_t* q;          // [B][Hq][128] bf16 queries
  const int32_t* seq_lens;
  const int32_t* block_table;
  const uint8_t* pool;        // INT2 pool
  const uint16_t* kv_pool;    // bf16 pool
  const uint16_t* r_v;        // INT2: value rotations [Hkv][128][128] (un-rotation in the merge)
  const uint16_t* win_k;      // INT2: bf16 window rings [B][W][Hkv][128]
  const uint16_t* win_v;
  float* part;                // [B][Hq][n_splits][130] split partials
  float* wpart;               // INT2: [B][Hq][130] window partials (unrotated domain)
  float* out;                 // [B][Hq][128]
  int64_t n_pages;
  int batch, hq, hkv, max_pages, max_len, window, split, n_splits;
  int gsub;                   // workgroups per KV head, each taking gw of its query heads
  int gw;                     // query heads a workgroup really has (<= G of its instantiation)
  float scale_log2;           // log2(e) / sqrt(d)
};

// Sequence length as the kernels see it: clamped to [0, max_len].
__device__ __forceinline__ int seq_len_of(const SplitParams& p, int b) {
  const int n = p.seq_lens[b];
  return n < 0 ? 0 : (n > p.max_len ? p.max_len : n);
}

// Combine the 4 waves' (m, l, acc) partials (LDS) into the workgroup partial.
template <int G>
__device__ __forceinline__ void combine_and_store(const SplitParams& p, const float* cm, const float* cl,
                                                  const float* cacc, int b, int hq0, int sp, int gw = G) {
  const int tid = threadIdx.x;
  for (int e = tid; e < gw * kD; e += 256) {
    const int g = e / kD, c = e % kD;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, cm[w * G + g]);
    float acc = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = cm[w * G + g] == kNegInf ? 0.f : exp2f(cm[w * G + g] - M);
      acc += f * cacc[(w * G + g) * kD + c];
      L += f * cl[w * G + g];
    }
    float* dst = p.part + (((int64_t)b * p.hq + hq0 + g) * p.n_splits + sp) * kPartStride;
    dst[2 + c] = acc;
    if (c == 0) {
      dst[0] = M;
      dst[1] = L;
    }
  }
}

// Raw bytes of one 128-token tile (8 pages) as one lane needs them.
struct Tile {
  uint2 kc[8];    // K row bytes 8lg..8lg+7 of token lr, per page
  uint2 meta[8];  // token lr's record {Ks, Kz, Vs, Vz} (any value past the history end)
  uint4 vlo[2], vhi[2];  // V words of channels 8lr..8lr+7, pages 2lg and 2lg+1
  uint32_t page_ok;      // bit pp: page pp of the tile exists in this split and in the pool
};

// Block-table entries of a wave's tiles.  The wave's k-th tile is tile
// wave + 4k of the split (the waves take tiles round robin); lane 8j + pp holds
// the page of page pp of the wave's tile k0 + j, or -1 when that page is past
// the split, past the table or outside the pool.  One load serves 8 tiles, so no
// tile waits on a block-table read before its own loads can start.
struct TileTable {
  int ent;        // this lane's entry
  uint64_t live;  // ballot of ent >= 0
};

__device__ __forceinline__ TileTable load_table(const SplitParams& p, const int* btr, int P0, int P1,
                                                int wave, int k0) {
  const int lane = threadIdx.x & 63;
  const int pg = P0 + 8 * (wave + 4 * (k0 + (lane >> 3))) + (lane & 7);
  int e = pg <= P1 ? btr[pg] : -1;
  e = (e >= 0 && e < p.n_pages) ? e : -1;
  return TileTable{e, __ballot(e >= 0)};
}

// All loads of one tile (j-th of its table chunk) are issued back to back with
// no branches: every page index is broadcast with readlane (so each page's block
// address is a scalar and a lane only adds its fixed offset), and a missing
// page is read as page 0 and masked, so the memory system sees the whole tile
// at once.
__device__ __forceinline__ void load_tile(const SplitParams& p, const TileTable& tt, int j, int h, int pbase,
                                          int t_end, int lg, int lr, Tile& t) {
  t.page_ok = (uint32_t)(tt.live >> (8 * j)) & 0xffu;
  const uint32_t off_k = kKCodes + 32 * lr + 8 * lg;
  const uint32_t off_m = kMeta + 8 * lr;
  const uint32_t off_v = kVCodes + 32 * lr;
  int pages[8];
#pragma unroll
  for (int pp = 0; pp < 8; ++pp) {
    const int e = __builtin_amdgcn_readlane(tt.ent, 8 * j + pp);
    pages[pp] = e < 0 ? 0 : e;
  }
#pragma unroll
  for (int pp = 0; pp < 8; ++pp) {
    const uint8_t* blk = p.pool + ((int64_t)pages[pp] * p.hkv + h) * kBlock;
    t.kc[pp] = *reinterpret_cast<const uint2*>(blk + off_k);
    t.meta[pp] = *reinterpret_cast<const uint2*>(blk + off_m);
  }
  // V words: lane group lg takes pages 2lg and 2lg + 1 (entries of lanes
  // 8j + 2lg + qq, fetched across lanes)
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    int pv = __builtin_amdgcn_ds_bpermute(4 * (8 * j + 2 * lg + qq), tt.ent);
    pv = pv < 0 ? 0 : pv;
    const uint8_t* blk = p.pool + ((int64_t)pv * p.hkv + h) * kBlock + off_v;
    t.vlo[qq] = *reinterpret_cast<const uint4*>(blk);
    t.vhi[qq] = *reinterpret_cast<const uint4*>(blk + 16);
  }
  // no use of the loaded registers here: the caller computes another tile
  // while these loads are in flight
}

// Pins a value at this point of the program.  The matrix instructions read
// their operands across all 64 lanes, so they must run with every lane active:
// without the pin the compiler may sink an MFMA whose result is only used under
// a per-lane condition into that condition's branch.
__device__ __forceinline__ float pin(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Running state of one wave: accumulators, running max, partial sums.
template <int NRG>
struct WaveState {
  f32x4 acc[NRG][8];
  float m_run[NRG], l_part[NRG], az_part[NRG];
};

template <int G, int NRG>
__device__ __forceinline__ void compute_tile(const SplitParams& p, const Tile& t, int pbase, int t_end, int lg,
                                             int lr, const i32x8* qa, const int* qsc, const float* qsr,
                                             uint8_t* wt, WaveState<NRG>& st) {
  const int slot_pos = 8 * (lr & 1) + (lr >> 1);  // k position of token lr within its page's 16
  // ---- scores: raw[rg][pp] = q'_(4rg+lg) . code(token lr of page pp) ----
  float raw[NRG][8];
#pragma unroll
  for (int pp = 0; pp < 8; ++pp) {
    i32x8 bk;
    bk[0] = (int)(t.kc[pp].x & 0x33333333u);
    bk[1] = (int)((t.kc[pp].x >> 2) & 0x33333333u);
    bk[2] = (int)(t.kc[pp].y & 0x33333333u);
    bk[3] = (int)((t.kc[pp].y >> 2) & 0x33333333u);
    bk[4] = bk[5] = bk[6] = bk[7] = 0;
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
      const f32x4 c = mfma_f8_f4(qa[rg], bk, f32x4{0.f, 0.f, 0.f, 0.f}, qsc[rg], kScaleCode);
      raw[rg][pp] = pin((c[0] + c[1]) + (c[2] + c[3]));
    }
  }
  // ---- online softmax, weights, w terms -> LDS ----
  // slots past the history end or on a missing page may hold anything: their
  // record must not reach the per-tile scale exponent or the sums
  uint2 meta[8];
#pragma unroll
  for (int pp = 0; pp < 8; ++pp) {
    const bool live = ((t.page_ok >> pp) & 1u) && (pbase + pp) * 16 + lr < t_end;
    meta[pp].x = live ? t.meta[pp].x : 0u;
    meta[pp].y = live ? t.meta[pp].y : 0u;
  }
  float wsum[NRG];
  float vsmax = 0.f;
#pragma unroll
  for (int pp = 0; pp < 8; ++pp) vsmax = fmaxf(vsmax, h2f((uint16_t)(meta[pp].y & 0xffffu)));
  vsmax = row_max16(vsmax);
  const int wexp = exponent_above(vsmax);  // every w = p vs <= vsmax < 2^wexp
  const float wmul = ldexpf(1.f, 7 - wexp);  // w * wmul < 128, exact (a power of two)
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) {
    const bool hv = 4 * rg + lg < p.gw;
    float lgt[8];
    float mx = kNegInf;
#pragma unroll
    for (int pp = 0; pp < 8; ++pp) {
      const int tok = (pbase + pp) * 16 + lr;
      const bool ok = hv && tok < t_end && ((t.page_ok >> pp) & 1u);
      const float ks = h2f((uint16_t)(meta[pp].x & 0xffffu));
      const float kz = h2f((uint16_t)(meta[pp].x >> 16));
      // computed on every lane, then masked: a select, not a branch
      const float v = pin((kz * qsr[rg] + ks * raw[rg][pp]) * p.scale_log2);
      lgt[pp] = ok ? v : kNegInf;
      mx = fmaxf(mx, lgt[pp]);
    }
    mx = row_max16(mx);
    const float m_new = fmaxf(st.m_run[rg], mx);
    if (__any(m_new > st.m_run[rg])) {
      const float alpha = (m_new == kNegInf) ? 1.f : exp2f(st.m_run[rg] - m_new);
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) st.acc[rg][nn] *= alpha;
      st.l_part[rg] *= alpha;
      st.az_part[rg] *= alpha;
      st.m_run[rg] = m_new;
    }
    float w[8];
    float ws = 0.f;
    const float m_safe = st.m_run[rg] == kNegInf ? 0.f : st.m_run[rg];  // exp2(-inf - m_safe) = 0
#pragma unroll
    for (int pp = 0; pp < 8; ++pp) {
      const float pv = exp2f(lgt[pp] - m_safe);
      const float vs = h2f((uint16_t)(meta[pp].y & 0xffffu));
      const float vz = h2f((uint16_t)(meta[pp].y >> 16));
      st.l_part[rg] += pv;
      st.az_part[rg] = fmaf(pv, fmaf(1.5f, vs, vz), st.az_part[rg]);
      w[pp] = pv * vs;
      ws += w[pp];
    }
    wsum[rg] = row_sum16(ws);
    uint8_t* tile_rg = wt + rg * 2048;
#pragma unroll
    for (int pp = 0; pp < 8; pp += 2) {
      uint32_t tt[4];
      split4(w[pp] * wmul, w[pp + 1] * wmul, tt);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint8_t* row = tile_rg + (4 * lg + j) * 128 + slot_pos;
        row[16 * pp] = (uint8_t)(tt[j] & 0xffu);
        row[16 * (pp + 1)] = (uint8_t)(tt[j] >> 8);
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // ---- values: acc[rg][nn] += w terms x V codes (channels 8lr + nn) ----
  const int wsc = clamp_scale(kScaleOne + wexp - 7 - 4 * (lr & 3));
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) {
    const uint8_t* row = wt + rg * 2048 + lr * 128;
    const uint4 a0 = *reinterpret_cast<const uint4*>(row + 16 * lg);
    const uint4 a1 = *reinterpret_cast<const uint4*>(row + 64 + 16 * lg);
    i32x8 wa;
    wa[0] = (int)a0.x;
    wa[1] = (int)a0.y;
    wa[2] = (int)a0.z;
    wa[3] = (int)a0.w;
    wa[4] = (int)a1.x;
    wa[5] = (int)a1.y;
    wa[6] = (int)a1.z;
    wa[7] = (int)a1.w;
    const float corr = 1.5f * wsum[rg];
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) {
      const uint32_t v0 = nn < 4 ? (&t.vlo[0].x)[nn] : (&t.vhi[0].x)[nn - 4];
      const uint32_t v1 = nn < 4 ? (&t.vlo[1].x)[nn] : (&t.vhi[1].x)[nn - 4];
      i32x8 bv;
      bv[0] = (int)(v0 & 0x33333333u);
      bv[1] = (int)((v0 >> 2) & 0x33333333u);
      bv[2] = (int)(v1 & 0x33333333u);
      bv[3] = (int)((v1 >> 2) & 0x33333333u);
      bv[4] = bv[5] = bv[6] = bv[7] = 0;
      st.acc[rg][nn] = mfma_f8_f4(wa, bv, st.acc[rg][nn], wsc, kScaleCode);
      st.acc[rg][nn][0] -= corr;
    }
  }
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ float wave_max64(float x) {
  x = row_max16(x);
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}


constexpr int kWinPass = 128;  // window tokens per pass (one per thread pair)

template <int GW>
constexpr int window_smem_bytes() { return (2 * GW * kD + kWinPass * 65 + 12 * GW) * 4; }

// bf16 window of one merge unit: positions [n - w, n) at ring slots pos % W,
// unrotated, for query heads hq0 .. hq0 + gw - 1; writes (m, l, acc[128]) per
// head to the window partials.  A pass takes up to 128 tokens with every load
// issued up front: thread pair (t, half) holds 64 dims of token t's key (for
// the scores) and stages the same dims of its value in LDS (for P V).
template <int GW>
__device__ void window_unit(const SplitParams& p, int b, int h, int hq0, int n, int w, float* sm) {
  constexpr int PER = (GW * kD + 255) / 256;
  const int tid = threadIdx.x, gw = p.gw, wave = tid >> 6;
  float* qs = sm;                                            // [GW][128]
  uint32_t* vw = reinterpret_cast<uint32_t*>(qs + GW * kD);  // [kWinPass][65] bf16 pairs
  float* ps = reinterpret_cast<float*>(vw + kWinPass * 65);  // [GW][kWinPass]
  float* red = ps + GW * kWinPass;                           // [4][GW]
  float* red2 = red + 4 * GW;                                // [4][GW]
  float* Mrun = red2 + 4 * GW;                               // [GW]
  float* Lrun = Mrun + GW;                                   // [GW]
  float* Mnew = Lrun + GW;                                   // [GW]
  float* Alph = Mnew + GW;                                   // [GW]
  for (int e = tid; e < GW * kD; e += 256)
    qs[e] = e < gw * kD ? bf16_to_f32(p.q[((int64_t)b * p.hq + hq0) * kD + e]) : 0.f;
  if (tid < GW) {
    Mrun[tid] = kNegInf;
    Lrun[tid] = 0.f;
  }
  float o2[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) o2[k] = 0.f;
  const int t = tid >> 1, hf = tid & 1;
  for (int cs = n - w; cs < n; cs += kWinPass) {
    const int nt = min(kWinPass, n - cs);
    const bool valid = t < nt;
    uint4 kk[8], vv[8];
    if (valid) {
      const int64_t row = (((int64_t)b * p.window + (cs + t) % p.window) * p.hkv + h) * kD + 64 * hf;
      const uint4* kr = reinterpret_cast<const uint4*>(p.win_k + row);
      const uint4* vr = reinterpret_cast<const uint4*>(p.win_v + row);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        kk[i] = kr[i];
        vv[i] = vr[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) kk[i] = vv[i] = make_uint4(0, 0, 0, 0);
    }
    __syncthreads();  // qs, Mrun ready; the previous pass is done with vw and ps
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t* dst = vw + t * 65 + 32 * hf + 4 * i;
      dst[0] = vv[i].x; dst[1] = vv[i].y; dst[2] = vv[i].z; dst[3] = vv[i].w;
    }
    float sc[GW];
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      const float* qg = qs + g * kD + 64 * hf;
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t u[4] = {kk[i].x, kk[i].y, kk[i].z, kk[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          d = fmaf(bf16lo(u[j]), qg[8 * i + 2 * j], fmaf(bf16hi(u[j]), qg[8 * i + 2 * j + 1], d));
      }
      d += dpp_f32<kDppSwap1>(d);  // the pair's two halves
      sc[g] = (valid && g < gw) ? d * p.scale_log2 : kNegInf;
      const float m = wave_max64(sc[g]);
      if ((tid & 63) == 0) red[wave * GW + g] = m;
    }
    __syncthreads();
    if (tid < GW) {
      const float mc = fmaxf(fmaxf(red[tid], red[GW + tid]), fmaxf(red[2 * GW + tid], red[3 * GW + tid]));
      const float mn = fmaxf(Mrun[tid], mc);
      Mnew[tid] = mn;
      Alph[tid] = mn == kNegInf ? 1.f : exp2f(Mrun[tid] - mn);
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      const float mn = Mnew[g];
      const float pv = sc[g] == kNegInf ? 0.f : exp2f(sc[g] - mn);
      if (hf == 0) ps[g * kWinPass + t] = pv;
    }
    __syncthreads();
    if (tid < GW) {
      float su = 0.f;
      for (int tt = 0; tt < nt; ++tt) su += ps[tid * kWinPass + tt];
      Lrun[tid] = Lrun[tid] * Alph[tid] + su;
      Mrun[tid] = Mnew[tid];
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = tid + 256 * k;
      const int g = e / kD, c = e % kD;
      float acc = o2[k] * Alph[g];
      const float* pg = ps + g * kWinPass;
      for (int tt = 0; tt < nt; ++tt) {
        const uint32_t x = vw[tt * 65 + (c >> 1)];
        acc = fmaf(pg[tt], (c & 1) ? bf16hi(x) : bf16lo(x), acc);
      }
      o2[k] = acc;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int e = tid + 256 * k;
    if (e >= gw * kD) break;
    const int g = e / kD, c = e % kD;
    float* dst = p.wpart + ((int64_t)b * p.hq + hq0 + g) * kPartStride;
    dst[2 + c] = o2[k];
    if (c == 0) {
      dst[0] = Mrun[g];
      dst[1] = Lrun[g];
    }
  }
}

// ---------------------------------------------------------------------------
// INT2 history split on the matrix cores.  Lane l = 16 lg + lr.
//   score MFMA output: head 4 rg + lg, token lr of the page;
//   value accumulators: head 4 rg + lg, channels 8 lr + n (n = 0..7);
//   loads per tile: K row bytes 8lg..8lg+7 of token lr and its metadata record
//   for each of the 8 pages; V words of channels 8lr..8lr+7 for pages 2lg, 2lg+1.
// The waves of a workgroup take the split's tiles round robin; each wave keeps
// the next tile's loads in flight while it computes the current one.
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256, G <= 4 ? 4 : 2) void int2_split_kernel(SplitParams p) {
  constexpr int NRG = (G + 3) / 4;                    // MFMA row groups of 4 heads
  constexpr int kTileBytes = 4 * NRG * 16 * 128;     // per-wave w-term tiles
  constexpr int kCombBytes = 4 * G * kD * 4 + 2 * 4 * G * 4;
  constexpr int kS1 = kTileBytes > kCombBytes ? kTileBytes : kCombBytes;
  constexpr int kSmem = kS1 > window_smem_bytes<G>() ? kS1 : window_smem_bytes<G>();

  // z = 0: the bf16 windows (x = sequence); they are dispatched before every
  // history split so that they overlap the history stream instead of trailing
  // it.  z = 1 + b: history split x of sequence b.
  const bool win_wg = blockIdx.z == 0;
  if (win_wg && (int)blockIdx.x >= p.batch) return;
  const int b = win_wg ? (int)blockIdx.x : (int)blockIdx.z - 1, h = blockIdx.y / p.gsub;
  const int sp = win_wg ? -1 : (int)blockIdx.x;
  const int sub = blockIdx.y % p.gsub;
  const int hq0 = h * p.gw * p.gsub + sub * p.gw;  // first query head of this workgroup
  const int n = seq_len_of(p, b);
  const int w = n < p.window ? n : p.window;
  const int hist = n - w;

  __shared__ __align__(16) uint8_t smem[kSmem];

  if (sp < 0) {  // the bf16 window of these heads, beside their history splits
    window_unit<G>(p, b, h, hq0, n, w, reinterpret_cast<float*>(smem));
    return;
  }
  const int t_begin = sp * p.split;
  if (t_begin >= hist) return;
  const int t_end = min(t_begin + p.split, hist);

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lg = lane >> 4, lr = lane & 15;

  // score operands prepared once per (sequence, KV head)
  i32x8 qa[NRG];
  int qsc[NRG];
  float qsr[NRG];
  const int ncb = (p.gw * p.gsub + 3) / 4;
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) {
    const int* src = p.qop + ((((int64_t)b * p.hkv + h) * ncb + (sub * p.gw) / 4 + rg) * 64 + lane) * 9;
#pragma unroll
    for (int i = 0; i < 8; ++i) qa[rg][i] = src[i];
    qsc[rg] = src[8];
    qsr[rg] = (4 * rg + lg < p.gw) ? p.qsum[(int64_t)b * p.hq + hq0 + 4 * rg + lg] : 0.f;
  }

  WaveState<NRG> st;
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) {
    st.m_run[rg] = kNegInf;
    st.l_part[rg] = 0.f;
    st.az_part[rg] = 0.f;
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) st.acc[rg][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  uint8_t* wt = smem + wave * (NRG * 2048);
  const int P0 = t_begin >> 4, P1 = (t_end - 1) >> 4;
  const int n_tiles = (P1 - P0 + 8) >> 3;
  const int* btr = p.block_table + (int64_t)b * p.max_pages;

  // The wave's tiles k = 0 .. ntw-1 are tiles wave + 4k of the split (at most
  // 4: a split holds at most 2048 tokens = 16 tiles).  One block-table load
  // covers them all, so a tile's loads never wait on a table read.  A wave keeps
  // one tile in registers: at ~122 VGPRs four waves share each SIMD, and the
  // other waves' work hides a wave's load latency (measured faster than keeping
  // two tiles per wave in flight at two waves per SIMD).
  const int ntw = wave < n_tiles ? (n_tiles - wave + 3) >> 2 : 0;
  const TileTable tab = load_table(p, btr, P0, P1, wave, 0);
  for (int k = 0; k < ntw; ++k) {
    const int pbase = P0 + 8 * (wave + 4 * k);
    Tile ta;
    load_tile(p, tab, k, h, pbase, t_end, lg, lr, ta);
    compute_tile<G, NRG>(p, ta, pbase, t_end, lg, lr, qa, qsc, qsr, wt, st);
  }

  // ---- per-wave partial -> LDS -> workgroup partial ----
  __syncthreads();  // every wave is done with its w-term tile before smem is reused
  float* cacc = reinterpret_cast<float*>(smem);  // [4][G][128]
  float* cm = cacc + 4 * G * kD;                 // [4][G]
  float* cl = cm + 4 * G;                        // [4][G]
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) {
    const float l = row_sum16(st.l_part[rg]), az = row_sum16(st.az_part[rg]);
    const int head = 4 * rg + lg;
    if (head < p.gw) {
#pragma unroll
      for (int nn = 0; nn < 8; ++nn)
        cacc[(wave * G + head) * kD + 8 * lr + nn] =
            (st.acc[rg][nn][0] + st.acc[rg][nn][1]) + (st.acc[rg][nn][2] + st.acc[rg][nn][3]) + az;
      if (lr == 0) {
        cm[wave * G + head] = st.m_run[rg];
        cl[wave * G + head] = l;
      }
    }
  }
  __syncthreads();
  combine_and_store<G>(p, cm, cl, cacc, b, hq0, sp, p.gw);
}

// ---------------------------------------------------------------------------
// bf16 comparator split: plain attention over bf16 pages, all n positions, on
// the matrix cores (v_mfma_f32_16x16x32_bf16).  Pool block per (page, KV head):
// K rows [16][128], then V transposed [128][16].  A tile is 32 tokens (2 pages).
//   scores: A = K (rows = 16 tokens), B = q^T (columns = query heads) -> lane
//           (g, r) holds tokens 4g .. 4g + 3 of head r;
//   P V:    A = p^T (rows = (head, hi|lo), k = 32 tokens), B = V (k = tokens,
//           columns = 16 channels) -> lane (g, r) holds channel 16c + r of rows
//           4g .. 4g + 3.
// The softmax weights go through a per-wave LDS tile as two bf16 rows each
// (p = hi + lo, about 16 significant bits); q is bf16 already, so the scores
// are exact products accumulated in fp32.
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void bf16_split_kernel(SplitParams p) {
  constexpr int NRG = (2 * G + 15) / 16;  // P V row groups: 8 heads x (hi, lo) rows each
  const int b = blockIdx.z, h = blockIdx.y, sp = blockIdx.x;
  const int n = seq_len_of(p, b);
  const int t_begin = sp * p.split;
  if (t_begin >= n) return;
  const int t_end = min(t_begin + p.split, n);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;

  __shared__ __align__(16) uint16_t pt[4][NRG][16][40];  // per wave: p^T rows x 32 tokens (bf16), padded rows
  __shared__ float alph[4][16];
  __shared__ float cm[4 * G], cl[4 * G];
  __shared__ float cacc[4 * G * kD];

  for (int e = tid; e < 4 * NRG * 16 * 40; e += 256) (&pt[0][0][0][0])[e] = 0;  // rows of absent heads stay 0
  if (tid < 64) (&alph[0][0])[tid] = 1.f;

  // B operand of the scores: column r = query head r, k-slots 8g .. 8g + 7 of each 32-dim chunk
  uint4 qb[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qb[s] = r < G ? *reinterpret_cast<const uint4*>(p.q + ((int64_t)b * p.hq + h * G + r) * kD + 32 * s + 8 * g)
                  : make_uint4(0, 0, 0, 0);

  float m_run = kNegInf, l_part = 0.f;  // head r
  f32x4 acc[NRG][8];
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[rg][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // block-table entries of the wave's tiles (tile k of the wave = tile wave + 4k,
  // pages P0 + 2 (wave + 4k) + {0, 1}): lane 2k + pp, at most 32 tiles (2048 tokens / 4 waves)
  const int P0 = t_begin >> 4, P1 = (t_end - 1) >> 4;
  const int n_tiles = (P1 - P0 + 2) >> 1;
  const int ntw = wave < n_tiles ? (n_tiles - wave + 3) >> 2 : 0;
  const int* btr = p.block_table + (int64_t)b * p.max_pages;
  int ent;
  {
    const int pg = P0 + 2 * (wave + 4 * (lane >> 1)) + (lane & 1);
    ent = pg <= P1 ? btr[pg] : -1;
    ent = (ent >= 0 && ent < p.n_pages) ? ent : -1;
  }
  const uint64_t live = __ballot(ent >= 0);
  __syncthreads();  // pt, alph initialised

  for (int k = 0; k < ntw; ++k) {
    const int pbase = P0 + 2 * (wave + 4 * k);
    const int ea = __builtin_amdgcn_readlane(ent, 2 * k), eb = __builtin_amdgcn_readlane(ent, 2 * k + 1);
    const int pg0 = ea < 0 ? 0 : ea, pg1 = eb < 0 ? 0 : eb;
    const uint32_t ok = (uint32_t)(live >> (2 * k)) & 3u;
    const uint16_t* blk0 = p.kv_pool + ((int64_t)pg0 * p.hkv + h) * (2 * kPage * kD);
    const uint16_t* blk1 = p.kv_pool + ((int64_t)pg1 * p.hkv + h) * (2 * kPage * kD);
    uint4 kk[2][4], vv[8];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      kk[0][s] = *reinterpret_cast<const uint4*>(blk0 + r * kD + 32 * s + 8 * g);
      kk[1][s] = *reinterpret_cast<const uint4*>(blk1 + r * kD + 32 * s + 8 * g);
    }
    const uint16_t* vblk = (g >> 1) ? blk1 : blk0;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      vv[c] = *reinterpret_cast<const uint4*>(vblk + kPage * kD + (16 * c + r) * kPage + 8 * (g & 1));

    // ---- scores and online softmax of head r ----
    float lg[2][4];
    float mx = kNegInf;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kk[pp][s]),
                                                     __builtin_bit_cast(bf16x8, qb[s]), sc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = (pbase + pp) * 16 + 4 * g + i;
        const bool valid = r < G && ((ok >> pp) & 1u) && tok < t_end;
        const float v = pin(sc[i] * p.scale_log2);
        lg[pp][i] = valid ? v : kNegInf;
        mx = fmaxf(mx, lg[pp][i]);
      }
    }
    mx = max_rows(mx);
    const float m_new = fmaxf(m_run, mx);
    const bool grow = __any(m_new > m_run);
    if (grow) {
      const float alpha = m_new == kNegInf ? 1.f : exp2f(m_run - m_new);
      l_part *= alpha;
      if (g == 0) alph[wave][r] = alpha;
      m_run = m_new;
    }
    const float m_safe = m_run == kNegInf ? 0.f : m_run;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      uint32_t hw[2], lw[2];
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const float p0 = exp2f(lg[pp][i] - m_safe), p1 = exp2f(lg[pp][i + 1] - m_safe);
        l_part += p0 + p1;
        const uint32_t h0 = bf16_rne_bits(p0), h1 = bf16_rne_bits(p1);
        const uint32_t l0 = bf16_rne_bits(p0 - bf16_to_f32(h0)), l1 = bf16_rne_bits(p1 - bf16_to_f32(h1));
        hw[i >> 1] = h0 | (h1 << 16);
        lw[i >> 1] = l0 | (l1 << 16);
      }
      if (r < G) {
        uint16_t* row = &pt[wave][r >> 3][2 * (r & 7)][16 * pp + 4 * g];
        *reinterpret_cast<uint2*>(row) = make_uint2(hw[0], hw[1]);
        *reinterpret_cast<uint2*>(row + 40) = make_uint2(lw[0], lw[1]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- P V ----
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
      if (grow) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = alph[wave][(8 * rg + 2 * g + (i >> 1)) & 15];
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[rg][c][i] *= a;
        }
      }
      const uint4 pa = *reinterpret_cast<const uint4*>(&pt[wave][rg][r][8 * g]);
#pragma unroll
      for (int c = 0; c < 8; ++c)
        acc[rg][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pa),
                                                             __builtin_bit_cast(bf16x8, vv[c]), acc[rg][c], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- per-wave partial -> LDS -> workgroup partial ----
  float l = l_part;
  {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(l), __float_as_uint(l), false, false);
    l = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto c2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
    l = __uint_as_float(c2[0]) + __uint_as_float(c2[1]);
  }
  if (g == 0 && r < G) {
    cm[wave * G + r] = m_run;
    cl[wave * G + r] = l;
  }
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int head = 8 * rg + 2 * g + j;
      if (head < G) {
#pragma unroll
        for (int c = 0; c < 8; ++c) cacc[(wave * G + head) * kD + 16 * c + r] = acc[rg][c][2 * j] + acc[rg][c][2 * j + 1];
      }
    }
  __syncthreads();
  combine_and_store<G>(p, cm, cl, cacc, b, h * G, sp);
}

// ---------------------------------------------------------------------------
// merge: one workgroup per (sequence, q head).  Log-sum-exp merge of the split
// partials; for the INT2 path the un-rotation by R_V^T and the bf16 window's
// partial, then the normalisation.  Every load the workgroup needs (the split
// partials, its 128 x 128 R_V tile, the window partial) is issued up front, so
// the kernel costs about one memory round trip.  A head with no position at
// all gets zeros.
// ---------------------------------------------------------------------------
constexpr int kMergeSplits = 64;  // splits whose accumulators a thread pair holds in registers per pass

__global__ __launch_bounds__(256) void merge_kernel(SplitParams p, int gq) {
  const int b = blockIdx.y, hq = blockIdx.x, h = hq / gq, tid = threadIdx.x;
  const bool int2 = p.r_v != nullptr;
  const int n = seq_len_of(p, b);
  const int w = int2 ? (n < p.window ? n : p.window) : 0;
  const int hist = n - w;
  const int ns = (hist + p.split - 1) / p.split;

  __shared__ float fs[kMergeSplits * 2];      // 2^(m_s - M), l_s of the current pass
  __shared__ float red[256];
  __shared__ float a1s[kD];
  __shared__ float o1p[16][kD + 4];
  __shared__ float Ms, Ls;

  // R_V tile loads first (INT2): thread (cg, jg) takes channels 8cg..8cg+7 of rows 8jg..8jg+7
  const int cg = tid & 15, jg = tid >> 4;
  uint4 rv[8];
  if (int2) {
    const uint16_t* r = p.r_v + ((int64_t)h * kD + 8 * jg) * kD + 8 * cg;
#pragma unroll
    for (int j = 0; j < 8; ++j) rv[j] = *reinterpret_cast<const uint4*>(r + j * kD);
  }
  // split partials: thread (c, half) sums channel c over the splits s = half, half + 2, ...
  const int c = tid & 127, half = tid >> 7;
  const float* base = p.part + ((int64_t)b * p.hq + hq) * p.n_splits * kPartStride;
  float M = kNegInf;
  for (int s = tid; s < ns; s += 256) M = fmaxf(M, base[s * kPartStride]);
  M = wave_max64(M);
  if ((tid & 63) == 0) red[tid >> 6] = M;
  __syncthreads();
  if (tid == 0) Ms = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  M = Ms;
  float acc = 0.f, lsum = 0.f;
  for (int s0 = 0; s0 < ns; s0 += kMergeSplits) {
    const int cnt = min(kMergeSplits, ns - s0);
    __syncthreads();
    if (tid < cnt) {
      const float* ps = base + (s0 + tid) * kPartStride;
      const float m = ps[0];
      fs[tid] = m == kNegInf ? 0.f : exp2f(m - M);
      fs[kMergeSplits + tid] = ps[1];
    }
    __syncthreads();
    float x[kMergeSplits / 2];
#pragma unroll
    for (int k = 0; k < kMergeSplits / 2; ++k) {
      const int s = 2 * k + half;
      x[k] = s < cnt ? base[(s0 + s) * kPartStride + 2 + c] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kMergeSplits / 2; ++k) {
      const int s = 2 * k + half;
      if (s < cnt) {
        acc = fmaf(fs[s], x[k], acc);
        if (c == 0) lsum = fmaf(fs[s], fs[kMergeSplits + s], lsum);
      }
    }
  }
  red[tid] = acc;
  if (c == 0) o1p[0][half] = lsum;
  __syncthreads();
  if (tid < kD) a1s[tid] = red[tid] + red[tid + 128];
  if (tid == 0) Ls = o1p[0][0] + o1p[0][1];
  __syncthreads();
  float* dst = p.out + ((int64_t)b * p.hq + hq) * kD;
  if (!int2) {
    if (tid < kD) dst[tid] = Ls > 0.f ? a1s[tid] / Ls : 0.f;
    return;
  }
  // o1 = R_V^T a1 from the register tile, partial sums over 8 rows per thread
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float aj = a1s[8 * jg + j];
    const uint32_t u[4] = {rv[j].x, rv[j].y, rv[j].z, rv[j].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = fmaf(bf16lo(u[i]), aj, o[2 * i]);
      o[2 * i + 1] = fmaf(bf16hi(u[i]), aj, o[2 * i + 1]);
    }
  }
  __syncthreads();  // o1p[0][0..1] (the l sums) were read
#pragma unroll
  for (int i = 0; i < 8; ++i) o1p[jg][8 * cg + i] = o[i];
  __syncthreads();
  if (tid < kD) {
    float o1 = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) o1 += o1p[k][tid];
    const float* wp = p.wpart + ((int64_t)b * p.hq + hq) * kPartStride;
    const float m1 = M, m2 = wp[0];
    const float Mx = fmaxf(m1, m2);
    const float f1 = m1 == kNegInf ? 0.f : exp2f(m1 - Mx);
    const float f2 = m2 == kNegInf ? 0.f : exp2f(m2 - Mx);
    const float den = f1 * Ls + f2 * wp[1];
    dst[tid] = den > 0.f ? (f1 * o1 + f2 * wp[2 + tid]) / den : 0.f;
  }
}

template <int G>
int launch_decode(bool int2, const SplitParams& sp, const uint16_t* r_k, int batch, hipStream_t s) {
  // INT2: at most 8 query heads per workgroup (register budget of the MFMA
  // tiles), and the 4-head instantiation for G < 4 masking the missing heads
  constexpr int GW = G > 8 ? 8 : (G < 4 ? 4 : G);
  SplitParams p2 = sp;
  if (int2) {
    p2.gw = G < GW ? G : GW;
    p2.gsub = G / p2.gw;
    prep_q_kernel<G><<<dim3(batch, sp.hkv), 256, 0, s>>>(r_k, sp.q, const_cast<float*>(sp.qsum),
                                                         const_cast<int*>(sp.qop), sp.hq, sp.hkv);
    if (hipGetLastError() != hipSuccess) return OSCAR_EHIP;
  }
  int slot = -1;
  timing_record_begin(s, int2 ? 1 : 2, &slot);
  if (int2)  // a leading z slab: one workgroup per (sequence, KV head, head subset) takes the bf16 window
    int2_split_kernel<GW><<<dim3(sp.n_splits > batch ? sp.n_splits : batch, sp.hkv * p2.gsub, batch + 1), 256, 0, s>>>(p2);
  else
    bf16_split_kernel<G><<<dim3(sp.n_splits, sp.hkv, batch), 256, 0, s>>>(sp);
  if (hipGetLastError() != hipSuccess) return OSCAR_EHIP;
  timing_record_end(s, slot);
  merge_kernel<<<dim3(sp.hq, batch), 256, 0, s>>>(sp, G);
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
  const SplitPlan plan = plan_splits(batch, shape->n_kv_heads, shape->n_q_heads / shape->n_kv_heads, max_seq_len,
                                     device_cu_count());
  const WorkspaceLayout wl = workspace_layout(batch, shape->n_q_heads, shape->n_kv_heads, plan);
  if (workspace_bytes < wl.total) return OSCAR_ENOSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return OSCAR_EINVAL;

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  SplitParams sp{};
  sp.qsum = reinterpret_cast<float*>(ws + wl.qsum);
  sp.qop = reinterpret_cast<int*>(ws + wl.qop);
  sp.q = q;
  sp.seq_lens = seq_lens;
  sp.block_table = block_table;
  sp.pool = pool;
  sp.kv_pool = kv_pool;
  sp.r_v = int2 ? r_v : nullptr;
  sp.win_k = win_k;
  sp.win_v = win_v;
  sp.part = reinterpret_cast<float*>(ws + wl.part);
  sp.wpart = reinterpret_cast<float*>(ws + wl.wpart);
  sp.out = out;
  sp.n_pages = n_pages;
  sp.batch = batch;
  sp.hq = shape->n_q_heads;
  sp.hkv = shape->n_kv_heads;
  sp.max_pages = max_pages_per_seq;
  sp.max_len = max_seq_len;
  sp.window = int2 ? shape->window : 0;
  sp.split = plan.split;
  sp.n_splits = plan.n_splits;
  sp.gsub = 1;
  sp.gw = shape->n_q_heads / shape->n_kv_heads;
  sp.scale_log2 = kLog2e / sqrtf((float)kD);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (shape->n_q_heads / shape->n_kv_heads) {
    case 1: return launch_decode<1>(int2, sp, r_k, batch, s);
    case 2: return launch_decode<2>(int2, sp, r_k, batch, s);
    case 4: return launch_decode<4>(int2, sp, r_k, batch, s);
    case 8: return launch_decode<8>(int2, sp, r_k, batch, s);
    case 16: return launch_decode<16>(int2, sp, r_k, batch, s);
  }
  return OSCAR_EUNSUPPORTED;
}

// bf16 comparator append: K rows into [page][Hkv] elements [16 slot][128],
// V into the transposed part, element 2048 + 16 c + slot.
__global__ __launch_bounds__(256) void bf16_append_kernel(const uint16_t* __restrict__ k_new,
                                                          const uint16_t* __restrict__ v_new, int64_t n_tokens,
                                                          const int32_t* seq_idx, const int32_t* pos, int batch,
                                                          const int32_t* block_table, int max_pages,
                                                          uint16_t* kv_pool, int64_t n_pages, int hkv) {
  // one thread per (token, head, 8-channel chunk of K or V)
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
  const uint4 src = reinterpret_cast<const uint4*>((kv ? v_new : k_new) + (t * hkv + h) * kD)[chunk];
  uint16_t* blk = kv_pool + ((int64_t)page * hkv + h) * (2 * kPage * kD);
  const int slot = ps & 15;
  if (kv == 0) {
    reinterpret_cast<uint4*>(blk + slot * kD)[chunk] = src;
  } else {
    const uint32_t w[4] = {src.x, src.y, src.z, src.w};
    uint16_t* vt = blk + kPage * kD + (8 * chunk) * kPage + slot;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vt[(2 * e) * kPage] = (uint16_t)(w[e] & 0xffffu);
      vt[(2 * e + 1) * kPage] = (uint16_t)(w[e] >> 16);
    }
  }
}

}  // namespace
}  // namespace oscar

extern "C" size_t oscar_decode_workspace_bytes(const oscar_shape* shape, int32_t batch, int32_t max_seq_len) {
  using namespace oscar;
  if (check_shape(shape) != OSCAR_OK || batch < 1 || max_seq_len < 1) return 0;
  return workspace_layout(batch, shape->n_q_heads, shape->n_kv_heads,
                          plan_splits(batch, shape->n_kv_heads, shape->n_q_heads / shape->n_kv_heads, max_seq_len,
                                      device_cu_count())).total;
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
