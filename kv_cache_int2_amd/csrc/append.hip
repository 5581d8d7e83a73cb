// Online rotate -> quantise -> pack of new K/V tokens into the paged INT2 cache.
// Method: P1 (gen-hub.ru, "Together AI открывает OSCAR…") «Что придумали в
// Together AI» (per-head rotation R = P_br H U^T of keys and values) and «Почему
// INT2 раньше не работал» (four levels); P2 (encorp.ai) «OSCAR има значение…»
// (recent tokens kept in bf16, history in INT2, paged storage).
//
// One workgroup = 4 waves = 64 tokens per iteration of one (KV head, K|V).
// R (128 x 128 bf16) is staged once per workgroup in LDS.  Each wave rotates 16
// tokens with v_mfma_f32_16x16x32_bf16: 8 output tiles x 4 k-steps.
//  - keys use A = R, B = X^T: a lane ends with 32 channels of ONE token, so the
//    per-token min/max needs 2 shuffles and the token-major K row is assembled
//    from 4 lanes' bytes;
//  - values use A = X, B = R^T: a lane ends with 4 tokens x 8 channels, so the
//    channel-major V words (16 slots x 2 bits) are assembled from 4 lanes and a
//    whole aligned page is written with plain stores; a partial page falls back
//    to per-token atomic and/or on the channel words.
// The k-slot -> input channel map (lane group g, step s, slot j -> 32g + 8s + j)
// is the same for both operands, so the hardware's internal k order is moot.
#include "common.h"

namespace oscar {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct AppendParams {
  const uint16_t* r[2];  // K, V rotations [Hkv][128][128]
  const uint16_t* x[2];  // k_new, v_new [T][Hkv][128]
  uint16_t* win[2];      // window rings [B][W][Hkv][128]
  const int32_t* seq_idx;
  const int32_t* pos;
  const int32_t* block_table;
  const int32_t* len_after;
  uint8_t* pool;
  int64_t n_tokens;
  int64_t n_pages;
  int batch, max_pages, hkv, window, tiles_per_wg;
};

constexpr int kRowU4 = 17;  // LDS row stride of R in uint4 (16 + 1 pad: 272 B)

__device__ __forceinline__ f32x4 mfma(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t encode(float v, float z, float s) {
  if (s == 0.f) return 0u;
  float t = rintf((v - z) / s);
  t = fminf(fmaxf(t, 0.f), 3.f);
  return (uint32_t)t;
}

// Resolve token `tok`: returns its block base (or nullptr if it must be skipped)
// and slot; also whether it enters the bf16 window and its window slot.
struct TokInfo {
  uint8_t* blk;
  int slot;
  int b;
  int pos;
  bool in_win;
};

__device__ __forceinline__ TokInfo resolve(const AppendParams& p, int64_t tok, int h) {
  TokInfo ti{nullptr, 0, 0, 0, false};
  if (tok >= p.n_tokens) return ti;
  int b = p.seq_idx[tok], ps = p.pos[tok];
  if (b < 0 || b >= p.batch || ps < 0 || (ps >> 4) >= p.max_pages) return ti;
  int page = p.block_table[(int64_t)b * p.max_pages + (ps >> 4)];
  if (page < 0 || page >= p.n_pages) return ti;
  ti.blk = p.pool + ((int64_t)page * p.hkv + h) * kBlock;
  ti.slot = ps & 15;
  ti.b = b;
  ti.pos = ps;
  ti.in_win = p.window > 0 && ps >= p.len_after[b] - p.window;
  return ti;
}

template <int KIND>
__device__ __forceinline__ void process_tile(const AppendParams& p, const uint4* r_lds, int64_t t0,
                                             int h, int lane) {
  const int g = lane >> 4, r = lane & 15;
  const int64_t tok = t0 + r;
  TokInfo ti = resolve(p, tok, h);
  const bool valid = tok < p.n_tokens;

  // X operand: token t0 + r, input channels 32g .. 32g + 31
  uint4 xv[4];
  const uint4* xp = reinterpret_cast<const uint4*>(p.x[KIND] + ((valid ? tok : 0) * p.hkv + h) * kD + 32 * g);
#pragma unroll
  for (int s = 0; s < 4; ++s) xv[s] = valid ? xp[s] : make_uint4(0, 0, 0, 0);

  f32x4 acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 rv = r_lds[(16 * m + r) * kRowU4 + 4 * g + s];
      acc[m] = KIND == 0 ? mfma(rv, xv[s], acc[m]) : mfma(xv[s], rv, acc[m]);
    }
  }

  // raw bf16 copy into the window ring (same for K and V)
  if (ti.blk && ti.in_win) {
    uint4* wp = reinterpret_cast<uint4*>(p.win[KIND] + (((int64_t)ti.b * p.window + ti.pos % p.window) * p.hkv + h) * kD + 32 * g);
#pragma unroll
    for (int s = 0; s < 4; ++s) wp[s] = xv[s];
  }

  if (KIND == 0) {
    // acc[m][i] = x'[token t0 + r][channel 16m + 4g + i]
    float mn = acc[0][0], mx = acc[0][0];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        mn = fminf(mn, acc[m][i]);
        mx = fmaxf(mx, acc[m][i]);
      }
    mn = fminf(mn, __shfl_xor(mn, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mn = fminf(mn, __shfl_xor(mn, 32));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float sigma = (mx - mn) / 3.0f;
    const uint16_t sb = f2h_bits(sigma), zb = f2h_bits(mn);
    const float sc = h2f(sb), z = h2f(zb);
    uint32_t dw[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      uint32_t byte = encode(acc[m][0], z, sc) | (encode(acc[m][1], z, sc) << 2) |
                      (encode(acc[m][2], z, sc) << 4) | (encode(acc[m][3], z, sc) << 6);
      uint32_t d = byte << (8 * g);
      d |= __shfl_xor(d, 16);
      d |= __shfl_xor(d, 32);
      dw[m] = d;
    }
    if (ti.blk) {
      uint2 out = make_uint2(dw[0], dw[1]);
      if (g == 1) out = make_uint2(dw[2], dw[3]);
      if (g == 2) out = make_uint2(dw[4], dw[5]);
      if (g == 3) out = make_uint2(dw[6], dw[7]);
      *reinterpret_cast<uint2*>(ti.blk + kKCodes + 32 * ti.slot + 8 * g) = out;
      if (g == 0) *reinterpret_cast<uint32_t*>(ti.blk + kMeta + 8 * ti.slot) = (uint32_t)sb | ((uint32_t)zb << 16);
    }
  } else {
    // acc[m][i] = x'[token t0 + 4g + i][channel 16m + r]
    float sc[4], z[4];
    uint16_t sbits[4], zbits[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mn = acc[0][i], mx = acc[0][i];
#pragma unroll
      for (int m = 1; m < 8; ++m) {
        mn = fminf(mn, acc[m][i]);
        mx = fmaxf(mx, acc[m][i]);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, o));
        mx = fmaxf(mx, __shfl_xor(mx, o));
      }
      const float sigma = (mx - mn) / 3.0f;
      sbits[i] = f2h_bits(sigma);
      zbits[i] = f2h_bits(mn);
      sc[i] = h2f(sbits[i]);
      z[i] = h2f(zbits[i]);
    }
    uint32_t code[8][4];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) code[m][i] = encode(acc[m][i], z[i], sc[i]);

    // fast path: the wave's 16 tokens are slots 0..15 of one page, in order
    const int b0 = __shfl(ti.b, 0), pos0 = __shfl(ti.pos, 0);
    uint8_t* blk0 = reinterpret_cast<uint8_t*>(__shfl(reinterpret_cast<uintptr_t>(ti.blk), 0));
    const bool mine = ti.blk != nullptr && ti.b == b0 && ti.pos == pos0 + r && (pos0 & 15) == 0;
    const bool full = __all(mine);
    // per-token info of the 4 tokens this lane holds codes for
    uint8_t* tblk[4];
    int tslot[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tblk[i] = reinterpret_cast<uint8_t*>(__shfl(reinterpret_cast<uintptr_t>(ti.blk), 4 * g + i));
      tslot[i] = __shfl(ti.slot, 4 * g + i);
    }
    if (full) {
      uint32_t w[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        uint32_t d = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) d |= code[m][i] << (2 * (4 * g + i));
        d |= __shfl_xor(d, 16);
        d |= __shfl_xor(d, 32);
        w[m] = d;
      }
      uint32_t* vw = reinterpret_cast<uint32_t*>(blk0 + kVCodes);
#pragma unroll
      for (int m = 0; m < 8; ++m)
        if ((m >> 1) == g) vw[16 * m + r] = w[m];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!tblk[i]) continue;
        uint32_t* vw = reinterpret_cast<uint32_t*>(tblk[i] + kVCodes);
        const uint32_t clr = ~(3u << (2 * tslot[i]));
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          atomicAnd(&vw[16 * m + r], clr);
          atomicOr(&vw[16 * m + r], code[m][i] << (2 * tslot[i]));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!tblk[i]) continue;
      if (r == i)
        *reinterpret_cast<uint32_t*>(tblk[i] + kMeta + 8 * tslot[i] + 4) = (uint32_t)sbits[i] | ((uint32_t)zbits[i] << 16);
    }
  }
}

__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  __shared__ uint4 r_lds[128 * kRowU4];
  const int h = blockIdx.y;
  const int kind = blockIdx.z;
  const uint4* rg = reinterpret_cast<const uint4*>(p.r[kind] + (int64_t)h * kD * kD);
  for (int i = threadIdx.x; i < 128 * 16; i += 256) r_lds[(i >> 4) * kRowU4 + (i & 15)] = rg[i];
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int it = 0; it < p.tiles_per_wg; ++it) {
    const int64_t t0 = ((int64_t)blockIdx.x * p.tiles_per_wg + it) * 64 + wave * 16;
    if (t0 >= p.n_tokens) break;
    if (kind == 0)
      process_tile<0>(p, r_lds, t0, h, lane);
    else
      process_tile<1>(p, r_lds, t0, h, lane);
  }
}

}  // namespace
}  // namespace oscar

extern "C" int oscar_quantize_append(const oscar_shape* shape, const uint16_t* r_k, const uint16_t* r_v,
                                     const uint16_t* k_new, const uint16_t* v_new, int64_t n_tokens,
                                     const int32_t* seq_idx, const int32_t* pos, int32_t batch,
                                     const int32_t* block_table, int32_t max_pages_per_seq,
                                     const int32_t* seq_len_after, uint8_t* pool, int64_t n_pages,
                                     uint16_t* win_k, uint16_t* win_v, void* stream) {
  using namespace oscar;
  int st = check_shape(shape);
  if (st != OSCAR_OK) return st;
  if (n_tokens < 0 || batch < 1 || max_pages_per_seq < 1 || n_pages < 1) return OSCAR_EINVAL;
  if (n_tokens == 0) return OSCAR_OK;
  if (!r_k || !r_v || !k_new || !v_new || !seq_idx || !pos || !block_table || !seq_len_after || !pool)
    return OSCAR_EINVAL;
  if (shape->window > 0 && (!win_k || !win_v)) return OSCAR_EINVAL;
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new) |
       reinterpret_cast<uintptr_t>(r_k) | reinterpret_cast<uintptr_t>(r_v) |
       reinterpret_cast<uintptr_t>(pool) | reinterpret_cast<uintptr_t>(win_k) |
       reinterpret_cast<uintptr_t>(win_v)) & 15)
    return OSCAR_EINVAL;
  AppendParams p;
  p.r[0] = r_k;
  p.r[1] = r_v;
  p.x[0] = k_new;
  p.x[1] = v_new;
  p.win[0] = win_k;
  p.win[1] = win_v;
  p.seq_idx = seq_idx;
  p.pos = pos;
  p.block_table = block_table;
  p.len_after = seq_len_after;
  p.pool = pool;
  p.n_tokens = n_tokens;
  p.n_pages = n_pages;
  p.batch = batch;
  p.max_pages = max_pages_per_seq;
  p.hkv = shape->n_kv_heads;
  p.window = shape->window;
  const int64_t tiles = (n_tokens + 63) / 64;
  p.tiles_per_wg = tiles >= 1024 ? 8 : (tiles >= 256 ? 4 : 1);
  dim3 grid((unsigned)((tiles + p.tiles_per_wg - 1) / p.tiles_per_wg), (unsigned)p.hkv, 2);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int slot = -1;
  timing_record_begin(s, 3, &slot);
  append_kernel<<<grid, 256, 0, s>>>(p);
  hipError_t e = hipGetLastError();
  timing_record_end(s, slot);
  return e == hipSuccess ? OSCAR_OK : OSCAR_EHIP;
}
