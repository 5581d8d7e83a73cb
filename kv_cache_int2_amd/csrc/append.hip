// Online rotate -> quantise -> pack of new K/V tokens into the paged INT2 cache.
// Method: P1 (gen-hub.ru, "Together AI открывает OSCAR…") «Что придумали в
// Together AI» (per-head rotation R = P_br H U^T of keys and values) and «Почему
// INT2 раньше не работал» (four levels); P2 (encorp.ai) «OSCAR има значение…»
// (recent tokens kept in bf16, history in INT2, paged storage).
//
// One workgroup = 4 waves = 64 tokens per iteration of one (KV head, K|V).
// R (128 x 128 bf16) is staged once per workgroup in LDS.  Each wave rotates its
// 16-token tile(s) with v_mfma_f32_16x16x32_bf16; every R tile read from LDS
// feeds every token tile of the wave.  One tile per wave by default: at ~114
// VGPRs four waves share each SIMD, which measured faster than two tiles per
// wave (fewer LDS reads of R) at two waves per SIMD.
//  - keys use A = R, B = X^T: a lane ends with channels 16m + 4g + i (m = 0..7,
//    i = 0..3) of ONE token, exactly the 8-byte segment g of the token's K row,
//    so it writes that segment itself;
//  - values use A = X, B = R^T: a lane ends with 4 tokens x 8 channels, so the
//    channel-major V words (16 slots x 2 bits) are OR-ed over the 4 lane groups
//    with permlane swaps and a whole aligned page is written with plain stores;
//    a partial page falls back to per-token atomic and/or on the channel words.
// The k-slot -> input channel map (lane group g, step s, slot j -> 32g + 8s + j)
// is the same for both operands, so the hardware's internal k order is moot.
// Groups: with NG = 128 / g groups per token, group j is rotated channels
// [g j, g (j + 1)); the channels 16m + .. a lane holds for accumulator m all fall
// in group m NG / 8, so each group's min and max are reduced on their own and
// every group of every token gets its own record at 1024 + 8 (NG slot + j).
// Codes: t = (x' - z) / s is evaluated as x' * (1/s) - z * (1/s) (one FMA; the
// reciprocal once per token); it differs from the quotient by a few ulp, so a
// code can only differ next to a rounding boundary.  The scale itself is the
// correctly rounded fp32 (max - min) / 3, as the definition has it.
#include "common.h"

namespace oscar {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct AppendParams {
  const uint16_t* r[2];  // K, V rotations [Hkv][128][128]
  const uint16_t* x[2];  // k_new, v_new [T][Hkv][128]
  uint16_t* win[2];      // bf16 rings [B][W + n_sink][Hkv][128]
  const int32_t* seq_idx;
  const int32_t* pos;
  const int32_t* block_table;
  const int32_t* len_after;
  uint8_t* pool;
  int block;   // bytes per (page, KV head) block: 1024 + 128 NG
  int64_t n_tokens;
  int64_t n_pages;
  int batch, max_pages, hkv, window, tiles_per_wg;
  int n_sink;  // leading positions also kept in bf16 (ring rows window + pos)
  int ring;    // ring rows per sequence: window + n_sink
  // layers appended in one launch: rotations, tokens, rings and pools stacked
  // layer-major with these strides (elements; pool in bytes); positions, block
  // table and lengths shared by all layers
  int64_t ls_rot, ls_x, ls_win, ls_pool;
};

constexpr int kRowU4 = 17;  // LDS row stride of R in uint4 (16 + 1 pad: 272 B)
#ifndef OSCAR_APPEND_TILES
#define OSCAR_APPEND_TILES 1
#endif
constexpr int kAppendTiles = OSCAR_APPEND_TILES;  // 16-token tiles per wave and iteration
constexpr int kAppendTokens = 4 * 16 * kAppendTiles;  // tokens per workgroup and iteration

__device__ __forceinline__ f32x4 mfma(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// code = clamp(rint(t), 0, 3) with t = x * inv - zi
__device__ __forceinline__ uint32_t encode(float v, float inv, float zi) {
  const float t = __builtin_amdgcn_fmed3f(fmaf(v, inv, -zi), 0.f, 3.f);
  return (uint32_t)__builtin_rintf(t);
}

// Scale and zero of a group from its min and max: s16 = fp16((max - min) / 3),
// z16 = fp16(min); codes are taken against the stored (fp16) values.  The
// division by 3 is q0 = d * fl(1/3) corrected once with the exact remainder
// d - 3 q0 (an FMA), which gives the correctly rounded quotient; 1/s is the
// hardware reciprocal (a code can only move next to a rounding boundary).
struct Quant {
  uint32_t sz;  // s16 | z16 << 16
  float inv, zi;
};
__device__ __forceinline__ Quant quant_params(float mn, float mx) {
  const float d = mx - mn;
  const float q0 = d * 0.333333343f;
  const float sigma = fmaf(fmaf(-3.0f, q0, d), 0.333333343f, q0);
  const uint16_t sb = f2h_bits(sigma), zb = f2h_bits(mn);
  const float sc = h2f(sb), z = h2f(zb);
  Quant q;
  q.sz = (uint32_t)sb | ((uint32_t)zb << 16);
  q.inv = sc > 0.f ? __builtin_amdgcn_rcpf(sc) : 0.f;  // a zero scale codes every channel 0
  q.zi = z * q.inv;
  return q;
}

template <int LANE>  // value of lane LANE of each quad, on all 4 lanes of the quad
__device__ __forceinline__ uint32_t quad_bcast(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, LANE * 0x55, 0xf, 0xf, true);
}

// Destination of one token (see resolve).
struct TokInfo {
  uint8_t* blk;
  int slot;
  int b;
  int pos;
  bool in_win;   // recent: ring row pos % window
  bool in_sink;  // sink: ring row window + pos
};

// Indices of the tokens of one wave's 16-token tile(s) (token t0 + 16 j + r):
// raw sequence and position (-1 past the last token), then block-table entry
// and sequence length.  The first tile's are loaded while the rotation is
// staged, so their chain of dependent loads is off the critical path.
struct TileIdx {
  int b[kAppendTiles], ps[kAppendTiles];
  int2 pl[kAppendTiles];  // lookup(b, ps)
};

__device__ __forceinline__ void load_idx(const AppendParams& p, int64_t t0, int lane, TileIdx& in) {
  const int r = lane & 15;
#pragma unroll
  for (int j = 0; j < kAppendTiles; ++j) {
    const int64_t tok = t0 + 16 * j + r;
    const bool valid = tok < p.n_tokens;
    in.b[j] = valid ? p.seq_idx[tok] : -1;
    in.ps[j] = valid ? p.pos[tok] : -1;
  }
}

// Block-table entry and length of a token's sequence (-1 when the token is
// skipped); loaded ahead, so only plain integers stay live until the token is
// written.
__device__ __forceinline__ int2 lookup(const AppendParams& p, int b, int ps) {
  if (b < 0 || b >= p.batch || ps < 0 || (ps >> 4) >= p.max_pages) return make_int2(-1, 0);
  return make_int2(p.block_table[(int64_t)b * p.max_pages + (ps >> 4)], p.len_after[b]);
}

// Where a token goes: its block base (nullptr if it must be skipped) and slot;
// also whether it enters the bf16 window and its window slot.
__device__ __forceinline__ TokInfo resolve(const AppendParams& p, int b, int ps, int2 pl, int h) {
  TokInfo ti{nullptr, 0, 0, 0, false, false};
  const int page = pl.x;
  if (page < 0 || page >= p.n_pages) return ti;
  ti.blk = p.pool + ((int64_t)page * p.hkv + h) * p.block;
  ti.slot = ps & 15;
  ti.b = b;
  ti.pos = ps;
  ti.in_win = p.window > 0 && ps >= pl.y - p.window;
  ti.in_sink = ps < p.n_sink;
  return ti;
}

// X operand of tile j of a wave: token t0 + 16 j + r, input channels
// 32 g .. 32 g + 31 (zero past the last token)
template <int KIND>
__device__ __forceinline__ void load_x(const AppendParams& p, int64_t t0, int h, int lane,
                                       uint4 (&xv)[kAppendTiles][4]) {
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int j = 0; j < kAppendTiles; ++j) {
    const int64_t tok = t0 + 16 * j + r;
    const bool valid = tok < p.n_tokens;
    const uint4* xp = reinterpret_cast<const uint4*>(p.x[KIND] + ((valid ? tok : 0) * p.hkv + h) * kD + 32 * g);
#pragma unroll
    for (int s = 0; s < 4; ++s) xv[j][s] = valid ? xp[s] : make_uint4(0, 0, 0, 0);
  }
}

// PRE: the tile's X rows were loaded by the caller (xpre); otherwise they are
// loaded here.
template <int KIND, int NG, bool PRE>
__device__ __forceinline__ void process_tiles(const AppendParams& p, const uint4* r_lds, const TileIdx& in,
                                              const uint4 (&xpre)[kAppendTiles][4], int64_t t0, int h, int lane) {
  constexpr int NT = kAppendTiles;
  constexpr int MPG = 8 / NG;  // accumulators m per group
  const int g = lane >> 4, r = lane & 15;
  uint4 xv[NT][4];
  if constexpr (PRE) {
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int s = 0; s < 4; ++s) xv[j][s] = xpre[j][s];
  } else {
    load_x<KIND>(p, t0, h, lane, xv);
  }

  f32x4 acc[NT][8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j][m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 rv = r_lds[(16 * m + r) * kRowU4 + 4 * g + s];
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[j][m] = KIND == 0 ? mfma(rv, xv[j][s], acc[j][m]) : mfma(xv[j][s], rv, acc[j][m]);
    }
  }

#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int64_t tj = t0 + 16 * j;
    if (tj >= p.n_tokens) break;  // uniform: the wave's tokens are contiguous
    const TokInfo ti = resolve(p, in.b[j], in.ps[j], in.pl[j], h);

    // raw bf16 copies into the ring (same for K and V): recent tokens, sinks
    if (ti.blk && ti.in_win) {
      uint4* wp = reinterpret_cast<uint4*>(p.win[KIND] + (((int64_t)ti.b * p.ring + ti.pos % p.window) * p.hkv + h) * kD + 32 * g);
#pragma unroll
      for (int s = 0; s < 4; ++s) wp[s] = xv[j][s];
    }
    if (ti.blk && ti.in_sink) {
      uint4* wp = reinterpret_cast<uint4*>(p.win[KIND] + (((int64_t)ti.b * p.ring + p.window + ti.pos) * p.hkv + h) * kD + 32 * g);
#pragma unroll
      for (int s = 0; s < 4; ++s) wp[s] = xv[j][s];
    }

    if (KIND == 0) {
      // acc[j][m][i] = x'[token tj + r][channel 16m + 4g + i]: row segment g
      Quant q[NG];
#pragma unroll
      for (int gr = 0; gr < NG; ++gr) {
        float mn = acc[j][gr * MPG][0], mx = acc[j][gr * MPG][0];
#pragma unroll
        for (int m = gr * MPG; m < (gr + 1) * MPG; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            mn = fminf(mn, acc[j][m][i]);
            mx = fmaxf(mx, acc[j][m][i]);
          }
        q[gr] = quant_params(min_rows(mn), max_rows(mx));
      }
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[m >> 2] |= encode(acc[j][m][i], q[m / MPG].inv, q[m / MPG].zi) << (8 * (m & 3) + 2 * i);
      if (ti.blk) {
        *reinterpret_cast<uint2*>(ti.blk + kKCodes + 32 * ti.slot + 8 * g) = make_uint2(w[0], w[1]);
        // lane group g < NG writes group g's K scale and zero
#pragma unroll
        for (int gr = 0; gr < NG; ++gr)
          if (g == gr) *reinterpret_cast<uint32_t*>(ti.blk + kMeta + 8 * (NG * ti.slot + gr)) = q[gr].sz;
      }
    } else {
      // acc[j][m][i] = x'[token tj + 4g + i][channel 16m + r]
      float mn[4][NG], mx[4][NG];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int gr = 0; gr < NG; ++gr) {
          float lo = acc[j][gr * MPG][i], hi = lo;
#pragma unroll
          for (int m = gr * MPG + 1; m < (gr + 1) * MPG; ++m) {
            lo = fminf(lo, acc[j][m][i]);
            hi = fmaxf(hi, acc[j][m][i]);
          }
          mn[i][gr] = row_min16(lo);
          mx[i][gr] = row_max16(hi);
        }
      // lane r of each row takes token 4g + (r & 3), group (r >> 2) mod NG; the
      // others then read them: within the quad (NG = 1) or the row
      const int mi = r & 3, mk = (r >> 2) % NG;
      float mn_l = mn[0][0], mx_l = mx[0][0];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int gr = 0; gr < NG; ++gr) {
          const bool sel = mi == i && mk == gr;
          mn_l = sel ? mn[i][gr] : mn_l;
          mx_l = sel ? mx[i][gr] : mx_l;
        }
      const Quant ql = quant_params(mn_l, mx_l);
      Quant q[4][NG];
      if constexpr (NG == 1) {
        q[0][0] = Quant{quad_bcast<0>(ql.sz), __uint_as_float(quad_bcast<0>(__float_as_uint(ql.inv))),
                        __uint_as_float(quad_bcast<0>(__float_as_uint(ql.zi)))};
        q[1][0] = Quant{quad_bcast<1>(ql.sz), __uint_as_float(quad_bcast<1>(__float_as_uint(ql.inv))),
                        __uint_as_float(quad_bcast<1>(__float_as_uint(ql.zi)))};
        q[2][0] = Quant{quad_bcast<2>(ql.sz), __uint_as_float(quad_bcast<2>(__float_as_uint(ql.inv))),
                        __uint_as_float(quad_bcast<2>(__float_as_uint(ql.zi)))};
        q[3][0] = Quant{quad_bcast<3>(ql.sz), __uint_as_float(quad_bcast<3>(__float_as_uint(ql.inv))),
                        __uint_as_float(quad_bcast<3>(__float_as_uint(ql.zi)))};
      } else {
        const int row0 = lane & 48;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int gr = 0; gr < NG; ++gr) {
            const int src = row0 + 4 * gr + i;
            q[i][gr] = Quant{(uint32_t)__shfl((int)ql.sz, src), __shfl(ql.inv, src), __shfl(ql.zi, src)};
          }
      }
      const bool rec_lane = r < 4 * NG;  // lane r stores the record of token 4g + mi, group mk
      // fast path: the tile's 16 tokens are slots 0..15 of one page, in order
      const int b0 = __builtin_amdgcn_readfirstlane(ti.b), pos0 = __builtin_amdgcn_readfirstlane(ti.pos);
      const uintptr_t bp = reinterpret_cast<uintptr_t>(ti.blk);
      uint8_t* blk0 = reinterpret_cast<uint8_t*>(
          ((uintptr_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(bp >> 32)) << 32) |
          (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bp));
      const bool mine = ti.blk != nullptr && ti.b == b0 && ti.pos == pos0 + r && (pos0 & 15) == 0;
      if (__all(mine)) {
        uint32_t w[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          uint32_t d = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) d |= encode(acc[j][m][i], q[i][m / MPG].inv, q[i][m / MPG].zi) << (2 * (4 * g + i));
          w[m] = or_rows(d);
        }
        uint32_t* vw = reinterpret_cast<uint32_t*>(blk0 + kVCodes);
#pragma unroll
        for (int m = 0; m < 8; ++m)
          if ((m >> 1) == g) vw[16 * m + r] = w[m];
        // token 4g + i is slot 4g + i
        if (rec_lane) *reinterpret_cast<uint32_t*>(blk0 + kMeta + 8 * (NG * (4 * g + mi) + mk) + 4) = ql.sz;
      } else {
        // per-token info of the 4 tokens this lane holds codes for
        uint8_t* tblk[4];
        int tslot[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          tblk[i] = reinterpret_cast<uint8_t*>(__shfl(bp, 4 * g + i));
          tslot[i] = __shfl(ti.slot, 4 * g + i);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (!tblk[i]) continue;
          uint32_t* vw = reinterpret_cast<uint32_t*>(tblk[i] + kVCodes);
          const uint32_t clr = ~(3u << (2 * tslot[i]));
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            atomicAnd(&vw[16 * m + r], clr);
            atomicOr(&vw[16 * m + r], encode(acc[j][m][i], q[i][m / MPG].inv, q[i][m / MPG].zi) << (2 * tslot[i]));
          }
          if (rec_lane && mi == i) *reinterpret_cast<uint32_t*>(tblk[i] + kMeta + 8 * (NG * tslot[i] + mk) + 4) = ql.sz;
        }
      }
    }
  }
}

// ONE: every workgroup has a single iteration (tiles_per_wg == 1, as for
// decode-time appends); its X rows then also go out before R is staged.
template <int NG, bool ONE>
__global__ __launch_bounds__(256, 4) void append_kernel(AppendParams p) {
  __shared__ uint4 r_lds[128 * kRowU4];
  const int h = blockIdx.y;
  const int kind = blockIdx.z & 1, layer = blockIdx.z >> 1;
  if (layer > 0) {  // static indices only: the parameters stay in scalar registers
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      p.r[k] += layer * p.ls_rot;
      p.x[k] += layer * p.ls_x;
      if (p.win[k]) p.win[k] += layer * p.ls_win;
    }
    p.pool += layer * p.ls_pool;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  auto tile0 = [&](int it) {
    return ((int64_t)blockIdx.x * p.tiles_per_wg + it) * kAppendTokens + wave * 16 * kAppendTiles;
  };
  // the first tile's token indices (and with ONE its rows) go out before the
  // rotation is staged
  TileIdx in;
  uint4 xv[kAppendTiles][4];
  const bool any = tile0(0) < p.n_tokens;  // uniform across the wave
  if (any) {
    load_idx(p, tile0(0), lane, in);
    if constexpr (ONE) {
      if (kind == 0)
        load_x<0>(p, tile0(0), h, lane, xv);
      else
        load_x<1>(p, tile0(0), h, lane, xv);
    }
  }
  const uint4* rg = reinterpret_cast<const uint4*>((kind ? p.r[1] : p.r[0]) + (int64_t)h * kD * kD);
  uint4 rr[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) rr[k] = rg[threadIdx.x + 256 * k];
  if (any) {
#pragma unroll
    for (int j = 0; j < kAppendTiles; ++j) in.pl[j] = lookup(p, in.b[j], in.ps[j]);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int i = threadIdx.x + 256 * k;
    r_lds[(i >> 4) * kRowU4 + (i & 15)] = rr[k];
  }
  __syncthreads();
  if constexpr (ONE) {
    if (any) {
      if (kind == 0)
        process_tiles<0, NG, true>(p, r_lds, in, xv, tile0(0), h, lane);
      else
        process_tiles<1, NG, true>(p, r_lds, in, xv, tile0(0), h, lane);
    }
    return;
  }
  TileIdx nxt;  // raw indices of the next tile, loaded while this one is processed
  for (int it = 0; it < p.tiles_per_wg; ++it) {
    const int64_t t0 = tile0(it);
    if (t0 >= p.n_tokens) break;
    if (it > 0) {
#pragma unroll
      for (int j = 0; j < kAppendTiles; ++j) {
        in.b[j] = nxt.b[j];
        in.ps[j] = nxt.ps[j];
        in.pl[j] = lookup(p, in.b[j], in.ps[j]);
      }
    }
    if (it + 1 < p.tiles_per_wg && tile0(it + 1) < p.n_tokens) load_idx(p, tile0(it + 1), lane, nxt);
    if (kind == 0)
      process_tiles<0, NG, false>(p, r_lds, in, xv, t0, h, lane);
    else
      process_tiles<1, NG, false>(p, r_lds, in, xv, t0, h, lane);
  }
}

}  // namespace
}  // namespace oscar

extern "C" int oscar_quantize_append_layers(const oscar_shape* shape, int32_t n_layers, const uint16_t* r_k,
                                            const uint16_t* r_v, const uint16_t* k_new, const uint16_t* v_new,
                                            int64_t n_tokens, const int32_t* seq_idx, const int32_t* pos,
                                            int32_t batch, const int32_t* block_table, int32_t max_pages_per_seq,
                                            const int32_t* seq_len_after, uint8_t* pool, int64_t n_pages,
                                            uint16_t* win_k, uint16_t* win_v, void* stream) {
  using namespace oscar;
  int st = check_shape(shape);
  if (st != OSCAR_OK) return st;
  if (n_tokens < 0 || batch < 1 || max_pages_per_seq < 1 || n_pages < 1) return OSCAR_EINVAL;
  if (n_layers < 1 || n_layers > 32767) return OSCAR_EINVAL;
  if (n_tokens == 0) return OSCAR_OK;
  if (!r_k || !r_v || !k_new || !v_new || !seq_idx || !pos || !block_table || !seq_len_after || !pool)
    return OSCAR_EINVAL;
  if (shape->window + shape->n_sink > 0 && (!win_k || !win_v)) return OSCAR_EINVAL;
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
  p.block = block_bytes(shape->group_size);
  p.n_tokens = n_tokens;
  p.n_pages = n_pages;
  p.batch = batch;
  p.max_pages = max_pages_per_seq;
  p.hkv = shape->n_kv_heads;
  p.window = shape->window;
  p.n_sink = shape->n_sink;
  p.ring = shape->window + shape->n_sink;
  p.ls_rot = (int64_t)p.hkv * kD * kD;
  p.ls_x = n_tokens * p.hkv * kD;
  p.ls_win = (int64_t)batch * p.ring * p.hkv * kD;
  p.ls_pool = n_pages * p.hkv * p.block;
  const int64_t tiles = (n_tokens + kAppendTokens - 1) / kAppendTokens;  // workgroup iterations
  p.tiles_per_wg = tiles >= 512 ? 4 : (tiles >= 128 ? 2 : 1);
  dim3 grid((unsigned)((tiles + p.tiles_per_wg - 1) / p.tiles_per_wg), (unsigned)p.hkv, 2 * (unsigned)n_layers);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const TimedLaunch tl = timing_events(3);
  const bool one = p.tiles_per_wg == 1;
  auto go = [&](auto kernel) { hipExtLaunchKernelGGL(kernel, grid, dim3(256), 0, s, tl.start, tl.stop, 0, p); };
  switch (kD / shape->group_size) {
    case 1: one ? go(append_kernel<1, true>) : go(append_kernel<1, false>); break;
    case 2: one ? go(append_kernel<2, true>) : go(append_kernel<2, false>); break;
    default: one ? go(append_kernel<4, true>) : go(append_kernel<4, false>); break;
  }
  return hipGetLastError() == hipSuccess ? OSCAR_OK : OSCAR_EHIP;
}

extern "C" int oscar_quantize_append(const oscar_shape* shape, const uint16_t* r_k, const uint16_t* r_v,
                                     const uint16_t* k_new, const uint16_t* v_new, int64_t n_tokens,
                                     const int32_t* seq_idx, const int32_t* pos, int32_t batch,
                                     const int32_t* block_table, int32_t max_pages_per_seq,
                                     const int32_t* seq_len_after, uint8_t* pool, int64_t n_pages,
                                     uint16_t* win_k, uint16_t* win_v, void* stream) {
  return oscar_quantize_append_layers(shape, 1, r_k, r_v, k_new, v_new, n_tokens, seq_idx, pos, batch, block_table,
                                      max_pages_per_seq, seq_len_after, pool, n_pages, win_k, win_v, stream);
}
