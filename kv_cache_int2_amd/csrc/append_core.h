#pragma once
// Device code of the append path, shared by the append kernel and the fused
// decode step (whose query-preparation kernel also appends each sequence's
// newest token).
// Online rotate -> quantise -> pack of new K/V tokens into the paged INT2 cache.
// Method: P1 (gen-hub.ru, "Together AI открывает OSCAR…") «Что придумали в
// Together AI» (per-head rotation R = P_br H U^T of keys and values) and «Почему
// INT2 раньше не работал» (four levels); P2 (encorp.ai) «OSCAR има значение…»
// (recent tokens kept in bf16, history in INT2, paged storage).
//
// One workgroup = 8 waves = 128 tokens per iteration of one (KV head, K|V).
// R (128 x 128 bf16) is staged once per workgroup in LDS.  Each wave rotates its
// 16-token tile(s) with v_mfma_f32_16x16x32_bf16; every R tile read from LDS
// feeds every token tile of the wave.  One tile per wave by default: at <= 128
// VGPRs four waves share each SIMD, which measured faster than two tiles per
// wave (fewer LDS reads of R) at two waves per SIMD.  A wave's next tile is
// loaded straight into its 4 KB of LDS while the current one is quantised, so
// the prefetch costs no VGPRs; R and the 8 tile buffers take 64 KB, two
// workgroups per CU.
//  - keys use A = R, B = X^T: a lane ends with channels 16m + 4g + i (m = 0..7,
//    i = 0..3) of ONE token, exactly the 8-byte segment g of the token's K row,
//    so it writes that segment itself;
//  - values use A = X, B = R^T: a lane ends with 4 tokens x 8 channels, that is
//    byte g (slots 4g .. 4g + 3) of 8 channel-major V words (16 slots x 2 bits),
//    and stores those bytes itself when the tile is a whole aligned page; a
//    partial page falls back to per-token atomic and/or on the channel words.
// The k-slot -> input channel map (lane group g, step s, slot j -> 32s + 8g + j)
// is the same for both operands, so the hardware's internal k order is moot;
// it makes the four lanes of a token read (and copy to the ring) one whole
// 64-byte line per step.
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
  int max_len;  // the fused decode step's max_seq_len (implicit token indices only)
  int ring;    // ring rows per sequence: window + n_sink
  // layers appended in one launch: rotations, tokens, rings and pools stacked
  // layer-major with these strides (elements; pool in bytes); positions, block
  // table and lengths shared by all layers
  int64_t ls_rot, ls_x, ls_win, ls_pool;
};

// f(integral_constant<int, k>) for k = 0 .. N-1, unrolled at compile time
template <int N, int K = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (K < N) {
    f(std::integral_constant<int, K>{});
    static_for<N, K + 1>(f);
  }
}

// R in LDS: row o (output channel) holds its 16 chunks of 8 bf16 (k) at chunk
// c ^ (o & 15), so the 16 rows a step reads at one chunk fall in 16 different
// bank groups; unpadded, R takes exactly 32 KiB and five workgroups fit a CU.
__device__ __forceinline__ int r_slot(int o, int c) { return o * 16 + (c ^ (o & 15)); }
#ifndef OSCAR_APPEND_TILES
#define OSCAR_APPEND_TILES 1
#endif
constexpr int kAppendTiles = OSCAR_APPEND_TILES;  // 16-token tiles per wave and iteration
constexpr int kAppendWaves = 8;                        // waves per workgroup
constexpr int kAppendThreads = 64 * kAppendWaves;
constexpr int kAppendTokens = kAppendWaves * 16 * kAppendTiles;  // tokens per workgroup and iteration

__device__ __forceinline__ f32x4 mfma(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Code of x' as a float's bits: u = kRound + clamp(rint(x' * inv - zi), 0, 3).
// Adding 1.5 * 2^23 rounds t (|t| < 2^22) to an integer, ties to even, in the
// low mantissa bits, so the bits of u are kRoundBits + code.  A packed word is
// then the sum of such bits shifted into place, less the shifted kRoundBits
// (a constant; all of it lies at bit 22 and up, before the shift).  A NaN
// t clamps to the low bound (v_med3 returns the smallest operand), code 0.
constexpr float kRound = 12582912.0f;
constexpr uint32_t kRoundBits = 0x4B400000u;
__device__ __forceinline__ uint32_t code_bits(float v, float inv, float zi) {
  const float u = fmaf(v, inv, -zi) + kRound;
  return __float_as_uint(__builtin_amdgcn_fmed3f(u, kRound, kRound + 3.0f));
}
// (x << S) + c as one v_lshl_add_u32: left to itself the compiler splits a chain
// of these into shifts and three-operand adds, one instruction more per pair.
template <int S>
__device__ __forceinline__ uint32_t lshl_add(uint32_t x, uint32_t c) {
  uint32_t d;
  asm("v_lshl_add_u32 %0, %1, %2, %3" : "=v"(d) : "v"(x), "n"(S), "v"(c));
  return d;
}
// sum of kRoundBits << s over the shifts 8 m + 2 i (m, i = 0..3) of a K word
constexpr uint32_t k_word_bias() {
  uint32_t c = 0;
  for (int m = 0; m < 4; ++m)
    for (int i = 0; i < 4; ++i) c += kRoundBits << (8 * m + 2 * i);
  return c;
}

// Order-preserving map of fp32 bits to int32 (its own inverse): integer
// min/max take a DPP operand for free, where fminf/fmaxf would first quiet
// both operands.  -0 orders just below +0.
__device__ __forceinline__ int f2key(float x) {
  const int b = __float_as_int(x);
  return b ^ ((b >> 31) & 0x7fffffff);
}
__device__ __forceinline__ float key2f(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7fffffff)); }
constexpr int kDppRor4 = 0x124, kDppRor8 = 0x128;  // row_ror by 4, 8 lanes

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

// Stores and atomics into the pool through global-memory pointers: they then
// compile to global rather than flat instructions (a flat one also counts
// against the LDS counter and may alias LDS, so the compiler waits for every
// load into LDS before it).  The pool pointer alone is not known to be global.
template <typename T>
__device__ __forceinline__ void st_global(uint8_t* a, T v) {
  *(__attribute__((address_space(1))) T*)a = v;
}
__device__ __forceinline__ void and_or_global(uint8_t* a, uint32_t clr, uint32_t set) {
  auto* w = (__attribute__((address_space(1))) uint32_t*)a;
  __hip_atomic_fetch_and(w, clr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_fetch_or(w, set, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// IMPLICIT (the fused decode step): token t is the newest token of sequence
// t, at position len_after[t] - 1; a sequence whose length is not in
// [1, max_len] gets none.  seq_idx and pos are not read.
template <bool IMPLICIT = false>
__device__ __forceinline__ void load_idx(const AppendParams& p, int64_t t0, int lane, TileIdx& in) {
  const int r = lane & 15;
#pragma unroll
  for (int j = 0; j < kAppendTiles; ++j) {
    const int64_t tok = t0 + 16 * j + r;
    const bool valid = tok < p.n_tokens;
    const int64_t tc = valid ? tok : p.n_tokens - 1;  // every lane loads: no branch
    int b, ps;
    if constexpr (IMPLICIT) {
      const int n = p.len_after[tc];
      b = (int)tc;
      ps = n >= 1 && n <= p.max_len ? n - 1 : -1;
    } else {
      b = p.seq_idx[tc];
      ps = p.pos[tc];
    }
    in.b[j] = valid ? b : -1;
    in.ps[j] = valid ? ps : -1;
  }
}

// Block-table entry and length of a token's sequence (-1 when the token is
// skipped); loaded ahead, so only plain integers stay live until the token is
// written.
__device__ __forceinline__ int2 lookup(const AppendParams& p, int b, int ps) {
  const bool ok = b >= 0 && b < p.batch && ps >= 0 && (ps >> 4) < p.max_pages;
  const int bc = ok ? b : 0, pc = ok ? ps >> 4 : 0;  // every lane loads: no branch
  const int page = p.block_table[(int64_t)bc * p.max_pages + pc], len = p.len_after[bc];
  return ok ? make_int2(page, len) : make_int2(-1, 0);
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
// 32 s + 8 g .. 32 s + 8 g + 7 at step s (zero past the last token)
template <int KIND>
__device__ __forceinline__ void load_x(const AppendParams& p, int64_t t0, int h, int lane,
                                       uint4 (&xv)[kAppendTiles][4]) {
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int j = 0; j < kAppendTiles; ++j) {
    // wave-uniform row base and a 32-bit lane offset (a token row is hkv * 256 B)
    const int64_t tj = t0 + 16 * j;
    const uint8_t* xb = reinterpret_cast<const uint8_t*>(p.x[KIND]) + (tj * p.hkv + h) * (2 * kD);
    const bool valid = tj + r < p.n_tokens;
    const uint32_t off = valid ? (uint32_t)r * (uint32_t)(p.hkv * 2 * kD) + 16u * g : 0u;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      xv[j][s] = valid ? *reinterpret_cast<const uint4*>(xb + off + 64 * s) : make_uint4(0, 0, 0, 0);
  }
}

// The same X operand staged in the wave's LDS buffer by direct global -> LDS
// loads: 16 bytes a lane, lane l's at buf[(4 j + s) 64 + l], so no VGPR holds
// the rows while they are in flight.  t0 must be a token of the launch.  A row
// past the last token reads the last token's row instead, so the loads take
// no branch: a count of loads in flight that does not depend on the data lets
// the compiler wait for exactly the older ones.
template <int KIND>
__device__ __forceinline__ void dma_x(const AppendParams& p, int64_t t0, int h, int lane, uint4* buf) {
  const int g = lane >> 4, r = lane & 15;
  const int64_t last = p.n_tokens - 1;
  const uint8_t* x = reinterpret_cast<const uint8_t*>(p.x[KIND]);
  const int64_t row = (int64_t)p.hkv * 2 * kD;
#pragma unroll
  for (int j = 0; j < kAppendTiles; ++j) {
    const int64_t tj = t0 + 16 * j < last ? t0 + 16 * j : last;  // uniform
    const uint8_t* xb = x + tj * row + h * (2 * kD);
    const int64_t nr = last - tj;  // rows left after tj
    const uint32_t off = (uint32_t)(r < nr ? r : nr) * (uint32_t)row + 16u * g;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(xb + off + 64 * s), buf + (4 * j + s) * 64, 16,
                                       0, 0);
  }
}
// A row past the last token holds a copy of the last token's row (dma_x): its
// results are never stored, and every reduction stays within one token, so
// it need not be zeroed.
__device__ __forceinline__ void read_x(int lane, const uint4* buf, uint4 (&xv)[kAppendTiles][4]) {
#pragma unroll
  for (int j = 0; j < kAppendTiles; ++j)
#pragma unroll
    for (int s = 0; s < 4; ++s) xv[j][s] = buf[(4 * j + s) * 64 + lane];
}

// Rotates, quantises and stores the tile(s) whose X operand is xv; after the
// rotation (the last read of R and of xv's LDS copy) calls after_mfma(), which
// may start the next tile's loads.
template <int KIND, int NG, typename AfterMfma>
__device__ __forceinline__ void process_tiles(const AppendParams& p, const uint4* r_lds, const TileIdx& in,
                                              const uint4 (&xv)[kAppendTiles][4], int64_t t0, int h, int lane,
                                              AfterMfma&& after_mfma) {
  constexpr int NT = kAppendTiles;
  constexpr int MPG = 8 / NG;  // accumulators m per group
  const int g = lane >> 4, r = lane & 15;

  f32x4 acc[NT][8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j][m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 rv = r_lds[r_slot(16 * m + r, 4 * s + g)];
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[j][m] = KIND == 0 ? mfma(rv, xv[j][s], acc[j][m]) : mfma(xv[j][s], rv, acc[j][m]);
    }
  }
  // the tiles' destinations are waited for before after_mfma's loads are
  // issued: a wait for an older load behind those loads would wait for them too
#pragma unroll
  for (int j = 0; j < NT; ++j) asm volatile("" ::"v"(in.pl[j].x), "v"(in.pl[j].y));
  after_mfma();

#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int64_t tj = t0 + 16 * j;
    if (tj >= p.n_tokens) break;  // uniform: the wave's tokens are contiguous
    const TokInfo ti = resolve(p, in.b[j], in.ps[j], in.pl[j], h);

    // raw bf16 copies into the ring (same for K and V): recent tokens, sinks
    if (ti.blk && ti.in_win) {
      uint4* wp = reinterpret_cast<uint4*>(p.win[KIND] + (((int64_t)ti.b * p.ring + ti.pos % p.window) * p.hkv + h) * kD);
#pragma unroll
      for (int s = 0; s < 4; ++s) wp[4 * s + g] = xv[j][s];
    }
    if (ti.blk && ti.in_sink) {
      uint4* wp = reinterpret_cast<uint4*>(p.win[KIND] + (((int64_t)ti.b * p.ring + p.window + ti.pos) * p.hkv + h) * kD);
#pragma unroll
      for (int s = 0; s < 4; ++s) wp[4 * s + g] = xv[j][s];
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
      constexpr uint32_t kBias = k_word_bias();
      uint32_t w[2] = {0u - kBias, 0u - kBias};
      static_for<32>([&](auto mi_) {
        constexpr int m = decltype(mi_)::value >> 2, i = decltype(mi_)::value & 3;
        w[m >> 2] = lshl_add<8 * (m & 3) + 2 * i>(code_bits(acc[j][m][i], q[m / MPG].inv, q[m / MPG].zi), w[m >> 2]);
      });
      if (ti.blk) {
        st_global(ti.blk + kKCodes + 32 * ti.slot + 8 * g, (uint64_t)w[1] << 32 | w[0]);
        // lane group g < NG writes group g's K scale and zero
#pragma unroll
        for (int gr = 0; gr < NG; ++gr)
          if (g == gr) st_global(ti.blk + kMeta + 8 * (NG * ti.slot + gr), q[gr].sz);
      }
    } else {
      // acc[j][m][i] = x'[token tj + 4g + i][channel 16m + r].  Per-token min
      // and max: over m in the lane, then over the row's 16 lanes.  Lanes r and
      // r^1 combine, and each keeps the tokens with i & 1 == r & 1; then lanes
      // r and r^2, keeping token i == r & 3; rotating the row by 4 and 8 lanes
      // finishes it.  Every lane ends with the min and max of each group of
      // token 4g + (r & 3).
      int kmn[4][NG], kmx[4][NG];
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
          kmn[i][gr] = f2key(lo);
          kmx[i][gr] = f2key(hi);
        }
      const bool odd1 = r & 1, odd2 = r & 2;
      int pmn[2][NG], pmx[2][NG];  // tokens 2 h + (r & 1)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int gr = 0; gr < NG; ++gr) {
          const int e0 = min(kmn[2 * h][gr], dpp_i32<kDppSwap1>(kmn[2 * h][gr]));
          const int e1 = min(kmn[2 * h + 1][gr], dpp_i32<kDppSwap1>(kmn[2 * h + 1][gr]));
          pmn[h][gr] = odd1 ? e1 : e0;
          const int f0 = max(kmx[2 * h][gr], dpp_i32<kDppSwap1>(kmx[2 * h][gr]));
          const int f1 = max(kmx[2 * h + 1][gr], dpp_i32<kDppSwap1>(kmx[2 * h + 1][gr]));
          pmx[h][gr] = odd1 ? f1 : f0;
        }
      Quant qo[NG];  // this lane's token 4g + (r & 3)
#pragma unroll
      for (int gr = 0; gr < NG; ++gr) {
        const int e0 = min(pmn[0][gr], dpp_i32<kDppSwap2>(pmn[0][gr]));
        const int e1 = min(pmn[1][gr], dpp_i32<kDppSwap2>(pmn[1][gr]));
        int lo = odd2 ? e1 : e0;
        const int f0 = max(pmx[0][gr], dpp_i32<kDppSwap2>(pmx[0][gr]));
        const int f1 = max(pmx[1][gr], dpp_i32<kDppSwap2>(pmx[1][gr]));
        int hi = odd2 ? f1 : f0;
        lo = min(lo, dpp_i32<kDppRor4>(lo));
        hi = max(hi, dpp_i32<kDppRor4>(hi));
        lo = min(lo, dpp_i32<kDppRor8>(lo));
        hi = max(hi, dpp_i32<kDppRor8>(hi));
        qo[gr] = quant_params(key2f(lo), key2f(hi));
      }
      // token 4g + i's inverse scale and scaled zero from lane i of the quad
      float inv[4][NG], zi[4][NG];
#pragma unroll
      for (int gr = 0; gr < NG; ++gr) {
        const uint32_t iv = __float_as_uint(qo[gr].inv), zv = __float_as_uint(qo[gr].zi);
        inv[0][gr] = __uint_as_float(quad_bcast<0>(iv));
        inv[1][gr] = __uint_as_float(quad_bcast<1>(iv));
        inv[2][gr] = __uint_as_float(quad_bcast<2>(iv));
        inv[3][gr] = __uint_as_float(quad_bcast<3>(iv));
        zi[0][gr] = __uint_as_float(quad_bcast<0>(zv));
        zi[1][gr] = __uint_as_float(quad_bcast<1>(zv));
        zi[2][gr] = __uint_as_float(quad_bcast<2>(zv));
        zi[3][gr] = __uint_as_float(quad_bcast<3>(zv));
      }
      const int mi = r & 3, mk = (r >> 2) % NG;
      uint32_t rec_sz = qo[0].sz;
#pragma unroll
      for (int gr = 1; gr < NG; ++gr) rec_sz = mk == gr ? qo[gr].sz : rec_sz;
      const bool rec_lane = r < 4 * NG;  // lane r stores the record of token 4g + mi, group mk
      // fast path: the tile's 16 tokens are slots 0..15 of one page, in order
      const int b0 = __builtin_amdgcn_readfirstlane(ti.b), pos0 = __builtin_amdgcn_readfirstlane(ti.pos);
      const uintptr_t bp = reinterpret_cast<uintptr_t>(ti.blk);
      uint8_t* blk0 = reinterpret_cast<uint8_t*>(
          ((uintptr_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(bp >> 32)) << 32) |
          (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bp));
      const bool mine = ti.blk != nullptr && ti.b == b0 && ti.pos == pos0 + r && (pos0 & 15) == 0;
      if (__all(mine)) {
        // byte g of channel word 16 m + r holds tokens 4g .. 4g + 3: the low
        // byte of the shifted code bits (kRoundBits lies above it)
        uint8_t* vb = blk0 + kVCodes + 4 * r + g;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          uint32_t d = code_bits(acc[j][m][0], inv[0][m / MPG], zi[0][m / MPG]);
          d = lshl_add<2>(code_bits(acc[j][m][1], inv[1][m / MPG], zi[1][m / MPG]), d);
          d = lshl_add<4>(code_bits(acc[j][m][2], inv[2][m / MPG], zi[2][m / MPG]), d);
          d = lshl_add<6>(code_bits(acc[j][m][3], inv[3][m / MPG], zi[3][m / MPG]), d);
          st_global(vb + 64 * m, (uint8_t)d);
        }
        // token 4g + i is slot 4g + i
        if (rec_lane) st_global(blk0 + kMeta + 8 * (NG * (4 * g + mi) + mk) + 4, rec_sz);
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
          uint8_t* vw = tblk[i] + kVCodes + 4 * r;  // channel word 16 m + r at vw + 64 m
          const uint32_t clr = ~(3u << (2 * tslot[i]));
#pragma unroll
          for (int m = 0; m < 8; ++m)
            and_or_global(vw + 64 * m, clr,
                          (code_bits(acc[j][m][i], inv[i][m / MPG], zi[i][m / MPG]) & 3u) << (2 * tslot[i]));
          if (rec_lane && mi == i) st_global(tblk[i] + kMeta + 8 * (NG * tslot[i] + mk) + 4, rec_sz);
        }
      }
    }
  }
}

// R of (head h, kind KIND) staged in LDS by THREADS threads: loaded into
// registers first (r_load), written swizzled after other loads have been
// issued (r_store); the caller passes the barrier.
template <int THREADS>
struct RStage {
  uint4 v[128 * 16 / THREADS];
};
template <int THREADS>
__device__ __forceinline__ void r_load(const uint16_t* r, int h, RStage<THREADS>& rs) {
  const uint4* rg = reinterpret_cast<const uint4*>(r + (int64_t)h * kD * kD);
#pragma unroll
  for (int k = 0; k < 128 * 16 / THREADS; ++k) rs.v[k] = rg[threadIdx.x + THREADS * k];
}
template <int THREADS>
__device__ __forceinline__ void r_store(uint4* r_lds, const RStage<THREADS>& rs) {
#pragma unroll
  for (int k = 0; k < 128 * 16 / THREADS; ++k) {
    const int i = threadIdx.x + THREADS * k;
    r_lds[r_slot(i >> 4, i & 15)] = rs.v[k];
  }
}

// A workgroup of THREADS / 64 waves with one 16-token tile per wave (the
// wave's first token t0): the tile's indices and rows go out before R is
// staged, so their latency overlaps its load.  Every thread of the workgroup
// calls it (it passes a barrier); r_lds is 32 KiB of LDS.
template <int KIND, int NG, int THREADS, bool IMPLICIT>
__device__ __forceinline__ void append_one(const AppendParams& p, uint4* r_lds, int h, int64_t t0, int lane) {
  TileIdx in;
  uint4 xv[kAppendTiles][4];
  const bool any = t0 < p.n_tokens;  // uniform across the wave
  if (any) {
    load_idx<IMPLICIT>(p, t0, lane, in);
    load_x<KIND>(p, t0, h, lane, xv);
  }
  RStage<THREADS> rs;
  r_load<THREADS>(p.r[KIND], h, rs);
  if (any) {
#pragma unroll
    for (int j = 0; j < kAppendTiles; ++j) in.pl[j] = lookup(p, in.b[j], in.ps[j]);
  }
  r_store<THREADS>(r_lds, rs);
  __syncthreads();
  if (any) process_tiles<KIND, NG>(p, r_lds, in, xv, t0, h, lane, [] {});
}

}  // namespace
}  // namespace oscar
