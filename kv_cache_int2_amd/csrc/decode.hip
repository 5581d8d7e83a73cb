// Decode attention over the mixed-precision paged cache: rotate q by the key
// transform, attend the INT2 history in the rotated domain (split over the
// context), merge the splits, un-rotate by the value transform and fold in the
// bf16 recent window.  Method: P1 (gen-hub.ru, "Together AI открывает OSCAR…")
// «Что придумали в Together AI»; P2 (encorp.ai) «OSCAR има значение…» and P4
// (aiforradalom.hu) «OSCAR: figyelem-tudatos…» (bf16 recent tokens, INT2
// history, paged attention).
//
// Kernels (one call = three launches on the caller's stream; L layers of a
// layer-batched call share them):
//   prep          grid (L B, Hkv, 1 + chunks): z = 0: q' = R_K q for the G heads
//                                         of a KV head, its group sums, the fp8
//                                         score operands and the tile prefix;
//                                         z > 0: one 32-token chunk of the bf16
//                                         window or sinks, partial per q head
//   int2_split    grid (2 per CU), persistent: equal shares of the flattened
//                                         history tiles of every (layer, sequence,
//                                         KV head group); partial (m, l, acc'[128])
//                                         per wave, q head and unit touched
//   merge         grid (Hq / mh, L B):    log-sum-exp merge of the partials,
//                                         R_V^T acc', window / sink chunks, normalise
// Scores are kept in the log2 domain: logit * log2(e) / sqrt(d).
//
// INT2 split kernel.  Both contractions of a 128-token tile (8 pages) run on the
// matrix cores as v_mfma_scale_f32_16x16x128_f8f6f4 with the packed 2-bit codes
// as the fp4 (e2m1) operand: a code c zero-extended to a nibble is exactly the
// e2m1 value c/2, so (w & 0x33333333) and ((w >> 2) & 0x33333333) turn 16 packed
// codes into two ready operand dwords.  The other operand is carried as fp8
// (e4m3) fixed-point digits: v 2^(3 - E) = d0 + d1/16 + d2/256 + d3/4096, one
// digit per MFMA row, the powers of two in the E8M0 operand scales; every
// product is a small multiple of one power of two, so the matrix cores sum them
// exactly.  q' (scores) takes signed digits |d_j| <= 8 (see digits_pair), E its
// head's exponent; the softmax weights (values), never negative, take the hex
// digits of one rounding to the 1/4096 grid as raw e4m3 bytes (see
// weight_fixed), E the exponent of the largest weight of the head in the tile.
// Rows are (head, digit): 4 heads per MFMA.
//   scores: A = q' digits [(head, digit) x 128 channels], B = K codes [128 x 16 tokens]
//   values: A = w digits  [(head, digit) x 128 tokens],  B = V codes [128 x 16 channels]
// The score output leaves one (head, token) per lane after an in-lane sum of
// the four digit rows, so the softmax runs on full lanes.  The w digits go to a
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
#include "append_core.h"

namespace oscar {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) loads of cache bytes: every byte of the paged pools
// is read once per decode, so the loads carry the non-temporal hint (measured on
// this part: scattered 1152- to 9216-byte blocks stream at ~6.3 TB/s with it
// against ~5.85 TB/s without).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 load_nt2(const void* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ uint4 load_nt4(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// The same loads through a buffer resource on a block whose base is uniform
// (a scalar register quad): the lane's 32-bit offset is the whole per-lane
// address, so no 64-bit vector address arithmetic is spent per load.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint8_t* blk) {
  // raw buffer, no stride, no range limit in practice; dword 3 as this
  // generation's raw buffer loads take it
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blk), 0, 0x7fffffff, 0x00020000);
}
constexpr int kBufNT = 2;  // cache policy: non-temporal
__device__ __forceinline__ uint2 buffer_nt2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kBufNT);
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ uint4 buffer_nt4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kBufNT);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

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

// Fixed-point digits of the fp8 (e4m3) operands of both INT2 contractions.  The
// scaled fp8 x fp4 MFMA sums a row's products exactly only while they span a
// narrow range: with products spread over the e4m3 range the measured sum is cut
// to ~2^-10 .. 2^-12 of the largest product, always downward.  So every fp8
// operand is a small integer: a value v with |v| < 2^E is written through
// x = v 2^(3 - E), |x| < 8, as x = d0 + d1/16 + d2/256 + d3/4096 with each d_j
// the RNE of the remaining residual (|d_j| <= 8, exact in e4m3); digit j sits in
// the MFMA row of term j, whose E8M0 scale is 2^(E - 3 - 4 j).  Every product is
// then an integer of magnitude <= 24 and every dot product exact; v is carried
// to 2^-13 of 2^E.
constexpr int kDigits = 4;

// Digits of a pair of values (|a|, |b| < 8): digit j of a in byte 0 and of b in
// byte 1 of out[j]; ra, rb the residuals left after the last digit (in units of
// 16^-(kDigits - 1)), so a = sum_j d_j 16^-j + ra 16^-(kDigits - 1).
__device__ __forceinline__ void digits_pair(float a, float b, uint32_t out[kDigits], float& ra, float& rb) {
#pragma unroll
  for (int j = 0; j < kDigits; ++j) {
    const float da = __builtin_rintf(a), db = __builtin_rintf(b);
    out[j] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(da, db, 0, false) & 0xffffu;
    a -= da;
    b -= db;
    if (j < kDigits - 1) {
      a *= 16.f;
      b *= 16.f;
    }
  }
  ra = a;
  rb = b;
}

// The split kernel's weights are never negative, so their digits need no sign:
// x = w 2^(3 - e) in [0, 8) is carried as X = rint(4096 x) < 2^16, whose four
// hexadecimal digits (X = 4096 d0 + 256 d1 + 16 d2 + d3, d0 <= 8, others
// <= 15) are the same 1/4096 grid the signed digits above reach.  An e4m3 byte
// n <= 16 is exactly n 2^-9 (the subnormals and the first binade are evenly
// spaced), so each digit, taken out of X as an integer, already is its fp8
// operand byte; the row's E8M0 scale carries the 2^9.  Adding 1.5 2^23 to
// 4096 x (one FMA; the product is exact, a power of two) rounds it to an
// integer, ties to even, in the low mantissa bits: the bits are kRoundBits + X.
// Every product with a code is then a multiple of 2^-10 of at most 22.5 2^-9,
// within the range the MFMA sums exactly.  (kRound = 1.5 2^23 and its bits
// kRoundBits come with the append's device code, which rounds the same way.)
constexpr int kDigitByteExp = 9;          // e4m3 byte n (n <= 16) reads as n 2^-9
constexpr int kMinWeightExp = -100;       // floor of a tile's weight exponent

// kRoundBits + rint(w fix): fix = 2^(15 - e) with every weight below 2^e
__device__ __forceinline__ uint32_t weight_fixed(float w, float fix) { return __float_as_uint(fmaf(w, fix, kRound)); }
// digit j (0 = most significant) of X from weight_fixed's bits, in the low
// byte (the fp8 operand byte; only that byte is stored): one bit-field
// extract (written out: the compiler would split it into a shift and an AND),
// and for digit 0 a plain shift (bits 16..21 of u are zero)
template <int J>
__device__ __forceinline__ uint32_t weight_digit(uint32_t u) {
  if constexpr (J == 0) {
    return u >> 12;
  } else if constexpr (J == 3) {
    return u & 15u;
  } else {
    uint32_t d;
    asm("v_bfe_u32 %0, %1, %2, 4" : "=v"(d) : "v"(u), "n"(12 - 4 * J));
    return d;
  }
}

// Row maxima as integer maxima, which take their DPP operand for free (a float
// max first quiets both operands).  Non-negative floats order as their bits;
// any float (-inf included) orders as b ^ ((b >> 31) & 0x7fffffff), which is its
// own inverse.
__device__ __forceinline__ int row_max16_i32(int v) {
  v = max(v, dpp_i32<kDppSwap1>(v));
  v = max(v, dpp_i32<kDppSwap2>(v));
  v = max(v, dpp_i32<kDppHalfMirror>(v));
  return max(v, dpp_i32<kDppMirror>(v));
}
__device__ __forceinline__ float row_max16_nonneg(float x) { return __int_as_float(row_max16_i32(__float_as_int(x))); }
__device__ __forceinline__ float row_max16_any(float x) {
  const int b = __float_as_int(x);
  const int k = row_max16_i32(b ^ ((b >> 31) & 0x7fffffff));
  return __int_as_float(k ^ ((k >> 31) & 0x7fffffff));
}

__device__ __forceinline__ int exponent_above(float x) {  // E with |x| < 2^E (0 for x == 0)
  int e = 0;
  frexpf(x, &e);
  return e;
}

struct SplitParams {
  const float* qsum;          // [B][Hq][ng]  (INT2 path) sums of q' over each quantisation group
  const int* qop;             // [B][Hkv][ceil(G/4)][64][9] (INT2 path)
  const uint16_t* q;          // [B][Hq][128] bf16 queries
  const int32_t* seq_lens;
  const int32_t* block_table;
  const uint8_t* pool;        // INT2 pool
  const uint16_t* kv_pool;    // bf16 pool
  const uint16_t* r_v;        // INT2: value rotations [Hkv][128][128] (un-rotation in the merge)
  const uint16_t* win_k;      // INT2: bf16 window rings [B][W][Hkv][128]
  const uint16_t* win_v;
  float* part;                // bf16: [B][Hq][n_splits][130]; INT2: [n_wg + units][gw][130] slot partials
  float* wpart;               // INT2: [B][Hq][n_wchunks][130] window, then sink chunk partials (plain domain)
  int* tile_prefix;           // INT2: [units + 1] first history tile of each unit in the flattened order
  float* out;                 // [B][Hq][128]
  int64_t n_pages;
  int batch, hq, hkv, max_pages, max_len, window, split, n_splits;
  int n_wchunks;              // INT2: 32-token chunks of the ring, ceil(W / 32) + ceil(n_sink / 32)
  int n_wwin;                 // INT2: the first ceil(W / 32) of them cover the window, the rest the sinks
  int n_sink;                 // INT2: leading positions kept in bf16 (ring rows W + pos)
  int ring;                   // INT2: ring rows per sequence, W + n_sink
  int gsub;                   // INT2 merge units per KV head, each taking gw of its query heads
  int gw;                     // query heads a unit really has (<= G of the kernel's instantiation)
  int n_wg;                   // INT2: persistent workgroups of the split kernel
  int hw;                     // INT2: KV heads a split workgroup reads side by side (1, 2 or 4)
  int block;                  // INT2: bytes per (page, KV head) block, 1024 + 128 ng
  int ng;                     // INT2: quantisation groups per token (1, 2 or 4)
  float scale_log2;           // log2(e) / sqrt(d)
  // INT2: layers decoded in one call.  q, out, r_v (and r_k), pool, the rings
  // and the per-layer workspace regions are stacked layer-major with these
  // strides (elements of each buffer's type; pool in bytes); the block table
  // and lengths are shared; the split partials and the tile prefix span all
  // layers (units layer-major).
  int n_layers;
  int64_t ls_q, ls_out, ls_rot, ls_pool, ls_win, ls_qsum, ls_qop, ls_wpart;
  // INT2: share weights of the split workgroups: wf for the first hf, ws for
  // the rest (see share_begin)
  int wf, ws, hf;
  // INT2, the fused decode step only (else null): the newest token of every
  // sequence, [B][Hkv][128] bf16, appended by the prep kernel while the window
  // chunks read it from here instead of the ring row being written
  const uint16_t* k_new;
  const uint16_t* v_new;
};

// The parameters of layer l: every per-layer buffer advanced by l strides.
// Without a branch, so that the kernel argument loads are issued together at
// the kernel's start rather than in dependent rounds.
__device__ __forceinline__ SplitParams layer_params(const SplitParams& p, int l) {
  SplitParams r = p;
  r.q += l * p.ls_q;
  r.out += l * p.ls_out;
  r.r_v += l * p.ls_rot;
  r.pool += l * p.ls_pool;
  r.win_k += l * p.ls_win;
  r.win_v += l * p.ls_win;
  r.qsum += l * p.ls_qsum;
  r.qop += l * p.ls_qop;
  r.wpart += l * p.ls_wpart;
  return r;
}

// Shares of the persistent split kernel.  Workgroup w takes the flattened tiles
// [share_begin(w), share_begin(w + 1)).  The first hf workgroups weigh wf, the
// others ws: workgroups w and w + hf share a CU, and the one dispatched first
// has the older waves, which win the CU's issue arbitration, so it streams
// faster and is given the larger share (with equal shares it finished ~15 us
// before its partner at 100K context, every CU alike).
struct ShareWeights {
  int wf, ws, hf, total;  // total = wf hf + ws (nw - hf) <= 26 x 2^16
};
// With fewer than 4 tiles per workgroup the shares are equal, so that every
// workgroup keeps at least one tile (the weights satisfy wf <= 3 ws).
__device__ __forceinline__ ShareWeights share_weights(const SplitParams& p, int64_t T, int nw) {
  const bool weigh = T >= 4 * (int64_t)nw;
  ShareWeights s;
  s.wf = weigh ? p.wf : 1;
  s.ws = weigh ? p.ws : 1;
  s.hf = p.hf < nw ? p.hf : nw;
  s.total = s.wf * s.hf + s.ws * (nw - s.hf);
  return s;
}
// floor(a / b) for 0 <= a < 2^52, 0 < b < 2^31: the fp64 quotient (correctly
// rounded, so at most one off after the floor) corrected with integer
// products, instead of a 64-bit integer division's long instruction sequence.
__device__ __forceinline__ int64_t div_floor(int64_t a, int64_t b) {
  int64_t q = (int64_t)((double)a / (double)b);
  if (q * b > a) q -= 1;
  else if ((q + 1) * b <= a) q += 1;
  return q;
}
__device__ __forceinline__ int64_t share_begin(const SplitParams& p, int64_t T, int nw, int w) {
  const ShareWeights s = share_weights(p, T, nw);
  const int cum = w <= s.hf ? s.wf * w : s.wf * s.hf + s.ws * (w - s.hf);
  return div_floor(T * cum, s.total);
}
// The workgroup whose share holds tile t (0 <= t < T): the largest w with
// share_begin(w) <= t, i.e. with cum(w) <= ((t + 1) total - 1) / T.
__device__ __forceinline__ int64_t share_owner(const SplitParams& p, int64_t T, int nw, int64_t t) {
  const ShareWeights s = share_weights(p, T, nw);
  const int c = (int)div_floor((t + 1) * s.total - 1, T);
  const int w = c < s.wf * s.hf ? c / s.wf : s.hf + (c - s.wf * s.hf) / s.ws;
  return w < nw - 1 ? w : nw - 1;
}

// Sequence length as the kernels see it: clamped to [0, max_len].
__device__ __forceinline__ int seq_len_of(const SplitParams& p, int b) {
  const int n = p.seq_lens[b];
  return n < 0 ? 0 : (n > p.max_len ? p.max_len : n);
}

// History tiles (128 tokens) of sequence b.
__device__ __forceinline__ int hist_tiles(const SplitParams& p, int b) {
  const int n = seq_len_of(p, b);
  const int hist = n - (n < p.window ? n : p.window);
  return (hist + 127) >> 7;
}

template <int GMAX>
constexpr int window_smem_bytes() { return (GMAX * kD + kWinChunk * 65 + GMAX * kWinChunk + 4 * GMAX) * 4; }

// One 32-token chunk of the bf16 ring of (sequence b, KV head h), unrotated,
// for the G <= GMAX query heads of h: chunk c < n_wwin covers window positions
// n - w + 32 c .. (ring rows pos % W), chunk n_wwin + c' the sink positions
// 32 c' .. below s = min(n_sink, n - w) (ring rows W + pos).
// Thread (t, part) = (tid / 8, tid % 8) loads dims 16 part .. 16 part + 15 of
// token t's key and value (all loads issued first); the 8 parts of a score are
// summed across lanes, V goes through LDS for P V.  Writes (m, l, acc[128]) of
// the chunk per head; an empty chunk writes m = -inf, l = 0, acc = 0.
template <int GMAX>
__device__ void window_chunk(const SplitParams& p, int b, int h, int c, int G, float* sm) {
  const int tid = threadIdx.x, wave = tid >> 6;
  const int n = seq_len_of(p, b);
  const int w = n < p.window ? n : p.window;
  const bool sink = c >= p.n_wwin;
  const int s_end = min(p.n_sink, n - w);  // sink positions [0, s_end)
  const int cs = sink ? kWinChunk * (c - p.n_wwin) : n - w + kWinChunk * c;
  const int nt = min(kWinChunk, (sink ? s_end : n) - cs);  // <= 0: empty chunk
  const int hq0 = h * G;
  float* dst0 = p.wpart + (((int64_t)b * p.hq + hq0) * p.n_wchunks + c) * kPartStride;
  const int64_t head_stride = (int64_t)p.n_wchunks * kPartStride;
  if (nt <= 0) {
    for (int e = tid; e < G * kPartStride; e += 256) {
      const int g = e / kPartStride, i = e % kPartStride;
      dst0[g * head_stride + i] = i == 0 ? kNegInf : 0.f;
    }
    return;
  }
  float* qs = sm;                                            // [G][128]
  uint32_t* vs = reinterpret_cast<uint32_t*>(qs + G * kD);   // [32][65] bf16 pairs
  float* ps = reinterpret_cast<float*>(vs + kWinChunk * 65);  // [GMAX][32]
  float* red = ps + GMAX * kWinChunk;                         // [4][GMAX]
  const int t = tid >> 3, part = tid & 7;
  const bool valid = t < nt;
  uint4 kk[2], vv[2];
  {
    // ring row of window position cs + t: (cs mod W) + t, less W once it
    // passes W (t < nt <= w <= W), instead of a per-lane division
    const int cw = sink ? 0 : cs % p.window;  // uniform
    const int slot = !valid ? 0 : sink ? p.window + cs + t : (cw + t >= p.window ? cw + t - p.window : cw + t);
    const int64_t row = (((int64_t)b * p.ring + slot) * p.hkv + h) * kD + 16 * part;
    const uint4* kr = reinterpret_cast<const uint4*>(p.win_k + row);
    const uint4* vr = reinterpret_cast<const uint4*>(p.win_v + row);
    // the fused step's newest token (position n - 1, appended by this launch
    // when the length is not clamped) comes from the new-token rows
    if (p.k_new && valid && cs + t == n - 1 && p.seq_lens[b] == n) {
      const int64_t nrow = ((int64_t)b * p.hkv + h) * kD + 16 * part;
      kr = reinterpret_cast<const uint4*>(p.k_new + nrow);
      vr = reinterpret_cast<const uint4*>(p.v_new + nrow);
    }
    kk[0] = kr[0]; kk[1] = kr[1];
    vv[0] = vr[0]; vv[1] = vr[1];
  }
  // the G heads' queries (contiguous rows), 8 channels a thread: one load in
  // flight with the key and value rows (a clamped one past 16 G threads)
  const uint4 qv = reinterpret_cast<const uint4*>(p.q + ((int64_t)b * p.hq + hq0) * kD)[tid < 16 * G ? tid : 0];
  if (tid < 16 * G) {
    const uint32_t u[4] = {qv.x, qv.y, qv.z, qv.w};
    float4* d = reinterpret_cast<float4*>(qs + 8 * tid);
    d[0] = make_float4(bf16lo(u[0]), bf16hi(u[0]), bf16lo(u[1]), bf16hi(u[1]));
    d[1] = make_float4(bf16lo(u[2]), bf16hi(u[2]), bf16lo(u[3]), bf16hi(u[3]));
  }
  {
    uint32_t* d = vs + t * 65 + 8 * part;
    const uint32_t u[8] = {vv[0].x, vv[0].y, vv[0].z, vv[0].w, vv[1].x, vv[1].y, vv[1].z, vv[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = valid ? u[i] : 0u;
  }
  __syncthreads();
  const uint32_t ku[8] = {kk[0].x, kk[0].y, kk[0].z, kk[0].w, kk[1].x, kk[1].y, kk[1].z, kk[1].w};
  float sc[GMAX];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g >= G) break;  // uniform
    const float* qg = qs + g * kD + 16 * part;
    float d = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) d = fmaf(bf16lo(ku[i]), qg[2 * i], fmaf(bf16hi(ku[i]), qg[2 * i + 1], d));
    d += dpp_f32<kDppSwap1>(d);
    d += dpp_f32<kDppSwap2>(d);
    d += dpp_f32<kDppHalfMirror>(d);  // the 8 parts of token t
    sc[g] = valid ? d * p.scale_log2 : kNegInf;
    const float m = wave_max64(sc[g]);
    if ((tid & 63) == 0) red[wave * GMAX + g] = m;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g >= G) break;
    const float m = fmaxf(fmaxf(red[g], red[GMAX + g]), fmaxf(red[2 * GMAX + g], red[3 * GMAX + g]));
    if (part == 0) ps[g * kWinChunk + t] = valid ? exp2f(sc[g] - m) : 0.f;
  }
  __syncthreads();
  for (int e = tid; e < G * kD; e += 256) {
    const int g = e >> 7, ch = e & (kD - 1);
    const float* pg = ps + g * kWinChunk;
    // all 32 rows with a fixed trip count (a token past nt has p = 0 and a zero
    // row), so the LDS reads are issued together rather than one per iteration
    float acc0 = 0.f, acc1 = 0.f, l = 0.f;
#pragma unroll
    for (int tt = 0; tt < kWinChunk; tt += 2) {
      const uint32_t x0 = vs[tt * 65 + (ch >> 1)], x1 = vs[(tt + 1) * 65 + (ch >> 1)];
      const float2 pp = *reinterpret_cast<const float2*>(pg + tt);
      acc0 = fmaf(pp.x, (ch & 1) ? bf16hi(x0) : bf16lo(x0), acc0);
      acc1 = fmaf(pp.y, (ch & 1) ? bf16hi(x1) : bf16lo(x1), acc1);
      l += pp.x + pp.y;
    }
    float* dst = dst0 + g * head_stride;
    dst[2 + ch] = acc0 + acc1;
    if (ch == 0) {
      dst[0] = fmaxf(fmaxf(red[g], red[GMAX + g]), fmaxf(red[2 * GMAX + g], red[3 * GMAX + g]));
      dst[1] = l;
    }
  }
}

// ---------------------------------------------------------------------------
// Query preparation, once per (sequence, KV head):
//   q' = R_K[h] q for its G <= 16 query heads on the matrix cores (bf16 in,
//   fp32 out; each wave 32 output channels);
//   q' is kept scaled by log2(e) / sqrt(d), so the scores come out in the log2
//   domain; qsum[head][j] = sum of that q' over the channels of quantisation
//   group j;
//   the fp8 score operand of every 4-head group: lane (lg, lr) holds digit lr % 4
//   of q'_(head lr / 4) at the 32 channels its k-slots map to, plus the row's
//   E8M0 scale (2^(E - 3 - 4 digit), |q'| < 2^E), exactly as the split kernel's
//   MFMA consumes it.
// ---------------------------------------------------------------------------
//
// NGA > 0 (the fused decode step, NGA quantisation groups per token): planes
// z = 1 + n_wchunks + kind also append the newest token of every sequence
// (kind 0: keys, 1: values) for KV head blockIdx.y, 64 sequences per
// workgroup, exactly as the append kernel would (its device code, 4 waves of
// one 16-token tile each).
template <int G, int NGA>
__global__ __launch_bounds__(256) void prep_kernel(SplitParams p0, const uint16_t* __restrict__ r_k0,
                                                   AppendParams ap) {
  constexpr int NCB = (G + 3) / 4;  // 4-head operand groups
  static_assert(G <= 16, "the heads are the 16 columns of one MFMA");
  constexpr int kQBytes = 2 * G * kD * 4 + G * 4;
  constexpr int kSmem0 = kQBytes > window_smem_bytes<G>() ? kQBytes : window_smem_bytes<G>();
  constexpr int kSmem = NGA > 0 && kSmem0 < 128 * 16 * 16 ? 128 * 16 * 16 : kSmem0;  // R of the append: 32 KiB
  __shared__ __align__(16) float smem_f[kSmem / 4];
  const int layer = blockIdx.x / p0.batch, b = blockIdx.x % p0.batch, h = blockIdx.y, tid = threadIdx.x;
  if constexpr (NGA > 0) {
    if ((int)blockIdx.z > p0.n_wchunks) {  // the newest tokens, one launch with the query preparation
      const int64_t t_wg = (int64_t)blockIdx.x * 64;
      if (t_wg >= ap.n_tokens) return;  // uniform over the workgroup
      const int64_t t0 = t_wg + 16 * (tid >> 6);
      uint4* r_lds = reinterpret_cast<uint4*>(smem_f);
      if ((int)blockIdx.z == p0.n_wchunks + 1)
        append_one<0, NGA, 256, true>(ap, r_lds, h, t0, tid & 63);
      else
        append_one<1, NGA, 256, true>(ap, r_lds, h, t0, tid & 63);
      return;
    }
  }
  const SplitParams p = layer_params(p0, layer);
  const uint16_t* r_k = r_k0 + layer * p0.ls_rot;
  const int hq = p.hq, hkv = p.hkv;
  if (blockIdx.z > 0) {  // chunk z - 1 of the bf16 window of this (sequence, KV head)
    window_chunk<G>(p, b, h, blockIdx.z - 1, G, smem_f);
    return;
  }
  // The rotation's operands go out first: the query rows and R_K rows below do
  // not depend on the tile prefix, so both wait on one round trip.
  // q' = R_K q on the matrix cores (v_mfma_f32_16x16x32_bf16, exact bf16
  // products, fp32 sums): wave v computes output channels 32 v .. 32 v + 31
  // as two 16-row blocks; A = rows of R_K, B = q^T with the G heads as
  // columns (zero past G).  Lane (g, r) supplies A row r and B column r at
  // k = 8 g .. 8 g + 7 of each 32-wide k step and ends with channels
  // 16 cb + 4 g + i of head r.
  const int mg = (tid & 63) >> 4, mr = tid & 15, mw = tid >> 6;
  uint4 bq[4], ra[2][4];
  {
    // rows past G read head 0's (a clamped row, no branch around the load)
    // and are zeroed before use
    const uint4* qrow = reinterpret_cast<const uint4*>(p.q + ((int64_t)b * hq + h * G + (mr < G ? mr : 0)) * kD);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) bq[ks] = qrow[4 * ks + mg];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const uint4* rrow = reinterpret_cast<const uint4*>(r_k + ((int64_t)h * kD + 16 * (2 * mw + blk) + mr) * kD);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) ra[blk][ks] = rrow[4 * ks + mg];
    }
  }
  // first history tile of the units (layer, b, head group, sub) in the
  // flattened order (layer-major, then sequence, KV head group, head subset),
  // written by the first head of each group; the last group also closes the
  // array.  Every layer has the same sequences, hence the same T tiles.
  if (tid < 64 && h % p.hw == 0) {  // wave 0: tiles of the sequences before b, of b and of all, summed across lanes
    int pb = 0, pt = 0, tb = 0;
    for (int bb = tid; bb < p.batch; bb += 64) {
      const int tt = hist_tiles(p, bb);
      pb += bb < b ? tt : 0;
      tb += bb == b ? tt : 0;
      pt += tt;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      pb += __shfl_xor(pb, o);
      tb += __shfl_xor(tb, o);
      pt += __shfl_xor(pt, o);
    }
    const int hgp = h / p.hw, per_seq = (hkv / p.hw) * p.gsub;
    const int64_t u0 = (int64_t)layer * p.batch * per_seq, t0 = (int64_t)layer * per_seq * pt;
    for (int sub = tid; sub < p.gsub; sub += 64)
      p.tile_prefix[u0 + (int64_t)b * per_seq + hgp * p.gsub + sub] =
          (int)(t0 + per_seq * pb + (hgp * p.gsub + sub) * tb);
    if (tid == 0 && layer == p.n_layers - 1 && b == p.batch - 1 && h == hkv - p.hw)
      p.tile_prefix[u0 + (int64_t)p.batch * per_seq] = (int)(t0 + (int64_t)per_seq * pt);
  }
  float (*qs)[kD] = reinterpret_cast<float (*)[kD]>(smem_f);
  int* qexp = reinterpret_cast<int*>(smem_f + 2 * G * kD);
  float* qsum_out = const_cast<float*>(p.qsum);
  int* qop = const_cast<int*>(p.qop);
  {
    if (mr >= G) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) bq[ks] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ra[blk][ks]),
                                                      __builtin_bit_cast(bf16x8, bq[ks]), acc, 0, 0, 0);
      if (mr < G) {
#pragma unroll
        for (int i = 0; i < 4; ++i) qs[mr][16 * (2 * mw + blk) + 4 * mg + i] = acc[i] * p.scale_log2;
      }
    }
  }
  __syncthreads();
  if (tid < G * 16) {  // 16 threads per head: group sums and max |q'|
    const int g = tid >> 4, j = tid & 15;
    const int tpg = 16 / p.ng;  // threads per group (8 channels each)
    float s = 0.f, mx = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      s += qs[g][8 * j + c];
      mx = fmaxf(mx, fabsf(qs[g][8 * j + c]));
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const float so = __shfl_xor(s, o);
      s = o < tpg ? s + so : s;
      mx = fmaxf(mx, __shfl_xor(mx, o));
    }
    if (j % tpg == 0) qsum_out[((int64_t)b * hq + h * G + g) * p.ng + j / tpg] = s;
    if (j == 0) qexp[g] = exponent_above(mx);
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  // item (cb, q4): dwords 2 q4 and 2 q4 + 1 of the operand (k-slots 8 q4 .. 8 q4 + 7)
  for (int it = wave; it < NCB * 4; it += 4) {
    const int cb = it >> 2, q4 = it & 3;
    const int head = 4 * cb + (lr >> 2), term = lr & 3;
    int op[2] = {0, 0};
    int sc = kScaleOne;
    if (head < G) {
      const int E = qexp[head];
      sc = clamp_scale(kScaleOne + E - 3 - 4 * term);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float a = ldexpf(qs[head][k_channel(k_of_fp8(lg, 8 * q4 + e))], 3 - E);
        const float c = ldexpf(qs[head][k_channel(k_of_fp8(lg, 8 * q4 + e + 1))], 3 - E);
        uint32_t t[kDigits];
        float ra, rc;
        digits_pair(a, c, t, ra, rc);
        op[e >> 2] |= (int)(t[term] << (8 * (e & 3)));
      }
    }
    int* dst = qop + ((((int64_t)b * hkv + h) * NCB + cb) * 64 + lane) * 9;
    dst[2 * q4] = op[0];
    dst[2 * q4 + 1] = op[1];
    if (q4 == 0) dst[8] = sc;
  }
}

// Combine the 4 waves' (m, l, acc) partials (LDS) into the workgroup partial
// (m, l, acc[128]) of each of the gw heads, written to dst0 + g * head_stride.
template <int G>
__device__ __forceinline__ void combine_and_store(const float* cm, const float* cl, const float* cacc, float* dst0,
                                                  int64_t head_stride, int gw) {
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
    float* dst = dst0 + g * head_stride;
    dst[2 + c] = acc;
    if (c == 0) {
      dst[0] = M;
      dst[1] = L;
    }
  }
}

// Raw bytes of one 128-token tile (8 pages) as one lane needs them; NG
// quantisation groups per token.
template <int NG>
struct Tile {
  uint2 kc[8];        // K row bytes 8lg..8lg+7 of token lr, per page
  uint4 rec[NG];      // 16 bytes of the tile's records (see load_tile); any value past the history end
  uint2 meta[8][NG];  // or, without the LDS spread: token lr's records, one per page and group
  uint4 vlo[2], vhi[2];  // V words of channels 4lr..4lr+3 (lo), 64+4lr..64+4lr+3 (hi), pages 2lg and 2lg+1
  uint32_t page_ok;      // bit pp: page pp of the tile exists in this split and in the pool
};

// Block-table entries of two consecutive tiles of a wave.  The wave's k-th
// tile is tile ph + ts k of the range (ph = the wave's phase, ts = the waves
// sharing its KV head, which take its tiles round robin);
// lane 8j + pp (j < 2) holds the page of page pp of the wave's tile k0 + j, or
// -1 when that page is past the history, the tile past the wave's range, or
// the entry outside the pool.  The entries are loaded one loop iteration ahead
// of their use (table_load, no branch: the index is clamped) and validated
// only when the iteration that uses them starts (table_ready), so no wait on
// the block table ever drains the tile loads in flight behind it.
struct TileTable {
  int ent;        // this lane's entry
  uint64_t live;  // ballot of ent >= 0
};

__device__ __forceinline__ int table_page(int P0, int ph, int ts, int k0) {
  const int lane = threadIdx.x & 63;
  return P0 + 8 * (ph + ts * (k0 + ((lane >> 3) & 1))) + (lane & 7);
}

__device__ __forceinline__ int table_load(const int* btr, int P0, int P1, int ph, int ts, int k0) {
  const int pg = table_page(P0, ph, ts, k0);
  return btr[pg < P1 ? pg : P1];
}

__device__ __forceinline__ TileTable table_ready(const SplitParams& p, int raw, int P0, int P1, int ph, int ts,
                                                 int k0, int ntw) {
  const int lane = threadIdx.x & 63;
  const int pg = table_page(P0, ph, ts, k0);
  const bool ok = lane < 16 && pg <= P1 && k0 + (lane >> 3) < ntw && raw >= 0 && raw < p.n_pages;
  return TileTable{ok ? raw : -1, __ballot(ok)};
}

// All loads of one tile (j-th of its table pair) are issued back to back with
// no branches: every page index is broadcast with readlane, so each page's block
// address is a scalar (base_h + page * stride, two scalar multiplies and an add)
// and every K-row and record load takes it as its base with the lane's fixed
// 32-bit offset; a missing page is read as page 0 and masked, so the memory
// system sees the whole tile at once.  base_h: the KV head's block in page 0;
// stride: bytes per page (all KV heads).
// REC: the records come as one 16-byte chunk per lane (spread through LDS by
// spread_records); otherwise each lane loads its token's records itself (the
// register-heavier instantiations, where the LDS spread's live range spills).
template <int NG, bool REC = true>
__device__ __forceinline__ void load_tile(const uint8_t* base_h, uint32_t stride, const TileTable& tt, int j, int lg,
                                          int lr, Tile<NG>& t) {
  t.page_ok = (uint32_t)(tt.live >> (8 * j)) & 0xffu;
  const uint32_t off_k = kKCodes + 32 * lr + 8 * lg;
  const uint32_t off_v = kVCodes + 16 * lr;  // 16 lanes read 256 contiguous bytes per half
#pragma unroll
  for (int pp = 0; pp < 8; ++pp) {
    const int e = __builtin_amdgcn_readlane(tt.ent, 8 * j + pp);
    const __amdgpu_buffer_rsrc_t blk = block_rsrc(base_h + (uint64_t)(uint32_t)(e < 0 ? 0 : e) * stride);
    t.kc[pp] = buffer_nt2(blk, off_k);
    if constexpr (!REC) {
      const uint32_t off_m = kMeta + 8 * NG * lr;
      if constexpr (NG == 1) {
        t.meta[pp][0] = buffer_nt2(blk, off_m);
      } else {
#pragma unroll
        for (int q2 = 0; q2 < NG; q2 += 2) {
          const uint4 m2 = buffer_nt4(blk, off_m + 8 * q2);
          t.meta[pp][q2] = make_uint2(m2.x, m2.y);
          t.meta[pp][q2 + 1] = make_uint2(m2.z, m2.w);
        }
      }
    }
  }
  // records: one 16-byte chunk per lane and group block, lane 8 p + c taking
  // chunk c of page p's 128 NG record bytes (every lane a distinct address;
  // the lanes of one token read them from LDS, see spread_records)
  if constexpr (REC) {
    const int lane = threadIdx.x & 63;
    const int pr = __builtin_amdgcn_ds_bpermute(4 * (8 * j + (lane >> 3)), tt.ent);
    const uint8_t* blk = base_h + (uint64_t)(uint32_t)(pr < 0 ? 0 : pr) * stride + kMeta + 16 * (lane & 7);
#pragma unroll
    for (int k = 0; k < NG; ++k) t.rec[k] = load_nt4(blk + 128 * k);
  }
  // V words: lane group lg takes pages 2lg and 2lg + 1 (entries of lanes
  // 8j + 2lg + qq, fetched across lanes)
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const int pv = __builtin_amdgcn_ds_bpermute(4 * (8 * j + 2 * lg + qq), tt.ent);
    const uint8_t* blk = base_h + (uint64_t)(uint32_t)(pv < 0 ? 0 : pv) * stride + off_v;
    t.vlo[qq] = load_nt4(blk);
    t.vhi[qq] = load_nt4(blk + 256);
  }
  // no use of the loaded registers here: the caller computes another tile
  // while these loads are in flight
}

// The same loads in two parts, for the loop that keeps one tile in flight:
// load_tile_k the K-code rows and the records (all that phase 1 of
// compute_tile reads), load_tile_v the V words (all that phase 2 reads).
template <int NG>
__device__ __forceinline__ void load_tile_k(const uint8_t* base_h, uint32_t stride, const TileTable& tt, int j, int lg,
                                            int lr, Tile<NG>& t) {
  t.page_ok = (uint32_t)(tt.live >> (8 * j)) & 0xffu;
  const uint32_t off_k = kKCodes + 32 * lr + 8 * lg;
  const uint32_t off_m = kMeta + 8 * NG * lr;
#pragma unroll
  for (int pp = 0; pp < 8; ++pp) {
    const int e = __builtin_amdgcn_readlane(tt.ent, 8 * j + pp);
    const __amdgpu_buffer_rsrc_t blk = block_rsrc(base_h + (uint64_t)(uint32_t)(e < 0 ? 0 : e) * stride);
    t.kc[pp] = buffer_nt2(blk, off_k);
    if constexpr (NG == 1) {
      t.meta[pp][0] = buffer_nt2(blk, off_m);
    } else {
#pragma unroll
      for (int q2 = 0; q2 < NG; q2 += 2) {
        const uint4 m2 = buffer_nt4(blk, off_m + 8 * q2);
        t.meta[pp][q2] = make_uint2(m2.x, m2.y);
        t.meta[pp][q2 + 1] = make_uint2(m2.z, m2.w);
      }
    }
  }
}
template <int NG>
__device__ __forceinline__ void load_tile_v(const uint8_t* base_h, uint32_t stride, const TileTable& tt, int j, int lg,
                                            int lr, Tile<NG>& t) {
  const uint32_t off_v = kVCodes + 16 * lr;
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const int pv = __builtin_amdgcn_ds_bpermute(4 * (8 * j + 2 * lg + qq), tt.ent);
    const uint8_t* blk = base_h + (uint64_t)(uint32_t)(pv < 0 ? 0 : pv) * stride + off_v;
    t.vlo[qq] = load_nt4(blk);
    t.vhi[qq] = load_nt4(blk + 256);
  }
}

// Pins a value at this point of the program.  The matrix instructions read
// their operands across all 64 lanes, so they must run with every lane active:
// without the pin the compiler may sink an MFMA whose result is only used under
// a per-lane condition into that condition's branch.
__device__ __forceinline__ float pin(float x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ void pin8(f32x4 (&c)[8]) {
  asm volatile("" : "+v"(c[0]), "+v"(c[1]), "+v"(c[2]), "+v"(c[3]), "+v"(c[4]), "+v"(c[5]), "+v"(c[6]), "+v"(c[7]));
}

// Running state of one wave: accumulators, running max, partial sums (the
// midpoint sums per quantisation group).
template <int NRG, int NG>
struct WaveState {
  f32x4 acc[NRG][8];
  float m_run[NRG], l_part[NRG], az_part[NRG][NG];
};

// Group of the K-operand dword half (0: bytes 0..3 of the row segment, 1: bytes
// 4..7) and its byte mask: byte m of a segment holds channels 16 m + 4 lg + i,
// so group jg of NG holds bytes [8 jg / NG, 8 (jg + 1) / NG).
template <int NG>
__device__ __forceinline__ void k_operand_group(const uint2 kc, int jg, i32x8& bk) {
  const uint32_t lo = kc.x & 0x33333333u, hi = (kc.x >> 2) & 0x33333333u;
  const uint32_t lo1 = kc.y & 0x33333333u, hi1 = (kc.y >> 2) & 0x33333333u;
  if constexpr (NG == 1) {
    bk[0] = (int)lo;
    bk[1] = (int)hi;
    bk[2] = (int)lo1;
    bk[3] = (int)hi1;
  } else {
    const int half = NG == 2 ? jg : jg >> 1;
    const uint32_t mask = NG == 2 ? 0xffffffffu : ((jg & 1) ? 0xffff0000u : 0x0000ffffu);
    bk[0] = half == 0 ? (int)(lo & mask) : 0;
    bk[1] = half == 0 ? (int)(hi & mask) : 0;
    bk[2] = half == 1 ? (int)(lo1 & mask) : 0;
    bk[3] = half == 1 ? (int)(hi1 & mask) : 0;
  }
  bk[4] = bk[5] = bk[6] = bk[7] = 0;
}

// The tile's records reach the lanes that use them through the wave's LDS
// region rb (128 NG bytes per page): token lr's records of page pp, one per
// group, into meta[pp][jg] ({Ks, Kz} in .x, {Vs, Vz} in .y).
template <int NG>
__device__ __forceinline__ void spread_records(const Tile<NG>& t, uint8_t* rb, int lr, uint2 (&meta)[8][NG]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < NG; ++k)
    *reinterpret_cast<uint4*>(rb + (lane >> 3) * 128 * NG + 128 * k + 16 * (lane & 7)) = t.rec[k];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int pp = 0; pp < 8; ++pp) {
    const uint8_t* src = rb + pp * 128 * NG + 8 * NG * lr;
    if constexpr (NG == 1) {
      meta[pp][0] = *reinterpret_cast<const uint2*>(src);
    } else {
#pragma unroll
      for (int q2 = 0; q2 < NG; q2 += 2) {
        const uint4 m2 = *reinterpret_cast<const uint4*>(src + 8 * q2);
        meta[pp][q2] = make_uint2(m2.x, m2.y);
        meta[pp][q2 + 1] = make_uint2(m2.z, m2.w);
      }
    }
  }
}

// What phase 1 of compute_tile leaves for phase 2, beside the wave's LDS
// digit tile: the weights' digit sums (midpoint correction) and exponents.
template <int NRG, int NG>
struct TileWeights {
  float wsum[NRG][NG];
  int wexp[NRG][NG];
};

// PHASE 0: the whole tile.  PHASE 1: scores, softmax and the weight digits
// only (reads the tile's K codes and records; leaves tw); PHASE 2: the value
// MFMAs only (reads the tile's V codes and tw), so that a caller can load the
// next tile's K part while phase 2 runs and its V part while phase 1 runs.
template <int G, int NRG, bool FULL, int NG, bool REC, int PHASE = 0>  // FULL: all 8 pages exist and every token is below t_end
__device__ __forceinline__ void compute_tile(const SplitParams& p, const Tile<NG>& t, int pbase, int t_beg, int t_end,
                                             int lg, int lr, const i32x8* qa, const int* qsc, const float (*qsr)[NG],
                                             uint8_t* wt, uint8_t* rb, WaveState<NRG, NG>& st,
                                             TileWeights<NRG, NG>* tw = nullptr) {
  float wsum[NRG][NG];  // sum of the weights as the digits carry them
  int wexp[NRG][NG];    // every weight of this lane's head and group below 2^wexp
  if constexpr (PHASE == 2) {
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
      for (int jg = 0; jg < NG; ++jg) {
        wsum[rg][jg] = tw->wsum[rg][jg];
        wexp[rg][jg] = tw->wexp[rg][jg];
      }
  }
  if constexpr (PHASE != 2) {
  uint2 meta[8][NG];
  if constexpr (REC) {
    spread_records(t, rb, lr, meta);
  } else {
#pragma unroll
    for (int pp = 0; pp < 8; ++pp)
#pragma unroll
      for (int jg = 0; jg < NG; ++jg) meta[pp][jg] = t.meta[pp][jg];
  }
  const int slot_pos = 8 * (lr & 1) + (lr >> 1);  // k position of token lr within its page's 16
  // slots past the history end or on a missing page may hold anything: their
  // records must not reach the per-tile scale exponent or the sums
  bool live[8];
#pragma unroll
  for (int pp = 0; pp < 8; ++pp) {
    const int tok = (pbase + pp) * 16 + lr;
    live[pp] = FULL || (((t.page_ok >> pp) & 1u) && tok >= t_beg && tok < t_end);
  }
  // ---- scores (log2 domain; q' and its group sums arrive scaled by log2(e)/sqrt(d)):
  // sc[rg][pp] = sum over groups jg of ks_jg (q'_(4rg+lg) . code) + kz_jg qsum_jg,
  // the dot product over group jg's channels of token lr of page pp ----
  float sc[NRG][8];
  if constexpr (NRG > 1) {  // registers: one page at a time, each score pinned
#pragma unroll
    for (int pp = 0; pp < 8; ++pp) {
#pragma unroll
      for (int jg = 0; jg < NG; ++jg) {
        i32x8 bk;
        k_operand_group<NG>(t.kc[pp], jg, bk);
        const float ks = h2f((uint16_t)(meta[pp][jg].x & 0xffffu));
        const float kz = h2f((uint16_t)(meta[pp][jg].x >> 16));
#pragma unroll
        for (int rg = 0; rg < NRG; ++rg) {
          const f32x4 c = mfma_f8_f4(qa[rg], bk, f32x4{0.f, 0.f, 0.f, 0.f}, qsc[rg], kScaleCode);
          const float term = fmaf(kz, qsr[rg][jg], ks * ((c[0] + c[1]) + (c[2] + c[3])));
          sc[rg][pp] = pin(jg == 0 ? term : sc[rg][pp] + term);
        }
      }
    }
  } else {
#pragma unroll
  for (int jg = 0; jg < NG; ++jg) {
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
      // the 8 pages' MFMAs first, all pinned at one point (every lane active),
      // then their sums: no result is waited for right behind its MFMA
      f32x4 c[8];
#pragma unroll
      for (int pp = 0; pp < 8; ++pp) {
        i32x8 bk;
        k_operand_group<NG>(t.kc[pp], jg, bk);
        c[pp] = mfma_f8_f4(qa[rg], bk, f32x4{0.f, 0.f, 0.f, 0.f}, qsc[rg], kScaleCode);
      }
      pin8(c);
#pragma unroll
      for (int pp = 0; pp < 8; ++pp) {
        const float ks = h2f((uint16_t)(meta[pp][jg].x & 0xffffu));
        const float kz = h2f((uint16_t)(meta[pp][jg].x >> 16));
        const float term = fmaf(kz, qsr[rg][jg], ks * ((c[pp][0] + c[pp][1]) + (c[pp][2] + c[pp][3])));
        sc[rg][pp] = jg == 0 ? term : sc[rg][pp] + term;
      }
    }
  }
  }
  // ---- online softmax, weights, weight digits -> LDS ----
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) {
    const bool hv = 4 * rg + lg < p.gw;
    float lgt[8];
    float mx = kNegInf;
#pragma unroll
    for (int pp = 0; pp < 8; ++pp) {
      // computed on every lane, then masked: a select, not a branch
      lgt[pp] = hv && live[pp] ? sc[rg][pp] : kNegInf;
      mx = fmaxf(mx, lgt[pp]);
    }
    mx = row_max16_any(mx);
    const float m_new = fmaxf(st.m_run[rg], mx);
    if (__any(m_new > st.m_run[rg])) {
      const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(st.m_run[rg] - m_new);
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) st.acc[rg][nn] *= alpha;
      st.l_part[rg] *= alpha;
#pragma unroll
      for (int jg = 0; jg < NG; ++jg) st.az_part[rg][jg] *= alpha;
      st.m_run[rg] = m_new;
    }
    const float m_safe = st.m_run[rg] == kNegInf ? 0.f : st.m_run[rg];  // exp2(-inf - m_safe) = 0
    float pv[8];
#pragma unroll
    for (int pp = 0; pp < 8; ++pp) {
      // the hardware exp2: p <= 1, and a p below 2^-126 may read as 0
      pv[pp] = __builtin_amdgcn_exp2f(lgt[pp] - m_safe);
      st.l_part[rg] += pv[pp];
    }
#pragma unroll
    for (int jg = 0; jg < NG; ++jg) {  // one group's weights at a time (registers)
      float w[8];
      float wmax = 0.f;
#pragma unroll
      for (int pp = 0; pp < 8; ++pp) {
        // value scale and zero of (page pp, group jg); a dead slot's record may
        // hold anything (NaN included), so it is replaced by zeros first
        const uint32_t vrec = live[pp] ? meta[pp][jg].y : 0u;
        const float vs = h2f((uint16_t)(vrec & 0xffffu)), vz = h2f((uint16_t)(vrec >> 16));
        st.az_part[rg][jg] = fmaf(pv[pp], fmaf(1.5f, vs, vz), st.az_part[rg][jg]);
        w[pp] = pv[pp] * vs;
        wmax = fmaxf(wmax, w[pp]);
      }
      // this head's weights in the tile are < 2^e.  The floor keeps 2^(15 - e)
      // finite: weights below 2^-100 then sit on a grid of 2^-115 (below
      // 2^-116 they code as 0), an absolute error under 2^-92 of the
      // partial's largest weight (p = 1 there, and a nonzero fp16 scale is at
      // least 2^-24)
      const int e = max(exponent_above(row_max16_nonneg(wmax)), kMinWeightExp);
      const float fix = ldexpf(1.f, 15 - e);  // w fix = 4096 w 2^(3 - e) < 2^15, exact
      uint32_t xsum = 0u;  // sum of the lane's kRoundBits + X (mod 2^32)
      uint8_t* col = wt + (rg * NG + jg) * 2048 + (4 * lg) * 128 + slot_pos;
#pragma unroll
      for (int pp = 0; pp < 8; ++pp) {
        const uint32_t u = weight_fixed(w[pp], fix);
        xsum += u;
        col[0 * 128 + 16 * pp] = (uint8_t)weight_digit<0>(u);
        col[1 * 128 + 16 * pp] = (uint8_t)weight_digit<1>(u);
        col[2 * 128 + 16 * pp] = (uint8_t)weight_digit<2>(u);
        col[3 * 128 + 16 * pp] = (uint8_t)weight_digit<3>(u);
      }
      // the digits carry X 2^(e - 15), not w: the correction below takes the
      // same sum, or its rounding would shift every channel alike (the 16 lanes'
      // X sum to below 2^22, exact in fp32)
      wsum[rg][jg] = row_sum16((float)(xsum - 8u * kRoundBits)) * ldexpf(1.f, e - 15);
      wexp[rg][jg] = e;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }  // phase 1
  if constexpr (PHASE == 1) {
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
      for (int jg = 0; jg < NG; ++jg) {
        tw->wsum[rg][jg] = wsum[rg][jg];
        tw->wexp[rg][jg] = wexp[rg][jg];
      }
    return;
  }

  // ---- values: acc[rg][nn] += weight digits x V codes (channel vch(nn) of
  // column lr: 4 lr + nn for nn < 4, 64 + 4 lr + nn - 4 above) ----
  // with NG > 1 the column's channel in the MFMAs nn < 4 belongs to group
  // lr NG / 32, in nn >= 4 to group NG / 2 + lr NG / 32.  The MFMA of group jg
  // scales the codes of the other groups' columns by 2^-127 (E8M0 0) instead of
  // 2 (its B scale is per lane, i.e. per column): their products with group jg's
  // weights land ~2^-128 below the true products, under fp32 resolution of any
  // accumulator they join, and no instruction is spent masking them.
  // A-operand scale of row lr (head lr / 4 of the row group, digit lr % 4, a
  // byte n of which reads n 2^-9): that head's exponent lives on the lanes of
  // row lr / 4
  const int src_row = 4 * 16 * (lr >> 2);
  const int grp_lo = lr * NG / 32, grp_hi = NG / 2 + lr * NG / 32;
  float corr_lo[NRG], corr_hi[NRG];
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg) corr_lo[rg] = corr_hi[rg] = 0.f;
#pragma unroll
  for (int jg = 0; jg < NG; ++jg) {
    const bool mine_lo = NG == 1 || grp_lo == jg, mine_hi = NG == 1 || grp_hi == jg;
    const int sb_lo = mine_lo ? kScaleCode : 0, sb_hi = mine_hi ? kScaleCode : 0;
    i32x8 wa[NRG];
    int wsc[NRG];
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
      const uint8_t* row = wt + (rg * NG + jg) * 2048 + lr * 128;
      const uint4 a0 = *reinterpret_cast<const uint4*>(row + 16 * lg);
      const uint4 a1 = *reinterpret_cast<const uint4*>(row + 64 + 16 * lg);
      wa[rg][0] = (int)a0.x;
      wa[rg][1] = (int)a0.y;
      wa[rg][2] = (int)a0.z;
      wa[rg][3] = (int)a0.w;
      wa[rg][4] = (int)a1.x;
      wa[rg][5] = (int)a1.y;
      wa[rg][6] = (int)a1.z;
      wa[rg][7] = (int)a1.w;
      const int eh = __builtin_amdgcn_ds_bpermute(src_row, wexp[rg][jg]);
      wsc[rg] = clamp_scale(kScaleOne + kDigitByteExp + eh - 3 - 4 * (lr & 3));
      corr_lo[rg] = mine_lo ? 1.5f * wsum[rg][jg] : corr_lo[rg];
      corr_hi[rg] = mine_hi ? 1.5f * wsum[rg][jg] : corr_hi[rg];
    }
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
#pragma unroll
      for (int rg = 0; rg < NRG; ++rg)
        st.acc[rg][nn] = mfma_f8_f4(wa[rg], bv, st.acc[rg][nn], wsc[rg], nn < 4 ? sb_lo : sb_hi);
    }
  }
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) st.acc[rg][nn][0] -= nn < 4 ? corr_lo[rg] : corr_hi[rg];
  __builtin_amdgcn_wave_barrier();
}



// ---------------------------------------------------------------------------
// INT2 history attention on the matrix cores, persistent.
// The history tiles (128 tokens) of every merge unit (sequence, group of hw
// adjacent KV heads, head subset) form one flattened sequence, unit after
// unit.  Workgroup w of the nw resident workgroups takes the tiles
// [share_begin(w), share_begin(w + 1)): a fixed share whatever the lengths,
// larger for the older of the two workgroups of a CU.  Each wave works alone
// (no barrier in the kernel): wave v takes KV head hw g + v % hw of group g and,
// of the range's tiles of a unit, those congruent to v / hw modulo 4 / hw, and
// writes one partial per unit its range touches, at (slot w + u, v) - unique,
// as consecutive ranges share at most one unit.  Handing steps out dynamically
// through device-scope atomics (a shared chunk counter, or per-wave claim words
// with stealing) measured slower than these static shares on this part.
// Lane l = 16 lg + lr:
//   score MFMA output: head 4 rg + lg, token lr of the page;
//   value accumulators: head 4 rg + lg, channels 4 lr + n and 64 + 4 lr + n (n = 0..3);
//   loads per tile: K row bytes 8lg..8lg+7 of token lr for each of the 8 pages,
//   the tile's records (one 16-byte chunk per lane);
//   V words of those 8 channels for pages 2lg, 2lg+1.
// Each wave keeps two tiles in flight (the loads of its next tile go out before
// the current one is computed); two workgroups per CU.
// ---------------------------------------------------------------------------
// The last unit u < units with tp[u] <= t (tp[0] = 0 <= t): a 64-way search,
// one round of loads per factor of 64 in the unit count.
__device__ __forceinline__ int find_unit(const int* tp, int units, int64_t t) {
  const int lane = threadIdx.x & 63;
  int a = 0, n = units;  // the answer lies in [a, a + n)
  while (n > 1) {
    const int step = (n + 63) >> 6;
    const bool ok = lane * step < n && tp[a + lane * step] <= t;
    const uint64_t m = __ballot(ok);  // lane 0 always set
    const int last = 63 - __builtin_clzll(m);
    a += last * step;
    n = min(step, n - last * step);
  }
  return a;
}

template <int G, int NG>
__global__ __launch_bounds__(256, 2) void int2_split_kernel(SplitParams p) {
  constexpr int NRG = (G + 3) / 4;  // MFMA row groups of 4 heads
  constexpr bool kRecLds = NRG == 1 && NG <= 2;  // records spread through LDS (see load_tile)
  __shared__ __align__(16) uint8_t smem[4 * NRG * NG * 2048];        // per-wave weight-digit tiles
  __shared__ __align__(16) uint8_t recs[kRecLds ? 4 * NG * 1024 : 16];  // per-wave record staging

  const int hg_per_seq = p.hkv / p.hw;  // KV head groups per sequence
  const int per_seq = hg_per_seq * p.gsub;
  const int units_layer = p.batch * per_seq;
  const int units = p.n_layers * units_layer;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lg = lane >> 4, lr = lane & 15;
  const int ts = 4 / p.hw;  // waves sharing a head (tile stride)
  uint8_t* wt = smem + wave * (NRG * NG * 2048);
  uint8_t* rb = recs + wave * (NG * 1024);
  const int ncb = (p.gw * p.gsub + 3) / 4;
  const int64_t wave_part = (int64_t)p.gw * kPartStride;  // floats of one wave's partial
  // equal shares [T w / nw, T (w + 1) / nw) of the T flattened tiles
  const int64_t T = p.tile_prefix[units];
  const int nw = (int)(T < p.n_wg ? T : p.n_wg);  // at least one tile per share
  const int w = blockIdx.x;

  // unit part [a, e) of the tiles [lo, hi) of the flattened order; false past the range
  auto segment = [&](int u, int64_t lo, int64_t hi, int& a, int& e) {
    const int64_t su = p.tile_prefix[u], su1 = p.tile_prefix[u + 1];
    if (su >= hi) return false;
    a = (int)((lo > su ? lo : su) - su);
    e = (int)((hi < su1 ? hi : su1) - su);
    return true;
  };
  // steps of phase ph in a unit part of tiles [a, e)
  auto steps_of = [&](int a, int e, int ph) { return ((e - a - ph + ts - 1) / ts + 1) >> 1; };

  // Empty partial (m = -inf, l = 0, acc = 0) of one wave.
  auto write_empty = [&](float* dst) {
    for (int i = lane; i < p.gw * kPartStride; i += 64) dst[i] = (i % kPartStride) == 0 ? kNegInf : 0.f;
  };

  // Steps [0, ns) of phase ph, KV head hv of the group, in tiles [a, e) of
  // unit u (indices within the unit); the wave's partial to dst.
  auto run_steps = [&](int ug, int a, int e, int ph, int hv, int ns, float* dst) {
    const int layer = ug / units_layer, u = ug % units_layer;
    const SplitParams pl = layer_params(p, layer);
    const int b = u / per_seq, hs = u % per_seq, hgp = hs / p.gsub, sub = hs % p.gsub;
    const int h = hgp * p.hw + hv;                   // the KV head
    const int hq0 = h * p.gw * p.gsub + sub * p.gw;  // first query head of the unit
    const int n = seq_len_of(p, b);
    const int t_end = n - (n < p.window ? n : p.window);  // history tokens
    const int t_beg = min(p.n_sink, t_end);               // the sinks before it are bf16
    const uint8_t* base_h = pl.pool + (size_t)h * p.block;  // head h's block of page 0
    const uint32_t stride = (uint32_t)(p.hkv * p.block);    // bytes per page

    // score operands prepared once per (sequence, KV head)
    i32x8 qa[NRG];
    int qsc[NRG];
    float qsr[NRG][NG];
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
      const int* src = pl.qop + ((((int64_t)b * p.hkv + h) * ncb + (sub * p.gw) / 4 + rg) * 64 + lane) * 9;
#pragma unroll
      for (int i = 0; i < 8; ++i) qa[rg][i] = src[i];
      qsc[rg] = src[8];
      const bool hv = 4 * rg + lg < p.gw;
      const float* qs = pl.qsum + ((int64_t)b * p.hq + hq0 + (hv ? 4 * rg + lg : 0)) * NG;
#pragma unroll
      for (int jg = 0; jg < NG; ++jg) qsr[rg][jg] = hv ? qs[jg] : 0.f;
    }
    WaveState<NRG, NG> st;
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
      st.m_run[rg] = kNegInf;
      st.l_part[rg] = 0.f;
#pragma unroll
      for (int jg = 0; jg < NG; ++jg) st.az_part[rg][jg] = 0.f;
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) st.acc[rg][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // (the weight-digit tiles need no clearing: every tile writes all their rows)

    // step s: the wave's tiles 2s and 2s + 1, i.e. tiles a + ph + ts k of the
    // unit; a step with one tile computes an empty (all-masked) second one
    const int P0 = 8 * a, P1 = (t_end - 1) >> 4;
    const int ntw = (e - a - ph + ts - 1) / ts;
    const int* btr = p.block_table + (int64_t)b * p.max_pages;
    auto pbase_of = [&](int k) { return P0 + 8 * (ph + ts * k); };
    TileTable tab = table_ready(p, table_load(btr, P0, P1, ph, ts, 0), P0, P1, ph, ts, 0, ntw);
    int raw_next = table_load(btr, P0, P1, ph, ts, 2);
    auto compute = [&](const Tile<NG>& t, int pbase) {
      compute_tile<G, NRG, false, NG, kRecLds>(p, t, pbase, t_beg, t_end, lg, lr, qa, qsc, qsr, wt, rb, st);
    };
    if constexpr (NRG > 1 || NG > 2) {
      // registers for one tile only, its two parts loaded a phase ahead: tile
      // k + 1's K codes and records go out while tile k's values are computed
      // (tile k's K part is dead by then), its V codes while its own scores
      // are.  Past the last step the table is empty and the loads re-read page
      // 0's blocks (cache resident), never computed.
      static_assert(!kRecLds, "the two-part loads read each token's records per lane");
      Tile<NG> t;
      TileWeights<NRG, NG> tw;
      auto phase1 = [&](int pbase) {
        compute_tile<G, NRG, false, NG, false, 1>(p, t, pbase, t_beg, t_end, lg, lr, qa, qsc, qsr, wt, rb, st, &tw);
      };
      auto phase2 = [&] {
        compute_tile<G, NRG, false, NG, false, 2>(p, t, 0, t_beg, t_end, lg, lr, qa, qsc, qsr, wt, rb, st, &tw);
      };
      load_tile_k<NG>(base_h, stride, tab, 0, lg, lr, t);
      load_tile_v<NG>(base_h, stride, tab, 0, lg, lr, t);
      for (int s = 0;; ++s) {
        const int k = 2 * s;
        phase1(pbase_of(k));
        load_tile_k<NG>(base_h, stride, tab, 1, lg, lr, t);
        phase2();
        load_tile_v<NG>(base_h, stride, tab, 1, lg, lr, t);
        phase1(pbase_of(k + 1));
        const bool more = s + 1 < ns;
        tab = table_ready(p, raw_next, P0, P1, ph, ts, k + 2, more ? ntw : 0);
        raw_next = table_load(btr, P0, P1, ph, ts, k + 4);
        load_tile_k<NG>(base_h, stride, tab, 0, lg, lr, t);
        phase2();
        load_tile_v<NG>(base_h, stride, tab, 0, lg, lr, t);
        if (!more) break;
      }
    } else {  // two tiles in flight per wave: tile k + 1's loads go out before tile k is computed
      Tile<NG> ta, tb;
      load_tile<NG, kRecLds>(base_h, stride, tab, 0, lg, lr, ta);
      for (int s = 0;; ++s) {
        const int k = 2 * s;
        load_tile<NG, kRecLds>(base_h, stride, tab, 1, lg, lr, tb);
        compute(ta, pbase_of(k));
        const bool more = s + 1 < ns;
        // past the last step the table is empty: tile k + 2 re-reads page 0's
        // block (cache resident) and is never computed
        tab = table_ready(p, raw_next, P0, P1, ph, ts, k + 2, more ? ntw : 0);
        raw_next = table_load(btr, P0, P1, ph, ts, k + 4);
        load_tile<NG, kRecLds>(base_h, stride, tab, 0, lg, lr, ta);
        compute(tb, pbase_of(k + 1));
        if (!more) break;
      }
    }

    // ---- the wave's partial: lane (lg, lr) holds channels 4 lr .. 4 lr + 3 and
    // 64 + 4 lr .. 64 + 4 lr + 3 of head 4 rg + lg ----
    // (the accumulators are pinned here, with every lane active: otherwise the
    // last tile's value MFMAs could be sunk into the per-lane store branch)
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
      for (int nn = 0; nn < 8; ++nn)
#pragma unroll
        for (int i = 0; i < 4; ++i) st.acc[rg][nn][i] = pin(st.acc[rg][nn][i]);
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
      const float l = row_sum16(st.l_part[rg]);
      // midpoint sums of the groups of this lane's two channel runs
      float az_lo = 0.f, az_hi = 0.f;
#pragma unroll
      for (int jg = 0; jg < NG; ++jg) {
        const float a = row_sum16(st.az_part[rg][jg]);
        az_lo = (NG == 1 || lr * NG / 32 == jg) ? a : az_lo;
        az_hi = (NG == 1 || NG / 2 + lr * NG / 32 == jg) ? a : az_hi;
      }
      const int head = 4 * rg + lg;
      if (head < p.gw) {
        float* d = dst + head * kPartStride;
#pragma unroll
        for (int nn = 0; nn < 8; nn += 2) {
          const float az = nn < 4 ? az_lo : az_hi;
          const float x0 = (st.acc[rg][nn][0] + st.acc[rg][nn][1]) + (st.acc[rg][nn][2] + st.acc[rg][nn][3]) + az;
          const float x1 =
              (st.acc[rg][nn + 1][0] + st.acc[rg][nn + 1][1]) + (st.acc[rg][nn + 1][2] + st.acc[rg][nn + 1][3]) + az;
          const int ch = nn < 4 ? 4 * lr + nn : 64 + 4 * lr + nn - 4;
          *reinterpret_cast<float2*>(d + 2 + ch) = make_float2(x0, x1);
        }
        if (lr == 0) *reinterpret_cast<float2*>(d) = make_float2(st.m_run[rg], l);
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // ---- the workgroup's range: one wave partial per unit it touches, at (w + u, wave) ----
  if (w < nw) {
    const int64_t lo = share_begin(p, T, nw, w), hi = share_begin(p, T, nw, w + 1);
    const int ph = wave / p.hw, hv = wave % p.hw;
    int a, e;
    for (int u = find_unit(p.tile_prefix, units, lo); u < units && segment(u, lo, hi, a, e); ++u) {
      if (e <= a) continue;
      float* dst = p.part + ((int64_t)(w + u) * 4 + wave) * wave_part;
      const int nst = steps_of(a, e, ph);
      if (nst > 0) run_steps(u, a, e, ph, hv, nst, dst);
      else write_empty(dst);
    }
  }
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
      kk[0][s] = load_nt4(blk0 + r * kD + 32 * s + 8 * g);
      kk[1][s] = load_nt4(blk1 + r * kD + 32 * s + 8 * g);
    }
    const uint16_t* vblk = (g >> 1) ? blk1 : blk0;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      vv[c] = load_nt4(vblk + kPage * kD + (16 * c + r) * kPage + 8 * (g & 1));

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
  combine_and_store<G>(cm, cl, cacc, p.part + (((int64_t)b * p.hq + h * G) * p.n_splits + sp) * kPartStride,
                       (int64_t)p.n_splits * kPartStride, G);
}

// ---------------------------------------------------------------------------
// merge: one workgroup per (sequence, group of MH q heads of one KV head);
// MH (1, 2 or 4, dividing G) is chosen on the host so that the grid still has
// about two workgroups per CU.  The 4 / MH waves of a head share its partials
// (wave s of the head takes partials s, s + 4 / MH, ...).  A pass of a wave
// covers up to NP of its partials, NP (8, 16 or 32) the smallest that holds
// them all when it can: the (m, l) of partial i0 + i sit on lane i, whose
// address the wave reads out of that lane for the accumulator loads
// (channels lane and lane + 64), and every load of a pass is issued before
// any is used; the passes keep a running max.  The short kernel's time is its
// serial instruction count, so nothing is executed for partials a wave does
// not have beyond the pass's padding.  The waves of a head meet in LDS
// (log-sum-exp over their (m, l, acc)).  INT2: the workgroup's R_V tile
// (loaded once for its MH heads) un-rotates every head, then the first wave of
// each head merges the window and sink chunk partials and normalises.  A head
// with no position at all gets zeros.
// ---------------------------------------------------------------------------
constexpr int kMergeWin = 4;    // window / sink chunk partials held in registers (a 128-token window)
constexpr int kMergeHeads = 4;  // q heads per workgroup at most

__device__ __forceinline__ const float* readlane_ptr(const float* p, int lane) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, lane), hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), lane);
  return reinterpret_cast<const float*>(((uint64_t)hi << 32) | lo);
}

template <int MH, bool INT2>
__global__ __launch_bounds__(256) void merge_kernel(SplitParams p0, int gq) {
  constexpr int LW = MH == 1 ? 2 : MH == 2 ? 1 : 0, WPH = 1 << LW;  // waves per head
  const int layer = blockIdx.y / p0.batch, b = blockIdx.y % p0.batch;
  const SplitParams p = layer_params(p0, layer);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = wave >> LW, sub = wave & (WPH - 1);  // head slot, this wave's share of its partials
  const bool lead = sub == 0;  // merges the window partials and stores the head
  const int hq = blockIdx.x * MH + m, h = hq / gq;  // one KV head for the workgroup (MH divides G)
  constexpr bool int2 = INT2;  // INT2 cache (partials in the rotated basis) or bf16 cache
  __shared__ float accs[4][kD];  // per wave: its (unnormalised) accumulator
  __shared__ float mls[4][2];    // per wave: its running max and sum
  __shared__ float o1p[MH][16][kD + 4];

  // The loads that depend on nothing else go out first, so that they are in
  // flight while the partials' places are looked up.
  // R_V tile (INT2): thread (cg, jg) takes channels 8cg..8cg+7 of rows 8jg..8jg+7
  const int cg = tid & 15, jg = tid >> 4;
  uint4 rv[8];
  if (int2) {
    const uint16_t* r = p.r_v + ((int64_t)h * kD + 8 * jg) * kD + 8 * cg;
#pragma unroll
    for (int j = 0; j < 8; ++j) rv[j] = *reinterpret_cast<const uint4*>(r + j * kD);
  }
  // window / sink chunk partials (INT2, first wave of a head): channels lane
  // and lane + 64 of the first kMergeWin chunks
  const float* wp = p.wpart + ((int64_t)b * p.hq + hq) * p.n_wchunks * kPartStride;
  const int nwc = int2 && lead ? p.n_wchunks : 0;
  // (m, l) are loaded per lane (lane & 1) and read out only where they are
  // used: as uniform values they would be scalar loads waited for at once
  float wv0[kMergeWin], wv1[kMergeWin], wml[kMergeWin];
#pragma unroll
  for (int cc = 0; cc < kMergeWin; ++cc) {
    const float* wc = wp + (cc < nwc ? cc : 0) * kPartStride;  // in the workspace even when unused
    wv0[cc] = wc[2 + lane];
    wv1[cc] = wc[2 + 64 + lane];
    wml[cc] = wc[lane & 1];
  }

  // partials of this head: INT2 - the wave partials (w + u, v) of the ts
  // waves v of this head in each workgroup w whose tile range touches unit u,
  // at p.part + ((4 (w + u) + v) gw + g) 130 (partial s: workgroup w_lo + s / ts,
  // wave hv + hw (s % ts)); bf16 - the splits of the sequence (partial s at
  // base + s 130)
  const float* base;
  int ns;
  int64_t stride;
  int ts = 1, hw = 1, w0 = 0;
  if (int2) {
    const int jq = hq % gq, hsub = jq / p.gw, g = jq % p.gw;
    const int per_seq = (p.hkv / p.hw) * p.gsub;
    const int u = (layer * p.batch + b) * per_seq + (h / p.hw) * p.gsub + hsub;
    const int64_t T = p.tile_prefix[p.n_layers * p.batch * per_seq];
    const int64_t nw = T < p.n_wg ? T : p.n_wg;
    const int64_t su = p.tile_prefix[u], su1 = p.tile_prefix[u + 1];
    int64_t w_lo = 0;
    ns = 0;
    // (T > 0 holds whenever su1 > su; testing it keeps T's load beside those
    // of su and su1 instead of a round trip later)
    if (su1 > su && T > 0) {  // workgroup of tile t: ((t + 1) nw - 1) / T
      w_lo = share_owner(p, T, (int)nw, su);
      ns = (int)(share_owner(p, T, (int)nw, su1 - 1) - w_lo + 1);
    }
    hw = p.hw;
    ts = 4 / hw;
    w0 = (int)(w_lo + u);
    base = p.part + ((int64_t)h % hw * p.gw + g) * kPartStride;
    stride = (int64_t)p.gw * kPartStride;
    ns *= ts;
  } else {
    const int n = seq_len_of(p, b);
    ns = (n + p.split - 1) / p.split;
    base = p.part + ((int64_t)b * p.hq + hq) * p.n_splits * kPartStride;
    stride = kPartStride;
  }
  const int tsh = ts == 4 ? 2 : ts == 2 ? 1 : 0;  // ts = 4 / hw: 1, 2 or 4
  // this wave's partials: s = sub + WPH i, i < nmine
  const int nmine = ns > sub ? (ns - sub + WPH - 1) >> LW : 0;

  float M = kNegInf, acc0 = 0.f, acc1 = 0.f, lsum = 0.f;  // M, lsum: the same on every lane
  auto pass = [&](int i0, auto np) {
    constexpr int NP = decltype(np)::value;
    const int cnt = min(NP, nmine - i0);
    // lane i: the wave's partial i0 + i, clamped (no branch around a load)
    const int s = sub + ((i0 + min(lane, cnt - 1)) << LW);
    const float* pl = base + (int64_t)(int2 ? 4 * (w0 + (s >> tsh)) + hw * (s & (ts - 1)) : s) * stride;
    const float2 mlv = *reinterpret_cast<const float2*>(pl);
    float x0[NP], x1[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const float* pk = readlane_ptr(pl, k);
      x0[k] = pk[2 + lane];
      x1[k] = pk[2 + 64 + lane];
    }
    const float ml = lane < cnt ? mlv.x : kNegInf;
    const float ll = lane < cnt ? mlv.y : 0.f;
    const float Mn = fmaxf(M, wave_max64(ml));
    const float alpha = M == kNegInf ? 0.f : exp2f(M - Mn);
    const float f = ml == kNegInf ? 0.f : exp2f(ml - Mn);  // weight of partial i0 + lane, 0 past cnt
    acc0 *= alpha;
    acc1 *= alpha;
    lsum = lsum * alpha + wave_sum64(f * ll);
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      // lanes past cnt carry weight 0 and the (finite) accumulator of a valid partial
      const float fk = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(f), k));
      acc0 = fmaf(fk, x0[k], acc0);
      acc1 = fmaf(fk, x1[k], acc1);
    }
    M = Mn;
  };
  if (nmine > 0) {
    if (nmine <= 8) {
      pass(0, std::integral_constant<int, 8>{});
    } else if (nmine <= 16) {
      pass(0, std::integral_constant<int, 16>{});
    } else {
      for (int i0 = 0; i0 < nmine; i0 += 32) pass(i0, std::integral_constant<int, 32>{});
    }
  }
  accs[wave][lane] = acc0;
  accs[wave][lane + 64] = acc1;
  if (lane == 0) {
    mls[wave][0] = M;
    mls[wave][1] = lsum;
  }
  __syncthreads();
  // the waves of head slot mm: weights relative to the head's max, and its (M, l)
  auto head_weights = [&](int mm, float* f, float& Mh, float& lh) {
    Mh = kNegInf;
#pragma unroll
    for (int s = 0; s < WPH; ++s) Mh = fmaxf(Mh, mls[(mm << LW) + s][0]);
    lh = 0.f;
#pragma unroll
    for (int s = 0; s < WPH; ++s) {
      const float ms = mls[(mm << LW) + s][0];
      f[s] = ms == kNegInf ? 0.f : exp2f(ms - Mh);
      lh = fmaf(f[s], mls[(mm << LW) + s][1], lh);
    }
  };
  float* dst = p.out + ((int64_t)b * p.hq + hq) * kD;
  if (!int2) {
    if (lead) {
      float f[WPH], Mh, lh;
      head_weights(m, f, Mh, lh);
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int s = 0; s < WPH; ++s) {
        a0 = fmaf(f[s], accs[wave + s][lane], a0);
        a1 = fmaf(f[s], accs[wave + s][lane + 64], a1);
      }
      dst[lane] = lh > 0.f ? a0 / lh : 0.f;
      dst[lane + 64] = lh > 0.f ? a1 / lh : 0.f;
    }
    return;
  }
  // o1 = R_V^T a1 of every head from the register tile, partial sums over 8 rows per thread
#pragma unroll
  for (int mm = 0; mm < MH; ++mm) {
    float f[WPH], Mh, lh;
    head_weights(mm, f, Mh, lh);
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float aj = 0.f;
#pragma unroll
      for (int s = 0; s < WPH; ++s) aj = fmaf(f[s], accs[(mm << LW) + s][8 * jg + j], aj);
      const uint32_t u[4] = {rv[j].x, rv[j].y, rv[j].z, rv[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] = fmaf(bf16lo(u[i]), aj, o[2 * i]);
        o[2 * i + 1] = fmaf(bf16hi(u[i]), aj, o[2 * i + 1]);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) o1p[mm][jg][8 * cg + i] = o[i];
  }
  __syncthreads();
  if (!lead) return;
  float fh[WPH], Mh, lh;
  head_weights(m, fh, Mh, lh);
  float o1[2] = {0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    o1[0] += o1p[m][k][lane];
    o1[1] += o1p[m][k][lane + 64];
  }
  float wm[kMergeWin], wl[kMergeWin];
#pragma unroll
  for (int cc = 0; cc < kMergeWin; ++cc) {
    const bool ok = cc < nwc;
    wm[cc] = ok ? __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(wml[cc]), 0)) : kNegInf;
    wl[cc] = ok ? __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(wml[cc]), 1)) : 0.f;
    wv0[cc] = ok ? wv0[cc] : 0.f;
    wv1[cc] = ok ? wv1[cc] : 0.f;
  }
  float Mx = Mh;
#pragma unroll
  for (int cc = 0; cc < kMergeWin; ++cc) Mx = fmaxf(Mx, wm[cc]);
  for (int cc = kMergeWin; cc < nwc; ++cc) Mx = fmaxf(Mx, wp[cc * kPartStride]);
  const float f1 = Mh == kNegInf ? 0.f : exp2f(Mh - Mx);
  float den = f1 * lh, num0 = f1 * o1[0], num1 = f1 * o1[1];
#pragma unroll
  for (int cc = 0; cc < kMergeWin; ++cc) {
    const float f2 = wm[cc] == kNegInf ? 0.f : exp2f(wm[cc] - Mx);
    den = fmaf(f2, wl[cc], den);
    num0 = fmaf(f2, wv0[cc], num0);
    num1 = fmaf(f2, wv1[cc], num1);
  }
  for (int cc = kMergeWin; cc < nwc; ++cc) {
    const float* wc = wp + cc * kPartStride;
    const float m2 = wc[0];
    const float f2 = m2 == kNegInf ? 0.f : exp2f(m2 - Mx);
    den = fmaf(f2, wc[1], den);
    num0 = fmaf(f2, wc[2 + lane], num0);
    num1 = fmaf(f2, wc[2 + 64 + lane], num1);
  }
  dst[lane] = den > 0.f ? num0 / den : 0.f;
  dst[lane + 64] = den > 0.f ? num1 / den : 0.f;
}

template <int G>
int launch_decode(bool int2, const SplitParams& sp, const uint16_t* r_k, int batch, hipStream_t s, TimedLaunch tl,
                  const AppendParams* ap) {
  if (int2) {
    // z = 0: rotated query and its MFMA operands, the tile prefix; z > 0: the
    // bf16 window chunks; with ap (the fused step) two more planes append the
    // newest tokens' keys and values
    const dim3 grid(batch * sp.n_layers, sp.hkv, 1 + sp.n_wchunks + (ap ? 2 : 0));
    if (!ap) {
      prep_kernel<G, 0><<<grid, 256, 0, s>>>(sp, r_k, AppendParams{});
    } else {
      switch (sp.ng) {
        case 1: prep_kernel<G, 1><<<grid, 256, 0, s>>>(sp, r_k, *ap); break;
        case 2: prep_kernel<G, 2><<<grid, 256, 0, s>>>(sp, r_k, *ap); break;
        default: prep_kernel<G, 4><<<grid, 256, 0, s>>>(sp, r_k, *ap); break;
      }
    }
    if (hipGetLastError() != hipSuccess) return OSCAR_EHIP;
  }
  if (int2) {
    constexpr int GW = G > 8 ? 8 : (G < 4 ? 4 : G);  // whole-token groups; 4 heads with finer groups
    auto go = [&](auto kernel) { launch(kernel, dim3(sp.n_wg), dim3(256), s, tl, sp); };
    switch (sp.ng) {
      case 1: go(int2_split_kernel<GW, 1>); break;
      case 2: go(int2_split_kernel<4, 2>); break;
      default: go(int2_split_kernel<4, 4>); break;
    }
  } else {
    launch(bf16_split_kernel<G>, dim3(sp.n_splits, sp.hkv, batch), dim3(256), s, tl, sp);
  }
  if (hipGetLastError() != hipSuccess) return OSCAR_EHIP;
  // heads per merge workgroup: the R_V tile is loaded once for all of them,
  // as long as about two workgroups per CU remain
  int mh = 1;
  const int64_t rows = (int64_t)batch * sp.n_layers;
  while (2 * mh <= kMergeHeads && 2 * mh <= G && rows * sp.hq / (2 * mh) >= 2 * (int64_t)device_cu_count())
    mh *= 2;
  const dim3 mgrid(sp.hq / mh, (unsigned)rows);
  auto merge = [&](auto kernel) { kernel<<<mgrid, 256, 0, s>>>(sp, G); };
  if (int2) {
    switch (mh) {
      case 1: merge(merge_kernel<1, true>); break;
      case 2: merge(merge_kernel<2, true>); break;
      default: merge(merge_kernel<4, true>); break;
    }
  } else {
    switch (mh) {
      case 1: merge(merge_kernel<1, false>); break;
      case 2: merge(merge_kernel<2, false>); break;
      default: merge(merge_kernel<4, false>); break;
    }
  }
  return hipGetLastError() == hipSuccess ? OSCAR_OK : OSCAR_EHIP;
}

}  // namespace

// Validation, split plan, workspace layout and the three launches of a decode
// call (declared in common.h).
int decode_common(bool int2, const oscar_shape* shape, const uint16_t* r_k, const uint16_t* r_v,
                  const uint16_t* q, int32_t batch, const int32_t* seq_lens, int32_t max_seq_len,
                  const int32_t* block_table, int32_t max_pages_per_seq, const uint8_t* pool,
                  const uint16_t* kv_pool, int64_t n_pages, const uint16_t* win_k, const uint16_t* win_v,
                  float* out, void* workspace, size_t workspace_bytes, void* stream, int n_layers, TimedLaunch tl,
                  bool int2_only, const uint16_t* k_new, const uint16_t* v_new) {
  int st = check_shape(shape);
  if (st != OSCAR_OK) return st;
  if (check_events(tl) != OSCAR_OK) return OSCAR_EINVAL;
  if (batch < 1 || max_seq_len < 0 || max_pages_per_seq < 1 || n_pages < 1) return OSCAR_EINVAL;
  if (n_layers < 1 || (!int2 && n_layers != 1) || (int64_t)n_layers * batch > 65535) return OSCAR_EINVAL;
  if (!q || !seq_lens || !block_table || !out || !workspace) return OSCAR_EINVAL;
  if (int2 && (!r_k || !r_v || !pool)) return OSCAR_EINVAL;
  if (int2 && shape->window + shape->n_sink > 0 && (!win_k || !win_v)) return OSCAR_EINVAL;
  if (!int2 && !kv_pool) return OSCAR_EINVAL;
  if ((int64_t)max_seq_len > (int64_t)max_pages_per_seq * kPage) return OSCAR_ENOSPACE;
  const bool fused = k_new != nullptr || v_new != nullptr;  // the decode step: append, then attend
  if (fused && (!int2 || n_layers != 1 || !k_new || !v_new)) return OSCAR_EINVAL;
  const int gqa = shape->n_q_heads / shape->n_kv_heads;
  const int n_cu = device_cu_count();
  const SplitPlan plan = plan_splits(batch, shape->n_kv_heads, gqa, max_seq_len, n_cu);
  const WorkspaceLayout wl = workspace_layout(batch, shape->n_q_heads, shape->n_kv_heads, shape->window, shape->n_sink,
                                              kD / shape->group_size, plan, n_cu, n_layers, int2_only);
  if (workspace_bytes < wl.total) return OSCAR_ENOSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return OSCAR_EINVAL;
  // rows are read as 16-byte vectors
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(r_k) | reinterpret_cast<uintptr_t>(r_v) |
       reinterpret_cast<uintptr_t>(pool) | reinterpret_cast<uintptr_t>(kv_pool) |
       reinterpret_cast<uintptr_t>(win_k) | reinterpret_cast<uintptr_t>(win_v) |
       reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15)
    return OSCAR_EINVAL;

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
  sp.tile_prefix = reinterpret_cast<int*>(ws + wl.tile_prefix);
  sp.out = out;
  sp.n_pages = n_pages;
  sp.batch = batch;
  sp.hq = shape->n_q_heads;
  sp.hkv = shape->n_kv_heads;
  sp.max_pages = max_pages_per_seq;
  sp.max_len = max_seq_len;
  sp.window = int2 ? shape->window : 0;
  sp.n_sink = int2 ? shape->n_sink : 0;
  sp.ring = sp.window + sp.n_sink;
  sp.n_wwin = (sp.window + kWinChunk - 1) / kWinChunk;
  sp.n_wchunks = sp.n_wwin + (sp.n_sink + kWinChunk - 1) / kWinChunk;
  sp.split = plan.split;
  sp.n_splits = plan.n_splits;
  // INT2: at most 8 (4 with finer groups) query heads per merge unit (register
  // budget of the MFMA tiles); G < 4 runs the 4-head instantiation masking the
  // missing heads
  sp.gw = int2 ? int2_unit_heads(gqa, kD / shape->group_size) : gqa;
  sp.gsub = gqa / sp.gw;
  sp.n_wg = int2 ? split_wg_count(gqa, n_cu) : 0;
  sp.hw = split_heads_per_wg(shape->n_kv_heads);
  // the older workgroup of each CU takes 1.5 times the share of the younger:
  // a sweep of 20:20 .. 26:14 at 100K context was fastest at 24:16 (split
  // 93.8 us against 98.1 us with equal shares)
  sp.wf = 24;
  sp.ws = 16;
  sp.hf = sp.n_wg / 2;
  sp.block = block_bytes(shape->group_size);
  sp.ng = kD / shape->group_size;
  // per-layer strides (layer-major stacking of every per-layer buffer)
  sp.n_layers = n_layers;
  sp.ls_q = (int64_t)batch * sp.hq * kD;
  sp.ls_out = (int64_t)batch * sp.hq * kD;
  sp.ls_rot = (int64_t)sp.hkv * kD * kD;
  sp.ls_pool = n_pages * sp.hkv * sp.block;
  sp.ls_win = (int64_t)batch * sp.ring * sp.hkv * kD;
  sp.ls_qsum = (int64_t)(align256((size_t)batch * sp.hq * sp.ng * sizeof(float)) / sizeof(float));
  sp.ls_qop = (int64_t)(align256((size_t)batch * sp.hkv * ((gqa + 3) / 4) * 64 * 9 * sizeof(int)) / sizeof(int));
  {
    const size_t nwp = (size_t)batch * sp.hq * sp.n_wchunks;
    sp.ls_wpart = (int64_t)(align256((nwp > 0 ? nwp : 1) * kPartStride * sizeof(float)) / sizeof(float));
  }
  sp.scale_log2 = kLog2e / sqrtf((float)kD);
  // the fused step's append: token b of k_new / v_new at position
  // seq_lens[b] - 1 of sequence b (seq_idx and pos implicit)
  AppendParams ap{};
  if (fused) {
    sp.k_new = k_new;
    sp.v_new = v_new;
    ap.r[0] = r_k;
    ap.r[1] = r_v;
    ap.x[0] = k_new;
    ap.x[1] = v_new;
    ap.win[0] = const_cast<uint16_t*>(win_k);
    ap.win[1] = const_cast<uint16_t*>(win_v);
    ap.block_table = block_table;
    ap.len_after = seq_lens;
    ap.pool = const_cast<uint8_t*>(pool);
    ap.block = sp.block;
    ap.n_tokens = batch;
    ap.n_pages = n_pages;
    ap.batch = batch;
    ap.max_pages = max_pages_per_seq;
    ap.hkv = sp.hkv;
    ap.window = sp.window;
    ap.tiles_per_wg = 1;
    ap.n_sink = sp.n_sink;
    ap.ring = sp.ring;
    ap.max_len = max_seq_len;
  }
  const AppendParams* app = fused ? &ap : nullptr;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (shape->n_q_heads / shape->n_kv_heads) {
    case 1: return launch_decode<1>(int2, sp, r_k, batch, s, tl, app);
    case 2: return launch_decode<2>(int2, sp, r_k, batch, s, tl, app);
    case 4: return launch_decode<4>(int2, sp, r_k, batch, s, tl, app);
    case 8: return launch_decode<8>(int2, sp, r_k, batch, s, tl, app);
    case 16: return launch_decode<16>(int2, sp, r_k, batch, s, tl, app);
  }
  return OSCAR_EUNSUPPORTED;
}

namespace {

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
  return oscar_decode_layers_workspace_bytes(shape, 1, batch, max_seq_len);
}

extern "C" size_t oscar_decode_layers_workspace_bytes(const oscar_shape* shape, int32_t n_layers, int32_t batch,
                                                      int32_t max_seq_len) {
  using namespace oscar;
  if (check_shape(shape) != OSCAR_OK || batch < 1 || max_seq_len < 0 || n_layers < 1) return 0;
  const int n_cu = device_cu_count();
  return workspace_layout(batch, shape->n_q_heads, shape->n_kv_heads, shape->window, shape->n_sink,
                          kD / shape->group_size,
                          plan_splits(batch, shape->n_kv_heads, shape->n_q_heads / shape->n_kv_heads, max_seq_len,
                                      n_cu),
                          n_cu, n_layers)
      .total;
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

extern "C" int oscar_decode_attn_layers(const oscar_shape* shape, int32_t n_layers, const uint16_t* r_k,
                                        const uint16_t* r_v, const uint16_t* q, int32_t batch,
                                        const int32_t* seq_lens, int32_t max_seq_len, const int32_t* block_table,
                                        int32_t max_pages_per_seq, const uint8_t* pool, int64_t n_pages,
                                        const uint16_t* win_k, const uint16_t* win_v, float* out, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  return oscar::decode_common(true, shape, r_k, r_v, q, batch, seq_lens, max_seq_len, block_table,
                              max_pages_per_seq, pool, nullptr, n_pages, win_k, win_v, out, workspace,
                              workspace_bytes, stream, n_layers);
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

extern "C" int oscar_decode_attn_timed(const oscar_shape* shape, const uint16_t* r_k, const uint16_t* r_v,
                                       const uint16_t* q, int32_t batch, const int32_t* seq_lens,
                                       int32_t max_seq_len, const int32_t* block_table, int32_t max_pages_per_seq,
                                       const uint8_t* pool, int64_t n_pages, const uint16_t* win_k,
                                       const uint16_t* win_v, float* out, void* workspace, size_t workspace_bytes,
                                       void* stream, void* ev_start, void* ev_stop) {
  return oscar::decode_common(true, shape, r_k, r_v, q, batch, seq_lens, max_seq_len, block_table,
                              max_pages_per_seq, pool, nullptr, n_pages, win_k, win_v, out, workspace,
                              workspace_bytes, stream, 1,
                              oscar::TimedLaunch{static_cast<hipEvent_t>(ev_start), static_cast<hipEvent_t>(ev_stop)});
}
extern "C" int oscar_decode_step(const oscar_shape* shape, const uint16_t* r_k, const uint16_t* r_v,
                                 const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q, int32_t batch,
                                 const int32_t* seq_lens, int32_t max_seq_len, const int32_t* block_table,
                                 int32_t max_pages_per_seq, uint8_t* pool, int64_t n_pages, uint16_t* win_k,
                                 uint16_t* win_v, float* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!k_new || !v_new) return OSCAR_EINVAL;
  return oscar::decode_common(true, shape, r_k, r_v, q, batch, seq_lens, max_seq_len, block_table,
                              max_pages_per_seq, pool, nullptr, n_pages, win_k, win_v, out, workspace,
                              workspace_bytes, stream, 1, oscar::TimedLaunch{nullptr, nullptr}, false, k_new, v_new);
}
extern "C" int oscar_decode_step_timed(const oscar_shape* shape, const uint16_t* r_k, const uint16_t* r_v,
                                       const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q,
                                       int32_t batch, const int32_t* seq_lens, int32_t max_seq_len,
                                       const int32_t* block_table, int32_t max_pages_per_seq, uint8_t* pool,
                                       int64_t n_pages, uint16_t* win_k, uint16_t* win_v, float* out,
                                       void* workspace, size_t workspace_bytes, void* stream, void* ev_start,
                                       void* ev_stop) {
  if (!k_new || !v_new) return OSCAR_EINVAL;
  return oscar::decode_common(true, shape, r_k, r_v, q, batch, seq_lens, max_seq_len, block_table,
                              max_pages_per_seq, pool, nullptr, n_pages, win_k, win_v, out, workspace,
                              workspace_bytes, stream, 1,
                              oscar::TimedLaunch{static_cast<hipEvent_t>(ev_start), static_cast<hipEvent_t>(ev_stop)},
                              false, k_new, v_new);
}

extern "C" int oscar_bf16_decode_attn_timed(const oscar_shape* shape, const uint16_t* q, int32_t batch,
                                            const int32_t* seq_lens, int32_t max_seq_len, const int32_t* block_table,
                                            int32_t max_pages_per_seq, const uint16_t* kv_pool, int64_t n_pages,
                                            float* out, void* workspace, size_t workspace_bytes, void* stream,
                                            void* ev_start, void* ev_stop) {
  return oscar::decode_common(false, shape, nullptr, nullptr, q, batch, seq_lens, max_seq_len, block_table,
                              max_pages_per_seq, nullptr, kv_pool, n_pages, nullptr, nullptr, out, workspace,
                              workspace_bytes, stream, 1,
                              oscar::TimedLaunch{static_cast<hipEvent_t>(ev_start), static_cast<hipEvent_t>(ev_stop)});
}
