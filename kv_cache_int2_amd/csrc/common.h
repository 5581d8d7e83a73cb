// Internal helpers shared by the library's translation units (host and device).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cstddef>
#include <cstdint>

#include "oscar.h"

namespace oscar {

constexpr int kD = 128;          // head dim
constexpr int kPage = 16;        // tokens per page
// K codes, V codes, records: the record {Ks, Kz, Vs, Vz} fp16 of group j of
// token t sits at kMeta + 8 (NG t + j), NG = 128 / group size
constexpr int kKCodes = 0, kVCodes = 512, kMeta = 1024;
inline int block_bytes(int group_size) { return kMeta + 8 * kPage * (kD / group_size); }
constexpr int kMaxWindow = 1024;
constexpr int kWinChunk = 32;  // window tokens per decode workgroup (one window partial each)
constexpr int kPartStride = 2 + kD;  // (m, l, acc[128]) per (batch, q head, split)
constexpr int kMaxSplit = 2048;      // tokens per split at most: 16 tiles of 128, 4 per wave

// Host-side shape check.  Returns OSCAR_OK or an error.
inline int check_shape(const oscar_shape* s) {
  if (!s) return OSCAR_EINVAL;
  if (s->n_kv_heads < 1 || s->n_q_heads < 1 || s->window < 0) return OSCAR_EINVAL;
  if (s->head_dim != kD || s->page_size != kPage) return OSCAR_EUNSUPPORTED;
  if (s->group_size != 32 && s->group_size != 64 && s->group_size != kD) return OSCAR_EUNSUPPORTED;
  if (s->n_q_heads % s->n_kv_heads) return OSCAR_EINVAL;
  int g = s->n_q_heads / s->n_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16) return OSCAR_EUNSUPPORTED;
  if (s->n_sink < 0) return OSCAR_EINVAL;
  if (s->window > kMaxWindow || s->n_sink > kMaxWindow) return OSCAR_EUNSUPPORTED;
  return OSCAR_OK;
}

// Split plan of the decode: every (sequence, KV head) history is cut into
// `n_splits` page-aligned ranges of `split` tokens; one workgroup per range.
struct SplitPlan {
  int split;     // tokens per split (multiple of 64)
  int n_splits;  // splits for the longest sequence
};

// Workgroups of the INT2 split kernel resident per compute unit: two 4-wave
// workgroups (its register budget, two tiles in flight per wave at G <= 4).
inline int split_wgs_per_cu(int /*gqa*/) { return 2; }

// The longest split (multiple of 64 in [256, 2048]) that still gives every
// resident workgroup slot of the device a range of the longest sequence.  A
// sweep at 100K context (B = 8) found the kernel throughput-bound: 1024- to
// 4096-token splits all land within 6 % of each other, the longest being
// fastest (fewest partials and per-workgroup prologues).
inline SplitPlan plan_splits(int batch, int n_kv_heads, int gqa, int max_tokens, int n_cu) {
  const long gsub = gqa > 8 ? gqa / 8 : 1;
  const long units = (long)batch * n_kv_heads * gsub;
  const long slots = (long)(n_cu > 0 ? n_cu : 256) * split_wgs_per_cu(gqa);
  long best = 256;
  for (long s = kMaxSplit; s >= 256; s -= 64) {
    if (units * (((long)max_tokens + s - 1) / s) >= slots) {
      best = s;
      break;
    }
  }
  const int n = max_tokens <= 0 ? 1 : (int)((max_tokens + best - 1) / best);
  return SplitPlan{(int)best, n < 1 ? 1 : n};
}

// Compute units of the current device (the split plan depends on it).
int device_cu_count();

// KV heads a workgroup of the INT2 split kernel reads side by side (its 4
// waves take one head each, or share one head round robin): adjacent heads'
// blocks of a page are adjacent in the pool, so 4 of them make one 4.6 KB read.
inline int split_heads_per_wg(int n_kv_heads) { return n_kv_heads % 4 == 0 ? 4 : (n_kv_heads % 2 == 0 ? 2 : 1); }

// Resident workgroups of the persistent INT2 split kernel.
// Query heads of one INT2 merge unit: up to 8 at whole-token groups, up to 4
// with finer groups (the per-group scores and weights of 8 heads exceed the
// split kernel's register budget; a KV head with more query heads is then read
// once per unit).
inline int int2_unit_heads(int gqa, int ng) {
  const int cap = ng > 1 ? 4 : 8;
  return gqa > cap ? cap : gqa;
}

inline int split_wg_count(int gqa, int n_cu) { return (n_cu > 0 ? n_cu : 256) * split_wgs_per_cu(gqa); }

// Workspace layout (bytes, each region 256-aligned):
//   qsum         float [B][Hq][ng]                  sums of the rotated query over each quantisation group
//   qop          int   [B][Hkv][ceil(G/4)][64][9]   per-lane fp8 score operand (8 dwords) + E8M0 scale
//   part         float  bf16 comparator: [B][Hq][n_splits][130] split partials (m, l, acc[128]);
//                       INT2: [n_wg + units][4][gw][130] partials of the persistent workgroups'
//                       waves (units = B Hkv / hw x Hq / (Hkv gw); hw KV heads per workgroup)
//   wpart        float [B][Hq][ceil(W/32) + ceil(n_sink/32)][130]  window, then sink chunk partials
//   tile_prefix  int   [units + 1]                  first history tile of each merge unit
inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }
struct WorkspaceLayout {
  size_t qsum, qop, part, wpart, tile_prefix, total;
};
// n_layers > 1 (INT2 only): the per-layer regions (qsum, qop, wpart) repeat
// for every layer; the split partials and the tile prefix cover the units of
// all layers.  The stride of a per-layer region is its size rounded to 256 B.
// int2_only: the partials region sized for the INT2 decode alone (the bf16
// comparator's split partials left out).
inline WorkspaceLayout workspace_layout(int batch, int n_q_heads, int n_kv_heads, int window, int n_sink, int ng,
                                        const SplitPlan& p, int n_cu, int n_layers = 1, bool int2_only = false) {
  const int gqa = n_q_heads / n_kv_heads;
  const size_t g4 = (size_t)((gqa + 3) / 4);
  const size_t gw = (size_t)int2_unit_heads(gqa, ng);
  const size_t L = (size_t)n_layers;
  const size_t units = L * batch * n_q_heads / (gw * (size_t)split_heads_per_wg(n_kv_heads));
  const size_t part_bf16 = int2_only ? 0 : (size_t)batch * n_q_heads * p.n_splits * kPartStride;
  const size_t n_wg = (size_t)split_wg_count(gqa, n_cu);
  const size_t part_int2 = (n_wg + units) * 4 * gw * kPartStride;
  WorkspaceLayout w{};
  w.qsum = 0;
  w.qop = w.qsum + L * align256((size_t)batch * n_q_heads * ng * sizeof(float));
  w.part = w.qop + L * align256((size_t)batch * n_kv_heads * g4 * 64 * 9 * sizeof(int));
  w.wpart = w.part + align256((part_bf16 > part_int2 ? part_bf16 : part_int2) * sizeof(float));
  const size_t n_wchunks = (size_t)((window + kWinChunk - 1) / kWinChunk + (n_sink + kWinChunk - 1) / kWinChunk);
  // at least one partial: the merge reads chunk 0 of its head unconditionally
  const size_t n_wparts = (size_t)batch * n_q_heads * n_wchunks;
  w.tile_prefix = w.wpart + L * align256((n_wparts > 0 ? n_wparts : 1) * kPartStride * sizeof(float));
  w.total = w.tile_prefix + align256((units + 1) * sizeof(int));
  return w;
}

// Event pair attached to the dispatch of a call's main kernel (both null when
// the call is not timed).  The kernel is launched with hipExtLaunchKernelGGL,
// which stamps the events at the dispatch's own start and end, so the pair
// spans the kernel and nothing queued around it.
struct TimedLaunch {
  hipEvent_t start, stop;
};
// OSCAR_OK when both events or neither are given.
int check_events(const TimedLaunch& t);

// Launches kernel on stream s; with events, through hipExtLaunchKernelGGL so
// that they are stamped at the dispatch's own start and end.  Without events
// the plain launch is used: attaching events delays the dispatch's start by
// about 6 us behind the preceding kernel on the same stream, a cost that only
// timed calls should pay.
template <typename Kernel, typename... Args>
inline void launch(Kernel kernel, dim3 grid, dim3 block, hipStream_t s, const TimedLaunch& tl, Args... args) {
  if (tl.start)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, tl.start, tl.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
}

// One decode call (INT2 with int2 set, else the bf16 comparator): argument
// checks, split plan, workspace layout (int2_only: without the comparator's
// partials) and the launches on `stream`.  Returns an oscar_status.
int decode_common(bool int2, const oscar_shape* shape, const uint16_t* r_k, const uint16_t* r_v,
                  const uint16_t* q, int32_t batch, const int32_t* seq_lens, int32_t max_seq_len,
                  const int32_t* block_table, int32_t max_pages_per_seq, const uint8_t* pool,
                  const uint16_t* kv_pool, int64_t n_pages, const uint16_t* win_k, const uint16_t* win_v,
                  float* out, void* workspace, size_t workspace_bytes, void* stream, int n_layers = 1,
                  TimedLaunch tl = TimedLaunch{nullptr, nullptr}, bool int2_only = false,
                  const uint16_t* k_new = nullptr, const uint16_t* v_new = nullptr);

}  // namespace oscar

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)
namespace oscar {

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {  // finite x: round to nearest even
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float h2f(uint16_t b) {
  _Float16 h = __builtin_bit_cast(_Float16, b);
  return (float)h;
}
__device__ __forceinline__ uint16_t f2h_bits(float x) {  // round to nearest even
  _Float16 h = (_Float16)x;
  return __builtin_bit_cast(uint16_t, h);
}

constexpr float kLog2e = 1.4426950408889634f;

// Lane permutations inside a 16-lane DPP row (one VALU operand modifier each).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xf, 0xf, true);
}
constexpr int kDppSwap1 = 0xB1;       // quad_perm [1, 0, 3, 2]
constexpr int kDppSwap2 = 0x4E;       // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // lane i <- 7 - i within each 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <- 15 - i within the row

// Max / sum over the 16 lanes of a row, every lane receiving the same result
// (each step combines two disjoint, already reduced groups of lanes, and
// a + b == b + a, so all lanes compute bitwise the same value).
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp_f32<kDppSwap1>(x));
  x = fmaxf(x, dpp_f32<kDppSwap2>(x));
  x = fmaxf(x, dpp_f32<kDppHalfMirror>(x));
  return fmaxf(x, dpp_f32<kDppMirror>(x));
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f32<kDppSwap1>(x);
  x += dpp_f32<kDppSwap2>(x);
  x += dpp_f32<kDppHalfMirror>(x);
  return x + dpp_f32<kDppMirror>(x);
}

// OR / min / max over the 4 rows of 16 lanes of a wave (v_permlane16_swap and
// v_permlane32_swap exchange whole rows): every lane receives the combination
// of its own and the 3 partner lanes 16, 32 and 48 apart.
__device__ __forceinline__ uint32_t or_rows(uint32_t d) {
  auto a = __builtin_amdgcn_permlane16_swap(d, d, false, false);
  d = a[0] | a[1];
  auto b = __builtin_amdgcn_permlane32_swap(d, d, false, false);
  return b[0] | b[1];
}
__device__ __forceinline__ float min_rows(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fminf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float max_rows(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row_min16(float x) {
  x = fminf(x, dpp_f32<kDppSwap1>(x));
  x = fminf(x, dpp_f32<kDppSwap2>(x));
  x = fminf(x, dpp_f32<kDppHalfMirror>(x));
  return fminf(x, dpp_f32<kDppMirror>(x));
}

__device__ __forceinline__ float sum_rows(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// max / sum over the 64 lanes of a wave (the same bits on every lane)
__device__ __forceinline__ float wave_max64(float x) {
  x = row_max16(x);
  return max_rows(x);
}
__device__ __forceinline__ float wave_sum64(float x) { return sum_rows(row_sum16(x)); }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

}  // namespace oscar
#endif
