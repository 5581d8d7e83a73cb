// The append kernel: new K/V tokens rotated, quantised and packed into the
// paged INT2 cache (and the bf16 window ring); the device code it runs is in
// append_core.h.
#include "append_core.h"

namespace oscar {
namespace {

// ONE: every workgroup has a single iteration (tiles_per_wg == 1, as for
// decode-time appends); its X rows then also go out before R is staged.
// Otherwise each wave's X rows go through its LDS buffer: the first tile's
// loads are issued before R is staged, each later tile's as soon as the
// previous tile's rotation is done, so they arrive while it is quantised and
// stored.
template <int NG, bool ONE>
__global__ __launch_bounds__(kAppendThreads) __attribute__((amdgpu_waves_per_eu(4))) void append_kernel(AppendParams p) {
  __shared__ uint4 r_lds[128 * 16];
  __shared__ uint4 x_lds[ONE ? 1 : kAppendWaves * kAppendTiles * 4 * 64];
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
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint4* xbuf = x_lds + (ONE ? 0 : wave * kAppendTiles * 4 * 64);
  auto tile0 = [&](int it) {
    return ((int64_t)blockIdx.x * p.tiles_per_wg + it) * kAppendTokens + wave * 16 * kAppendTiles;
  };
  // one copy of the body per kind (K or V), so that no value crosses a
  // branch on it
  auto body = [&](auto kind_c) {
    constexpr int KIND = decltype(kind_c)::value;
    if constexpr (ONE) {
      append_one<KIND, NG, kAppendThreads, false>(p, r_lds, h, tile0(0), lane);
      return;
    }
    // the first tile's token indices and rows go out before the rotation is
    // staged
    TileIdx in;
    uint4 xv[kAppendTiles][4];
    const bool any = tile0(0) < p.n_tokens;  // uniform across the wave
    if (any) {
      load_idx(p, tile0(0), lane, in);
      dma_x<KIND>(p, tile0(0), h, lane, xbuf);
    }
    RStage<kAppendThreads> rs;
    r_load<kAppendThreads>(p.r[KIND], h, rs);
    if (any) {
#pragma unroll
      for (int j = 0; j < kAppendTiles; ++j) in.pl[j] = lookup(p, in.b[j], in.ps[j]);
    }
    r_store<kAppendThreads>(r_lds, rs);
    __syncthreads();
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
      // the next tile of this workgroup's run, or this one again after its
      // last (loaded, never used), so that no load depends on a branch
      const bool more = it + 1 < p.tiles_per_wg && tile0(it + 1) < p.n_tokens;
      const int64_t tn = more ? tile0(it + 1) : t0;
      load_idx(p, tn, lane, nxt);
      read_x(lane, xbuf, xv);
      process_tiles<KIND, NG>(p, r_lds, in, xv, t0, h, lane, [&] { dma_x<KIND>(p, tn, h, lane, xbuf); });
    }
    // the last loads into LDS land before the workgroup's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  if (kind == 0)
    body(std::integral_constant<int, 0>{});
  else
    body(std::integral_constant<int, 1>{});
}

}  // namespace
}  // namespace oscar

namespace oscar {
namespace {

int append_impl(const oscar_shape* shape, int32_t n_layers, const uint16_t* r_k, const uint16_t* r_v,
                const uint16_t* k_new, const uint16_t* v_new, int64_t n_tokens, const int32_t* seq_idx,
                const int32_t* pos, int32_t batch, const int32_t* block_table, int32_t max_pages_per_seq,
                const int32_t* seq_len_after, uint8_t* pool, int64_t n_pages, uint16_t* win_k, uint16_t* win_v,
                void* stream, TimedLaunch tl) {
  int st = check_shape(shape);
  if (st != OSCAR_OK) return st;
  if (check_events(tl) != OSCAR_OK) return OSCAR_EINVAL;
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
  // One launch-wide round of workgroups: as many as the device holds at once
  // (2 per CU), each taking an equal run of 128-token iterations of one KV
  // head, K or V, so the rotation is staged once per run and no partly filled
  // second round trails the first (measured with 4-wave workgroups: 76 us for
  // 65536 tokens x 8 heads, against 82 us with 4 iterations per workgroup).
  const int64_t tiles = (n_tokens + kAppendTokens - 1) / kAppendTokens;  // iterations per (head, K|V)
  const int64_t slots = 2 * (int64_t)device_cu_count();
  const int64_t streams = 2 * (int64_t)p.hkv * n_layers;
  const int64_t tpw = (tiles * streams + slots - 1) / slots;
  p.tiles_per_wg = (int)(tpw < 1 ? 1 : (tpw > tiles ? tiles : (tpw > (1 << 30) ? (1 << 30) : tpw)));
  dim3 grid((unsigned)((tiles + p.tiles_per_wg - 1) / p.tiles_per_wg), (unsigned)p.hkv, 2 * (unsigned)n_layers);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool one = p.tiles_per_wg == 1;
  auto go = [&](auto kernel) { launch(kernel, grid, dim3(kAppendThreads), s, tl, p); };
  switch (kD / shape->group_size) {
    case 1: one ? go(append_kernel<1, true>) : go(append_kernel<1, false>); break;
    case 2: one ? go(append_kernel<2, true>) : go(append_kernel<2, false>); break;
    default: one ? go(append_kernel<4, true>) : go(append_kernel<4, false>); break;
  }
  return hipGetLastError() == hipSuccess ? OSCAR_OK : OSCAR_EHIP;
}

}  // namespace
}  // namespace oscar

extern "C" int oscar_quantize_append_layers(const oscar_shape* shape, int32_t n_layers, const uint16_t* r_k,
                                            const uint16_t* r_v, const uint16_t* k_new, const uint16_t* v_new,
                                            int64_t n_tokens, const int32_t* seq_idx, const int32_t* pos,
                                            int32_t batch, const int32_t* block_table, int32_t max_pages_per_seq,
                                            const int32_t* seq_len_after, uint8_t* pool, int64_t n_pages,
                                            uint16_t* win_k, uint16_t* win_v, void* stream) {
  return oscar::append_impl(shape, n_layers, r_k, r_v, k_new, v_new, n_tokens, seq_idx, pos, batch, block_table,
                            max_pages_per_seq, seq_len_after, pool, n_pages, win_k, win_v, stream,
                            oscar::TimedLaunch{nullptr, nullptr});
}

extern "C" int oscar_quantize_append(const oscar_shape* shape, const uint16_t* r_k, const uint16_t* r_v,
                                     const uint16_t* k_new, const uint16_t* v_new, int64_t n_tokens,
                                     const int32_t* seq_idx, const int32_t* pos, int32_t batch,
                                     const int32_t* block_table, int32_t max_pages_per_seq,
                                     const int32_t* seq_len_after, uint8_t* pool, int64_t n_pages,
                                     uint16_t* win_k, uint16_t* win_v, void* stream) {
  return oscar::append_impl(shape, 1, r_k, r_v, k_new, v_new, n_tokens, seq_idx, pos, batch, block_table,
                            max_pages_per_seq, seq_len_after, pool, n_pages, win_k, win_v, stream,
                            oscar::TimedLaunch{nullptr, nullptr});
}

extern "C" int oscar_quantize_append_timed(const oscar_shape* shape, const uint16_t* r_k, const uint16_t* r_v,
                                           const uint16_t* k_new, const uint16_t* v_new, int64_t n_tokens,
                                           const int32_t* seq_idx, const int32_t* pos, int32_t batch,
                                           const int32_t* block_table, int32_t max_pages_per_seq,
                                           const int32_t* seq_len_after, uint8_t* pool, int64_t n_pages,
                                           uint16_t* win_k, uint16_t* win_v, void* stream, void* ev_start,
                                           void* ev_stop) {
  return oscar::append_impl(shape, 1, r_k, r_v, k_new, v_new, n_tokens, seq_idx, pos, batch, block_table,
                            max_pages_per_seq, seq_len_after, pool, n_pages, win_k, win_v, stream,
                            oscar::TimedLaunch{static_cast<hipEvent_t>(ev_start), static_cast<hipEvent_t>(ev_stop)});
}
