// Decode attention without a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  The decode's scratch regions (rotated
// query operands, split partials, window partials, tile prefix) live in a fixed
// device array of this library instead of a caller workspace.
//
// The array's device address is looked up once per device, with that device
// current (hipGetSymbolAddress), and only that address is handed to the
// kernels: in host code the array's name is a host-side stand-in, not a device
// address.  Every region the kernels read is written earlier in the same call,
// so nothing needs clearing between calls.  Every call on a device shares that
// device's array: calls that overlap on one device race.
#include <mutex>

#include "common.h"

namespace oscar {
namespace {

constexpr size_t kScratchBytes = (size_t)OSCAR_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of the scratch array, or nullptr on failure.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace oscar

extern "C" size_t oscar_decode_noalloc_scratch_bytes(const oscar_shape* shape, int32_t batch, int32_t max_seq_len) {
  using namespace oscar;
  if (check_shape(shape) != OSCAR_OK || batch < 1 || max_seq_len < 0) return 0;
  const int n_cu = device_cu_count();
  return workspace_layout(batch, shape->n_q_heads, shape->n_kv_heads, shape->window, shape->n_sink,
                          kD / shape->group_size,
                          plan_splits(batch, shape->n_kv_heads, shape->n_q_heads / shape->n_kv_heads, max_seq_len,
                                      n_cu),
                          n_cu, 1, true)
      .total;
}

extern "C" int oscar_decode_attn_noalloc(const oscar_shape* shape, const uint16_t* r_k, const uint16_t* r_v,
                                         const uint16_t* q, int32_t batch, const int32_t* seq_lens,
                                         int32_t max_seq_len, const int32_t* block_table, int32_t max_pages_per_seq,
                                         const uint8_t* pool, int64_t n_pages, const uint16_t* win_k,
                                         const uint16_t* win_v, float* out, void* stream) {
  using namespace oscar;
  const int st = check_shape(shape);
  if (st != OSCAR_OK) return st;
  if (batch < 1 || max_seq_len < 0) return OSCAR_EINVAL;
  if (oscar_decode_noalloc_scratch_bytes(shape, batch, max_seq_len) > kScratchBytes) return OSCAR_ENOSPACE;
  void* ws = scratch_on_current_device();
  if (!ws) return OSCAR_EHIP;
  return decode_common(true, shape, r_k, r_v, q, batch, seq_lens, max_seq_len, block_table, max_pages_per_seq, pool,
                       nullptr, n_pages, win_k, win_v, out, ws, kScratchBytes, stream, 1,
                       TimedLaunch{nullptr, nullptr}, true);
}
