// Measurement helpers, the device's compute-unit count and status strings: a
// streaming copy kernel (HBM probe and the known-size reference for HBM traffic
// counters), a timed wait kernel that holds a stream without touching memory,
// and opt-in event pairs attached to the dispatch of the main kernel of each
// append / decode call.
#include <vector>

#include "common.h"

namespace oscar {
namespace {

struct Timing {
  bool on = false;
  int capacity = 0;
  int used = 0;
  std::vector<hipEvent_t> start, stop;
  std::vector<int> kind;
};
Timing g_timing;

__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

// One wave that returns once `ticks` of the constant-rate wall clock have
// passed, sleeping between reads; at most `max_iter` sleeps, so it also ends
// should the clock not advance.
__global__ __launch_bounds__(64) void wait_kernel(uint64_t ticks, int64_t max_iter) {
  const uint64_t t0 = wall_clock64();
  for (int64_t i = 0; i < max_iter; ++i) {
    if (wall_clock64() - t0 >= ticks) break;
    __builtin_amdgcn_s_sleep(32);
  }
}

}  // namespace

int device_cu_count() {
  // cached per device: an attribute query per decode call would be a needless
  // runtime round trip
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
  if (dev < 64) cached[dev] = n;
  return n;
}

TimedLaunch timing_events(int kind) {
  TimedLaunch t{nullptr, nullptr};
  if (!g_timing.on || g_timing.used >= g_timing.capacity) return t;
  const int slot = g_timing.used++;
  g_timing.kind[slot] = kind;
  t.start = g_timing.start[slot];
  t.stop = g_timing.stop[slot];
  return t;
}

}  // namespace oscar

extern "C" int oscar_timing_begin(int32_t capacity) {
  using oscar::g_timing;
  if (capacity < 1 || g_timing.on) return OSCAR_EINVAL;
  g_timing.start.assign(capacity, nullptr);
  g_timing.stop.assign(capacity, nullptr);
  g_timing.kind.assign(capacity, 0);
  for (int i = 0; i < capacity; ++i) {
    if (hipEventCreate(&g_timing.start[i]) != hipSuccess || hipEventCreate(&g_timing.stop[i]) != hipSuccess)
      return OSCAR_EHIP;
  }
  g_timing.capacity = capacity;
  g_timing.used = 0;
  g_timing.on = true;
  return OSCAR_OK;
}

extern "C" int oscar_timing_end(float* ms, int32_t* kinds, int32_t capacity, int32_t* n) {
  using oscar::g_timing;
  if (!g_timing.on) return OSCAR_EINVAL;
  int status = OSCAR_OK;
  int k = 0;
  for (int i = 0; i < g_timing.used; ++i) {
    if (hipEventSynchronize(g_timing.stop[i]) != hipSuccess) {
      status = OSCAR_EHIP;
      continue;
    }
    float t = 0.f;
    if (hipEventElapsedTime(&t, g_timing.start[i], g_timing.stop[i]) != hipSuccess) status = OSCAR_EHIP;
    if (ms && kinds && k < capacity) {
      ms[k] = t;
      kinds[k] = g_timing.kind[i];
      ++k;
    }
  }
  if (n) *n = k;
  for (int i = 0; i < g_timing.capacity; ++i) {
    (void)hipEventDestroy(g_timing.start[i]);
    (void)hipEventDestroy(g_timing.stop[i]);
  }
  g_timing = oscar::Timing{};
  return status;
}

extern "C" int oscar_hbm_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || (bytes & 15) || ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15))
    return OSCAR_EINVAL;
  if (bytes == 0) return OSCAR_OK;
  const int64_t n = (int64_t)(bytes / 16);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  oscar::copy_kernel<<<(unsigned)blocks, 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4*>(src), static_cast<uint4*>(dst), n);
  return hipGetLastError() == hipSuccess ? OSCAR_OK : OSCAR_EHIP;
}

extern "C" int oscar_gpu_wait(int64_t microseconds, void* stream) {
  if (microseconds < 0 || microseconds > 10000000) return OSCAR_EINVAL;
  if (microseconds == 0) return OSCAR_OK;
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return OSCAR_EHIP;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz < 1) return OSCAR_EHIP;
  const uint64_t ticks = (uint64_t)microseconds * (uint64_t)khz / 1000u;
  // a sleep of 32 x 64 clocks lasts >= 0.5 us below 4 GHz: 64 sleeps per us are ample
  oscar::wait_kernel<<<1, 64, 0, reinterpret_cast<hipStream_t>(stream)>>>(ticks, 64 * microseconds + 64);
  return hipGetLastError() == hipSuccess ? OSCAR_OK : OSCAR_EHIP;
}

extern "C" const char* oscar_strerror(int status) {
  switch (status) {
    case OSCAR_OK: return "ok";
    case OSCAR_EINVAL: return "invalid argument";
    case OSCAR_EUNSUPPORTED: return "unsupported shape";
    case OSCAR_EHIP: return "HIP runtime or launch failure";
    case OSCAR_ENOSPACE: return "workspace too small or sequence longer than the block table";
    case OSCAR_EIO: return "file could not be opened, read or written";
    case OSCAR_EFORMAT: return "not a rotation file of this format, damaged, or not matching the shape";
  }
  return "unknown status";
}
