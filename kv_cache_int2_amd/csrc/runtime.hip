// Measurement helpers, the device's compute-unit count and status strings: a
// streaming copy kernel (the known-size reference for HBM traffic counters), a
// streaming read kernel over whole or scattered blocks (the in-session HBM
// ceilings of the decode's access shapes), a timed wait kernel that holds a
// stream without touching memory, and thin wrappers of HIP events for the
// timed entry points.  The library keeps no timing state of its own: the
// caller creates the events and passes them to each timed call.
#include "common.h"

namespace oscar {
namespace {

__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

// Read probe.  The blocks (cpb 16-byte chunks each) are concatenated in table
// order and workgroup w reads the chunks [w N / nw, (w + 1) N / nw) of that
// stream, 8 loads of 16 bytes in flight per thread; chunk c lies in block
// c / cpb of the table (found in fp64, exact after one correction since the
// quotient is off by less than one).  Without a table, chunk c is src[c].  The
// XOR of everything a workgroup read goes to sink[w], so no load can be dropped.
constexpr int kReadUnroll = 8;
template <bool NT>  // NT: the loads carry the non-temporal hint, as the decode's do
__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ src, const int32_t* __restrict__ blocks,
                                                   int64_t n_blocks, int cpb, double inv_cpb,
                                                   uint32_t* __restrict__ sink) {
  const int64_t N = n_blocks * cpb;
  const int64_t lo = N * blockIdx.x / gridDim.x, hi = N * (blockIdx.x + 1) / gridDim.x;
  uint32_t x = 0;
  for (int64_t c0 = lo + threadIdx.x; c0 < hi; c0 += 256 * kReadUnroll) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int j = 0; j < kReadUnroll; ++j) {
      const int64_t c = c0 + 256 * j;
      const int64_t cc = c < hi ? c : hi - 1;  // a clamped duplicate past the range is read but not used
      int64_t at = cc;
      if (blocks) {
        int64_t blk = (int64_t)((double)cc * inv_cpb);
        int64_t off = cc - blk * cpb;
        if (off < 0) {
          blk -= 1;
          off += cpb;
        } else if (off >= cpb) {
          blk += 1;
          off -= cpb;
        }
        at = (int64_t)blocks[blk] * cpb + off;
      }
      if constexpr (NT) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + at));
        v[j] = make_uint4(t[0], t[1], t[2], t[3]);
      } else {
        v[j] = src[at];
      }
    }
#pragma unroll
    for (int j = 0; j < kReadUnroll; ++j)
      x ^= c0 + 256 * j < hi ? (v[j].x ^ v[j].y ^ v[j].z ^ v[j].w) : 0u;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
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

int check_events(const TimedLaunch& t) {
  return (t.start == nullptr) == (t.stop == nullptr) ? OSCAR_OK : OSCAR_EINVAL;
}

}  // namespace oscar

extern "C" int oscar_event_create(void** event) {
  if (!event) return OSCAR_EINVAL;
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return OSCAR_EHIP;
  *event = e;
  return OSCAR_OK;
}

extern "C" int oscar_event_destroy(void* event) {
  if (!event) return OSCAR_EINVAL;
  return hipEventDestroy(static_cast<hipEvent_t>(event)) == hipSuccess ? OSCAR_OK : OSCAR_EHIP;
}

extern "C" int oscar_event_elapsed_ms(void* start, void* stop, float* ms) {
  if (!start || !stop || !ms) return OSCAR_EINVAL;
  if (hipEventSynchronize(static_cast<hipEvent_t>(stop)) != hipSuccess) return OSCAR_EHIP;
  return hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop)) == hipSuccess
             ? OSCAR_OK
             : OSCAR_EHIP;
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

namespace oscar {
namespace {
int hbm_read(bool nt, const void* src, int64_t block_bytes, const int32_t* blocks, int64_t n_blocks, uint32_t* sink,
             int32_t n_workgroups, void* stream) {
  if (!src || !sink || block_bytes < 16 || (block_bytes & 15) || block_bytes > (1 << 20) || n_blocks < 0 ||
      n_workgroups < 0 || n_workgroups > OSCAR_READ_MAX_WORKGROUPS || (reinterpret_cast<uintptr_t>(src) & 15))
    return OSCAR_EINVAL;
  if (n_blocks == 0) return OSCAR_OK;
  const int cpb = (int)(block_bytes / 16);
  if (n_blocks > ((int64_t)1 << 40) / cpb) return OSCAR_EINVAL;
  const int wg = n_workgroups > 0 ? n_workgroups : 8 * device_cu_count();
  auto kernel = nt ? read_kernel<true> : read_kernel<false>;
  kernel<<<(unsigned)wg, 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(static_cast<const uint4*>(src), blocks,
                                                                         n_blocks, cpb, 1.0 / (double)cpb, sink);
  return hipGetLastError() == hipSuccess ? OSCAR_OK : OSCAR_EHIP;
}
}  // namespace
}  // namespace oscar

extern "C" int oscar_hbm_read(const void* src, int64_t block_bytes, const int32_t* blocks, int64_t n_blocks,
                              uint32_t* sink, int32_t n_workgroups, void* stream) {
  return oscar::hbm_read(false, src, block_bytes, blocks, n_blocks, sink, n_workgroups, stream);
}

extern "C" int oscar_hbm_read_nt(const void* src, int64_t block_bytes, const int32_t* blocks, int64_t n_blocks,
                                 uint32_t* sink, int32_t n_workgroups, void* stream) {
  return oscar::hbm_read(true, src, block_bytes, blocks, n_blocks, sink, n_workgroups, stream);
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
