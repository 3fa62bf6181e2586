// Gather-read ceiling probe (measurement only; built as libspdec_probe.so,
// apart from libspdec.so and its C ABI).
//
// Streams a list of equal-size blocks at arbitrary byte offsets from one or
// two bases, exactly as the library's streaming kernels walk their lists
// (every wave owns one contiguous range of list entries, reads the entries'
// offsets 64 at a time, one per lane, with the next window's offsets in
// flight, and covers each block with 16-byte non-temporal loads), and does
// nothing with the data except fold it into one word per wave. Timed on the
// same lists as the kernels (the sparse decode's kept K and V pages, the
// scoring pass's page summaries), it gives the HBM rate a gather of that
// shape reaches on the device, which the kernels' rates are set against.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kWave = 64;
constexpr int kThreads = 256;
constexpr int kInFlight = 8;         // 16-byte loads per lane in flight
constexpr int kSinkWords = 1 << 16;  // one folded word per wave, modulo this

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 load_nt(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// S = 16-byte segments per block.
template <int S>
__global__ __launch_bounds__(kThreads) void gather_probe_kernel(const char* __restrict__ b0,
                                                                const char* __restrict__ b1,
                                                                const int64_t* __restrict__ off, int64_t n,
                                                                uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x % kWave;
  const int64_t nw = (int64_t)gridDim.x * (kThreads / kWave);
  const int64_t w = (int64_t)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  const int64_t per = (n + nw - 1) / nw;
  const int64_t i0 = min(n, w * per), i1 = min(n, i0 + per);
  uint32_t acc = 0;
  int64_t cur = off[min(i0 + lane, n - 1)];
  for (int64_t wb = i0; wb < i1; wb += kWave) {
    const int64_t nxt = off[min(wb + kWave + lane, n - 1)];  // next window, in flight
    const int nb = (int)min<int64_t>(kWave, i1 - wb);
    const int nseg = nb * S;
    for (int e0 = 0; e0 < nseg; e0 += kWave * kInFlight) {
      u32x4 v0[kInFlight], v1[kInFlight];
      bool ok[kInFlight];
#pragma unroll
      for (int k = 0; k < kInFlight; ++k) {
        const int e = e0 + k * kWave + lane;
        ok[k] = e < nseg;
        const int blk = min(e / S, nb - 1);
        const int64_t o = __shfl(cur, blk) + (int64_t)(e % S) * 16;
        v0[k] = load_nt(b0 + o);
        if (b1 != nullptr) v1[k] = load_nt(b1 + o);
      }
#pragma unroll
      for (int k = 0; k < kInFlight; ++k) {
        if (ok[k]) {
          acc ^= v0[k].x ^ v0[k].y ^ v0[k].z ^ v0[k].w;
          if (b1 != nullptr) acc ^= v1[k].x ^ v1[k].y ^ v1[k].z ^ v1[k].w;
        }
      }
    }
    cur = nxt;
  }
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) acc ^= __shfl_xor(acc, o);
  if (lane == 0) sink[w % kSinkWords] = acc;
}

template <int S>
hipError_t launch(const char* b0, const char* b1, const int64_t* off, int64_t n, uint32_t* sink, hipStream_t s) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(&gather_probe_kernel<S>),
                                                     kThreads, 0);
  if (e != hipSuccess) return e;
  const int grid = cus * (per_cu > 0 ? per_cu : 1);
  hipLaunchKernelGGL((gather_probe_kernel<S>), dim3(grid), dim3(kThreads), 0, s, b0, b1, off, n, sink);
  return hipGetLastError();
}

}  // namespace

// Reads n blocks of block_bytes (a power of two from 512 to 16384) at byte
// offsets off[0 .. n) (device int64, each a multiple of 16 and the block
// inside the base's allocation) from base0 and, when base1 is not null, from
// base1 at the same offsets. sink: device uint32 [65536], overwritten. Returns
// 0, -1 for bad arguments (nothing launched), -4 for a launch failure.
extern "C" int spdec_probe_gather(const void* base0, const void* base1, const int64_t* off, int64_t n,
                                  int block_bytes, uint32_t* sink, hipStream_t stream) {
  if (base0 == nullptr || off == nullptr || sink == nullptr || n < 1) return -1;
  const char* b0 = static_cast<const char*>(base0);
  const char* b1 = static_cast<const char*>(base1);
  hipStream_t s = stream;
  hipError_t e;
  switch (block_bytes) {
    case 512: e = launch<32>(b0, b1, off, n, sink, s); break;
    case 1024: e = launch<64>(b0, b1, off, n, sink, s); break;
    case 2048: e = launch<128>(b0, b1, off, n, sink, s); break;
    case 4096: e = launch<256>(b0, b1, off, n, sink, s); break;
    case 8192: e = launch<512>(b0, b1, off, n, sink, s); break;
    case 16384: e = launch<1024>(b0, b1, off, n, sink, s); break;
    default: return -1;
  }
  return e == hipSuccess ? 0 : -4;
}

extern "C" int spdec_probe_sink_words(void) { return kSinkWords; }
