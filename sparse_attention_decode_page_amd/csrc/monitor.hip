// Streaming tail monitor of the per-token acceptance (Sparrow project page,
// "Control Study 1": training stays stable while the lower 5th percentile of
// the per-token mismatch over the rollout's tokens stays above a threshold,
// 0.86 in its takeaway).
//
// The monitor keeps the per-token acceptance values of a rollout in a device
// ring of `capacity` values (the most recent ones once more are appended), so
// every decode step appends its batch on the device and the statistics are
// taken on the device too, with no host round trip:
//   * append: the new values are written at the ring's head and the 64-bit
//     count of values appended so far advances (one workgroup for a decode
//     step's batch);
//   * stats: the mean (fp64, fixed order) and the exact lower 5th percentile
//     with linear interpolation between the order statistics at rank
//     0.05 * (n - 1), n = min(count, capacity) (numpy's default). The
//     percentile is a radix select over the values' 32-bit order-preserving
//     keys: three histogram passes of 11, 11 and 10 bits across the whole
//     device (integer atomics: exact and order-free), each pass restricted
//     to the keys whose leading bits the previous passes fixed; the last
//     kernel finds the order statistic at rank floor(0.05 (n - 1)), takes the
//     next one (when no tie covers it) as the next occupied bin of the last
//     histogram or the smallest larger key the third pass saw past the
//     fixed prefix, and interpolates in fp64 with one rounding.
// Every kernel reads the previous passes' histograms itself, so a call is four
// launches and no host work; the final one-workgroup kernel clears the
// histograms, so the workspace is ready for the next call.
#include <limits.h>

#include "common.h"
#include "launch.h"

namespace spdec {

namespace {

constexpr int kMonThreads = 256;
constexpr int kMonPer = 16;                             // values per thread per workgroup
constexpr int kMonTile = kMonThreads * kMonPer;         // values per workgroup
constexpr int kMonBins0 = 2048, kMonBins1 = 2048, kMonBins2 = 1024;  // 11 + 11 + 10 bits
constexpr int kMonAppendThreads = 1024;
constexpr int kMonPass1Groups = 128;

// Workspace layout (64-bit words first):
//   [0]            count of values appended so far
//   [8 .. 8+G)     fp64 partial sums of the first pass, one per workgroup
//   [8+G .. 8+2G)  per workgroup of the third pass: the smallest keys above
//                  the lower order statistic's 22-bit prefix, inside and past
//                  its 11-bit leading bin (as complements, 0 = none)
// then three u32 histograms (zero between calls), then the ring of floats.
struct MonLayout {
  unsigned long long* count;
  double* partial;
  unsigned int* next_min;
  unsigned int* h0;
  unsigned int* h1;
  unsigned int* h2;
  float* ring;
};

constexpr size_t kMonMaxGroups = (size_t)1 << 16;  // capacity <= kMonMaxGroups * kMonTile

size_t mon_header_bytes() {
  return (8 + 2 * kMonMaxGroups) * sizeof(unsigned long long) +
         (size_t)(kMonBins0 + kMonBins1 + kMonBins2) * sizeof(unsigned int);
}

MonLayout mon_layout(void* ws) {
  MonLayout m;
  unsigned long long* w = reinterpret_cast<unsigned long long*>(ws);
  m.count = w;
  m.partial = reinterpret_cast<double*>(w + 8);
  m.next_min = reinterpret_cast<unsigned int*>(w + 8 + kMonMaxGroups);
  m.h0 = reinterpret_cast<unsigned int*>(w + 8 + 2 * kMonMaxGroups);
  m.h1 = m.h0 + kMonBins0;
  m.h2 = m.h1 + kMonBins1;
  m.ring = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + ((mon_header_bytes() + 255) & ~(size_t)255));
  return m;
}

// Order-preserving key of a float (-0 and +0 share one key; NaN never occurs:
// acceptance values are finite).
__device__ __forceinline__ uint32_t mon_key(float x) { return score_key(x); }
__device__ __forceinline__ float mon_value(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ int mon_n(const MonLayout& m, int capacity) {
  const unsigned long long c = *m.count;
  return c < (unsigned long long)capacity ? (int)c : capacity;
}

// Value i of a batch is appended value c + i (c = values appended before), at
// slot (c + i) mod capacity. Of a batch longer than the ring only its last
// capacity values are written (the earlier ones would be overwritten by the
// same batch). UPDATE: this (single) workgroup also advances the count;
// otherwise a grid writes and mon_count_kernel advances it afterwards.
template <bool UPDATE>
__global__ __launch_bounds__(kMonAppendThreads) void mon_append_kernel(MonLayout m, int capacity,
                                                                       const float* __restrict__ alpha, int n) {
  const unsigned long long c = *m.count;
  const int head = (int)(c % (unsigned long long)capacity);
  const int first = n > capacity ? n - capacity : 0;
  const int stride = gridDim.x * kMonAppendThreads;
  for (int i = first + (int)(blockIdx.x * kMonAppendThreads + threadIdx.x); i < n; i += stride) {
    const int slot = (int)(((long long)head + i) % capacity);
    m.ring[slot] = alpha[i];
  }
  if (UPDATE) {
    __syncthreads();
    if (threadIdx.x == 0) *m.count = c + (unsigned long long)n;
  }
}

__global__ void mon_count_kernel(MonLayout m, int n) {
  if (threadIdx.x == 0) *m.count += (unsigned long long)n;
}

// Inclusive scan of per-thread counts over the block (fixed order).
__device__ __forceinline__ unsigned int block_scan_u32(unsigned int x, unsigned int* s_tot) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const unsigned int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) s_tot[wave] = x;
  __syncthreads();
  unsigned int base = 0;
  for (int w = 0; w < wave; ++w) base += s_tot[w];
  __syncthreads();
  return base + x;
}

// The bin of histogram h (NB bins) holding rank `rank` (0-based) and the count
// of keys in the bins below it; every thread gets the same answer.
template <int NB>
__device__ void find_bin(const unsigned int* h, unsigned int rank, int* s_bin, unsigned int* s_below,
                         unsigned int* s_tot, int* bin, unsigned int* below) {
  constexpr int per = NB / kMonThreads;  // bins per thread, in order
  unsigned int c[per];
  unsigned int tot = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    c[i] = h[threadIdx.x * per + i];
    tot += c[i];
  }
  const unsigned int incl = block_scan_u32(tot, s_tot);
  unsigned int run = incl - tot;
  if (run <= rank && rank < incl) {  // exactly one thread holds the rank
#pragma unroll
    for (int i = 0; i < per; ++i) {
      if (rank < run + c[i]) {
        *s_bin = threadIdx.x * per + i;
        *s_below = run;
        break;
      }
      run += c[i];
    }
  }
  __syncthreads();
  *bin = *s_bin;
  *below = *s_below;
}

// Rank of the lower order statistic: floor(0.05 (n - 1)), in fp64 as the
// interpolation position is computed.
__device__ __forceinline__ unsigned int lower_rank(int n) {
  return (unsigned int)floor(0.05 * (double)(n - 1));
}

// Pass 0 (P = 0), 1, 2: histogram of the key digit of pass P over the keys
// whose leading digits equal those fixed by the earlier passes (found here
// from the earlier histograms), workgroup g taking tiles g, g + G, ...;
// pass 0 also writes the workgroup's fp64 sum, pass 2 the smallest keys past
// the fixed 22-bit prefix (inside and past its leading 11-bit bin), from
// which the final pass takes the next order statistic when no tie covers it.
template <int P>
__global__ __launch_bounds__(kMonThreads) void mon_hist_kernel(MonLayout m, int capacity) {
  constexpr int NB = P == 2 ? kMonBins2 : 2048;
  __shared__ unsigned int s_h[NB];
  __shared__ unsigned int s_tot[kMonThreads / kWave];
  __shared__ int s_bin;
  __shared__ unsigned int s_below;
  __shared__ double s_sum[kMonThreads / kWave];
  __shared__ unsigned int s_min[2][kMonThreads / kWave];
  const int n = mon_n(m, capacity);
  if ((int)blockIdx.x * kMonTile >= n) return;
  for (int i = threadIdx.x; i < NB; i += kMonThreads) s_h[i] = 0u;
  int bin0 = 0, bin1 = 0;
  if (P >= 1) {
    const unsigned int rank = lower_rank(n);
    unsigned int below0;
    find_bin<kMonBins0>(m.h0, rank, &s_bin, &s_below, s_tot, &bin0, &below0);
    if (P >= 2) {
      unsigned int below1;
      find_bin<kMonBins1>(m.h1, rank - below0, &s_bin, &s_below, s_tot, &bin1, &below1);
    }
  }
  __syncthreads();
  double sum = 0.0;
  // Pass 0: the leading 11 bits (sign, exponent, 2 mantissa bits) of values
  // in a narrow range take few distinct bins, so each thread counts runs of
  // equal bins in a register and adds a run to LDS when its bin changes.
  uint32_t run_bin = 0u, run_cnt = 0u;
  uint32_t min_in = UINT_MAX, min_past = UINT_MAX;  // pass 2
  const uint32_t prefix22 = ((uint32_t)bin0 << 11) | (uint32_t)bin1;
  for (int base = blockIdx.x * kMonTile; base < n; base += gridDim.x * kMonTile) {
#pragma unroll
    for (int j = 0; j < kMonPer; ++j) {
      const int i = base + j * kMonThreads + (int)threadIdx.x;
      if (i < n) {
        const float v = m.ring[i];
        const uint32_t k = mon_key(v);
        if (P == 0) {
          const uint32_t bin = k >> 21;
          sum += (double)v;
          if (bin != run_bin) {
            if (run_cnt != 0u) atomicAdd(&s_h[run_bin], run_cnt);
            run_bin = bin;
            run_cnt = 0u;
          }
          ++run_cnt;
        } else if (P == 1) {
          if ((int)(k >> 21) == bin0) atomicAdd(&s_h[(k >> 10) & 2047u], 1u);
        } else {
          const uint32_t p22 = k >> 10;
          if (p22 == prefix22) atomicAdd(&s_h[k & 1023u], 1u);
          else if (p22 > prefix22 && (int)(k >> 21) == bin0) min_in = min(min_in, k);
          else if ((int)(k >> 21) > bin0) min_past = min(min_past, k);
        }
      }
    }
  }
  if (P == 0) {
    if (run_cnt != 0u) atomicAdd(&s_h[run_bin], run_cnt);
    sum = group_sum<kWave>(sum);
    if (threadIdx.x % kWave == 0) s_sum[threadIdx.x / kWave] = sum;
  }
  if (P == 2) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      min_in = min(min_in, (uint32_t)__shfl_xor((int)min_in, off));
      min_past = min(min_past, (uint32_t)__shfl_xor((int)min_past, off));
    }
    if (threadIdx.x % kWave == 0) {
      s_min[0][threadIdx.x / kWave] = min_in;
      s_min[1][threadIdx.x / kWave] = min_past;
    }
  }
  __syncthreads();
  unsigned int* gh = P == 0 ? m.h0 : (P == 1 ? m.h1 : m.h2);
  for (int i = threadIdx.x; i < NB; i += kMonThreads)
    if (s_h[i] != 0u) atomicAdd(&gh[i], s_h[i]);
  if (P == 0 && threadIdx.x == 0) {
    double t = 0.0;
    for (int w = 0; w < kMonThreads / kWave; ++w) t += s_sum[w];
    m.partial[blockIdx.x] = t;
  }
  if (P == 2 && threadIdx.x == 0) {
    for (int w = 1; w < kMonThreads / kWave; ++w) {
      min_in = min(min_in, s_min[0][w]);
      min_past = min(min_past, s_min[1][w]);
    }
    m.next_min[2 * blockIdx.x + 0] = min_in;
    m.next_min[2 * blockIdx.x + 1] = min_past;
  }
}

// Final step, one workgroup: the lower order statistic from the three
// histograms; when no tie covers the next rank, the next order statistic is
// the next occupied bin of the last histogram if there is one, else the
// smallest key the third pass found past the 22-bit prefix. The mean sums the
// first pass's workgroup sums (thread t takes workgroups t, t + 256, ... in
// order, then the threads in order). Interpolation in fp64, one rounding;
// the histograms are cleared for the next call.
__global__ __launch_bounds__(kMonThreads) void mon_final_kernel(MonLayout m, int capacity, int groups2,
                                                                float* __restrict__ out) {
  __shared__ unsigned int s_tot[kMonThreads / kWave];
  __shared__ int s_bin;
  __shared__ unsigned int s_below;
  __shared__ unsigned int s_next[2];
  __shared__ double s_part[kMonThreads / kWave];
  const int n = mon_n(m, capacity);
  if (n == 0) {  // empty window: no statistic (the controller skips a non-finite value)
    if (threadIdx.x == 0) {
      out[0] = NAN;
      out[1] = NAN;
    }
    return;
  }
  const unsigned int rank = lower_rank(n);
  int b0, b1, b2;
  unsigned int below0, below1, below2;
  find_bin<kMonBins0>(m.h0, rank, &s_bin, &s_below, s_tot, &b0, &below0);
  find_bin<kMonBins1>(m.h1, rank - below0, &s_bin, &s_below, s_tot, &b1, &below1);
  find_bin<kMonBins2>(m.h2, rank - below0 - below1, &s_bin, &s_below, s_tot, &b2, &below2);
  const uint32_t klo = ((uint32_t)b0 << 21) | ((uint32_t)b1 << 10) | (uint32_t)b2;
  const unsigned int le = below0 + below1 + below2 + m.h2[b2];  // keys <= klo
  const bool need_next = rank + 1 < (unsigned int)n && le <= rank + 1;
  if (threadIdx.x == 0) {
    s_next[0] = UINT_MAX;
    s_next[1] = UINT_MAX;
  }
  __syncthreads();
  if (need_next) {
    // the next occupied bin of the last histogram
    uint32_t nb = UINT_MAX;
    for (int i = b2 + 1 + (int)threadIdx.x; i < kMonBins2; i += kMonThreads)
      if (m.h2[i] != 0u) nb = min(nb, (uint32_t)i);
    // else the third pass's smallest keys past the prefix, inside then past the leading bin
    const int g2 = min(groups2, (n + kMonTile - 1) / kMonTile);
    uint32_t mi = UINT_MAX, mp = UINT_MAX;
    for (int g = threadIdx.x; g < g2; g += kMonThreads) {
      mi = min(mi, m.next_min[2 * g + 0]);
      mp = min(mp, m.next_min[2 * g + 1]);
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      nb = min(nb, (uint32_t)__shfl_xor((int)nb, off));
      mi = min(mi, (uint32_t)__shfl_xor((int)mi, off));
      mp = min(mp, (uint32_t)__shfl_xor((int)mp, off));
    }
    if (threadIdx.x % kWave == 0) {
      atomicMin(&s_next[0], nb != UINT_MAX ? (((klo >> 10) << 10) | nb) : UINT_MAX);
      atomicMin(&s_next[1], min(mi, mp));
    }
  }
  double sum = 0.0;
  const int g0 = (n + kMonTile - 1) / kMonTile;
  for (int g = threadIdx.x; g < g0; g += kMonThreads) sum += m.partial[g];
  sum = group_sum<kWave>(sum);
  if (threadIdx.x % kWave == 0) s_part[threadIdx.x / kWave] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double pos = 0.05 * (double)(n - 1);
    const double frac = pos - floor(pos);
    const double vlo = (double)mon_value(klo);
    double vhi = vlo;
    if (need_next) vhi = (double)mon_value(s_next[0] != UINT_MAX ? s_next[0] : s_next[1]);
    sum = 0.0;
    for (int w = 0; w < kMonThreads / kWave; ++w) sum += s_part[w];
    out[0] = (float)(sum / (double)n);
    out[1] = (float)(vlo + frac * (vhi - vlo));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kMonBins0 + kMonBins1 + kMonBins2; i += kMonThreads) m.h0[i] = 0u;
}

__global__ void mon_reset_kernel(MonLayout m) {
  if (threadIdx.x == 0) *m.count = 0ull;
}

int mon_groups(int capacity) { return (capacity + kMonTile - 1) / kMonTile; }

}  // namespace

size_t monitor_workspace_bytes(int capacity) {
  return ((mon_header_bytes() + 255) & ~(size_t)255) + (size_t)capacity * sizeof(float);
}

hipError_t launch_monitor_reset(void* ws, int capacity, hipStream_t s) {
  (void)capacity;
  hipLaunchKernelGGL(mon_reset_kernel, dim3(1), dim3(kWave), 0, s, mon_layout(ws));
  return hipGetLastError();
}

hipError_t launch_monitor_append(void* ws, int capacity, const float* alpha, int n, hipStream_t s) {
  const MonLayout m = mon_layout(ws);
  const int written = n < capacity ? n : capacity;
  constexpr int kOneGroup = 16 * kMonAppendThreads;
  if (written <= kOneGroup) {
    hipLaunchKernelGGL((mon_append_kernel<true>), dim3(1), dim3(kMonAppendThreads), 0, s, m, capacity, alpha, n);
  } else {
    const int groups = (written + kOneGroup - 1) / kOneGroup;
    hipLaunchKernelGGL((mon_append_kernel<false>), dim3(groups), dim3(kMonAppendThreads), 0, s, m, capacity, alpha, n);
    hipLaunchKernelGGL(mon_count_kernel, dim3(1), dim3(kWave), 0, s, m, n);
  }
  return hipGetLastError();
}

hipError_t launch_monitor_stats(void* ws, int capacity, float* out, hipStream_t s) {
  const MonLayout m = mon_layout(ws);
  const int g = mon_groups(capacity);
  // The second pass adds a histogram of up to 2048 occupied bins per
  // workgroup: fewer workgroups, each over several tiles, keep those device
  // atomics few.
  const int g1 = g < kMonPass1Groups ? g : kMonPass1Groups;
  hipLaunchKernelGGL((mon_hist_kernel<0>), dim3(g), dim3(kMonThreads), 0, s, m, capacity);
  hipLaunchKernelGGL((mon_hist_kernel<1>), dim3(g1), dim3(kMonThreads), 0, s, m, capacity);
  hipLaunchKernelGGL((mon_hist_kernel<2>), dim3(g), dim3(kMonThreads), 0, s, m, capacity);
  hipLaunchKernelGGL(mon_final_kernel, dim3(1), dim3(kMonThreads), 0, s, m, capacity, g, out);
  return hipGetLastError();
}

}  // namespace spdec
