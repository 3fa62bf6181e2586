// Per-token sparse-vs-dense acceptance over the vocabulary.
//
// alpha_r = sum_v min(softmax(a_r/T)_v, softmax(b_r/T)_v) = 1 - TV(p, q)
// (Sparrow project page, "Insights": the per-token mismatch of the sparse
// actor against the dense policy; the wispaper blog calls it the acceptance
// rate). Each row is split into 2048-entry chunks so a few rows still fill the
// GPU:
//   pass 1: per chunk, the max and sum of 2^(x - max) of both rows (x = logit*log2e/T);
//   pass 2: per chunk, the row's global normalisers from the pass-1 partials
//           (fixed order), then sum_v min(p_v, q_v) over the chunk;
//   pass 3: per row, the chunk sums in index order, clamped to [0, 1].
// No float atomics: results are run-to-run identical.
#include "common.h"
#include "launch.h"

namespace spdec {

namespace {

constexpr int kAccThreads = 256;
// Entries per thread per row: 2048-entry chunks give 64 rows of 151936 about
// four rounds of workgroups, so the loads of a later round overlap the
// arithmetic of an earlier one (one round of 8192-entry chunks ran 6% slower).
constexpr int kAccPer = 8;
constexpr int kAccChunk = kAccThreads * kAccPer;
// Pass 1 reads the logits with ordinary loads (cached on the memory side) and
// pass 2 visits the chunks in reverse order (below), so the chunks read last,
// the likeliest still to be cached, come first: about a quarter off pass 2.
// Its L2 misses are unchanged (the counters show the full rows fetched again),
// so the saving is in the last-level cache beyond the L2.
constexpr bool kPass1Stream = false;
constexpr bool kPass2Stream = false;

struct AccArgs {
  const float* a;
  const float* b;
  int rows, vocab, nchunk;
  int64_t stride;
  float c;        // log2(e) / T
  float* part;    // [rows][nchunk][4]: max_a, sum_a, max_b, sum_b
  float* csum;    // [rows][nchunk]
  float* alpha;   // [rows]
};

// Thread t loads entries base + 4t + 1024j .. +3, j = 0..kAccPer/4-1 (16-byte loads).
// STREAM selects the non-temporal hint (data read once from HBM).
template <bool ALIGNED, bool STREAM>
__device__ __forceinline__ void load_row(const float* row, int vocab, int base, float* x) {
#pragma unroll
  for (int j = 0; j < kAccPer / 4; ++j) {
    const int idx = base + 4 * (int)threadIdx.x + 4 * kAccThreads * j;
    if (ALIGNED && idx + 3 < vocab) {
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      const f32x4* p = reinterpret_cast<const f32x4*>(row + idx);
      const f32x4 v = STREAM ? __builtin_nontemporal_load(p) : *p;
      x[4 * j + 0] = v.x;
      x[4 * j + 1] = v.y;
      x[4 * j + 2] = v.z;
      x[4 * j + 3] = v.w;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) x[4 * j + u] = (idx + u < vocab) ? row[idx + u] : -INFINITY;
    }
  }
}

// Fixed-order block reductions (wave butterfly, then waves in index order).
__device__ __forceinline__ float block_max(float v, float* sh) {
  v = group_max<kWave>(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (threadIdx.x % kWave == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int i = 1; i < kAccThreads / kWave; ++i) r = fmaxf(r, sh[i]);
  return r;
}

__device__ __forceinline__ float block_sum(float v, float* sh) {
  v = group_sum<kWave>(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (threadIdx.x % kWave == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int i = 1; i < kAccThreads / kWave; ++i) r += sh[i];
  return r;
}

// Entries times c, each a rounded product (never fused into a later
// subtraction), so both passes see the same scaled values.
__device__ __forceinline__ void scale_entries(float* va, float* vb, float c) {
#pragma clang fp contract(off)
#pragma unroll
  for (int i = 0; i < kAccPer; ++i) {
    va[i] = va[i] * c;
    vb[i] = vb[i] * c;
  }
}

// Pass 1 on one chunk: loads both rows' entries (scaled by c) into va, vb and
// writes the chunk's (max, sum) pair of each row.
template <bool ALIGNED>
__device__ __forceinline__ void chunk_stats(const AccArgs& x, int r, int ch, float* va, float* vb, float* sh) {
  const int base = ch * kAccChunk;
  load_row<ALIGNED, kPass1Stream>(x.a + (int64_t)r * x.stride, x.vocab, base, va);
  load_row<ALIGNED, kPass1Stream>(x.b + (int64_t)r * x.stride, x.vocab, base, vb);
  scale_entries(va, vb, x.c);
  float ma = va[0], mb = vb[0];
#pragma unroll
  for (int i = 1; i < kAccPer; ++i) { ma = fmaxf(ma, va[i]); mb = fmaxf(mb, vb[i]); }
  ma = block_max(ma, sh);
  mb = block_max(mb, sh);
  float sa = 0.f, sb = 0.f;
#pragma unroll
  for (int i = 0; i < kAccPer; ++i) { sa += fast_exp2(va[i] - ma); sb += fast_exp2(vb[i] - mb); }
  sa = block_sum(sa, sh);
  sb = block_sum(sb, sh);
  if (threadIdx.x == 0) {
    float* p = x.part + ((int64_t)r * x.nchunk + ch) * 4;
    p[0] = ma; p[1] = sa; p[2] = mb; p[3] = sb;
  }
}

// The row normalisers from the pass-1 partials (fixed order), by the first wave.
__device__ __forceinline__ void row_norms(const AccArgs& x, int r, float* s_norm) {
  if (threadIdx.x < kWave) {
    // Lane i folds chunks i, i+64, ...
    const float* p = x.part + (int64_t)r * x.nchunk * 4;
    float ma = kNegBig, mb = kNegBig;
    for (int j = threadIdx.x; j < x.nchunk; j += kWave) { ma = fmaxf(ma, p[4 * j]); mb = fmaxf(mb, p[4 * j + 2]); }
    ma = group_max<kWave>(ma);
    mb = group_max<kWave>(mb);
    float sa = 0.f, sb = 0.f;
    for (int j = threadIdx.x; j < x.nchunk; j += kWave) {
      sa = fmaf(fast_exp2(p[4 * j] - ma), p[4 * j + 1], sa);
      sb = fmaf(fast_exp2(p[4 * j + 2] - mb), p[4 * j + 3], sb);
    }
    sa = group_sum<kWave>(sa);
    sb = group_sum<kWave>(sb);
    if (threadIdx.x == 0) { s_norm[0] = ma; s_norm[1] = 1.f / sa; s_norm[2] = mb; s_norm[3] = 1.f / sb; }
  }
  __syncthreads();
}

// Pass 2 on one chunk from its scaled entries: sum_v min(p_v, q_v).
__device__ __forceinline__ void chunk_min(const AccArgs& x, int r, int ch, const float* va, const float* vb,
                                          const float* s_norm, float* sh) {
  const float ma = s_norm[0], ia = s_norm[1], mb = s_norm[2], ib = s_norm[3];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kAccPer; ++i) s += fminf(fast_exp2(va[i] - ma) * ia, fast_exp2(vb[i] - mb) * ib);
  s = block_sum(s, sh);
  if (threadIdx.x == 0) x.csum[(int64_t)r * x.nchunk + ch] = s;
}

// Pass 3 for one row: the chunk sums in index order, clamped, by one wave.
__device__ __forceinline__ void row_final(const AccArgs& x, int r) {
  float s = 0.f;
  for (int j = threadIdx.x; j < x.nchunk; j += kWave) s += x.csum[(int64_t)r * x.nchunk + j];
  s = group_sum<kWave>(s);
  if (threadIdx.x == 0) x.alpha[r] = fminf(1.f, fmaxf(0.f, s));
}

template <bool ALIGNED>
__global__ __launch_bounds__(kAccThreads) void acc_stats_kernel(AccArgs x) {
  __shared__ float sh[kAccThreads / kWave];
  float va[kAccPer], vb[kAccPer];
  chunk_stats<ALIGNED>(x, blockIdx.y, blockIdx.x, va, vb, sh);
}

template <bool ALIGNED>
__global__ __launch_bounds__(kAccThreads) void acc_min_kernel(AccArgs x) {
  __shared__ float sh[kAccThreads / kWave];
  __shared__ float s_norm[4];
  // Chunks in reverse order of pass 1. The map keeps the linear id's class
  // mod 8, so a chunk is read by the same XCD in both passes (workgroups are
  // dealt to the XCDs round-robin by linear id).
  const int N = gridDim.x * gridDim.y;
  const int i = blockIdx.y * gridDim.x + blockIdx.x;
  const int N8 = N & ~7;
  const int item = i < N8 ? (N8 - 8 - (i & ~7)) + (i & 7) : i;
  const int r = item / gridDim.x, ch = item % gridDim.x;
  // The chunk's logits are requested first; the row normalisers are folded
  // from the pass-1 partials while those loads are in flight.
  float va[kAccPer], vb[kAccPer];
  const int base = ch * kAccChunk;
  load_row<ALIGNED, kPass2Stream>(x.a + (int64_t)r * x.stride, x.vocab, base, va);
  load_row<ALIGNED, kPass2Stream>(x.b + (int64_t)r * x.stride, x.vocab, base, vb);
  row_norms(x, r, s_norm);
  scale_entries(va, vb, x.c);
  chunk_min(x, r, ch, va, vb, s_norm, sh);
}

__global__ __launch_bounds__(kWave) void acc_final_kernel(AccArgs x) { row_final(x, blockIdx.x); }

// Tail statistics of the per-token acceptance (Sparrow project page,
// "Control Study 1": the lower 5th percentile of the mismatch is the stability
// signal; its takeaway threshold is 0.86): the mean and the 5th percentile
// (linear interpolation between order statistics, rank 0.05 * (n - 1)) of n
// values, in one workgroup. The values are sorted in LDS (bitonic, padded to a
// power of two with +inf); the mean and the interpolation run in fp64 and are
// rounded once, so both equal the exact statistics of the fp32 inputs up to
// that rounding.
constexpr int kTailThreads = 1024;

__global__ __launch_bounds__(kTailThreads) void tail_stats_kernel(const float* __restrict__ alpha, int n,
                                                                  float* __restrict__ out) {
  __shared__ float s[kTailMaxRows];
  __shared__ double s_sum[kTailThreads / kWave];
  int n2 = 1;
  while (n2 < n) n2 <<= 1;
  double part = 0.0;
  for (int i = threadIdx.x; i < n2; i += kTailThreads) {
    const float v = i < n ? alpha[i] : INFINITY;
    s[i] = v;
    if (i < n) part += (double)v;
  }
  part = group_sum<kWave>(part);
  if (threadIdx.x % kWave == 0) s_sum[threadIdx.x / kWave] = part;
  __syncthreads();
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n2; i += kTailThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const float a = s[i], b = s[ixj];
          const bool up = (i & k) == 0;
          if ((a > b) == up) { s[i] = b; s[ixj] = a; }
        }
      }
      __syncthreads();
    }
  }
  if (threadIdx.x == 0) {
    double sum = 0.0;
    for (int w = 0; w < kTailThreads / kWave; ++w) sum += s_sum[w];
    const double pos = 0.05 * (double)(n - 1);
    const int lo = (int)floor(pos);
    const int hi = min(lo + 1, n - 1);
    out[0] = (float)(sum / n);
    out[1] = (float)((double)s[lo] + (pos - lo) * ((double)s[hi] - (double)s[lo]));
  }
}

int nchunks(int vocab) { return (vocab + kAccChunk - 1) / kAccChunk; }

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

size_t acceptance_workspace_bytes(int rows, int vocab) {
  const size_t n = (size_t)rows * nchunks(vocab);
  return align256(n * 4 * sizeof(float)) + align256(n * sizeof(float));
}

hipError_t launch_tail_stats(const float* alpha, int n, float* out, hipStream_t s) {
  hipLaunchKernelGGL(tail_stats_kernel, dim3(1), dim3(kTailThreads), 0, s, alpha, n, out);
  return hipGetLastError();
}

hipError_t launch_acceptance(const float* a, const float* b, int rows, int vocab, int64_t stride, float temperature,
                             float* alpha, void* ws, hipStream_t s) {
  AccArgs x;
  x.a = a;
  x.b = b;
  x.rows = rows;
  x.vocab = vocab;
  x.nchunk = nchunks(vocab);
  x.stride = stride;
  x.c = kLog2e / temperature;
  const size_t n = (size_t)rows * x.nchunk;
  x.part = reinterpret_cast<float*>(ws);
  x.csum = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + align256(n * 4 * sizeof(float)));
  x.alpha = alpha;
  const bool aligned = (reinterpret_cast<uintptr_t>(a) % 16 == 0) && (reinterpret_cast<uintptr_t>(b) % 16 == 0) &&
                       (stride % 4 == 0);
  dim3 grid(x.nchunk, rows);
  if (aligned) {
    hipLaunchKernelGGL((acc_stats_kernel<true>), grid, dim3(kAccThreads), 0, s, x);
    hipLaunchKernelGGL((acc_min_kernel<true>), grid, dim3(kAccThreads), 0, s, x);
  } else {
    hipLaunchKernelGGL((acc_stats_kernel<false>), grid, dim3(kAccThreads), 0, s, x);
    hipLaunchKernelGGL((acc_min_kernel<false>), grid, dim3(kAccThreads), 0, s, x);
  }
  hipLaunchKernelGGL(acc_final_kernel, dim3(rows), dim3(kWave), 0, s, x);
  return hipGetLastError();
}

}  // namespace spdec
