// Per-token sparse-vs-dense acceptance over the vocabulary.
//
// alpha_r = sum_v min(softmax(a_r/T)_v, softmax(b_r/T)_v) = 1 - TV(p, q)
// (Sparrow project page, "Insights": the per-token mismatch of the sparse
// actor against the dense policy; the wispaper blog calls it the acceptance
// rate). The min needs both rows' global normalisers, which are known only
// once every entry of the row has been seen. Two decompositions:
//
//   * single read (every row split into at most a few thousand chunks in all,
//     e.g. 64 rows of 151936): one workgroup per chunk of 10240 entries holds
//     its entries of both rows in registers. It publishes its chunk's
//     (max, sum of 2^(x - max)) pair per row, waits for the other chunks of
//     its row, folds the row normalisers from the published pairs in a fixed
//     order, and sums min(p, q) over the entries it already holds. Chunk sums
//     meet in one 64-bit word per row (an arrival count above a fixed-point
//     sum), and the workgroup that arrives last writes alpha. Every logit is
//     read from HBM once. The wait is bounded: a workgroup that stops waiting
//     reads the whole row itself and computes the same pairs, so the result
//     never depends on how many workgroups are resident at once.
//   * two passes (more chunks than fit on the chip at once): pass 1 writes
//     per-chunk pairs, pass 2 re-reads the chunk and folds the normalisers,
//     pass 3 sums the chunk sums of each row in index order.
//
// No float atomics: results are run-to-run identical in either form.
#include "common.h"
#include "launch.h"

namespace spdec {

namespace {

constexpr int kAccThreads = 256;
constexpr int kAccWaves = kAccThreads / kWave;

// ------------------------------------------------------------ row helpers ---

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Thread t loads entries base + 4t + 1024j .. +3, j = 0..PER/4-1; entries
// past the vocabulary read as -inf (zero probability). ALIGNED: rows 16-byte
// aligned and vocab % 4 == 0, so every 16-byte load lies wholly inside or
// wholly past the row; the ones past it read the row's last 16 bytes instead
// (in bounds, no branch) and are replaced by -inf.
template <int PER, bool ALIGNED>
__device__ __forceinline__ void load_row(const float* row, int vocab, int base, float* x) {
#pragma unroll
  for (int j = 0; j < PER / 4; ++j) {
    const int idx = base + 4 * (int)threadIdx.x + 4 * kAccThreads * j;
    if (ALIGNED) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(row + min(idx, vocab - 4));
      const bool in = idx < vocab;
      x[4 * j + 0] = in ? v.x : -INFINITY;
      x[4 * j + 1] = in ? v.y : -INFINITY;
      x[4 * j + 2] = in ? v.z : -INFINITY;
      x[4 * j + 3] = in ? v.w : -INFINITY;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) x[4 * j + u] = (idx + u < vocab) ? row[idx + u] : -INFINITY;
    }
  }
}

// Fixed-order block reductions (wave butterfly, then waves in index order).
// Every thread returns the same value. `sh` holds one float per wave.
__device__ __forceinline__ float block_max(float v, float* sh) {
  v = group_max<kWave>(v);
  __syncthreads();
  if (threadIdx.x % kWave == 0) sh[threadIdx.x / kWave] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int i = 1; i < kAccWaves; ++i) r = fmaxf(r, sh[i]);
  return r;
}

__device__ __forceinline__ float block_sum(float v, float* sh) {
  v = group_sum<kWave>(v);
  __syncthreads();
  if (threadIdx.x % kWave == 0) sh[threadIdx.x / kWave] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int i = 1; i < kAccWaves; ++i) r += sh[i];
  return r;
}

// Entries times c = log2(e)/T, each a rounded product (never fused into a
// later subtraction), so every path sees the same scaled values.
template <int N>
__device__ __forceinline__ void scale_entries(float* v, float c) {
#pragma clang fp contract(off)
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = v[i] * c;
}

// A chunk's (max, sum of 2^(x - max)) of one row from its scaled entries:
// per thread in entry order, then across the block.
template <int PER>
__device__ __forceinline__ void chunk_pair(const float* v, float* sh, float& m, float& s) {
  float t = v[0];
#pragma unroll
  for (int i = 1; i < PER; ++i) t = fmaxf(t, v[i]);
  m = block_max(t, sh);
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) acc += fast_exp2(v[i] - m);
  s = block_sum(acc, sh);
}

// sum_v min(p_v, q_v) over the thread's entries, then across the block.
template <int PER>
__device__ __forceinline__ float chunk_min(const float* va, const float* vb, const float* nrm, float* sh) {
  const float ma = nrm[0], ia = nrm[1], mb = nrm[2], ib = nrm[3];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) s += fminf(fast_exp2(va[i] - ma) * ia, fast_exp2(vb[i] - mb) * ib);
  return block_sum(s, sh);
}

// ------------------------------------------------------------ single read ---

// Entries per thread per row: both rows' 2 x 40 values stay in registers
// (under 128 VGPRs, four waves per SIMD), so 64 rows of 151936 take 15
// chunks each, 960 workgroups: one resident round on 256 compute units.
constexpr int kOnePer = 40;
constexpr int kOneChunk = kAccThreads * kOnePer;  // 10240 entries
// Chunks per row of the single read: one wave holds a row's pairs
// (vocabularies up to 655360 entries).
constexpr int kOneMaxChunks = kWave;
// Fixed-point scale of the chunk sums (each in [0, 1]) and the arrival count
// above them in the per-row word: sums stay below 2^49, counts below 2^11.
constexpr int kFixBits = 48;
constexpr int kCountShift = 53;

struct OneArgs {
  const float* a;
  const float* b;
  int rows, vocab, nchunk;
  int64_t stride;
  float c;                    // log2(e) / T
  unsigned long long* pairs;  // [rows][2][nchunk]: (max, sum) of row a, then of row b; 0 = not yet written
  unsigned long long* word;   // [rows]: arrival count << 53 | fixed-point sum of the chunk sums
  float* alpha;               // [rows]
  int spin_limit;             // polls of the row's pairs before a workgroup reads the row itself
  int* fallbacks;             // nullable: workgroups that stopped waiting
};

// A published pair: the max and the sum in one 64-bit word. The sum is at
// least 1 (the maximal entry contributes 2^0), so a written word is never 0.
__device__ __forceinline__ unsigned long long pack_pair(float m, float s) {
  return ((unsigned long long)__float_as_uint(m) << 32) | __float_as_uint(s);
}
__device__ __forceinline__ float pair_max(unsigned long long w) { return __uint_as_float((uint32_t)(w >> 32)); }
__device__ __forceinline__ float pair_sum(unsigned long long w) { return __uint_as_float((uint32_t)w); }

__device__ __forceinline__ unsigned long long load_coherent(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Two block reductions at once (rows a and b); `sh` holds two floats per wave.
__device__ __forceinline__ void block_max2(float& x, float& y, float* sh) {
  x = group_max<kWave>(x);
  y = group_max<kWave>(y);
  __syncthreads();
  if (threadIdx.x % kWave == 0) {
    sh[threadIdx.x / kWave] = x;
    sh[kAccWaves + threadIdx.x / kWave] = y;
  }
  __syncthreads();
  x = sh[0];
  y = sh[kAccWaves];
#pragma unroll
  for (int i = 1; i < kAccWaves; ++i) {
    x = fmaxf(x, sh[i]);
    y = fmaxf(y, sh[kAccWaves + i]);
  }
}

__device__ __forceinline__ void block_sum2(float& x, float& y, float* sh) {
  x = group_sum<kWave>(x);
  y = group_sum<kWave>(y);
  __syncthreads();
  if (threadIdx.x % kWave == 0) {
    sh[threadIdx.x / kWave] = x;
    sh[kAccWaves + threadIdx.x / kWave] = y;
  }
  __syncthreads();
  x = sh[0];
  y = sh[kAccWaves];
#pragma unroll
  for (int i = 1; i < kAccWaves; ++i) {
    x += sh[i];
    y += sh[kAccWaves + i];
  }
}

// A thread's share of a chunk pair: its max t over its scaled entries, and
// the sum of 2^(x - t) in entry order. No barrier: a thread goes on as soon
// as its own loads have arrived. t starts at the finite sentinel, so a thread
// whose entries all lie past the vocabulary (-inf) gets weights and a sum of
// 0, not NaN. WEIGHTS: v is left holding the weights 2^(x - t).
template <int PER, bool WEIGHTS>
__device__ __forceinline__ void thread_pair(float* v, float& t, float& s) {
#pragma clang fp contract(off)
  t = kNegBig;
#pragma unroll
  for (int i = 0; i < PER; ++i) t = fmaxf(t, v[i]);
  s = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const float e = fast_exp2(v[i] - t);
    if (WEIGHTS) v[i] = e;
    s += e;
  }
}

// The chunk pairs of both rows from the threads' shares (ta, sa), (tb, sb):
// max m of the thread maxima, then the sum of 2^(t - m) * s over the block.
__device__ __forceinline__ void chunk_pairs(float ta, float sa, float tb, float sb, float* sh, float& ma, float& za,
                                            float& mb, float& zb) {
#pragma clang fp contract(off)
  ma = ta;
  mb = tb;
  block_max2(ma, mb, sh);
  za = fast_exp2(ta - ma) * sa;
  zb = fast_exp2(tb - mb) * sb;
  block_sum2(za, zb, sh);
}

// Pairs of every chunk of row r, computed from HBM by this workgroup alone
// with the arithmetic of the published ones (each thread's entries in the
// same order, read in pieces of 8, then the same block reductions), so they
// are bitwise equal. Thread j keeps chunk j's pairs in `out`.
template <bool ALIGNED>
__device__ void row_pairs_direct(const OneArgs& x, int r, float* sh, unsigned long long* out_a,
                                 unsigned long long* out_b) {
#pragma clang fp contract(off)
  constexpr int PIECE = 8;
  const float* ra = x.a + (int64_t)r * x.stride;
  const float* rb = x.b + (int64_t)r * x.stride;
  for (int j = 0; j < x.nchunk; ++j) {
    const int base = j * kOneChunk;
    float t[2], acc[2];
#pragma unroll
    for (int row = 0; row < 2; ++row) {
      const float* src = row == 0 ? ra : rb;
      float m = kNegBig;
#pragma unroll 1
      for (int p = 0; p < kOnePer / PIECE; ++p) {
        float v[PIECE];
        load_row<PIECE, ALIGNED>(src, x.vocab, base + 4 * kAccThreads * (PIECE / 4) * p, v);
        scale_entries<PIECE>(v, x.c);
#pragma unroll
        for (int i = 0; i < PIECE; ++i) m = fmaxf(m, v[i]);
      }
      float s = 0.f;
#pragma unroll 1
      for (int p = 0; p < kOnePer / PIECE; ++p) {
        float v[PIECE];
        load_row<PIECE, ALIGNED>(src, x.vocab, base + 4 * kAccThreads * (PIECE / 4) * p, v);
        scale_entries<PIECE>(v, x.c);
#pragma unroll
        for (int i = 0; i < PIECE; ++i) s += fast_exp2(v[i] - m);
      }
      t[row] = m;
      acc[row] = s;
    }
    float ma, za, mb, zb;
    chunk_pairs(t[0], acc[0], t[1], acc[1], sh, ma, za, mb, zb);
    if (threadIdx.x == j) {
      out_a[j] = pack_pair(ma, za);
      out_b[j] = pack_pair(mb, zb);
    }
  }
}

// One workgroup per (row, chunk); at most the device's resident workgroups in
// all, so on an otherwise idle device every chunk of a row runs at once.
template <bool ALIGNED>
__global__ __launch_bounds__(kAccThreads) void acc_one_read_kernel(OneArgs x) {
  __shared__ float sh[2 * kAccWaves];
  __shared__ unsigned long long s_pa[kOneMaxChunks], s_pb[kOneMaxChunks];
  __shared__ int s_ready, s_last;
  const int r = blockIdx.x / x.nchunk, ch = blockIdx.x % x.nchunk;
  const int lane = threadIdx.x % kWave;
  float va[kOnePer], vb[kOnePer];
  load_row<kOnePer, ALIGNED>(x.a + (int64_t)r * x.stride, x.vocab, ch * kOneChunk, va);
  load_row<kOnePer, ALIGNED>(x.b + (int64_t)r * x.stride, x.vocab, ch * kOneChunk, vb);
  scale_entries<kOnePer>(va, x.c);
  scale_entries<kOnePer>(vb, x.c);
  float ta, sa, tb, sb;
  thread_pair<kOnePer, true>(va, ta, sa);
  thread_pair<kOnePer, true>(vb, tb, sb);
  float ma, za, mb, zb;
  chunk_pairs(ta, sa, tb, sb, sh, ma, za, mb, zb);

  unsigned long long* row_pairs = x.pairs + (int64_t)r * 2 * x.nchunk;
  if (threadIdx.x == 0) {
    store_coherent(row_pairs + ch, pack_pair(ma, za));
    store_coherent(row_pairs + x.nchunk + ch, pack_pair(mb, zb));
  }
  // The first wave waits until every chunk of the row has published its
  // pairs (lane j watches chunk j), at most spin_limit polls.
  if (threadIdx.x < kWave) {
    unsigned long long wa = lane < x.nchunk ? 0ull : 1ull, wb = wa;
    bool ready = false;
    for (int it = 0;; ++it) {
      if (wa == 0ull) wa = load_coherent(row_pairs + lane);
      if (wb == 0ull) wb = load_coherent(row_pairs + x.nchunk + lane);
      if (__all(wa != 0ull && wb != 0ull)) { ready = true; break; }
      if (it >= x.spin_limit) break;
      __builtin_amdgcn_s_sleep(1);
    }
    if (lane < x.nchunk) {
      s_pa[lane] = wa;
      s_pb[lane] = wb;
    }
    if (lane == 0) s_ready = ready ? 1 : 0;
  }
  __syncthreads();
  if (!s_ready) {
    // Not every chunk of the row is running: compute the row's pairs here.
    row_pairs_direct<ALIGNED>(x, r, sh, s_pa, s_pb);
    if (threadIdx.x == 0) {
      // Make sure this workgroup's own published pairs have landed before any
      // of its waves arrives (the last arrival clears them): an exchange is
      // ordered after the earlier store to the same word and returns once
      // performed.
      unsigned long long t0 = __hip_atomic_exchange(row_pairs + ch, pack_pair(ma, za), __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
      unsigned long long t1 = __hip_atomic_exchange(row_pairs + x.nchunk + ch, pack_pair(mb, zb),
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      asm volatile("" ::"v"(t0), "v"(t1));
      if (x.fallbacks != nullptr) atomicAdd(x.fallbacks, 1);
    }
    __syncthreads();
  }
  // Row normalisers, folded by every wave alike from the pairs in LDS (lane j
  // holds chunk j): max, then the sum of 2^(m_j - M) * z_j, butterflies in a
  // fixed order.
  float ka, kb;
  {
#pragma clang fp contract(off)
    const bool in = lane < x.nchunk;
    const float pa = in ? pair_max(s_pa[lane]) : kNegBig, qa = in ? pair_sum(s_pa[lane]) : 0.f;
    const float pb = in ? pair_max(s_pb[lane]) : kNegBig, qb = in ? pair_sum(s_pb[lane]) : 0.f;
    const float Ma = group_max<kWave>(pa), Mb = group_max<kWave>(pb);
    const float Za = group_sum<kWave>(fast_exp2(pa - Ma) * qa);
    const float Zb = group_sum<kWave>(fast_exp2(pb - Mb) * qb);
    // p_v = 2^(x_v - t) * 2^(t - M) / Z with t the thread's reference: va,
    // vb hold the weights 2^(x_v - t), so one factor per thread and row remains.
    ka = fast_exp2(ta - Ma) * (1.f / Za);
    kb = fast_exp2(tb - Mb) * (1.f / Zb);
  }
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < kOnePer; ++i) part += fminf(va[i] * ka, vb[i] * kb);
  const float cs = block_sum(part, sh);

  // One arrival per chunk with its sum in fixed point: integer addition is
  // exact and order-free, so the row's total does not depend on arrival
  // order. The last of the row's nchunk arrivals writes alpha and clears the
  // row's pairs (every other chunk of the row has folded them by then: its
  // arrival carries a sum computed from them) and its word.
  if (threadIdx.x == 0) {
    const unsigned long long fx = __double2ull_rn((double)cs * (double)(1ull << kFixBits));
    const unsigned long long old = atomicAdd(x.word + r, (1ull << kCountShift) + fx);
    const bool last = (int)(old >> kCountShift) == x.nchunk - 1;
    if (last) {
      const unsigned long long tot = (old & ((1ull << kCountShift) - 1)) + fx;
      const float a = (float)((double)tot * (1.0 / (double)(1ull << kFixBits)));
      x.alpha[r] = fminf(1.f, fmaxf(0.f, a));
      store_coherent(x.word + r, 0ull);
    }
    s_last = last ? 1 : 0;
  }
  __syncthreads();
  if (s_last)
    for (int k = threadIdx.x; k < 2 * x.nchunk; k += kAccThreads) store_coherent(row_pairs + k, 0ull);
}

// ------------------------------------------------------------- two passes ---

// 2048-entry chunks: 64 rows of 151936 make about four rounds of workgroups,
// so the loads of a later round overlap the arithmetic of an earlier one.
constexpr int kTwoPer = 8;
constexpr int kTwoChunk = kAccThreads * kTwoPer;

struct TwoArgs {
  const float* a;
  const float* b;
  int rows, vocab, nchunk;
  int64_t stride;
  float c;
  float* part;    // [rows][nchunk][4]: max_a, sum_a, max_b, sum_b
  float* csum;    // [rows][nchunk]
  float* alpha;   // [rows]
};

template <bool ALIGNED>
__global__ __launch_bounds__(kAccThreads) void acc_stats_kernel(TwoArgs x) {
  __shared__ float sh[kAccWaves];
  const int r = blockIdx.y, ch = blockIdx.x;
  float va[kTwoPer], vb[kTwoPer];
  load_row<kTwoPer, ALIGNED>(x.a + (int64_t)r * x.stride, x.vocab, ch * kTwoChunk, va);
  load_row<kTwoPer, ALIGNED>(x.b + (int64_t)r * x.stride, x.vocab, ch * kTwoChunk, vb);
  scale_entries<kTwoPer>(va, x.c);
  scale_entries<kTwoPer>(vb, x.c);
  float ma, sa, mb, sb;
  chunk_pair<kTwoPer>(va, sh, ma, sa);
  chunk_pair<kTwoPer>(vb, sh, mb, sb);
  if (threadIdx.x == 0) {
    float* p = x.part + ((int64_t)r * x.nchunk + ch) * 4;
    p[0] = ma; p[1] = sa; p[2] = mb; p[3] = sb;
  }
}

template <bool ALIGNED>
__global__ __launch_bounds__(kAccThreads) void acc_min_kernel(TwoArgs x) {
  __shared__ float sh[kAccWaves];
  __shared__ float s_norm[4];
  const int r = blockIdx.y, ch = blockIdx.x;
  // The chunk's logits are requested first; the row normalisers are folded
  // from the pass-1 pairs (first wave, lane i takes chunks i, i + 64, ...)
  // while those loads are in flight.
  float va[kTwoPer], vb[kTwoPer];
  load_row<kTwoPer, ALIGNED>(x.a + (int64_t)r * x.stride, x.vocab, ch * kTwoChunk, va);
  load_row<kTwoPer, ALIGNED>(x.b + (int64_t)r * x.stride, x.vocab, ch * kTwoChunk, vb);
  if (threadIdx.x < kWave) {
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
  scale_entries<kTwoPer>(va, x.c);
  scale_entries<kTwoPer>(vb, x.c);
  const float s = chunk_min<kTwoPer>(va, vb, s_norm, sh);
  if (threadIdx.x == 0) x.csum[(int64_t)r * x.nchunk + ch] = s;
}

// Pass 3 for one row: the chunk sums in index order, clamped, by one wave.
__global__ __launch_bounds__(kWave) void acc_final_kernel(TwoArgs x) {
  const int r = blockIdx.x;
  float s = 0.f;
  for (int j = threadIdx.x; j < x.nchunk; j += kWave) s += x.csum[(int64_t)r * x.nchunk + j];
  s = group_sum<kWave>(s);
  if (threadIdx.x == 0) x.alpha[r] = fminf(1.f, fmaxf(0.f, s));
}

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

// ----------------------------------------------------------------- layout ---
//
// Workspace: [sync region, kAccSyncBytes][two-pass pairs and chunk sums].
// The sync region (single-read pairs and per-row words) sits at a fixed
// offset and size for every shape, so a workspace reused across shapes never
// finds the two-pass data there; it must be zero before the first call, and
// every call leaves it zero.
constexpr int kOneMaxItems = 4096;  // chunks in all (above any resident grid here)
constexpr int kOneMaxRows = 4096;

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int two_chunks(int vocab) { return (vocab + kTwoChunk - 1) / kTwoChunk; }
int one_chunks(int vocab) { return (vocab + kOneChunk - 1) / kOneChunk; }

// Resident workgroups of the single-read kernel on the current device (0 on error).
int one_read_capacity(bool aligned) {
  const void* k = aligned ? reinterpret_cast<const void*>(acc_one_read_kernel<true>)
                          : reinterpret_cast<const void*>(acc_one_read_kernel<false>);
  int grid = 0;
  if (persistent_grid(k, kAccThreads, 0, &grid) != hipSuccess) return 0;
  return grid;
}

}  // namespace

size_t acceptance_sync_bytes() {
  return align256((size_t)kOneMaxItems * 2 * sizeof(unsigned long long) + (size_t)kOneMaxRows * sizeof(unsigned long long));
}

size_t acceptance_workspace_bytes(int rows, int vocab) {
  const size_t n = (size_t)rows * two_chunks(vocab);
  return acceptance_sync_bytes() + align256(n * 4 * sizeof(float)) + align256(n * sizeof(float));
}

hipError_t launch_tail_stats(const float* alpha, int n, float* out, hipStream_t s) {
  hipLaunchKernelGGL(tail_stats_kernel, dim3(1), dim3(kTailThreads), 0, s, alpha, n, out);
  return hipGetLastError();
}

hipError_t launch_acceptance(const float* a, const float* b, int rows, int vocab, int64_t stride, float temperature,
                             float* alpha, void* ws, hipStream_t s, const AcceptanceDiag* diag) {
  const bool aligned = (reinterpret_cast<uintptr_t>(a) % 16 == 0) && (reinterpret_cast<uintptr_t>(b) % 16 == 0) &&
                       (stride % 4 == 0) && (vocab % 4 == 0);
  const float c = kLog2e / temperature;
  const int n1 = one_chunks(vocab);
  const int64_t items = (int64_t)rows * n1;
  bool one = diag != nullptr && diag->force_path >= 0 ? diag->force_path == 1 : true;
  if (one) {
    const int cap = one_read_capacity(aligned);
    one = items <= cap && items <= kOneMaxItems && rows <= kOneMaxRows && n1 <= kOneMaxChunks;
    if (diag != nullptr && diag->force_path == 1 && !one) return hipErrorInvalidValue;
  }
  if (diag != nullptr && diag->path != nullptr) *diag->path = one ? 1 : 2;
  if (one) {
    OneArgs x;
    x.a = a;
    x.b = b;
    x.rows = rows;
    x.vocab = vocab;
    x.nchunk = n1;
    x.stride = stride;
    x.c = c;
    x.pairs = reinterpret_cast<unsigned long long*>(ws);
    x.word = x.pairs + (size_t)kOneMaxItems * 2;
    x.alpha = alpha;
    x.spin_limit = diag != nullptr && diag->spin_limit >= 0 ? diag->spin_limit : kAcceptanceSpinLimit;
    x.fallbacks = diag != nullptr ? diag->fallbacks : nullptr;
    if (aligned)
      hipLaunchKernelGGL((acc_one_read_kernel<true>), dim3((unsigned)items), dim3(kAccThreads), 0, s, x);
    else
      hipLaunchKernelGGL((acc_one_read_kernel<false>), dim3((unsigned)items), dim3(kAccThreads), 0, s, x);
    return hipGetLastError();
  }
  TwoArgs x;
  x.a = a;
  x.b = b;
  x.rows = rows;
  x.vocab = vocab;
  x.nchunk = two_chunks(vocab);
  x.stride = stride;
  x.c = c;
  const size_t n = (size_t)rows * x.nchunk;
  char* base = reinterpret_cast<char*>(ws) + acceptance_sync_bytes();
  x.part = reinterpret_cast<float*>(base);
  x.csum = reinterpret_cast<float*>(base + align256(n * 4 * sizeof(float)));
  x.alpha = alpha;
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
