// Exact speculative sampling over the verifier's and the drafter's logits.
//
// After the dense verification pass (S3R page, abstract: drafted tokens are
// accepted by exact speculative sampling, so the emitted tokens follow the
// dense policy; the method is that of the two speculative-decoding papers the
// citation-map page lists by title), for every sequence b with k drafted
// tokens x_0 .. x_{k-1}:
//   draft i is kept when u_i * q_i(x_i) < p_i(x_i), p_i = softmax(verifier
//   logits / T), q_i = softmax(drafter logits / T), for i = 0, 1, ... until the
//   first rejection j; the next token is then drawn from max(0, p_j - q_j),
//   or from p_k when all k drafts are kept.
// A draw with uniform u takes the first token whose running sum of the
// weights exceeds u times their total (token order).
//
// Four passes, all fp32 with fixed reduction orders (run-to-run identical):
//   1. per (row, 8192-entry chunk): max and sum of 2^(x - max), x = logit * log2(e) / T,
//      for the k + 1 verifier rows and the k drafter rows of every sequence;
//   2. one wave per sequence: row normalisers from the chunk partials, the
//      accept chain, the row to draw from;
//   3. per (sequence, chunk): the sum of the draw weights of the chunk;
//   4. one workgroup per sequence: the chunk holding the draw, then an ordered
//      scan inside it.
#include <limits.h>

#include "common.h"
#include "launch.h"

namespace spdec {

namespace {

constexpr int kSpecThreads = 256;
constexpr int kSpecPer = 32;                          // entries per thread and chunk
constexpr int kSpecChunk = kSpecThreads * kSpecPer;   // 8192
constexpr int kSpecMaxDraft = 64;

struct SpecArgs {
  const float* p;        // verifier logits, row (b, i) at p + (b * (k + 1) + i) * stride
  const float* q;        // drafter logits, row (b, i) at q + (b * k + i) * stride
  int batch, k, vocab, nchunk;
  int64_t stride;
  const int32_t* draft;  // [batch][k]
  const float* u_accept; // [batch][k]
  const float* u_sample; // [batch]
  float c;               // log2(e) / T
  int32_t* n_accepted;   // [batch]
  int32_t* token;        // [batch]
  float* part;           // [rows][nchunk][2]: rows = batch*(k+1) verifier rows, then batch*k drafter rows
  float* draw;           // [batch][4]: max_p, 1/sum_p, max_q, 1/sum_q of the draw row
  int32_t* draw_row;     // [batch][2]: verifier row index, drafter row index (-1: draw from p alone)
  float* csum;           // [batch][nchunk]
};

__device__ __forceinline__ const float* row_ptr(const SpecArgs& a, int row) {
  const int prow = a.batch * (a.k + 1);
  return row < prow ? a.p + (int64_t)row * a.stride : a.q + (int64_t)(row - prow) * a.stride;
}

__device__ __forceinline__ float block_reduce_max(float v, float* sh) {
  v = group_max<kWave>(v);
  __syncthreads();
  if (threadIdx.x % kWave == 0) sh[threadIdx.x / kWave] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int i = 1; i < kSpecThreads / kWave; ++i) r = fmaxf(r, sh[i]);
  return r;
}

__device__ __forceinline__ float block_reduce_sum(float v, float* sh) {
  v = group_sum<kWave>(v);
  __syncthreads();
  if (threadIdx.x % kWave == 0) sh[threadIdx.x / kWave] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int i = 1; i < kSpecThreads / kWave; ++i) r += sh[i];
  return r;
}

// Pass 4 layout: thread t covers entries base + t * kSpecPer .. + kSpecPer - 1
// (contiguous, so a thread's entries are in token order for the scan).
struct LoadRun {
  __device__ __forceinline__ void operator()(const float* row, int vocab, int base, float* x) const {
    const int i0 = base + (int)threadIdx.x * kSpecPer;
#pragma unroll
    for (int e = 0; e < kSpecPer; ++e) x[e] = (i0 + e < vocab) ? row[i0 + e] : -INFINITY;
  }
};

// Passes 1 and 3 layout (order-free reductions): thread t loads entries
// base + 4t + 1024j .. +3 with 16-byte loads, one contiguous KiB per wave
// instruction; ALIGNED when rows and stride allow 16-byte loads.
template <bool ALIGNED>
__device__ __forceinline__ void load_spread(const float* row, int vocab, int base, float* x) {
#pragma unroll
  for (int j = 0; j < kSpecPer / 4; ++j) {
    const int idx = base + 4 * (int)threadIdx.x + 4 * kSpecThreads * j;
    if (ALIGNED && idx + 3 < vocab) {
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + idx));
      x[4 * j + 0] = v.x;
      x[4 * j + 1] = v.y;
      x[4 * j + 2] = v.z;
      x[4 * j + 3] = v.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * j + e] = (idx + e < vocab) ? row[idx + e] : -INFINITY;
    }
  }
}

template <bool ALIGNED>
struct LoadSpread {
  __device__ __forceinline__ void operator()(const float* row, int vocab, int base, float* x) const {
    load_spread<ALIGNED>(row, vocab, base, x);
  }
};

template <bool ALIGNED>
__global__ __launch_bounds__(kSpecThreads) void spec_stats_kernel(SpecArgs a) {
  __shared__ float sh[kSpecThreads / kWave];
  const int row = blockIdx.y, ch = blockIdx.x;
  float x[kSpecPer];
  load_spread<ALIGNED>(row_ptr(a, row), a.vocab, ch * kSpecChunk, x);
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < kSpecPer; ++e) { x[e] *= a.c; mx = fmaxf(mx, x[e]); }
  mx = block_reduce_max(mx, sh);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < kSpecPer; ++e) s += exp2f(x[e] - mx);
  s = block_reduce_sum(s, sh);
  if (threadIdx.x == 0) {
    a.part[((int64_t)row * a.nchunk + ch) * 2 + 0] = mx;
    a.part[((int64_t)row * a.nchunk + ch) * 2 + 1] = s;
  }
}

// One wave per sequence. Every row's normaliser is folded at once (eight
// lanes per row, eight rows per pass) and the logits at the drafted tokens
// are fetched up front, so the accept chain itself is a short scan over
// values already on chip.
__global__ __launch_bounds__(kWave) void spec_decide_kernel(SpecArgs a) {
  __shared__ float s_M[2 * kSpecMaxDraft + 1], s_Z[2 * kSpecMaxDraft + 1];
  __shared__ float s_lp[kSpecMaxDraft], s_lq[kSpecMaxDraft];
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int k = a.k;
  const int nrows = 2 * k + 1;  // rows 0..k: verifier rows of b; k+1..2k: drafter rows of b
  auto global_row = [&](int r) { return r <= k ? b * (k + 1) + r : a.batch * (k + 1) + b * k + (r - k - 1); };
  // Logits at the drafts (lanes 0..k-1: verifier, lanes 32..32+k-1: drafter).
  for (int i = lane % 32; i < k; i += 32) {
    const int x = min(max(a.draft[b * k + i], 0), a.vocab - 1);
    const int r = lane < 32 ? i : k + 1 + i;
    const float v = row_ptr(a, global_row(r))[x];
    if (lane < 32) s_lp[i] = v; else s_lq[i] = v;
  }
  // Row normalisers.
  const int sub = lane % 8;
  for (int base = 0; base < nrows; base += 8) {
    const int r = base + lane / 8;
    float m = -INFINITY, z = 0.f;
    if (r < nrows) {
      const float* pr = a.part + (int64_t)global_row(r) * a.nchunk * 2;
      for (int j = sub; j < a.nchunk; j += 8) m = fmaxf(m, pr[2 * j]);
    }
    m = group_max<8>(m);
    if (r < nrows) {
      const float* pr = a.part + (int64_t)global_row(r) * a.nchunk * 2;
      for (int j = sub; j < a.nchunk; j += 8) z += exp2f(pr[2 * j] - m) * pr[2 * j + 1];
    }
    z = group_sum<8>(z);
    if (r < nrows && sub == 0) { s_M[r] = m; s_Z[r] = z; }
  }
  __syncthreads();
  int kept = k;
  {  // products rounded on their own, as in the draw weights
#pragma clang fp contract(off)
    for (int i = 0; i < k; ++i) {
      const float px = exp2f(s_lp[i] * a.c - s_M[i]) / s_Z[i];
      const float qx = exp2f(s_lq[i] * a.c - s_M[k + 1 + i]) / s_Z[k + 1 + i];
      if (!(a.u_accept[b * k + i] * qx < px)) { kept = i; break; }
    }
  }
  if (lane == 0) {
    a.n_accepted[b] = kept;
    a.draw_row[2 * b + 0] = global_row(kept);
    a.draw_row[2 * b + 1] = kept < k ? global_row(k + 1 + kept) : -1;
    a.draw[4 * b + 0] = s_M[kept];
    a.draw[4 * b + 1] = 1.f / s_Z[kept];
    a.draw[4 * b + 2] = kept < k ? s_M[k + 1 + kept] : 0.f;
    a.draw[4 * b + 3] = kept < k ? 1.f / s_Z[k + 1 + kept] : 1.f;
  }
}

// Draw weights of sequence b's draw row at the entries LOAD places in w:
// p_v, or max(0, p_v - q_v) after a rejection unless from_p (the same fp32
// operations for every entry in both layouts).
// Every product is rounded on its own (no fused multiply-add), so identical
// verifier and drafter rows give a residual of exact zeros.
template <typename Load>
__device__ __forceinline__ void draw_weights(const SpecArgs& a, int b, int base, float* w, Load load,
                                             bool from_p = false) {
#pragma clang fp contract(off)
  const int prow = a.draw_row[2 * b + 0], qrow = from_p ? -1 : a.draw_row[2 * b + 1];
  const float Mp = a.draw[4 * b + 0], iZp = a.draw[4 * b + 1];
  float x[kSpecPer];
  load(row_ptr(a, prow), a.vocab, base, x);
#pragma unroll
  for (int e = 0; e < kSpecPer; ++e) w[e] = exp2f(x[e] * a.c - Mp) * iZp;
  if (qrow >= 0) {
    const float Mq = a.draw[4 * b + 2], iZq = a.draw[4 * b + 3];
    load(row_ptr(a, qrow), a.vocab, base, x);
#pragma unroll
    for (int e = 0; e < kSpecPer; ++e) w[e] = fmaxf(w[e] - exp2f(x[e] * a.c - Mq) * iZq, 0.f);
  }
}

template <bool ALIGNED>
__global__ __launch_bounds__(kSpecThreads) void spec_chunk_kernel(SpecArgs a) {
  __shared__ float sh[kSpecThreads / kWave];
  const int b = blockIdx.y, ch = blockIdx.x;
  float w[kSpecPer];
  draw_weights(a, b, ch * kSpecChunk, w, LoadSpread<ALIGNED>());
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < kSpecPer; ++e) s += w[e];
  s = block_reduce_sum(s, sh);
  if (threadIdx.x == 0) a.csum[(int64_t)b * a.nchunk + ch] = s;
}

// Inclusive scan over the block in thread order (wave scans, then the wave
// totals in order): the same fixed order on every run.
__device__ __forceinline__ float block_incl_scan(float x, float* s_tot) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) s_tot[wave] = x;
  __syncthreads();
  float base = 0.f;
  for (int w = 0; w < wave; ++w) base += s_tot[w];
  return base + x;
}

// The chunk holding the draw of target u * total over chunk sums cs (wave 0,
// in chunk order): s_pick (or the last chunk with weight when rounding left
// the target past the total, then s_before = -1; -1 when no chunk has weight),
// s_before = the running sum before the picked chunk, s_target.
__device__ __forceinline__ void pick_chunk(const float* cs, int nchunk, float u, int* s_pick, float* s_before,
                                           float* s_target) {
  const int lane = threadIdx.x % kWave;
  float total = 0.f;  // chunk sums in order (lane-strided partial sums folded in lane order)
  for (int j0 = 0; j0 < nchunk; j0 += kWave) {
    float v = j0 + lane < nchunk ? cs[j0 + lane] : 0.f;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const float y = __shfl_up(v, off);
      if (lane >= off) v += y;
    }
    total += __shfl(v, kWave - 1);
  }
  const float target = u * total;
  int pick = -1, last = -1;
  float before = 0.f, run = 0.f;
  for (int j0 = 0; j0 < nchunk && pick < 0; j0 += kWave) {
    const float c = j0 + lane < nchunk ? cs[j0 + lane] : 0.f;
    float incl = c;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const float y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    const uint64_t hit = __ballot(c > 0.f && run + incl > target);
    const uint64_t pos = __ballot(c > 0.f);
    if (pos) last = j0 + 63 - __clzll((long long)pos);
    if (hit) {
      const int l = __ffsll((long long)hit) - 1;
      pick = j0 + l;
      before = run + __shfl(incl - c, l);
    }
    run += __shfl(incl, kWave - 1);
  }
  if (lane == 0) {
    *s_pick = pick >= 0 ? pick : last;
    *s_before = pick >= 0 ? before : -1.f;  // -1: rounding left the target past the total
    *s_target = target;
  }
}

// One workgroup per sequence: the chunk holding the draw (wave 0 scans the
// chunk sums in order), then the chunk's weights staged through LDS so each
// thread owns 32 consecutive tokens, a block scan in token order, and the
// first token whose running sum passes the target. A rejection whose residual
// has no weight anywhere (p_j <= q_j at every token, p_j = q_j up to
// rounding) draws from p_j instead: its chunk sums are taken here first.
__global__ __launch_bounds__(kSpecThreads) void spec_sample_kernel(SpecArgs a) {
  __shared__ float s_w[kSpecChunk];
  __shared__ float s_tot[kSpecThreads / kWave];
  __shared__ float s_before, s_target;
  __shared__ int s_pick, s_res[2];
  const int b = blockIdx.x;
  float* cs = a.csum + (int64_t)b * a.nchunk;
  if (threadIdx.x < kWave) pick_chunk(cs, a.nchunk, a.u_sample[b], &s_pick, &s_before, &s_target);
  if (threadIdx.x == 0) {
    s_res[0] = INT_MAX;
    s_res[1] = -1;
  }
  __syncthreads();
  const bool from_p = s_pick < 0 && a.draw_row[2 * b + 1] >= 0;
  if (from_p) {
    for (int ch = 0; ch < a.nchunk; ++ch) {
      float w[kSpecPer];
      draw_weights(a, b, ch * kSpecChunk, w, LoadSpread<false>(), true);
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < kSpecPer; ++e) t += w[e];
      t = block_reduce_sum(t, s_tot);
      if (threadIdx.x == 0) cs[ch] = t;
    }
    __threadfence_block();
    __syncthreads();
    if (threadIdx.x < kWave) pick_chunk(cs, a.nchunk, a.u_sample[b], &s_pick, &s_before, &s_target);
    __syncthreads();
  }
  const int pick = s_pick;
  if (pick < 0) {  // no weight anywhere (cannot happen for finite logits: p has positive mass)
    if (threadIdx.x == 0) a.token[b] = -1;
    return;
  }
  const float before = s_before, target = s_target;
  {  // weights of the chunk, loaded coalesced, staged in token order
    float w[kSpecPer];
    draw_weights(a, b, pick * kSpecChunk, w, LoadSpread<false>(), from_p);
#pragma unroll
    for (int j = 0; j < kSpecPer / 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) s_w[4 * threadIdx.x + 4 * kSpecThreads * j + e] = w[4 * j + e];
  }
  __syncthreads();
  float w[kSpecPer];
  float tot = 0.f;
#pragma unroll
  for (int e = 0; e < kSpecPer; ++e) {
    w[e] = s_w[threadIdx.x * kSpecPer + e];
    tot += w[e];
  }
  const float incl = block_incl_scan(tot, s_tot);
  const int i0 = pick * kSpecChunk + (int)threadIdx.x * kSpecPer;
  int found = INT_MAX, lastpos = -1;
  float run = (before < 0.f ? 0.f : before) + (incl - tot);
#pragma unroll
  for (int e = 0; e < kSpecPer; ++e) {
    if (w[e] > 0.f && i0 + e < a.vocab) lastpos = i0 + e;
    run += w[e];
    if (before >= 0.f && found == INT_MAX && run > target && w[e] > 0.f) found = i0 + e;
  }
  if (found != INT_MAX) atomicMin(&s_res[0], found);
  if (lastpos >= 0) atomicMax(&s_res[1], lastpos);
  __syncthreads();
  if (threadIdx.x == 0) a.token[b] = s_res[0] != INT_MAX ? s_res[0] : s_res[1];
}

size_t align256s(size_t v) { return (v + 255) & ~(size_t)255; }
int spec_chunks(int vocab) { return (vocab + kSpecChunk - 1) / kSpecChunk; }

}  // namespace

size_t spec_accept_workspace_bytes(int batch, int k, int vocab) {
  const size_t nch = spec_chunks(vocab);
  const size_t rows = (size_t)batch * (2 * k + 1);
  return align256s(rows * nch * 2 * sizeof(float)) + align256s((size_t)batch * 4 * sizeof(float)) +
         align256s((size_t)batch * 2 * sizeof(int32_t)) + align256s((size_t)batch * nch * sizeof(float));
}

hipError_t launch_spec_accept(const float* p, const float* q, int batch, int k, int vocab, int64_t stride,
                              const int32_t* draft, const float* u_accept, const float* u_sample, float temperature,
                              int32_t* n_accepted, int32_t* token, void* ws, hipStream_t s) {
  SpecArgs a;
  a.p = p;
  a.q = q;
  a.batch = batch;
  a.k = k;
  a.vocab = vocab;
  a.nchunk = spec_chunks(vocab);
  a.stride = stride;
  a.draft = draft;
  a.u_accept = u_accept;
  a.u_sample = u_sample;
  a.c = kLog2e / temperature;
  a.n_accepted = n_accepted;
  a.token = token;
  const size_t rows = (size_t)batch * (2 * k + 1);
  char* base = reinterpret_cast<char*>(ws);
  a.part = reinterpret_cast<float*>(base);
  base += align256s(rows * a.nchunk * 2 * sizeof(float));
  a.draw = reinterpret_cast<float*>(base);
  base += align256s((size_t)batch * 4 * sizeof(float));
  a.draw_row = reinterpret_cast<int32_t*>(base);
  base += align256s((size_t)batch * 2 * sizeof(int32_t));
  a.csum = reinterpret_cast<float*>(base);
  const bool aligned = (reinterpret_cast<uintptr_t>(p) % 16 == 0) && (reinterpret_cast<uintptr_t>(q) % 16 == 0) &&
                       (stride % 4 == 0);
  if (aligned) {
    hipLaunchKernelGGL((spec_stats_kernel<true>), dim3(a.nchunk, (unsigned)rows), dim3(kSpecThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((spec_stats_kernel<false>), dim3(a.nchunk, (unsigned)rows), dim3(kSpecThreads), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(spec_decide_kernel, dim3(batch), dim3(kWave), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (aligned) {
    hipLaunchKernelGGL((spec_chunk_kernel<true>), dim3(a.nchunk, batch), dim3(kSpecThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((spec_chunk_kernel<false>), dim3(a.nchunk, batch), dim3(kSpecThreads), 0, s, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(spec_sample_kernel, dim3(batch), dim3(kSpecThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace spdec
