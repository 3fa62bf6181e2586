// Top-B page selection in one workgroup (device code shared by the select
// kernels and the fused sparse-path kernel).
//
// Selection (Top-k pages under a KV budget, Sparrow project page "Control
// Study 2"; sink and local pages always kept): the K - 2 largest scores of
// the middle pages 1 .. P-2, ties to the lower index, emitted ascending.
#pragma once

#include "common.h"

namespace spdec {
namespace {

__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Top-B select for P - 2 <= NT * KPT middle pages, one workgroup of NT threads
// per (sequence, KV head), keys in registers. Thread t holds the keys of
// middle pages [t*KPT, t*KPT + KPT) (index order, so the compaction emits
// ascending pages). Radix digits are taken on
// key - min_key: the span of real scores is a few exponent steps, so the first
// 8-bit digit already spreads the keys over the histogram and 2-3 passes
// usually suffice.
template <int NT>
struct TopBShared {
  uint32_t hist[256];
  uint32_t red[NT / kWave][2];
  int digit, above;
  int wave_sums[NT / kWave][2];
};

// The keys of middle pages 1 .. M (M = P - 2) and their block minimum and
// significant bit count.
template <int KPT, int NT>
__device__ __forceinline__ void load_keys(const float* srow, int M, uint32_t (&key)[KPT], uint32_t& kmin, int& nbits,
                                          TopBShared<NT>& sh) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int i0 = tid * KPT;
  kmin = 0xFFFFFFFFu;
  uint32_t kmax = 0u;
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const int i = i0 + r;
    key[r] = i < M ? score_key(srow[i + 1]) : 0u;
    if (i < M) { kmin = min(kmin, key[r]); kmax = max(kmax, key[r]); }
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
  }
  if (lane == 0) { sh.red[wave][0] = kmin; sh.red[wave][1] = kmax; }
  __syncthreads();
  kmin = sh.red[0][0];
  kmax = sh.red[0][1];
#pragma unroll
  for (int w = 1; w < NT / kWave; ++w) { kmin = min(kmin, sh.red[w][0]); kmax = max(kmax, sh.red[w][1]); }
  const uint32_t span = kmax - kmin;
  nbits = span == 0 ? 0 : 32 - __clz((int)span);
  __syncthreads();  // red is reused
}

template <int KPT, int NT>
__device__ __forceinline__ void write_selected(const uint32_t (&key)[KPT], int M, int need, uint32_t T, int eq_take,
                                               int32_t* out, TopBShared<NT>& sh);

// Writes the `need` highest keys of the middle pages (equal keys in page
// order) ascending to out[1 .. need].
template <int KPT, int NT>
__device__ __forceinline__ void emit_top(const uint32_t (&key)[KPT], int M, int need, uint32_t kmin, int nbits,
                                         int32_t* out, TopBShared<NT>& sh) {
  const int tid = threadIdx.x;
  const int i0 = tid * KPT;
  uint32_t prefix = 0, mask = 0;
  int remaining = need;
  for (int hi = nbits; hi > 0; hi -= 8) {
    const int lo = max(hi - 8, 0);
    const uint32_t dmask = (1u << (hi - lo)) - 1u;
    for (int i = tid; i < 256; i += NT) sh.hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const uint32_t off = key[r] - kmin;
      if (i0 + r < M && (off & mask) == prefix) atomicAdd(&sh.hist[(off >> lo) & dmask], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      const int top = 255 - 4 * tid;
      const int c0 = sh.hist[top], c1 = sh.hist[top - 1], c2 = sh.hist[top - 2], c3 = sh.hist[top - 3];
      const int tot = c0 + c1 + c2 + c3;
      const int incl = wave_incl_scan(tot);
      const int excl = incl - tot;
      if (excl < remaining && remaining <= incl) {
        const int rr = remaining - excl;
        int digit, above;
        if (rr <= c0) { digit = top; above = excl; }
        else if (rr <= c0 + c1) { digit = top - 1; above = excl + c0; }
        else if (rr <= c0 + c1 + c2) { digit = top - 2; above = excl + c0 + c1; }
        else { digit = top - 3; above = excl + c0 + c1 + c2; }
        sh.digit = digit;
        sh.above = above;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sh.digit << lo;
    mask |= dmask << lo;
    remaining -= sh.above;
    __syncthreads();
  }
  write_selected<KPT, NT>(key, M, need, kmin + prefix, remaining, out, sh);
}

// Writes the middle pages with key > T and the first eq_take pages with key
// == T (page order) ascending to out[1 .. need].
template <int KPT, int NT>
__device__ __forceinline__ void write_selected(const uint32_t (&key)[KPT], int M, int need, uint32_t T, int eq_take,
                                               int32_t* out, TopBShared<NT>& sh) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int i0 = tid * KPT;
  int gt = 0, eq = 0;
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    if (i0 + r < M) { gt += key[r] > T; eq += key[r] == T; }
  }
  const int gt_incl = wave_incl_scan(gt);
  const int eq_incl = wave_incl_scan(eq);
  if (lane == kWave - 1) { sh.wave_sums[wave][0] = gt_incl; sh.wave_sums[wave][1] = eq_incl; }
  __syncthreads();
  int gt_before = gt_incl - gt, eq_before = eq_incl - eq;
  for (int w = 0; w < wave; ++w) { gt_before += sh.wave_sums[w][0]; eq_before += sh.wave_sums[w][1]; }
  int pos = 1 + gt_before + min(eq_before, eq_take);
  int eq_seen = eq_before;
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    if (i0 + r < M) {
      bool take = key[r] > T;
      if (key[r] == T) { take = eq_seen < eq_take; ++eq_seen; }
      if (take && pos <= need) out[pos++] = i0 + r + 1;
    }
  }
}

}  // namespace
}  // namespace spdec
