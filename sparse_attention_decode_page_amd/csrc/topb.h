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

// Inclusive prefix sum over the wave on DPP (no LDS traffic): Hillis-Steele
// shifts inside each 16-lane row, then row 0's total into row 1 and row 2's
// into row 3 (row_bcast:15), then rows 0-1's total into rows 2 and 3
// (row_bcast:31). Lanes a step does not write take the `old` operand, 0.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Minimum and maximum over the wave, returned wave-uniform: butterflies
// inside each 16-lane row on DPP, then the four rows' results read out.
__device__ __forceinline__ void wave_min_max(uint32_t& lo, uint32_t& hi) {
  auto step = [&](auto ctrl) {
    constexpr int C = decltype(ctrl)::value;
    lo = min(lo, (uint32_t)__builtin_amdgcn_mov_dpp((int)lo, C, 0xF, 0xF, false));
    hi = max(hi, (uint32_t)__builtin_amdgcn_mov_dpp((int)hi, C, 0xF, 0xF, false));
  };
  step(std::integral_constant<int, kQuadSwap1>{});
  step(std::integral_constant<int, kQuadSwap2>{});
  step(std::integral_constant<int, kRowHalfMirror>{});
  step(std::integral_constant<int, kRowMirror>{});
  uint32_t l = (uint32_t)__builtin_amdgcn_readlane((int)lo, 0), h = (uint32_t)__builtin_amdgcn_readlane((int)hi, 0);
#pragma unroll
  for (int r = 16; r < kWave; r += 16) {
    l = min(l, (uint32_t)__builtin_amdgcn_readlane((int)lo, r));
    h = max(h, (uint32_t)__builtin_amdgcn_readlane((int)hi, r));
  }
  lo = l;
  hi = h;
}

// Top-B select for P - 2 <= NT * kpt middle pages, one workgroup of NT threads
// per (sequence, KV head), keys in registers (up to KPT per thread). Thread t
// holds the keys of middle pages [t*kpt, t*kpt + kpt) (index order, so the
// compaction emits ascending pages); kpt <= KPT may be chosen per unit so that
// a register array sized for the longest list spreads a shorter one over all
// threads. Radix digits are taken on
// key - min_key: the span of real scores is a few exponent steps, so the first
// 8-bit digit already spreads the keys over the histogram and 2-3 passes
// usually suffice.
// Keys this thread holds: middle pages tid*kpt .. of M, at most kpt.
template <int KPT>
__device__ __forceinline__ int held_keys(int M, int kpt) {
  return min(max(M - (int)threadIdx.x * kpt, 0), min(kpt, KPT));
}

template <int NT>
struct TopBShared {
  uint32_t hist[3][256];  // radix pass p counts into hist[p % 3]
  uint32_t red[NT / kWave][2];
  int digit, above;
  int wave_sums[NT / kWave][2];
};

// The keys of middle pages 1 .. M (M = P - 2) and their block minimum and
// significant bit count.
template <int KPT, int NT>
__device__ __forceinline__ void load_keys(const float* srow, int M, uint32_t (&key)[KPT], uint32_t& kmin, int& nbits,
                                          TopBShared<NT>& sh, int kpt = KPT) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int i0 = tid * kpt, nv = held_keys<KPT>(M, kpt);
  kmin = 0xFFFFFFFFu;
  uint32_t kmax = 0u;
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    key[r] = r < nv ? score_key(srow[i0 + r + 1]) : 0u;
    if (r < nv) { kmin = min(kmin, key[r]); kmax = max(kmax, key[r]); }
  }
  wave_min_max(kmin, kmax);
  if (lane == 0) { sh.red[wave][0] = kmin; sh.red[wave][1] = kmax; }
  for (int i = tid; i < 256; i += NT) sh.hist[0][i] = 0;  // the first radix pass's counts
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
                                               int32_t* out, TopBShared<NT>& sh, int kpt = KPT);

// Writes the `need` highest keys of the middle pages (equal keys in page
// order) ascending to out[1 .. need].
//
// One barrier per radix pass: pass p counts into hist[p % 3] while clearing
// hist[(p + 1) % 3] (last read by pass p - 2's scans, which every wave
// finished before the barrier of pass p - 1), and after the barrier every
// wave scans the 256 counts itself, so the cut digit needs no broadcast. The
// passes stop early once every key left under the resolved prefix is taken.
template <int KPT, int NT>
__device__ __forceinline__ void emit_top(const uint32_t (&key)[KPT], int M, int need, uint32_t kmin, int nbits,
                                         int32_t* out, TopBShared<NT>& sh, int kpt = KPT) {
  const int tid = threadIdx.x, lane = tid % kWave;
  const int nv = held_keys<KPT>(M, kpt);
  uint32_t prefix = 0, mask = 0;
  int remaining = need;
  uint32_t T = kmin;  // cut key: all keys above it are taken, then eq_take keys equal to it
  int eq_take = 0;
  int p = 0;
  for (int hi = nbits; hi > 0; hi -= 8, ++p) {
    const int lo = max(hi - 8, 0);
    const uint32_t dmask = (1u << (hi - lo)) - 1u;
    uint32_t* H = sh.hist[p % 3];
    for (int i = tid; i < 256; i += NT) sh.hist[(p + 1) % 3][i] = 0;
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const uint32_t off = key[r] - kmin;
      if (r < nv && (off & mask) == prefix) atomicAdd(&H[(off >> lo) & dmask], 1u);
    }
    __syncthreads();
    // Lane l of every wave holds digits 255-4l .. 252-4l; the cut is the digit
    // at which the count of higher keys first reaches `remaining`.
    const int top = 255 - 4 * lane;
    const int c0 = H[top], c1 = H[top - 1], c2 = H[top - 2], c3 = H[top - 3];
    const int tot = c0 + c1 + c2 + c3;
    const int incl = wave_incl_scan(tot);
    const int excl = incl - tot;
    const bool mine = excl < remaining && remaining <= incl;
    int digit = 0, above = 0, cnt = 0;
    if (mine) {
      const int rr = remaining - excl;
      if (rr <= c0) { digit = top; above = excl; cnt = c0; }
      else if (rr <= c0 + c1) { digit = top - 1; above = excl + c0; cnt = c1; }
      else if (rr <= c0 + c1 + c2) { digit = top - 2; above = excl + c0 + c1; cnt = c2; }
      else { digit = top - 3; above = excl + c0 + c1 + c2; cnt = c3; }
    }
    const int src = __builtin_ctzll(__ballot(mine));  // exactly one lane: 0 < remaining <= total
    digit = __builtin_amdgcn_readlane(digit, src);
    above = __builtin_amdgcn_readlane(above, src);
    cnt = __builtin_amdgcn_readlane(cnt, src);
    prefix |= (uint32_t)digit << lo;
    mask |= dmask << lo;
    remaining -= above;
    if (cnt == remaining && prefix != 0) {
      // Every key under the prefix is taken: keys >= kmin + prefix, none by tie.
      T = kmin + prefix - 1u;
      eq_take = 0;
      remaining = 0;
      break;
    }
    T = kmin + prefix;
    eq_take = remaining;
  }
  if (nbits == 0) eq_take = remaining;  // every key equal: take the first `need` in page order
  write_selected<KPT, NT>(key, M, need, T, eq_take, out, sh, kpt);
}

// Writes the middle pages with key > T and the first eq_take pages with key
// == T (page order) ascending to out[1 .. need].
template <int KPT, int NT>
__device__ __forceinline__ void write_selected(const uint32_t (&key)[KPT], int M, int need, uint32_t T, int eq_take,
                                               int32_t* out, TopBShared<NT>& sh, int kpt) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int i0 = tid * kpt, nv = held_keys<KPT>(M, kpt);
  int gt = 0, eq = 0;
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    if (r < nv) { gt += key[r] > T; eq += key[r] == T; }
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
    if (r < nv) {
      bool take = key[r] > T;
      if (key[r] == T) { take = eq_seen < eq_take; ++eq_seen; }
      if (take && pos <= need) out[pos++] = i0 + r + 1;
    }
  }
}

}  // namespace
}  // namespace spdec
