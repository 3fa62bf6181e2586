// Score-mass (top-p) page selection of one (sequence, KV head) in one
// workgroup (device code shared by the top-p select kernel and the fused
// top-p selection). The RTPurbo abstract argues for a dynamic top-p over a
// fixed top-k; the page-level form keeps pages 0 and P-1 and takes the middle
// pages in the Top-B order.
//
// The page masses w = exp(c (s - max s)) (fp64, so w <= 1) are summed as
// 2^-48 fixed-point integers: integer sums do not depend on their order,
// which keeps the histograms deterministic under LDS atomics. MSB-first radix
// passes on the keys find the smallest count of middle pages, in the Top-B
// order, whose mass with the two forced pages reaches ceil(top_p * total);
// the count is capped, and emit_top writes that many pages exactly as the
// Top-B select would.
#pragma once

#include "common.h"
#include "topb.h"

namespace spdec {
namespace {

constexpr double kMassOne = 281474976710656.0;  // 2^48

template <int NT>
struct ToppShared {
  TopBShared<NT> sh;
  unsigned long long mass[256];
  unsigned long long msum[NT / kWave];
  float fmax[NT / kWave];
  unsigned long long mabove, wtie;
  int cabove, found;
};

// The top-p selection of a unit with P pages from its scores srow[0 .. P)
// (global memory or LDS): the kept pages, ascending, into out[0 .. K) and K
// into *cnt, the count capped at kcap (2 <= kcap <= P). Middle page i (page
// i + 1) is held by thread i / kpt (kpt <= KPT keys per thread, chosen per
// unit so that a short list spreads over every thread).
template <int KPT, int NT>
__device__ __forceinline__ void topp_cut(const float* srow, int P, int kcap, float top_p, float score_scale,
                                         int32_t* out, int32_t* cnt, ToppShared<NT>& ts, int kpt = KPT) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  if (P <= 2) {
    if (tid < P) out[tid] = tid;
    if (tid == 0) *cnt = P;
    return;
  }
  const int M = P - 2;
  const int nv = held_keys<KPT>(M, kpt);  // keys this thread holds
  uint32_t key[KPT], kmin;
  int nbits;
  load_keys<KPT, NT>(srow, M, key, kmin, nbits, ts.sh, kpt);

  // Masses: the largest score, then fixed-point w for the middle pages.
  float mx = -INFINITY;
  for (int i = tid; i < P; i += NT) mx = fmaxf(mx, srow[i]);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) ts.fmax[wave] = mx;
  __syncthreads();
  mx = ts.fmax[0];
#pragma unroll
  for (int w = 1; w < NT / kWave; ++w) mx = fmaxf(mx, ts.fmax[w]);
  const double cs = (double)score_scale, dm = (double)mx;
  auto fixed_mass = [&](float s) {
    return (unsigned long long)(exp(cs * ((double)s - dm)) * kMassOne + 0.5);
  };
  // Up to 16 keys per thread the masses stay in registers; 32 recompute them
  // (the same value every time) rather than spill. Masses come from the keys
  // the thread holds (key_score inverts score_key; a zero keeps its mass).
  constexpr bool kKeep = KPT <= 16;
  unsigned long long wf[kKeep ? KPT : 1];
  auto mass_of = [&](int r) -> unsigned long long {
    if constexpr (kKeep) {
      return wf[r];
    } else {
      uint32_t k = key[r];
      asm volatile("" : "+v"(k));  // computed where it is used, not carried from an earlier loop
      return r < nv ? fixed_mass(key_score(k)) : 0ull;
    }
  };
  unsigned long long local = 0;
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const unsigned long long m = r < nv ? fixed_mass(key_score(key[r])) : 0ull;
    if constexpr (kKeep) wf[r] = m;
    local += m;
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) local += __shfl_xor(local, off);
  if (lane == 0) ts.msum[wave] = local;
  __syncthreads();
  unsigned long long middle = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) middle += ts.msum[w];
  const unsigned long long forced = fixed_mass(srow[0]) + fixed_mass(srow[P - 1]);
  const double tgt = ceil((double)top_p * (double)(forced + middle));
  int k_mass;
  uint32_t T_mass = 0;
  int eq_mass = 0;
  if ((double)forced >= tgt) {
    k_mass = 0;
  } else {
    // Mass still needed from the middle pages (the crossing exists unless
    // rounding put the target above the whole mass: then every page is kept).
    unsigned long long rem = (unsigned long long)tgt - forced;
    uint32_t prefix = 0, mask = 0;
    int cnt_above = 0;
    bool found = rem <= middle;
    for (int hi = nbits; hi > 0 && found; hi -= 8) {
      const int lo = max(hi - 8, 0);
      const uint32_t dmask = (1u << (hi - lo)) - 1u;
      // hist[2]: the Top-B passes below clear it before they use it; load_keys cleared hist[0] for them.
      for (int i = tid; i < 256; i += NT) { ts.sh.hist[2][i] = 0; ts.mass[i] = 0ull; }
      if (tid == 0) ts.found = 0;
      __syncthreads();
#pragma unroll
      for (int r = 0; r < KPT; ++r) {
        const uint32_t off = key[r] - kmin;
        if (r < nv && (off & mask) == prefix) {
          const uint32_t d = (off >> lo) & dmask;
          atomicAdd(&ts.sh.hist[2][d], 1u);
          atomicAdd(&ts.mass[d], mass_of(r));
        }
      }
      __syncthreads();
      if (tid < kWave) {
        const int top = 255 - 4 * tid;
        const unsigned long long m0 = ts.mass[top], m1 = ts.mass[top - 1], m2 = ts.mass[top - 2], m3 = ts.mass[top - 3];
        const unsigned long long tot = m0 + m1 + m2 + m3;
        unsigned long long incl = tot;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
          const unsigned long long y = __shfl_up(incl, off);
          if (lane >= off) incl += y;
        }
        const unsigned long long excl = incl - tot;
        const int c0 = ts.sh.hist[2][top], c1 = ts.sh.hist[2][top - 1], c2 = ts.sh.hist[2][top - 2];
        const int ctot = c0 + c1 + c2 + ts.sh.hist[2][top - 3];
        const int cincl = wave_incl_scan(ctot);
        const int cexcl = cincl - ctot;
        if (excl < rem && rem <= incl) {
          const unsigned long long rr = rem - excl;
          int digit;
          unsigned long long above;
          int cab;
          if (rr <= m0) { digit = top; above = excl; cab = cexcl; }
          else if (rr <= m0 + m1) { digit = top - 1; above = excl + m0; cab = cexcl + c0; }
          else if (rr <= m0 + m1 + m2) { digit = top - 2; above = excl + m0 + m1; cab = cexcl + c0 + c1; }
          else { digit = top - 3; above = excl + m0 + m1 + m2; cab = cexcl + c0 + c1 + c2; }
          ts.sh.digit = digit;
          ts.mabove = above;
          ts.cabove = cab;
          ts.found = 1;
        }
      }
      __syncthreads();
      found = ts.found != 0;
      if (found) {
        prefix |= (uint32_t)ts.sh.digit << lo;
        mask |= dmask << lo;
        rem -= ts.mabove;
        cnt_above += ts.cabove;
      }
      __syncthreads();
    }
    if (found) {
      // Pages with the threshold key share one score, hence one mass.
      const uint32_t T = kmin + prefix;
#pragma unroll
      for (int r = 0; r < KPT; ++r)
        if (r < nv && key[r] == T) ts.wtie = mass_of(r);
      __syncthreads();
      const unsigned long long wt = ts.wtie;
      eq_mass = wt > 0 ? (int)((rem + wt - 1) / wt) : M;
      k_mass = cnt_above + eq_mass;
      T_mass = T;
    } else {
      k_mass = M;
    }
  }
  const int need = min(min(k_mass, M), kcap - 2);
  const int K = need + 2;
  if (tid == 0) {
    out[0] = 0;
    out[K - 1] = P - 1;
    *cnt = K;
  }
  if (need == 0) return;
  if (need == k_mass && k_mass < M) {
    // The mass decided the count: its threshold key and tie share are the
    // Top-B order's cut for exactly this many pages.
    write_selected<KPT, NT>(key, M, need, T_mass, eq_mass, out, ts.sh, kpt);
  } else {
    emit_top<KPT, NT>(key, M, need, kmin, nbits, out, ts.sh, kpt);
  }}

}  // namespace
}  // namespace spdec
