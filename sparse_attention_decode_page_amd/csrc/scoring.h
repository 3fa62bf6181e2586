// Page scoring of one segment of a unit's pages by one wave (device code
// shared by the scoring kernels and the fused sparse-path kernel).
//
// Score (Quest-style bound; Quest is cited by title on the Sparrow citation-map
// page): s_p = sum_h sum_d max(q_hd*kmax_pd, q_hd*kmin_pd) over the G query
// heads of a KV head, computed as sum_d (kmax_pd*Qpos_d + kmin_pd*Qneg_d) with
// Qpos_d = sum_h max(q_hd,0), Qneg_d = sum_h min(q_hd,0), accumulated in fp64
// and rounded once.
#pragma once

#include "common.h"
#include "launch.h"

namespace spdec {
namespace {

// One wave scores pages [pb, pe) (pe > pb) of unit (b, g) into srow[pb .. pe)
// (srow: global or LDS). The summaries are streamed with 16-byte
// non-temporal loads, PPI pages per load instruction, in batches of BATCH
// instructions with the next batch in flight; page-table entries come 64 at a
// time, one per lane, read at clamped indices so that no load waits on a
// branch, the next window fetched a window ahead and together with the query
// loads (one wait per segment start).
template <typename T, int D, int G>
__device__ __forceinline__ void score_segment(const CacheView& c, const void* qv, int b, int g, int pb, int pe,
                                              float* srow, int lane) {
  constexpr int VEC = T::VEC;
  constexpr int LPT = D / VEC;
  constexpr int PPI = kWave / LPT;
  constexpr int BATCH = 4;  // load instructions (pairs) in flight per batch
  static_assert((BATCH * PPI) <= kWave && kWave % (BATCH * PPI) == 0, "batches tile a page-table window");
  using S = typename T::storage;
  const int sub = lane % LPT;
  const int d0 = sub * VEC;
  const S* q = reinterpret_cast<const S*>(qv);
  const S* mm = reinterpret_cast<const S*>(c.kminmax);
  const int32_t* ptab = c.page_table + (int64_t)b * c.max_pages;
  const int nbatch = (pe - pb + BATCH * PPI - 1) / (BATCH * PPI);
  auto window_raw = [&](int wi) -> int { return ptab[min(pb + wi * kWave + lane, pe - 1)]; };
  auto window_of = [&](int wi, int t) -> int {
    return (pb + wi * kWave + lane < pe && t >= 0 && t < c.num_phys) ? t : -1;
  };
  auto fetch_window = [&](int wi) -> int { return window_of(wi, window_raw(wi)); };
  int raw0 = window_raw(0), raw1 = window_raw(1);
  // The query group's signed sums (loads in flight with the windows').
  u32x4 qraw[G];
#pragma unroll
  for (int h = 0; h < G; ++h) qraw[h] = load16(q + ((int64_t)b * c.hq + g * G + h) * D + d0);
  hold(raw0);
  hold(raw1);
#pragma unroll
  for (int h = 0; h < G; ++h) hold(qraw[h]);
  double qpos[VEC], qneg[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) { qpos[e] = 0.0; qneg[e] = 0.0; }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float f[VEC];
    unpack<T>(qraw[h], f);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      qpos[e] += (double)fmaxf(f[e], 0.f);
      qneg[e] += (double)fminf(f[e], 0.f);
    }
  }
  int win0 = window_of(0, raw0), win1 = window_of(1, raw1);
  int cur_win = 0;
  auto issue = [&](int bt, u32x4* lo, u32x4* hi, int* phys) {
    const int wi = (bt * BATCH * PPI) / kWave;  // a batch never straddles two windows
    const int wsrc = wi == cur_win ? win0 : win1;
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int pl = (bt * BATCH + i) * PPI + lane / LPT;  // page offset in the segment
      phys[i] = __shfl(wsrc, pl & (kWave - 1));
      const int64_t row = ((int64_t)(phys[i] < 0 ? 0 : phys[i]) * c.hkv + g) * 2 * D + d0;
      lo[i] = load16_stream(mm + row);
      hi[i] = load16_stream(mm + row + D);
    }
  };
  u32x4 loA[BATCH], hiA[BATCH], loB[BATCH], hiB[BATCH];
  int phA[BATCH], phB[BATCH];
  issue(0, loA, hiA, phA);
  for (int bt = 0; bt < nbatch; ++bt) {
    const int wnext = ((bt + 1) * BATCH * PPI) / kWave;
    if (wnext != cur_win && bt + 1 < nbatch) {  // next batch opens a new window
      win0 = win1;
      cur_win = wnext;
      win1 = fetch_window(wnext + 1);
    }
    if (bt + 1 < nbatch) issue(bt + 1, loB, hiB, phB);
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      float fl[VEC], fh[VEC];
      unpack<T>(loA[i], fl);
      unpack<T>(hiA[i], fh);
      double sc = 0.0;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        sc = fma((double)fh[e], qpos[e], sc);
        sc = fma((double)fl[e], qneg[e], sc);
      }
      sc = group_sum<LPT>(sc);
      const int pl = (bt * BATCH + i) * PPI + lane / LPT;
      if (sub == 0 && phA[i] >= 0 && pb + pl < pe) srow[pb + pl] = (float)sc;
    }
#pragma unroll
    for (int i = 0; i < BATCH; ++i) { loA[i] = loB[i]; hiA[i] = hiB[i]; phA[i] = phB[i]; }
  }
}

}  // namespace
}  // namespace spdec
