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
// instruction pairs, over windows of 64 pages whose page-table entries come
// one per lane. Batches alternate between two register sets: the next batch
// is issued before the current one is used, always (past the segment end the
// loads read a valid row that is never used), and each window's entries are
// read two windows ahead, so the loads in flight never sit behind a branch
// and the wait before a batch covers only that batch's loads. Page p's score
// goes to srow[p - srow_base] and, when ptab_out (LDS) is given, its
// page-table entry as read to ptab_out[p - srow_base].
template <typename T, int D, int G>
__device__ __forceinline__ void score_segment(const CacheView& c, const void* qv, int b, int g, int pb, int pe,
                                              float* srow, int lane, int* ptab_out = nullptr, int srow_base = 0) {
  constexpr int VEC = T::VEC;
  constexpr int LPT = D / VEC;
  constexpr int PPI = kWave / LPT;
  constexpr int BATCH = 4;                  // load instruction pairs per batch
  constexpr int NBW = kWave / (BATCH * PPI);  // batches per window
  static_assert(NBW >= 2 && NBW % 2 == 0 && kWave % (BATCH * PPI) == 0, "batches tile a window in pairs");
  using S = typename T::storage;
  const int sub = lane % LPT;
  const int d0 = sub * VEC;
  const S* q = reinterpret_cast<const S*>(qv);
  const S* mm = reinterpret_cast<const S*>(c.kminmax);
  const int32_t* ptab = c.page_table + (int64_t)b * c.max_pages;
  const int nwin = (pe - pb + kWave - 1) / kWave;
  // Page-table entries of window wi, one per lane (index clamped into the segment).
  auto window_raw = [&](int wi) -> int { return ptab[min(pb + wi * kWave + lane, pe - 1)]; };
  auto window_of = [&](int wi, int t) -> int {
    return (pb + wi * kWave + lane < pe && t >= 0 && t < c.num_phys) ? t : -1;
  };
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
  // Batch j of a window: pages (j*BATCH + i)*PPI + lane/LPT of the window, i < BATCH.
  auto issue = [&](int j, int wv, u32x4* lo, u32x4* hi, int* phys) {
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      phys[i] = __shfl(wv, (j * BATCH + i) * PPI + lane / LPT);
      const int64_t row = ((int64_t)(phys[i] < 0 ? 0 : phys[i]) * c.hkv + g) * 2 * D + d0;
      lo[i] = load16_stream(mm + row);
      hi[i] = load16_stream(mm + row + D);
    }
  };
  auto consume = [&](int wi, int j, const u32x4* lo, const u32x4* hi, const int* phys) {
    if (pb + wi * kWave + j * BATCH * PPI >= pe) return;  // batch past the segment end
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      float fl[VEC], fh[VEC];
      unpack<T>(lo[i], fl);
      unpack<T>(hi[i], fh);
      double sc = 0.0;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        sc = fma((double)fh[e], qpos[e], sc);
        sc = fma((double)fl[e], qneg[e], sc);
      }
      sc = group_sum<LPT>(sc);
      const int p = pb + wi * kWave + (j * BATCH + i) * PPI + lane / LPT;
      if (sub == 0 && phys[i] >= 0 && p < pe) srow[p - srow_base] = (float)sc;
    }
  };
  u32x4 loA[BATCH], hiA[BATCH], loB[BATCH], hiB[BATCH];
  int phA[BATCH], phB[BATCH];
  auto keep_window = [&](int wi, int raw) {
    if (ptab_out != nullptr && pb + wi * kWave + lane < pe) ptab_out[pb + wi * kWave + lane - srow_base] = raw;
  };
  keep_window(0, raw0);
  int win = window_of(0, raw0);
  issue(0, win, loA, hiA, phA);
  for (int wi = 0; wi < nwin; ++wi) {
    const int raw2 = window_raw(wi + 2);
    const int win_next = window_of(wi + 1, raw1);  // past the end: no page (-1)
    keep_window(wi + 1, raw1);
#pragma unroll
    for (int j = 0; j < NBW; j += 2) {
      issue(j + 1, win, loB, hiB, phB);
      consume(wi, j, loA, hiA, phA);
      if (j + 2 < NBW) issue(j + 2, win, loA, hiA, phA);
      else issue(0, win_next, loA, hiA, phA);
      consume(wi, j + 1, loB, hiB, phB);
    }
    win = win_next;
    raw1 = raw2;
  }
}

}  // namespace
}  // namespace spdec
