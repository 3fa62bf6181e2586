// Attention over one unit's kept-page list by the waves of one workgroup
// (device code shared by the one-kernel sparse step and the sliced step).
//
// Each wave streams a contiguous range of the list's entries with the decode's
// window code (stream_window.h) into its own online-softmax partial; the
// partials meet in LDS and are folded in wave order:
//   M = max_w m_w,  l = sum_w 2^(m_w - M) l_w,  acc = sum_w 2^(m_w - M) acc_w
// (m in log2 units of the scaled scores).
#pragma once

#include "common.h"
#include "launch.h"
#include "stream_window.h"

namespace spdec {
namespace {

template <int D, int G, int NW>
struct WaveParts {
  float acc[NW][G][D];
  float ml[NW][G][2];
};

// One wave's partial over entries [e0, e1) of `list` (logical pages, LDS) of
// unit (b, g) with L tokens in P pages. An entry's physical page comes from
// lphys (nullable, LDS: the page-table entry of each list entry), else from
// ptab (nullable, LDS: the unit's page-table row), else from the page table.
// Leaves the closed partial in m, lsum, acc (m = kNegBig, zeros for an empty
// range).
template <int D, int G>
__device__ __forceinline__ void stream_list_range(const CacheView& c, const void* q, float qk_scale, int b, int g,
                                                  int L, int P, const int* list, const int* lphys, const int* ptab,
                                                  int e0, int e1, int lane, float (&m)[G], float (&lsum)[G],
                                                  float (&acc)[G][8]) {
  constexpr int NJ = D / 32;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
    lsum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
  if (e0 >= e1) return;
  const int r16 = lane % 16, q4 = lane / 16;
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(q);
  u32x4 qa[NJ];  // A operands: row r16 holds query head r16 % G
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj)
    qa[jj] = load16(qp + ((int64_t)b * c.hq + g * G + r16 % G) * D + 32 * jj + 8 * q4);
  for (int wb = e0; wb < e1; wb += kWave) {
    // Window of up to 64 entries: lane i holds entry wb+i's physical page and valid tokens.
    const int nwin = min(kWave, e1 - wb);
    const int ei = min(wb + lane, e1 - 1);
    const int logical = list[ei];
    const int ph = lphys != nullptr ? lphys[ei]
                   : ptab != nullptr
                       ? ptab[min(max(logical, 0), P - 1)]
                       : c.page_table[(int64_t)b * c.max_pages + min(max(logical, 0), c.max_pages - 1)];
    const bool ok = lane < nwin && logical >= 0 && logical < P && ph >= 0 && ph < c.num_phys;
    const int phys_w = ok ? ph : 0;
    const int valid_w = ok ? min(c.page_size, L - logical * c.page_size) : 0;
    stream_window<D, G>(c, g, nwin, phys_w, valid_w, qa, qk_scale, lane, m, lsum, acc);
  }
  close_segment<D, G>(lsum, acc);
}

// Stores wave `wave`'s closed partial into the workgroup's LDS slots.
template <int D, int G, int NW>
__device__ __forceinline__ void store_wave_part(WaveParts<D, G, NW>& parts, int wave, int lane, const float (&m)[G],
                                                const float (&lsum)[G], const float (&acc)[G][8]) {
  constexpr int LPT = D / 8;
  const int vsub = lane % LPT, vtok = lane / LPT;
  if (vtok == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) parts.acc[wave][h][8 * vsub + e] = acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      parts.ml[wave][h][0] = m[h];
      parts.ml[wave][h][1] = lsum[h];
    }
  }
}

// The waves' partials of head h, channel d folded in wave order (after a
// barrier that follows every store_wave_part).
template <int D, int G, int NW>
__device__ __forceinline__ void fold_wave_parts(const WaveParts<D, G, NW>& parts, int h, int d, float& M, float& Ls,
                                                float& o) {
  M = kNegBig;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, parts.ml[w][h][0]);
  Ls = 0.f;
  o = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float wt = exp2f(parts.ml[w][h][0] - M);
    Ls = fmaf(wt, parts.ml[w][h][1], Ls);
    o = fmaf(wt, parts.acc[w][h][d], o);
  }
}

}  // namespace
}  // namespace spdec
