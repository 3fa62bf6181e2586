// Score-mass (top-p) page selection.
//
// The RTPurbo abstract on the first page of the source set argues that the
// useful token budget depends strongly on the query, so a dynamic top-p
// selection suits better than a fixed top-k. The page-level form here is a
// reading: the page scores (the same Quest-style bounds the Top-B selection
// uses) act as logits of the pages' attention mass, w_p = exp(c (s_p - max s)),
// pages 0 and P-1 are always kept, and the other pages are taken in the Top-B
// order (score descending, lower index first) until the kept mass reaches
// top_p times the total, at most the per-sequence cap.
//
// One workgroup per (sequence, KV head): the middle pages' (score key, page)
// pairs are sorted in LDS (bitonic, descending on a 64-bit key that puts the
// lower page first on equal scores), their masses are summed in fp64 in the
// sorted order with fixed-order block scans (deterministic), the first
// position where the kept mass reaches the target fixes the count, and the
// kept pages are written ascending by an ordered compaction over page flags.
#include "common.h"
#include "launch.h"

namespace spdec {

namespace {

__device__ __forceinline__ double wave_incl_scan_f64(double x) {
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const double y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ int wave_incl_scan_i32(int x) {
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ int page_of(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }

template <int NT, int MAXM>
__global__ __launch_bounds__(NT) void select_topp_kernel(CacheView c, const float* __restrict__ scores, float top_p,
                                                         float score_scale, const int32_t* __restrict__ budget,
                                                         int cap, int32_t* __restrict__ sel_idx,
                                                         int32_t* __restrict__ sel_cnt) {
  constexpr int NW = NT / kWave;
  __shared__ uint64_t s_key[MAXM];
  __shared__ uint8_t s_flag[MAXM];
  __shared__ double s_dsum[NW];
  __shared__ int s_isum[NW];
  __shared__ float s_fmax[NW];
  __shared__ int s_first[NW];
  const int unit = blockIdx.x;
  const int b = unit / c.hkv;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int L = c.seq_lens[b];
  const int P = min((max(L, 0) + c.page_size - 1) >> c.ps_log2, c.max_pages);
  int32_t* out = sel_idx + (int64_t)unit * cap;
  if (P <= 2) {
    if (tid < P) out[tid] = tid;
    if (tid == 0) sel_cnt[unit] = P;
    return;
  }
  const int kcap = min(min(budget != nullptr ? max(budget[b], 2) : cap, cap), P);
  const float* srow = scores + (int64_t)unit * c.max_pages;
  const int M = P - 2;
  int N2 = 1;
  while (N2 < M) N2 <<= 1;

  // Largest score of the P pages.
  float mx = -INFINITY;
  for (int i = tid; i < P; i += NT) mx = fmaxf(mx, srow[i]);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) s_fmax[wave] = mx;
  // Keys of the middle pages 1 .. P-2 (padding sorts last).
  for (int i = tid; i < N2; i += NT) {
    uint64_t k = 0;
    if (i < M) {
      const int page = i + 1;
      k = ((uint64_t)score_key(srow[page]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)page);
      s_flag[i] = 0;
    }
    s_key[i] = k;
  }
  __syncthreads();
  mx = s_fmax[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) mx = fmaxf(mx, s_fmax[w]);

  // Bitonic sort, descending.
  for (int kk = 2; kk <= N2; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int t = tid; t < N2 / 2; t += NT) {
        const int i = ((t & ~(jj - 1)) << 1) | (t & (jj - 1));
        const int l = i + jj;
        const uint64_t x = s_key[i], y = s_key[l];
        const bool desc = (i & kk) == 0;
        if (desc ? (x < y) : (x > y)) {
          s_key[i] = y;
          s_key[l] = x;
        }
      }
      __syncthreads();
    }
  }

  // Masses in the sorted order: thread tid owns sorted positions [j0, j1).
  const double cs = (double)score_scale, dm = (double)mx;
  auto mass = [&](int page) { return exp(cs * ((double)srow[page] - dm)); };
  const int per = (M + NT - 1) / NT;
  const int j0 = min(tid * per, M), j1 = min(j0 + per, M);
  double local = 0.0;
  for (int j = j0; j < j1; ++j) local += mass(page_of(s_key[j]));
  const double incl = wave_incl_scan_f64(local);
  if (lane == kWave - 1) s_dsum[wave] = incl;
  __syncthreads();
  double before = incl - local, mid_total = 0.0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w < wave) before += s_dsum[w];
    mid_total += s_dsum[w];
  }
  const double forced = mass(0) + mass(P - 1);
  const double target = (double)top_p * (forced + mid_total);

  // First sorted position at which the kept mass reaches the target.
  int first = M;
  if (!(forced >= target)) {
    double run = forced + before;
    for (int j = j0; j < j1; ++j) {
      run += mass(page_of(s_key[j]));
      if (run >= target) {
        first = j;
        break;
      }
    }
  } else {
    first = -1;
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) first = min(first, __shfl_xor(first, off));
  if (lane == 0) s_first[wave] = first;
  __syncthreads();
  first = s_first[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) first = min(first, s_first[w]);
  const int k = min(first + 1, min(M, kcap - 2));  // middle pages kept

  for (int j = tid; j < k; j += NT) s_flag[page_of(s_key[j]) - 1] = 1;
  __syncthreads();
  // Ordered compaction of the flagged middle pages, ascending.
  const int i0 = min(tid * per, M), i1 = min(i0 + per, M);
  int cnt = 0;
  for (int i = i0; i < i1; ++i) cnt += s_flag[i];
  const int cincl = wave_incl_scan_i32(cnt);
  if (lane == kWave - 1) s_isum[wave] = cincl;
  __syncthreads();
  int pos = 1 + cincl - cnt;
  for (int w = 0; w < wave; ++w) pos += s_isum[w];
  for (int i = i0; i < i1; ++i)
    if (s_flag[i]) out[pos++] = i + 1;
  if (tid == 0) {
    out[0] = 0;
    out[k + 1] = P - 1;
    sel_cnt[unit] = k + 2;
  }
}

}  // namespace

hipError_t launch_select_top_p(const CacheView& c, const void* q, float top_p, float score_scale,
                               const int32_t* budget, int max_budget, int32_t* sel_idx, int32_t* sel_cnt,
                               float* scores_out, void* ws, hipStream_t s) {
  float* scores = scores_out ? scores_out : reinterpret_cast<float*>(ws);
  hipError_t e = launch_score(c, q, scores, s);
  if (e != hipSuccess) return e;
  const dim3 grid(c.batch * c.hkv);
  if (c.max_pages - 2 <= 2048) {
    hipLaunchKernelGGL((select_topp_kernel<256, 2048>), grid, dim3(256), 0, s, c, scores, top_p, score_scale, budget,
                       max_budget, sel_idx, sel_cnt);
  } else {
    hipLaunchKernelGGL((select_topp_kernel<512, kTopPMaxMiddle>), grid, dim3(512), 0, s, c, scores, top_p,
                       score_scale, budget, max_budget, sel_idx, sel_cnt);
  }
  return hipGetLastError();
}

}  // namespace spdec
