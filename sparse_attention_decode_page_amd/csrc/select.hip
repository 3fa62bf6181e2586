// Page scoring and top-B page selection.
//
// Score (Quest-style bound; Quest is cited by title on the Sparrow citation-map
// page): s_p = sum_h sum_d max(q_hd*kmax_pd, q_hd*kmin_pd) over the G query
// heads of a KV head. Because kmax >= kmin, the maximum picks kmax exactly when
// q_hd > 0, so s_p = sum_d (kmax_pd*Qpos_d + kmin_pd*Qneg_d) with
// Qpos_d = sum_h max(q_hd,0) and Qneg_d = sum_h min(q_hd,0): two FMAs per
// channel and page instead of 2G. Scoring is a GEMV over 2*D values per page,
// so it streams the page summaries with 16-byte loads and reduces across lanes.
// The sum is accumulated in fp64 and rounded once, so each fp32 score is the
// correctly rounded bound even when products cancel. Vector fp64 FMA runs at
// half the fp32 rate on this chip (78.6 vs 157.3 TFLOP/s); at 2*D FMAs (one
// flop per byte) per 4*D-byte bf16 summary, streaming at 8 TB/s takes about a
// tenth of the fp64 rate, so the pass stays bound by HBM, not ALU.
//
// Selection (Top-k pages under a KV budget, Sparrow project page "Control
// Study 2"; sink/local pages always kept): K = min(max(budget,2), cap, P);
// pages 0 and P-1 are forced, the other K-2 are the largest scores of 1..P-2
// with ties to the lower index. An MSB-first 8-bit radix select on
// order-preserving uint32 keys (offset by the unit's smallest key, so only the
// significant bits take passes: usually 2-3) with LDS histograms finds the
// cut key T and how many keys equal to T are taken; one ordered compaction
// then emits the kept pages already ascending, and equal keys are taken in
// index order, which is the tie rule.
#include "common.h"
#include "launch.h"
#include "scoring.h"
#include "topb.h"
#include "topp.h"

namespace spdec {

namespace {

constexpr int kScorePages = 256;   // pages per scoring workgroup
// Each of the 4 waves scores kScorePages/4 pages, PPI (>= 1) per load.
static_assert(kScorePages % 64 == 0 && kScorePages >= 64, "pages per scoring workgroup");

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void score_pages_kernel(CacheView c, const void* __restrict__ qv,
                                                          float* __restrict__ scores) {
  constexpr int VEC = T::VEC;
  constexpr int LPT = D / VEC;      // lanes per page summary row
  constexpr int PPI = kWave / LPT;  // pages per load instruction
  constexpr int ITERS = kScorePages / 4 / PPI;
  using S = typename T::storage;
  const int unit = blockIdx.y;
  const int b = unit / c.hkv;
  const int g = unit % c.hkv;
  const int L = c.seq_lens[b];
  const int P = min((L + c.page_size - 1) >> c.ps_log2, c.max_pages);
  const int p_begin = blockIdx.x * kScorePages;
  if (p_begin >= P) return;

  __shared__ int s_phys[kScorePages];
  for (int i = threadIdx.x; i < kScorePages; i += blockDim.x) {
    const int p = p_begin + i;
    int phys = -1;
    if (p < P) phys = c.page_table[(int64_t)b * c.max_pages + p];
    s_phys[i] = (phys >= 0 && phys < c.num_phys) ? phys : -1;
  }

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int sub = lane % LPT;
  const int d0 = sub * VEC;
  double qpos[VEC], qneg[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) { qpos[e] = 0.0; qneg[e] = 0.0; }
  const S* q = reinterpret_cast<const S*>(qv);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float f[VEC];
    unpack<T>(load16(q + ((int64_t)b * c.hq + g * G + h) * D + d0), f);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      qpos[e] += (double)fmaxf(f[e], 0.f);
      qneg[e] += (double)fminf(f[e], 0.f);
    }
  }
  __syncthreads();

  const S* mm = reinterpret_cast<const S*>(c.kminmax);
  float* srow = scores + (int64_t)unit * c.max_pages;
#pragma unroll 4
  for (int it = 0; it < ITERS; ++it) {
    const int pl = wave * (kScorePages / 4) + it * PPI + lane / LPT;
    const int phys = s_phys[pl];
    const int64_t row = ((int64_t)(phys < 0 ? 0 : phys) * c.hkv + g) * 2 * D + d0;
    const u32x4 lo = load16_stream(mm + row);
    const u32x4 hi = load16_stream(mm + row + D);
    float fl[VEC], fh[VEC];
    unpack<T>(lo, fl);
    unpack<T>(hi, fh);
    double s = 0.0;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      s = fma((double)fh[e], qpos[e], s);
      s = fma((double)fl[e], qneg[e], s);
    }
    s = group_sum<LPT>(s);
    const int p = p_begin + pl;
    if (sub == 0 && phys >= 0 && p < P) srow[p] = (float)s;
  }
}

// Persistent form of the scoring pass: the (sequence, KV head, page) triples
// are laid end to end and every wave scores one contiguous range of R pages,
// so all waves stream until the end instead of finishing in ragged rounds.
// A workgroup first builds the prefix of per-unit page counts in LDS; a wave
// binary-searches its first unit and walks units until its range ends.
constexpr int kStreamMinPages = 16;

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void score_stream_kernel(CacheView c, const void* __restrict__ qv,
                                                           float* __restrict__ scores) {
  extern __shared__ int s_pre[];  // units + 1
  __shared__ int s_tmp[256 / kWave];
  const int units = c.batch * c.hkv;
  // Four units per thread per pass with clamped (always valid) indices, so
  // that every load of a pass is in flight at once.
  for (int u0 = threadIdx.x; u0 < units; u0 += 4 * blockDim.x) {
    int L[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) L[k] = c.seq_lens[min(u0 + k * (int)blockDim.x, units - 1) / c.hkv];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int u = u0 + k * (int)blockDim.x;
      if (u < units) s_pre[u] = min((max(L[k], 0) + c.page_size - 1) >> c.ps_log2, c.max_pages);
    }
  }
  __syncthreads();
  block_exclusive_scan(s_pre, units, s_tmp);
  const int total = s_pre[units];
  const int lane = threadIdx.x % kWave;
  const int wpb = blockDim.x / kWave;
  const int64_t nw = (int64_t)gridDim.x * wpb;
  const int64_t w = (int64_t)blockIdx.x * wpb + threadIdx.x / kWave;
  const int64_t R = max<int64_t>((total + nw - 1) / nw, kStreamMinPages);
  if (w * R >= total) return;
  int pos = (int)(w * R);
  const int end = (int)min<int64_t>(pos + R, total);
  int u = find_unit(s_pre, units, pos);
  while (pos < end) {
    while (s_pre[u + 1] <= pos) ++u;  // units with no entry have no segment
    const int ubase = s_pre[u];
    const int seg_end = min(end, s_pre[u + 1]);
    score_segment<T, D, G>(c, qv, u / c.hkv, u % c.hkv, pos - ubase, seg_end - ubase,
                           scores + (int64_t)u * c.max_pages, lane);
    pos = seg_end;
    ++u;
  }
}

// Scoring for groups of N consecutive sequences that share their leading
// pages (a prompt sampled N times). Two kinds of units share one stream-K
// space: (group, KV head) units over the group's shared pages, read once
// through the first member's page table and bounded against all N members'
// queries, then (sequence, KV head) units over each sequence's own pages.
// A wave keeps the signed query sums of its unit's members in wave-private
// LDS (only its lanes' channels) and, for every batch of page summaries,
// loops over the members. The arithmetic per (member, page) is the
// single-sequence scoring's: fp64 accumulation in the same order, rounded
// once, so the scores are bit-identical to it.
constexpr int kSharedScoreMaxMembers = 8;

// Orders one wave's LDS writes before its lanes' later reads (and the reverse).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, int G>
__global__ __launch_bounds__(256) void score_grouped_kernel(CacheView c, const void* __restrict__ qv,
                                                            float* __restrict__ scores,
                                                            const int32_t* __restrict__ shared_pages, int N) {
  constexpr int VEC = BF16::VEC;
  constexpr int LPT = D / VEC;
  constexpr int PPI = kWave / LPT;
  constexpr int BATCH = 4;
  static_assert((BATCH * PPI) <= kWave && kWave % (BATCH * PPI) == 0, "batches tile a page-table window");
  using S = BF16::storage;
  extern __shared__ int s_dyn[];  // s_pre: units + 1, then s_first: groups
  __shared__ int s_tmp[256 / kWave];
  // [wave][member][pair k][channel chunk]: pairs 0 .. VEC/2-1 hold the
  // positive sums of the chunk's channels 2k, 2k+1, pairs VEC/2 .. VEC-1 the
  // negative ones. Chunk-minor, so a wave's 16-byte reads are consecutive.
  __shared__ double2 s_qs[256 / kWave][kSharedScoreMaxMembers][VEC][LPT];
  const int groups = c.batch / N;
  const int units_sh = groups * c.hkv;
  const int units = units_sh + c.batch * c.hkv;
  int* s_pre = s_dyn;
  int* s_first = s_dyn + units + 1;
  // Unit sizes. Four units per thread per pass with clamped (always valid)
  // indices, so that every load of a pass is in flight at once.
  for (int u0 = threadIdx.x; u0 < units; u0 += 4 * blockDim.x) {
    int L[4], Sh[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int u = min(u0 + k * (int)blockDim.x, units - 1);
      const int b = u < units_sh ? (u / c.hkv) * N : (u - units_sh) / c.hkv;
      L[k] = c.seq_lens[b];
      Sh[k] = shared_pages[b / N];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int u = u0 + k * (int)blockDim.x;
      if (u < units) {
        const int P = min((max(L[k], 0) + c.page_size - 1) >> c.ps_log2, c.max_pages);
        const int S = max(Sh[k], 0);
        s_pre[u] = u < units_sh ? min(S, P) : max(P - S, 0);
        if (u < units_sh && u % c.hkv == 0) s_first[u / c.hkv] = S;
      }
    }
  }
  __syncthreads();
  block_exclusive_scan(s_pre, units, s_tmp);
  const int total = s_pre[units];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int wpb = blockDim.x / kWave;
  const int64_t nw = (int64_t)gridDim.x * wpb;
  const int64_t w = (int64_t)blockIdx.x * wpb + wave;
  const int64_t R = max<int64_t>((total + nw - 1) / nw, kStreamMinPages);
  if (w * R >= total) return;
  int pos = (int)(w * R);
  const int end = (int)min<int64_t>(pos + R, total);
  int u = find_unit(s_pre, units, pos);
  const int sub = lane % LPT;
  const int d0 = sub * VEC;
  const S* q = reinterpret_cast<const S*>(qv);
  const S* mm = reinterpret_cast<const S*>(c.kminmax);
  while (pos < end) {
    while (s_pre[u + 1] <= pos) ++u;  // units with no entry have no segment
    int b0, g, members, first;
    if (u < units_sh) {
      b0 = (u / c.hkv) * N;
      g = u % c.hkv;
      members = N;
      first = 0;
    } else {
      b0 = (u - units_sh) / c.hkv;
      g = (u - units_sh) % c.hkv;
      members = 1;
      first = s_first[b0 / N];
    }
    const int ubase = s_pre[u];
    const int seg_end = min(end, s_pre[u + 1]);
    const int pb = pos - ubase, pe = seg_end - ubase;
    const int32_t* ptab = c.page_table + (int64_t)b0 * c.max_pages + first;
    // Pages [pb, pe) of this unit's list (pe > pb); page-table entries come
    // 64 at a time, one per lane, read at clamped indices so that no load
    // waits on a branch.
    const int nbatch = (pe - pb + BATCH * PPI - 1) / (BATCH * PPI);
    auto window_raw = [&](int wi) -> int { return ptab[min(pb + wi * kWave + lane, pe - 1)]; };
    auto window_of = [&](int wi, int t) -> int {
      return (pb + wi * kWave + lane < pe && t >= 0 && t < c.num_phys) ? t : -1;
    };
    auto fetch_window = [&](int wi) -> int { return window_of(wi, window_raw(wi)); };
    int raw0 = window_raw(0), raw1 = window_raw(1);
    // Members' signed query sums for this wave's channel chunks, loaded
    // together with the page-table windows.
    constexpr int MPL = (kSharedScoreMaxMembers + PPI - 1) / PPI;  // members per lane
    u32x4 qraw[MPL][G];
#pragma unroll
    for (int k = 0; k < MPL; ++k) {
      const int i = min(lane / LPT + k * PPI, members - 1);
#pragma unroll
      for (int h = 0; h < G; ++h) qraw[k][h] = load16(q + ((int64_t)(b0 + i) * c.hq + g * G + h) * D + d0);
    }
    hold(raw0);
    hold(raw1);
#pragma unroll
    for (int k = 0; k < MPL; ++k) {
#pragma unroll
      for (int h = 0; h < G; ++h) hold(qraw[k][h]);
    }
    wave_sync();  // the previous unit's reads of s_qs are done
#pragma unroll
    for (int k = 0; k < MPL; ++k) {
      const int i = lane / LPT + k * PPI;
      double qpos[VEC], qneg[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) { qpos[e] = 0.0; qneg[e] = 0.0; }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float f[VEC];
        unpack<BF16>(qraw[k][h], f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          qpos[e] += (double)fmaxf(f[e], 0.f);
          qneg[e] += (double)fminf(f[e], 0.f);
        }
      }
      if (i < members) {
#pragma unroll
        for (int kk = 0; kk < VEC / 2; ++kk) {
          s_qs[wave][i][kk][sub] = make_double2(qpos[2 * kk], qpos[2 * kk + 1]);
          s_qs[wave][i][VEC / 2 + kk][sub] = make_double2(qneg[2 * kk], qneg[2 * kk + 1]);
        }
      }
    }
    wave_sync();
    int win0 = window_of(0, raw0), win1 = window_of(1, raw1);
    int cur_win = 0;
    auto issue = [&](int bt, u32x4* lo, u32x4* hi, int* phys) {
      const int wi = (bt * BATCH * PPI) / kWave;
      const int wsrc = wi == cur_win ? win0 : win1;
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        const int pl = (bt * BATCH + i) * PPI + lane / LPT;
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
      if (wnext != cur_win && bt + 1 < nbatch) {
        win0 = win1;
        cur_win = wnext;
        win1 = fetch_window(wnext + 1);
      }
      if (bt + 1 < nbatch) issue(bt + 1, loB, hiB, phB);
      double fl[BATCH][VEC], fh[BATCH][VEC];
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        float tl[VEC], th[VEC];
        unpack<BF16>(loA[i], tl);
        unpack<BF16>(hiA[i], th);
#pragma unroll
        for (int e = 0; e < VEC; ++e) { fl[i][e] = (double)tl[e]; fh[i][e] = (double)th[e]; }
      }
      int st_ph = phA[0];
#pragma unroll
      for (int i = 1; i < BATCH; ++i) st_ph = sub == i ? phA[i] : st_ph;
      const int st_page = pb + (bt * BATCH + sub) * PPI + lane / LPT;
      const bool st_ok = sub < BATCH && st_ph >= 0 && st_page < pe;
      float* srow_m = scores + ((int64_t)b0 * c.hkv + g) * c.max_pages + first + st_page;
      for (int m = 0; m < members; ++m) {
        double qp[VEC], qn[VEC];
#pragma unroll
        for (int k = 0; k < VEC / 2; ++k) {
          const double2 a = s_qs[wave][m][k][sub];
          const double2 b = s_qs[wave][m][VEC / 2 + k][sub];
          qp[2 * k] = a.x; qp[2 * k + 1] = a.y;
          qn[2 * k] = b.x; qn[2 * k + 1] = b.y;
        }
        // BATCH independent chains, each in the single-sequence order.
        double sc[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i) sc[i] = 0.0;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
#pragma unroll
          for (int i = 0; i < BATCH; ++i) {
            sc[i] = fma(fh[i][e], qp[e], sc[i]);
            sc[i] = fma(fl[i][e], qn[e], sc[i]);
          }
        }
        // Every lane of a page's chunk group holds the page's sum; lane sub
        // (< BATCH) of each group stores the score of its group's page in
        // slot sub: one store instruction per member and batch.
        float v = 0.f;
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
          const float r = (float)group_sum<LPT>(sc[i]);
          v = sub == i ? r : v;
        }
        if (st_ok) srow_m[(int64_t)m * c.hkv * c.max_pages] = v;
      }
#pragma unroll
      for (int i = 0; i < BATCH; ++i) { loA[i] = loB[i]; hiA[i] = hiB[i]; phA[i] = phB[i]; }
    }
    pos = seg_end;
    ++u;
  }
}

template <int KPT, int NT>
__global__ __launch_bounds__(NT) void select_topk_reg_kernel(CacheView c, const int32_t* __restrict__ budget,
                                                           int cap, const float* __restrict__ scores,
                                                           int32_t* __restrict__ sel_idx,
                                                           int32_t* __restrict__ sel_cnt) {
  __shared__ TopBShared<NT> sh;
  const int unit = blockIdx.x;
  const int b = unit / c.hkv;
  const int tid = threadIdx.x;
  const int L = c.seq_lens[b];
  const int P = min((max(L, 0) + c.page_size - 1) >> c.ps_log2, c.max_pages);
  int32_t* out = sel_idx + (int64_t)unit * cap;
  const int K = min(min(max(budget[b], 2), cap), P);
  if (K >= P) {
    for (int i = tid; i < P; i += NT) out[i] = i;
    if (tid == 0) sel_cnt[unit] = P;
    return;
  }
  if (tid == 0) {
    out[0] = 0;
    out[K - 1] = P - 1;
    sel_cnt[unit] = K;
  }
  if (K == 2) return;
  uint32_t key[KPT], kmin;
  int nbits;
  load_keys<KPT, NT>(scores + (int64_t)unit * c.max_pages, P - 2, key, kmin, nbits, sh);
  emit_top<KPT, NT>(key, P - 2, K - 2, kmin, nbits, out, sh);
}

// Score-mass (top-p) selection over the same keys (topp.h), one workgroup
// per unit reading the unit's scores.
template <int KPT, int NT>
__global__ __launch_bounds__(NT) void select_topp_reg_kernel(CacheView c, const float* __restrict__ scores,
                                                           float top_p, float score_scale,
                                                           const int32_t* __restrict__ budget, int cap,
                                                           int32_t* __restrict__ sel_idx,
                                                           int32_t* __restrict__ sel_cnt) {
  __shared__ ToppShared<NT> ts;
  const int unit = blockIdx.x;
  const int b = unit / c.hkv;
  const int L = c.seq_lens[b];
  const int P = min((max(L, 0) + c.page_size - 1) >> c.ps_log2, c.max_pages);
  const int kcap = min(min(budget != nullptr ? max(budget[b], 2) : cap, cap), P);
  topp_cut<KPT, NT>(scores + (int64_t)unit * c.max_pages, P, kcap, top_p, score_scale, sel_idx + (int64_t)unit * cap,
                    sel_cnt + unit, ts);
}

template <typename T, int D, int G>
hipError_t score_launch(const CacheView& c, const void* q, float* scores, hipStream_t s) {
  const int units = c.batch * c.hkv;
  if (units <= kMaxStreamUnits) {
    const size_t lds = (size_t)(units + 1) * sizeof(int);
    int grid = 0;
    hipError_t e = persistent_grid(reinterpret_cast<const void*>(&score_stream_kernel<T, D, G>), 256, lds, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((score_stream_kernel<T, D, G>), dim3(grid), dim3(256), lds, s, c, q, scores);
  } else {
    dim3 grid((c.max_pages + kScorePages - 1) / kScorePages, units);
    hipLaunchKernelGGL((score_pages_kernel<T, D, G>), grid, dim3(256), 0, s, c, q, scores);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t score_impl(const CacheView& c, const void* q, float* scores, hipStream_t s) {
  switch (c.group) {
    case 1: return score_launch<T, D, 1>(c, q, scores, s);
    case 2: return score_launch<T, D, 2>(c, q, scores, s);
    case 4: return score_launch<T, D, 4>(c, q, scores, s);
    default: return score_launch<T, D, 8>(c, q, scores, s);
  }
}

template <int D, int G>
hipError_t score_shared_launch(const CacheView& c, const void* q, float* scores, const int32_t* shared_pages, int N,
                               hipStream_t s) {
  const int units = (c.batch / N + c.batch) * c.hkv;
  const size_t lds = (size_t)(units + 1 + c.batch / N) * sizeof(int);
  int grid = 0;
  hipError_t e = persistent_grid(reinterpret_cast<const void*>(&score_grouped_kernel<D, G>), 256, lds, &grid);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((score_grouped_kernel<D, G>), dim3(grid), dim3(256), lds, s, c, q, scores, shared_pages, N);
  return hipGetLastError();
}

template <int D>
hipError_t score_shared_impl(const CacheView& c, const void* q, float* scores, const int32_t* shared_pages, int N,
                             hipStream_t s) {
  switch (c.group) {
    case 1: return score_shared_launch<D, 1>(c, q, scores, shared_pages, N, s);
    case 2: return score_shared_launch<D, 2>(c, q, scores, shared_pages, N, s);
    case 4: return score_shared_launch<D, 4>(c, q, scores, shared_pages, N, s);
    default: return score_shared_launch<D, 8>(c, q, scores, shared_pages, N, s);
  }
}

hipError_t launch_topk(const CacheView& c, const int32_t* budget, int max_budget, const float* scores,
                       int32_t* sel_idx, int32_t* sel_cnt, hipStream_t s);

}  // namespace

size_t select_workspace_bytes(const CacheView& c) {
  return (size_t)c.batch * c.hkv * c.max_pages * sizeof(float);
}

hipError_t launch_score(const CacheView& c, const void* q, float* scores, hipStream_t s) {
  if (c.dtype == SPDEC_BF16)
    return c.head_dim == 64 ? score_impl<BF16, 64>(c, q, scores, s) : score_impl<BF16, 128>(c, q, scores, s);
  return c.head_dim == 64 ? score_impl<F32, 64>(c, q, scores, s) : score_impl<F32, 128>(c, q, scores, s);
}

hipError_t launch_select(const CacheView& c, const void* q, const int32_t* budget, int max_budget, int32_t* sel_idx,
                         int32_t* sel_cnt, float* scores_out, void* ws, hipStream_t s) {
  float* scores = scores_out ? scores_out : reinterpret_cast<float*>(ws);
  hipError_t e = launch_score(c, q, scores, s);
  if (e != hipSuccess) return e;
  return launch_topk(c, budget, max_budget, scores, sel_idx, sel_cnt, s);
}

hipError_t launch_select_top_p(const CacheView& c, const void* q, float top_p, float score_scale,
                               const int32_t* budget, int max_budget, int32_t* sel_idx, int32_t* sel_cnt,
                               float* scores_out, void* ws, hipStream_t s) {
  if (path_fused_supported(c, max_budget))
    return launch_select_topp_fused(c, q, top_p, score_scale, budget, max_budget, sel_idx, sel_cnt, scores_out, s);
  float* scores = scores_out ? scores_out : reinterpret_cast<float*>(ws);
  hipError_t e = launch_score(c, q, scores, s);
  if (e != hipSuccess) return e;
  // Size classes as for the Top-B select (8-32 keys per thread).
  const int middle = c.max_pages - 2;
  const dim3 grid(c.batch * c.hkv);
  if (middle <= 256 * 8) {
    hipLaunchKernelGGL((select_topp_reg_kernel<8, 256>), grid, dim3(256), 0, s, c, scores, top_p, score_scale, budget,
                       max_budget, sel_idx, sel_cnt);
  } else if (middle <= 1024 * 8) {
    hipLaunchKernelGGL((select_topp_reg_kernel<8, 1024>), grid, dim3(1024), 0, s, c, scores, top_p, score_scale,
                       budget, max_budget, sel_idx, sel_cnt);
  } else if (middle <= 1024 * 16) {
    hipLaunchKernelGGL((select_topp_reg_kernel<16, 1024>), grid, dim3(1024), 0, s, c, scores, top_p, score_scale,
                       budget, max_budget, sel_idx, sel_cnt);
  } else {
    hipLaunchKernelGGL((select_topp_reg_kernel<32, 1024>), grid, dim3(1024), 0, s, c, scores, top_p, score_scale,
                       budget, max_budget, sel_idx, sel_cnt);
  }
  return hipGetLastError();
}

bool select_shared_supported(const CacheView& c, int group_size) {
  return c.dtype == SPDEC_BF16 && group_size >= 1 && group_size <= kSharedScoreMaxMembers &&
         c.batch % group_size == 0 && (int64_t)(c.batch / group_size + c.batch) * c.hkv <= kMaxStreamUnits;
}

hipError_t launch_select_shared(const CacheView& c, const void* q, const int32_t* budget, int max_budget,
                                int group_size, const int32_t* shared_pages, int32_t* sel_idx, int32_t* sel_cnt,
                                float* scores_out, void* ws, hipStream_t s) {
  float* scores = scores_out ? scores_out : reinterpret_cast<float*>(ws);
  hipError_t e = c.head_dim == 64 ? score_shared_impl<64>(c, q, scores, shared_pages, group_size, s)
                                  : score_shared_impl<128>(c, q, scores, shared_pages, group_size, s);
  if (e != hipSuccess) return e;
  return launch_topk(c, budget, max_budget, scores, sel_idx, sel_cnt, s);
}

namespace {

hipError_t launch_topk(const CacheView& c, const int32_t* budget, int max_budget, const float* scores,
                       int32_t* sel_idx, int32_t* sel_cnt, hipStream_t s) {
  // Keys per thread stay at 8-32: lists longer than 2048 middle pages take
  // 1024-thread workgroups (with few sequences, each unit's select is then
  // spread over four times the lanes).
  const int middle = c.max_pages - 2;
  const dim3 sgrid(c.batch * c.hkv);
  if (middle <= 256 * 8) {
    hipLaunchKernelGGL((select_topk_reg_kernel<8, 256>), sgrid, dim3(256), 0, s, c, budget, max_budget, scores,
                       sel_idx, sel_cnt);
    return hipGetLastError();
  }
  if (middle <= 1024 * 8) {
    hipLaunchKernelGGL((select_topk_reg_kernel<8, 1024>), sgrid, dim3(1024), 0, s, c, budget, max_budget, scores,
                       sel_idx, sel_cnt);
    return hipGetLastError();
  }
  if (middle <= 1024 * 16) {
    hipLaunchKernelGGL((select_topk_reg_kernel<16, 1024>), sgrid, dim3(1024), 0, s, c, budget, max_budget, scores,
                       sel_idx, sel_cnt);
    return hipGetLastError();
  }
  if (middle <= 1024 * 32) {
    hipLaunchKernelGGL((select_topk_reg_kernel<32, 1024>), sgrid, dim3(1024), 0, s, c, budget, max_budget, scores,
                       sel_idx, sel_cnt);
    return hipGetLastError();
  }
  // The ABI caps the page table at 32768 pages, so the forms above cover every list.
  return hipGetLastError();
}

}  // namespace

}  // namespace spdec
