// The sparse path (page scores, Top-B selection, attention over the kept
// pages, merge) in one kernel, for batches of at least one (sequence, KV head)
// unit per compute unit.
//
// Each workgroup (eight waves) owns one unit and runs every step of it with
// the intermediate data in LDS: the waves score the unit's pages into LDS
// (scoring.h), the workgroup selects the Top-B from them (topb.h, ties to the
// lower index, emitted ascending into an LDS list), the waves split the kept
// pages and stream them (stream_window.h), and their partials are merged in
// wave order. No workgroup reads what another wrote, so there is no exchange
// between workgroups and one launch replaces four. Workgroup i takes the unit
// of rank i when units are ordered by the bytes they read (largest first,
// ties to the lower sequence): the dispatcher starts the largest units first
// and the smaller ones fill the compute units as they free up, and units in
// different steps keep HBM busy while others are in their latency-bound
// steps (selection, the first page-table lookups).
//
// Scores, selection and the per-chunk softmax arithmetic are those of
// spdec_select_pages and spdec_sparse_decode; only the split of a unit's
// kept pages into chunks differs, so outputs agree to rounding.
#include "common.h"
#include "launch.h"
#include "scoring.h"
#include "topb.h"
#include "topp.h"
#include "unit_stream.h"

namespace spdec {

namespace {

constexpr int kPathThreads = 512;
constexpr int kPathWaves = kPathThreads / kWave;
// Top-B keys per thread: a unit spreads its P - 2 middle pages over all
// threads, ceil((P - 2) / kPathThreads) each, in registers sized for up to
// 2048 middle pages or for kPathMaxPages pages (the smaller size has the
// shorter loops).
constexpr int kPathKeysShort = 4;
constexpr int kPathKeys = (kPathMaxPages + kPathThreads - 1) / kPathThreads;
static_assert(kPathKeys * kPathThreads + 2 >= kPathMaxPages, "the key registers hold every middle page");

// The need highest of the M = P - 2 middle pages' scores in s_score[1 .. P-1]
// into out[1 .. need], ascending (ties to the lower page).
template <int KPT>
__device__ __forceinline__ void path_top(const float* s_score, int M, int need, int32_t* out,
                                         TopBShared<kPathThreads>& sh) {
  uint32_t key[KPT], kmin;
  int nbits;
  const int kpt = (M + kPathThreads - 1) / kPathThreads;
  load_keys<KPT, kPathThreads>(s_score, M, key, kmin, nbits, sh, kpt);
  emit_top<KPT, kPathThreads>(key, M, need, kmin, nbits, out, sh, kpt);
}

struct PathArgs {
  CacheView c;
  const void* q;
  const int32_t* budget;
  int cap;          // max_budget_pages: row stride of sel_idx
  float qk_scale;   // softmax scale * log2(e)
  int32_t* sel_idx;
  int32_t* sel_cnt;
  float* scores;    // nullable: [batch][Hkv][max_pages]
  float* out;
  float* lse;       // nullable
  int lpt;          // 1: workgroups take units largest first (more units than compute units)
  int stream;       // 1: the whole step; 0: the selection only (no attention)
  int topp;         // 1: the score-mass (top-p) selection only; budget then nullable (caps)
  float top_p, score_scale;
};

// Tokens L, pages P and kept pages K of sequence b, and the bytes one of its
// units reads in units of 4*D bytes (a page summary, or one token's K and V
// row; the summaries only for the selection alone).
__device__ __forceinline__ long long path_work(const PathArgs& a, int b, int& L, int& P, int& K) {
  const CacheView& c = a.c;
  L = max(c.seq_lens[b], 0);
  P = min((L + c.page_size - 1) >> c.ps_log2, c.max_pages);
  K = min(min(a.budget != nullptr ? max(a.budget[b], 2) : a.cap, a.cap), P);
  if (a.topp) return P > 2 ? (long long)P : 0ll;  // the masses need every page's score
  const bool scored = K < P && K > 2;
  return (scored ? (long long)P : 0ll) + (a.stream ? (long long)min(L, K * c.page_size) : 0ll);
}

// s_rank[t] = rank of sequence t when sequences are ordered by path_work,
// largest first, ties to the lower index. The comparisons are split over all
// threads (parts = kPathThreads / B per sequence) and their counts added in
// LDS. Thread t < B (B <= kPathThreads) returns sequence t's L, P, K. Ends
// with a barrier.
__device__ __forceinline__ void rank_sequences(const PathArgs& a, long long* s_work, int* s_rank, int& L, int& P,
                                               int& K) {
  const int tid = threadIdx.x, B = a.c.batch;
  if (tid < B) {
    s_work[tid] = path_work(a, tid, L, P, K);
    s_rank[tid] = 0;
  }
  __syncthreads();
  const int parts = max(1, kPathThreads / B);
  const int chunk = (B + parts - 1) / parts;
  for (int i = tid; i < B * parts; i += kPathThreads) {
    const int t = i % B, part = i / B;
    const long long wt = s_work[t];
    const int lo = part * chunk, hi = min(B, lo + chunk);
    int r = 0;
#pragma unroll 8
    for (int t2 = lo; t2 < hi; ++t2) {
      const long long w2 = s_work[t2];
      r += (w2 > wt || (w2 == wt && t2 < t)) ? 1 : 0;
    }
    if (r != 0) atomicAdd(&s_rank[t], r);
  }
  __syncthreads();
}

// LDS of the per-unit selection.
struct UnitSelectShared {
  float score[kPathMaxPages];
  int list[kPathMaxPages];
  long long work[kPathMaxSeqs];
  int rank[kPathMaxSeqs];
  TopBShared<kPathThreads> sh;
  int seq, L, P, K;
};

// The workgroup's unit (b, g) with its L tokens in P pages, and its kept pages
// (K, ascending) in sm.list, also written to sel_idx / sel_cnt. ptab
// (nullable, LDS) receives the unit's page-table row when the pages are
// scored. Returns false, after writing sel_cnt = 0, for a unit with no token.
// The workgroup's unit: sequence b, KV head g, with L tokens in P pages and K
// (the Top-B count, or the cap for the top-p selection).
__device__ __forceinline__ void unit_resolve(const PathArgs& a, UnitSelectShared& sm, int& b, int& g, int& L, int& P,
                                             int& K) {
  const CacheView& c = a.c;
  const int tid = threadIdx.x;
  const int B = c.batch;
  // The unit: KV head blockIdx % Hkv of the sequence of rank blockIdx / Hkv
  // (with no more units than compute units every unit starts at once, and the
  // rank is the sequence index). The thread that found the unit's sequence
  // passes its shape on in LDS.
  const int want = blockIdx.x / c.hkv;
  g = blockIdx.x % c.hkv;
  if (a.lpt) {
    int tL = 0, tP = 0, tK = 0;
    rank_sequences(a, sm.work, sm.rank, tL, tP, tK);
    if (tid < B && sm.rank[tid] == want) {
      sm.seq = tid;
      sm.L = tL;
      sm.P = tP;
      sm.K = tK;
    }
  } else if (tid == 0) {
    int tL, tP, tK;
    path_work(a, want, tL, tP, tK);
    sm.seq = want;
    sm.L = tL;
    sm.P = tP;
    sm.K = tK;
  }
  __syncthreads();
  b = sm.seq;
  L = sm.L;
  P = sm.P;
  K = sm.K;
}

// The scores of pages [0, P) of unit (b, g) into sm.score, the eight waves
// taking a contiguous share each (ptab, nullable LDS, receives the unit's
// page-table row); written to a.scores too when asked for. Ends with a barrier.
template <int D, int G>
__device__ __forceinline__ void unit_scores(const PathArgs& a, UnitSelectShared& sm, int* ptab, int b, int g, int P,
                                            bool needed) {
  const CacheView& c = a.c;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  if (needed || a.scores != nullptr) {
    const int per = (P + kPathWaves - 1) / kPathWaves;
    const int p0 = min(P, wave * per), p1 = min(P, p0 + per);
    if (p0 < p1) score_segment<BF16, D, G>(c, a.q, b, g, p0, p1, sm.score, lane, ptab);
  }
  __syncthreads();
  if (a.scores != nullptr)
    for (int i = tid; i < P; i += kPathThreads) a.scores[((int64_t)b * c.hkv + g) * c.max_pages + i] = sm.score[i];
}

template <int D, int G>
__device__ __forceinline__ bool unit_selection(const PathArgs& a, UnitSelectShared& sm, int* ptab, int& b, int& g,
                                               int& L, int& P, int& K) {
  const CacheView& c = a.c;
  const int tid = threadIdx.x;
  unit_resolve(a, sm, b, g, L, P, K);
  const int u = b * c.hkv + g;
  if (P == 0) {
    if (tid == 0) a.sel_cnt[u] = 0;
    return false;
  }

  // Scores of the unit's pages (needed by the select, or asked for).
  const bool select = K < P && K > 2;
  unit_scores<D, G>(a, sm, ptab, b, g, P, select);

  // The kept pages, ascending, into list[0 .. K).
  if (K >= P) {
    for (int i = tid; i < P; i += kPathThreads) sm.list[i] = i;
  } else {
    if (tid == 0) {
      sm.list[0] = 0;
      sm.list[K - 1] = P - 1;
    }
    if (select) {
      if (P - 2 <= kPathKeysShort * kPathThreads)
        path_top<kPathKeysShort>(sm.score, P - 2, K - 2, sm.list, sm.sh);
      else
        path_top<kPathKeys>(sm.score, P - 2, K - 2, sm.list, sm.sh);
    }
  }
  __syncthreads();
  for (int i = tid; i < K; i += kPathThreads) a.sel_idx[(int64_t)u * a.cap + i] = sm.list[i];
  if (tid == 0) a.sel_cnt[u] = K;
  return true;
}

template <int D, int G>
__global__ __launch_bounds__(kPathThreads) void sparse_path_kernel(PathArgs a) {
  const CacheView& c = a.c;
  __shared__ UnitSelectShared sm;
  __shared__ int s_ptab[kPathMaxPages];  // the unit's page-table row, when the scoring pass read it
  __shared__ WaveParts<D, G, kPathWaves> s_parts;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  int b, g, L, P, K;
  const bool any = unit_selection<D, G>(a, sm, s_ptab, b, g, L, P, K);
  float* out_rows = a.out + ((int64_t)b * c.hq + g * G) * D;
  float* lse_rows = a.lse != nullptr ? a.lse + (int64_t)b * c.hq + g * G : nullptr;
  if (!any) {  // no token: no page, zero output, lse = ln 0
    for (int i = tid; i < G * D; i += kPathThreads) out_rows[i] = 0.f;
    if (lse_rows != nullptr && tid < G) lse_rows[tid] = -INFINITY;
    return;
  }
  const bool select = K < P && K > 2;
  const int* s_list = sm.list;

  // Attention over the kept pages: wave w streams entries [w*per, (w+1)*per).
  float m[G], lsum[G], acc[G][8];
  const int per = (K + kPathWaves - 1) / kPathWaves;
  const int e0 = min(K, wave * per), e1 = min(K, e0 + per);
  stream_list_range<D, G>(c, a.q, a.qk_scale, b, g, L, P, s_list, nullptr, select ? s_ptab : nullptr, e0, e1, lane, m, lsum,
                          acc);
  store_wave_part<D, G, kPathWaves>(s_parts, wave, lane, m, lsum, acc);
  __syncthreads();

  // Merge of the waves' partials in wave order: o = sum_w 2^(m_w - M) acc_w /
  // sum_w 2^(m_w - M) l_w, lse = ln2 (M + log2 sum_w 2^(m_w - M) l_w).
  for (int i = tid; i < G * D; i += kPathThreads) {
    const int h = i / D, d = i % D;
    float M, Ls, o;
    fold_wave_parts<D, G, kPathWaves>(s_parts, h, d, M, Ls, o);
    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
    out_rows[h * D + d] = o * inv;
    if (lse_rows != nullptr && d == 0) lse_rows[h] = Ls > 0.f ? (M + log2f(Ls)) * kLn2 : -INFINITY;
  }
}

// The selection alone (spdec_select_pages) in one kernel: each workgroup
// scores its unit's pages into LDS and takes the Top-B there, so the scores
// never go through HBM (unless asked for) and one launch replaces two.
template <int D, int G>
__global__ __launch_bounds__(kPathThreads) void select_path_kernel(PathArgs a) {
  __shared__ UnitSelectShared sm;
  int b, g, L, P, K;
  unit_selection<D, G>(a, sm, nullptr, b, g, L, P, K);
}

// The score-mass (top-p) selection (spdec_select_pages_top_p) in one kernel:
// each workgroup scores its unit's pages into LDS and takes the top-p cut
// there.
template <int D, int G>
__global__ __launch_bounds__(kPathThreads) void select_topp_path_kernel(PathArgs a) {
  __shared__ UnitSelectShared sm;
  __shared__ ToppShared<kPathThreads> ts;
  int b, g, L, P, K;
  unit_resolve(a, sm, b, g, L, P, K);
  unit_scores<D, G>(a, sm, nullptr, b, g, P, P > 2);
  const int64_t u = (int64_t)b * a.c.hkv + g;
  // keys spread over every thread: ceil((P - 2) / 512) each, in registers for up to 2048 or 4094 middle pages
  const int kpt = max(1, (P - 2 + kPathThreads - 1) / kPathThreads);
  if (P - 2 <= kPathKeysShort * kPathThreads)
    topp_cut<kPathKeysShort, kPathThreads>(sm.score, P, K, a.top_p, a.score_scale, a.sel_idx + u * a.cap,
                                           a.sel_cnt + u, ts, kpt);
  else
    topp_cut<kPathKeys, kPathThreads>(sm.score, P, K, a.top_p, a.score_scale, a.sel_idx + u * a.cap,
                                      a.sel_cnt + u, ts, kpt);
}

template <int D>
hipError_t path_launch(const PathArgs& a, hipStream_t s) {
  const dim3 grid(a.c.batch * a.c.hkv), block(kPathThreads);
  if (a.topp) {
    switch (a.c.group) {
      case 1: hipLaunchKernelGGL((select_topp_path_kernel<D, 1>), grid, block, 0, s, a); break;
      case 2: hipLaunchKernelGGL((select_topp_path_kernel<D, 2>), grid, block, 0, s, a); break;
      default: hipLaunchKernelGGL((select_topp_path_kernel<D, 4>), grid, block, 0, s, a); break;
    }
  } else if (a.stream) {
    switch (a.c.group) {
      case 1: hipLaunchKernelGGL((sparse_path_kernel<D, 1>), grid, block, 0, s, a); break;
      case 2: hipLaunchKernelGGL((sparse_path_kernel<D, 2>), grid, block, 0, s, a); break;
      default: hipLaunchKernelGGL((sparse_path_kernel<D, 4>), grid, block, 0, s, a); break;
    }
  } else {
    switch (a.c.group) {
      case 1: hipLaunchKernelGGL((select_path_kernel<D, 1>), grid, block, 0, s, a); break;
      case 2: hipLaunchKernelGGL((select_path_kernel<D, 2>), grid, block, 0, s, a); break;
      default: hipLaunchKernelGGL((select_path_kernel<D, 4>), grid, block, 0, s, a); break;
    }
  }
  return hipGetLastError();
}

}  // namespace

bool path_fused_supported(const CacheView& c, int max_budget) {
  const int cus = device_compute_units();
  return cus > 0 && c.dtype == SPDEC_BF16 && c.group <= 4 && c.max_pages <= kPathMaxPages &&
         max_budget <= kPathMaxPages && c.batch <= kPathMaxSeqs && (int64_t)c.batch * c.hkv >= cus;
}

hipError_t launch_sparse_path_fused(const CacheView& c, const void* q, const int32_t* budget, int max_budget,
                                    float scale, int32_t* sel_idx, int32_t* sel_cnt, float* scores, float* out,
                                    float* lse, hipStream_t s) {
  PathArgs a;
  a.c = c;
  a.q = q;
  a.budget = budget;
  a.cap = max_budget;
  a.qk_scale = scale * kLog2e;
  a.sel_idx = sel_idx;
  a.sel_cnt = sel_cnt;
  a.scores = scores;
  a.out = out;
  a.lse = lse;
  a.lpt = (int64_t)c.batch * c.hkv > device_compute_units() ? 1 : 0;
  a.stream = out != nullptr ? 1 : 0;
  a.topp = 0;
  a.top_p = a.score_scale = 0.f;
  return c.head_dim == 64 ? path_launch<64>(a, s) : path_launch<128>(a, s);
}

hipError_t launch_select_topp_fused(const CacheView& c, const void* q, float top_p, float score_scale,
                                    const int32_t* budget, int max_budget, int32_t* sel_idx, int32_t* sel_cnt,
                                    float* scores, hipStream_t s) {
  PathArgs a;
  a.c = c;
  a.q = q;
  a.budget = budget;
  a.cap = max_budget;
  a.qk_scale = 0.f;
  a.sel_idx = sel_idx;
  a.sel_cnt = sel_cnt;
  a.scores = scores;
  a.out = nullptr;
  a.lse = nullptr;
  a.lpt = (int64_t)c.batch * c.hkv > device_compute_units() ? 1 : 0;
  a.stream = 0;
  a.topp = 1;
  a.top_p = top_p;
  a.score_scale = score_scale;
  return c.head_dim == 64 ? path_launch<64>(a, s) : path_launch<128>(a, s);
}

}  // namespace spdec
