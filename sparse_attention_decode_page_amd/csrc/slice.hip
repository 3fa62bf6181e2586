// The sparse path for batches of few (sequence, KV head) units: each unit is
// cut into S page slices, S workgroups per unit, so that every compute unit
// takes part although the units are far fewer than the compute units.
//
// Selection (Top-k pages under a KV budget, Sparrow project page "Control
// Study 2"; sink and local pages always kept) in two steps, with no exchange
// inside a kernel:
//   1. slice_score_kernel: workgroup (unit, s) scores pages
//      [s*per, (s+1)*per) into LDS (the scoring segment) and keeps the
//      slice's own top need = K - 2 middle pages by (score desc, index asc),
//      the slice's candidates (all its middle pages when it has no more).
//      Every page of the unit's global top need is among its slice's
//      candidates: a page the slice dropped has need pages of its own slice
//      above it in the same order.
//   2. slice_select_kernel: each workgroup of the unit takes the same top
//      need of the unit's candidates (in page order, so the order's ties
//      are the global tie rule) with the Top-B cut, which gives exactly the
//      selection of spdec_select_pages; workgroup 0 writes it. In the
//      streaming form workgroup s then attends over entries
//      [s*K/S, (s+1)*K/S) of the list (the decode's window code) and stores
//      its partial in the decode's partial layout, which the stream merge
//      folds in slice order. (Folding the partials in the unit's last
//      workgroup to finish instead, behind device-scope stores and an
//      arrival counter, saved 1 µs of 61 on the 131K-token cache: the
//      exchange costs about what the merge launch does.)
#include <algorithm>

#include "common.h"
#include "launch.h"
#include "scoring.h"
#include "topb.h"
#include "unit_stream.h"

namespace spdec {

namespace {

constexpr int kSliceThreads = 512;
constexpr int kSliceWaves = kSliceThreads / kWave;
constexpr int kSliceKeysShort = 4;
constexpr int kSliceKeys = (kSliceMaxCand + kSliceThreads - 1) / kSliceThreads;
static_assert(kSliceKeys * kSliceThreads >= kSliceMaxCand, "the key registers hold every candidate");
static_assert(kSliceKeys * kSliceThreads >= kSliceMaxPages, "the key registers hold a slice's middle pages");

struct SliceArgs {
  CacheView c;
  const void* q;
  const int32_t* budget;
  int cap;            // max_budget_pages: row stride of sel_idx
  int S;              // slices per unit
  int per;            // pages per slice
  int cstride;        // candidate slots per slice (cap - 2)
  float qk_scale;     // softmax scale * log2(e)
  int32_t* cand_page; // [units][S][cstride]
  float* cand_score;  // [units][S][cstride]
  int32_t* cand_phys; // [units][S][cstride]: the candidate's page-table entry
  int32_t* cand_cnt;  // [units][S]
  int32_t* sel_idx;
  int32_t* sel_cnt;
  float* scores;      // nullable: [batch][Hkv][max_pages]
  float* part_acc;    // [units][S][G][D]
  float* part_ml;     // [units][S][G][2]
  int32_t* count;     // [units]: partials written (S; 0 for a unit with no token)
};

__device__ __forceinline__ void unit_shape(const SliceArgs& a, int u, int& b, int& g, int& L, int& P, int& K) {
  const CacheView& c = a.c;
  b = u / c.hkv;
  g = u % c.hkv;
  L = max(c.seq_lens[b], 0);
  P = min((L + c.page_size - 1) >> c.ps_log2, c.max_pages);
  K = min(min(max(a.budget[b], 2), a.cap), P);
}

// The need highest of M keys whose scores are srow[1 .. M] into out[1 .. need]
// as positions 1 .. M, ascending (ties to the lower position).
template <int KPT>
__device__ __forceinline__ void slice_top(const float* srow, int M, int need, int32_t* out,
                                          TopBShared<kSliceThreads>& sh) {
  uint32_t key[KPT], kmin;
  int nbits;
  const int kpt = (M + kSliceThreads - 1) / kSliceThreads;
  load_keys<KPT, kSliceThreads>(srow, M, key, kmin, nbits, sh, kpt);
  emit_top<KPT, kSliceThreads>(key, M, need, kmin, nbits, out, sh, kpt);
}

template <int D, int G>
__global__ __launch_bounds__(kSliceThreads) void slice_score_kernel(SliceArgs a) {
  const CacheView& c = a.c;
  __shared__ float s_buf[kSliceMaxPages + 1];  // s_buf[1 + p - p0]: page p's score
  __shared__ int s_ph[kSliceMaxPages];          // s_ph[p - p0]: page p's page-table entry
  __shared__ int s_pos[kSliceMaxPages + 1];
  __shared__ TopBShared<kSliceThreads> sh;
  float* s_score = s_buf + 1;
  const int units = c.batch * c.hkv;
  const int u = blockIdx.x % units, s = blockIdx.x / units;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  int b, g, L, P, K;
  unit_shape(a, u, b, g, L, P, K);
  const bool select = K < P && K > 2;
  const int need = K - 2;
  const int p0 = min(P, s * a.per), p1 = min(P, p0 + a.per);
  int32_t* cnt_out = a.cand_cnt + (int64_t)u * a.S + s;
  if (p0 >= p1 || (!select && a.scores == nullptr)) {
    if (tid == 0) *cnt_out = 0;
    return;
  }
  const int wper = (p1 - p0 + kSliceWaves - 1) / kSliceWaves;
  const int w0 = min(p1, p0 + wave * wper), w1 = min(p1, w0 + wper);
  if (w0 < w1) score_segment<BF16, D, G>(c, a.q, b, g, w0, w1, s_score, lane, s_ph, p0);
  __syncthreads();
  if (a.scores != nullptr)
    for (int p = p0 + tid; p < p1; p += kSliceThreads) a.scores[(int64_t)u * c.max_pages + p] = s_score[p - p0];
  if (!select) {
    if (tid == 0) *cnt_out = 0;
    return;
  }
  // The slice's middle pages [m0, m1) and its candidates.
  const int m0 = max(p0, 1), m1 = min(p1, P - 1);
  const int M = max(m1 - m0, 0);
  const int n = min(need, M);
  int32_t* cp = a.cand_page + ((int64_t)u * a.S + s) * a.cstride;
  float* cs = a.cand_score + ((int64_t)u * a.S + s) * a.cstride;
  int32_t* cph = a.cand_phys + ((int64_t)u * a.S + s) * a.cstride;
  if (n == M) {
    for (int i = tid; i < M; i += kSliceThreads) {
      cp[i] = m0 + i;
      cs[i] = s_score[m0 + i - p0];
      cph[i] = s_ph[m0 + i - p0];
    }
  } else {
    // srow[1 + i] = score of middle page m0 + i
    const float* srow = s_score + (m0 - p0) - 1;
    if (M <= kSliceKeysShort * kSliceThreads)
      slice_top<kSliceKeysShort>(srow, M, n, s_pos, sh);
    else
      slice_top<kSliceKeys>(srow, M, n, s_pos, sh);
    __syncthreads();
    for (int i = tid; i < n; i += kSliceThreads) {
      const int page = m0 + s_pos[i + 1] - 1;
      cp[i] = page;
      cs[i] = s_score[page - p0];
      cph[i] = s_ph[page - p0];
    }
  }
  if (tid == 0) *cnt_out = n;
}

template <int D, int G, bool STREAM>
__global__ __launch_bounds__(kSliceThreads) void slice_select_kernel(SliceArgs a) {
  const CacheView& c = a.c;
  __shared__ float s_cs[kSliceMaxCand + 1];  // s_cs[1 + i]: candidate i's score
  __shared__ int s_cp[kSliceMaxCand + 1];    // s_cp[1 + i]: candidate i's page
  __shared__ int s_cph[kSliceMaxCand + 1];   // s_cph[1 + i]: candidate i's page-table entry
  __shared__ int s_list[kSliceMaxList];
  __shared__ int s_lph[kSliceMaxList];       // page-table entry of each s_list page
  __shared__ int s_pre[kSliceMaxS + 1];
  __shared__ TopBShared<kSliceThreads> sh;
  __shared__ WaveParts<D, G, kSliceWaves> s_parts;
  const int units = c.batch * c.hkv;
  const int u = blockIdx.x % units, s = STREAM ? blockIdx.x / units : 0;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  int b, g, L, P, K;
  unit_shape(a, u, b, g, L, P, K);
  if (P == 0) {  // no token: no page; the merge writes zeros and lse = ln 0
    if (s == 0 && tid == 0) {
      a.sel_cnt[u] = 0;
      if (STREAM) a.count[u] = 0;
    }
    return;
  }
  const bool select = K < P && K > 2;
  // The kept pages, ascending, into s_list[0 .. K), with their page-table
  // entries in s_lph when K < P (the candidates carry theirs from scoring).
  if (K >= P) {
    for (int i = tid; i < P; i += kSliceThreads) s_list[i] = i;
  } else {
    if (tid == 0) {
      const int32_t* prow = c.page_table + (int64_t)b * c.max_pages;
      s_list[0] = 0;
      s_list[K - 1] = P - 1;
      s_lph[0] = prow[0];
      s_lph[K - 1] = prow[P - 1];
    }
    if (select) {
      // Every slot of the unit's slices is requested together with the slices'
      // counts (one round trip), then the counted ones are packed in slice
      // order straight from the registers.
      const int nslot = a.S * a.cstride;
      if (tid < a.S) s_pre[tid] = a.cand_cnt[(int64_t)u * a.S + tid];
      const int64_t ubase = (int64_t)u * a.S * a.cstride;
      constexpr int kSlotsPerThread = (kSliceMaxCand + kSliceThreads - 1) / kSliceThreads;
      int pk[kSlotsPerThread], ph[kSlotsPerThread];
      float sk[kSlotsPerThread];
#pragma unroll
      for (int r = 0; r < kSlotsPerThread; ++r) {
        const int i = tid + r * kSliceThreads;
        if (i < nslot) {
          pk[r] = a.cand_page[ubase + i];
          sk[r] = a.cand_score[ubase + i];
          ph[r] = a.cand_phys[ubase + i];
        }
      }
      __syncthreads();
      // Lane j of every wave: slice j's count and the counts before it.
      const int cj = lane < a.S ? s_pre[lane] : 0;
      const int incl = wave_incl_scan(cj);
      const int Mc = __builtin_amdgcn_readlane(incl, a.S - 1);
#pragma unroll
      for (int r = 0; r < kSlotsPerThread; ++r) {
        const int i = tid + r * kSliceThreads;
        const int j = min(i / a.cstride, a.S - 1);
        const int before = __shfl(incl - cj, j);
        const int cnt = __shfl(cj, j);
        const int k = i - j * a.cstride;
        if (i < nslot && k < cnt) {
          s_cp[1 + before + k] = pk[r];
          s_cs[1 + before + k] = sk[r];
          s_cph[1 + before + k] = ph[r];
        }
      }
      __syncthreads();
      if (Mc <= kSliceKeysShort * kSliceThreads)
        slice_top<kSliceKeysShort>(s_cs, Mc, K - 2, s_list, sh);
      else
        slice_top<kSliceKeys>(s_cs, Mc, K - 2, s_list, sh);
      __syncthreads();
      for (int i = 1 + tid; i < K - 1; i += kSliceThreads) {
        const int ci = s_list[i];
        s_list[i] = s_cp[ci];
        s_lph[i] = s_cph[ci];
      }
    }
  }
  __syncthreads();
  if (s == 0) {
    for (int i = tid; i < K; i += kSliceThreads) a.sel_idx[(int64_t)u * a.cap + i] = s_list[i];
    if (tid == 0) {
      a.sel_cnt[u] = K;
      if (STREAM) a.count[u] = a.S;
    }
  }
  if constexpr (STREAM) {
    // This slice's entries, split over the waves.
    const int eper = (K + a.S - 1) / a.S;
    const int s0 = min(K, s * eper), s1 = min(K, s0 + eper);
    const int wper = (s1 - s0 + kSliceWaves - 1) / kSliceWaves;
    const int e0 = min(s1, s0 + wave * wper), e1 = min(s1, e0 + wper);
    float m[G], lsum[G], acc[G][8];
    stream_list_range<D, G>(c, a.q, a.qk_scale, b, g, L, P, s_list, K < P ? s_lph : nullptr, nullptr, e0, e1, lane, m,
                            lsum, acc);
    store_wave_part<D, G, kSliceWaves>(s_parts, wave, lane, m, lsum, acc);
    __syncthreads();
    const int64_t slot = (int64_t)u * a.S + s;
    for (int i = tid; i < G * D; i += kSliceThreads) {
      const int h = i / D, d = i % D;
      float M, Ls, o;
      fold_wave_parts<D, G, kSliceWaves>(s_parts, h, d, M, Ls, o);
      a.part_acc[(slot * G + h) * D + d] = o;
      if (d == 0) {
        a.part_ml[(slot * G + h) * 2 + 0] = M;
        a.part_ml[(slot * G + h) * 2 + 1] = Ls;
      }
    }
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct SliceLayout {
  size_t cand_page, cand_score, cand_phys, cand_cnt, part_acc, part_ml, count, total;
};

// Workspace regions, each sized for any S the form takes: S * (max_budget - 2)
// <= kSliceMaxCand candidate slots and S <= kSliceMaxS slices per unit.
SliceLayout slice_layout(const CacheView& c) {
  const size_t units = (size_t)c.batch * c.hkv;
  SliceLayout l;
  size_t off = 0;
  l.cand_page = off;
  off += align256(units * kSliceMaxCand * sizeof(int32_t));
  l.cand_score = off;
  off += align256(units * kSliceMaxCand * sizeof(float));
  l.cand_phys = off;
  off += align256(units * kSliceMaxCand * sizeof(int32_t));
  l.cand_cnt = off;
  off += align256(units * kSliceMaxS * sizeof(int32_t));
  l.part_acc = off;
  off += align256(units * kSliceMaxS * c.group * c.head_dim * sizeof(float));
  l.part_ml = off;
  off += align256(units * kSliceMaxS * c.group * 2 * sizeof(float));
  l.count = off;
  off += align256(units * sizeof(int32_t));
  l.total = off;
  return l;
}

bool slice_shape_ok(const CacheView& c, int max_budget) {
  const int64_t units = (int64_t)c.batch * c.hkv;
  return c.dtype == SPDEC_BF16 && c.group <= 4 && units >= 1 && units <= kSliceMaxUnits && max_budget >= 2 &&
         max_budget <= kSliceMaxList;
}

template <int D, int G>
hipError_t slice_launch(const SliceArgs& a, bool stream, hipStream_t s) {
  const int units = a.c.batch * a.c.hkv;
  hipLaunchKernelGGL((slice_score_kernel<D, G>), dim3(units * a.S), dim3(kSliceThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (stream)
    hipLaunchKernelGGL((slice_select_kernel<D, G, true>), dim3(units * a.S), dim3(kSliceThreads), 0, s, a);
  else
    hipLaunchKernelGGL((slice_select_kernel<D, G, false>), dim3(units), dim3(kSliceThreads), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t slice_launch_g(const SliceArgs& a, bool stream, hipStream_t s) {
  switch (a.c.group) {
    case 1: return slice_launch<D, 1>(a, stream, s);
    case 2: return slice_launch<D, 2>(a, stream, s);
    default: return slice_launch<D, 4>(a, stream, s);
  }
}

}  // namespace

int slice_count(const CacheView& c, int max_budget, int cus) {
  const int64_t units = (int64_t)c.batch * c.hkv;
  if (!slice_shape_ok(c, max_budget) || cus < 1) return 0;
  int S = (int)std::min<int64_t>(kSliceMaxS, cus / units);
  if (S < 2) return 0;
  // every slice's pages and every unit's candidates must fit the LDS arrays
  while (S <= kSliceMaxS && (c.max_pages + S - 1) / S > kSliceMaxPages) ++S;
  if (S > kSliceMaxS || (int64_t)S * (max_budget - 2) > kSliceMaxCand) return 0;
  return S;
}

size_t slice_workspace_bytes(const CacheView& c, int max_budget) {
  return slice_shape_ok(c, max_budget) ? slice_layout(c).total : 0;
}

hipError_t launch_slice_path(const CacheView& c, const void* q, const int32_t* budget, int max_budget, int S,
                             float scale, int32_t* sel_idx, int32_t* sel_cnt, float* scores, float* out, float* lse,
                             void* ws, hipStream_t s) {
  const SliceLayout l = slice_layout(c);
  char* base = static_cast<char*>(ws);
  SliceArgs a;
  a.c = c;
  a.q = q;
  a.budget = budget;
  a.cap = max_budget;
  a.S = S;
  a.per = (c.max_pages + S - 1) / S;
  a.cstride = std::max(max_budget - 2, 1);
  a.qk_scale = scale * kLog2e;
  a.cand_page = reinterpret_cast<int32_t*>(base + l.cand_page);
  a.cand_score = reinterpret_cast<float*>(base + l.cand_score);
  a.cand_phys = reinterpret_cast<int32_t*>(base + l.cand_phys);
  a.cand_cnt = reinterpret_cast<int32_t*>(base + l.cand_cnt);
  a.sel_idx = sel_idx;
  a.sel_cnt = sel_cnt;
  a.scores = scores;
  a.part_acc = reinterpret_cast<float*>(base + l.part_acc);
  a.part_ml = reinterpret_cast<float*>(base + l.part_ml);
  a.count = reinterpret_cast<int32_t*>(base + l.count);
  const bool stream = out != nullptr;
  hipError_t e = c.head_dim == 64 ? slice_launch_g<64>(a, stream, s) : slice_launch_g<128>(a, stream, s);
  if (e != hipSuccess || !stream) return e;
  return launch_stream_merge(c, sel_cnt, max_budget, S, a.part_acc, a.part_ml, a.count, out, lse, s);
}

}  // namespace spdec
