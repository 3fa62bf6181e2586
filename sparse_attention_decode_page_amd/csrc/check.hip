// Device-side check of the data preconditions that the hot calls assume and
// do not test: sequence lengths within the page table, live page-table entries
// within the pool, selections of the form the Top-B selection writes, finite
// queries, and the shared leading pages of grouped samples.
//
// The checker reads only the page table, the lengths, the selection, the query
// and the shared-page counts, each inside its declared extent whatever values
// those arrays hold: indices come from the descriptor's sizes, and values read
// from the arrays are only compared, never dereferenced. It never reads the KV
// pools or page summaries, so a cache with bad entries can be checked safely.
#include "common.h"
#include "launch.h"

namespace spdec {

namespace {

constexpr int kCheckThreads = 256;

__global__ void check_init_kernel(int32_t* __restrict__ report, int batch) {
  if (threadIdx.x < SPDEC_CHECK_WORDS) report[threadIdx.x] = threadIdx.x == SPDEC_CHECK_FIRST ? batch : 0;
}

// One workgroup per sequence b.
__global__ __launch_bounds__(kCheckThreads) void check_kernel(CacheView c, const void* __restrict__ q,
                                                              const int32_t* __restrict__ sel_idx,
                                                              const int32_t* __restrict__ sel_cnt, int max_budget,
                                                              int group_size, const int32_t* __restrict__ shared_pages,
                                                              int32_t* __restrict__ report) {
  __shared__ int counts[5];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid < 5) counts[tid] = 0;
  __syncthreads();

  const int64_t max_tokens = (int64_t)c.max_pages * c.page_size;
  const int L = c.seq_lens[b];
  const int Lc = L < 0 ? 0 : (int64_t)L > max_tokens ? (int)max_tokens : L;
  const int P = (Lc + c.page_size - 1) >> c.ps_log2;
  const int32_t* pt = c.page_table + (int64_t)b * c.max_pages;
  if (tid == 0 && Lc != L) counts[0] = 1;

  int bad = 0;
  for (int p = tid; p < P; p += kCheckThreads) {
    const int32_t e = pt[p];
    bad += (e < 0 || (int64_t)e >= c.num_phys) ? 1 : 0;
  }
  if (bad) atomicAdd(&counts[1], bad);

  if (sel_idx != nullptr) {
    const int cap = P < max_budget ? P : max_budget;
    for (int g = 0; g < c.hkv; ++g) {
      const int64_t row = (int64_t)b * c.hkv + g;
      const int cnt = sel_cnt[row];
      const int n = cnt < 0 ? 0 : cnt > max_budget ? max_budget : cnt;
      const int32_t* s = sel_idx + row * max_budget;
      int rb = (tid == 0 && (cnt < 0 || cnt > cap)) ? 1 : 0;
      for (int i = tid; i < n; i += kCheckThreads) {
        const int32_t v = s[i];
        if (v < 0 || v >= P || (i > 0 && v <= s[i - 1])) rb = 1;
      }
      if (__syncthreads_or(rb) && tid == 0) counts[2] += 1;
    }
  }

  if (q != nullptr) {
    const int64_t n = (int64_t)c.hq * c.head_dim;
    int nf = 0;
    if (c.dtype == SPDEC_BF16) {
      const uint16_t* x = static_cast<const uint16_t*>(q) + (int64_t)b * n;
      for (int64_t i = tid; i < n; i += kCheckThreads) nf += ((x[i] & 0x7f80u) == 0x7f80u) ? 1 : 0;
    } else {
      const uint32_t* x = static_cast<const uint32_t*>(q) + (int64_t)b * n;
      for (int64_t i = tid; i < n; i += kCheckThreads) nf += ((x[i] & 0x7f800000u) == 0x7f800000u) ? 1 : 0;
    }
    if (nf) atomicAdd(&counts[3], nf);
  }

  if (shared_pages != nullptr && b % group_size == 0) {
    const int S = shared_pages[b / group_size];
    int gb = (tid == 0 && (S < 0 || S > c.max_pages)) ? 1 : 0;
    const int Sc = S < 0 ? 0 : S > c.max_pages ? c.max_pages : S;
    for (int m = 0; m < group_size; ++m) {
      const int Lm = c.seq_lens[b + m];
      const int Lmc = Lm < 0 ? 0 : (int64_t)Lm > max_tokens ? (int)max_tokens : Lm;
      if (tid == 0 && (int64_t)Sc * c.page_size > Lmc) gb = 1;  // shared pages are full in every member
      const int32_t* ptm = c.page_table + (int64_t)(b + m) * c.max_pages;
      for (int p = tid; p < Sc; p += kCheckThreads)
        if (ptm[p] != pt[p]) gb = 1;
    }
    if (__syncthreads_or(gb) && tid == 0) counts[4] = 1;
  } else {
    __syncthreads();
  }
  __syncthreads();

  if (tid == 0) {
    int any = 0;
    for (int k = 0; k < 5; ++k) {
      if (counts[k]) atomicAdd(&report[k], counts[k]);
      any |= counts[k];
    }
    if (any) atomicMin(&report[SPDEC_CHECK_FIRST], b);
  }
}

}  // namespace

hipError_t launch_check(const CacheView& c, const void* q, const int32_t* sel_idx, const int32_t* sel_cnt,
                        int max_budget, int group_size, const int32_t* shared_pages, int32_t* report, hipStream_t s) {
  hipLaunchKernelGGL(check_init_kernel, dim3(1), dim3(64), 0, s, report, c.batch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(check_kernel, dim3(c.batch), dim3(kCheckThreads), 0, s, c, q, sel_idx, sel_cnt, max_budget,
                     group_size, shared_pages, report);
  return hipGetLastError();
}

}  // namespace spdec
