// Dense decode for groups of sequences that share their leading pages.
//
// In group-based RL rollouts every prompt is sampled N times; the N sequences
// share the prompt's KV (the same physical pages in every page table). The
// cost model on the Sparrow project page ("Control Study 2") charges the
// prompt terms once rather than once per sample; a per-sequence decode reads
// the prompt pages N times. Here the attention of sequence b over its pages
// splits at the group's shared-page count S:
//   * prefix pass: pages 0 .. S-1, read once per (group, KV head) for the
//     N * G query rows of the group (the multi-row stream kernel);
//   * suffix pass: pages S .. P_b - 1 of each sequence (the single-query
//     dense stream kernel with its list starting at page S);
//   * merge: for every (sequence, query head) the partials of both passes by
//     log-sum-exp, chunks in a fixed order.
// The result is the dense decode of every sequence (the same softmax over the
// same tokens), up to rounding.
#include "common.h"
#include "launch.h"

namespace spdec {

namespace {

struct SharedMergeArgs {
  CacheView c;
  int group_size;
  const int32_t* shared;
  int jmax_p, rows_p;         // prefix: [groups * hkv][jmax_p][rows_p][D]
  const float* acc_p;
  const float* ml_p;
  const int* count_p;
  int jmax_s;                 // suffix: [batch * hkv][jmax_s][G][D]
  const float* acc_s;
  const float* ml_s;
  const int* count_s;
  float* out;                 // [batch][Hq][D]
  float* lse;                 // [batch][Hq] or null
};

// The leading kSharedMergePre chunks of each pass (slots below that pass's
// jmax lie inside the workspace) are requested together with the chunk
// counts, so a merge over that many chunks per pass costs one round trip.
constexpr int kSharedMergePre = 8;

template <int D>
__global__ __launch_bounds__(kWave) void shared_merge_kernel(SharedMergeArgs a) {
  constexpr int DPL = D / kWave;
  constexpr int NP = kSharedMergePre;
  const CacheView& c = a.c;
  const int bh = blockIdx.x;
  const int b = bh / c.hq, h = bh % c.hq;
  const int g = h / c.group, hh = h % c.group;
  const int n = b / a.group_size, i = b % a.group_size;
  const int lane = threadIdx.x;
  const int up = n * c.hkv + g, us = b * c.hkv + g;
  const int rp = i * c.group + hh;
  auto ml_p = [&](int j) { return a.ml_p + (((int64_t)up * a.jmax_p + j) * a.rows_p + rp) * 2; };
  auto ml_s = [&](int j) { return a.ml_s + (((int64_t)us * a.jmax_s + j) * c.group + hh) * 2; };
  auto acc_p = [&](int j) { return a.acc_p + (((int64_t)up * a.jmax_p + j) * a.rows_p + rp) * D + lane * DPL; };
  auto acc_s = [&](int j) { return a.acc_s + (((int64_t)us * a.jmax_s + j) * c.group + hh) * D + lane * DPL; };
  // Requested up front, at clamped slots: lane j's (m, l) of both passes and
  // the leading accumulators of both passes.
  const float* mlp0 = ml_p(min(lane, a.jmax_p - 1));
  const float* mls0 = ml_s(min(lane, a.jmax_s - 1));
  const float mp0 = mlp0[0], lp0 = mlp0[1], ms0 = mls0[0], ls0 = mls0[1];
  float pre_p[NP][DPL], pre_s[NP][DPL];
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const float* sp = acc_p(min(k, a.jmax_p - 1));
    const float* ss = acc_s(min(k, a.jmax_s - 1));
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      pre_p[k][e] = sp[e];
      pre_s[k][e] = ss[e];
    }
  }
  // Entry counts exactly as the two passes derived them.
  const int b0 = n * a.group_size;
  const int L0 = max(c.seq_lens[b0], 0);
  const int P0 = min((L0 + c.page_size - 1) >> c.ps_log2, c.max_pages);
  const int S = max(a.shared[n], 0);
  const int np = min(S, P0);
  const int L = max(c.seq_lens[b], 0);
  const int P = min((L + c.page_size - 1) >> c.ps_log2, c.max_pages);
  const int ns = max(P - S, 0);
  const int Jp = np > 0 ? min(max(a.count_p[up], 0), a.jmax_p) : 0;
  const int Js = ns > 0 ? min(max(a.count_s[us], 0), a.jmax_s) : 0;
  const int J = Jp + Js;
  // Chunk j of the merge order: prefix chunk j for j < Jp, else suffix chunk j - Jp.
  auto ml_of = [&](int j) -> const float* { return j < Jp ? ml_p(j) : ml_s(j - Jp); };
  // Lane j's own chunk (j < 64): prefix slot j, or suffix slot j - Jp, which
  // lane j - Jp requested.
  const float msh = __shfl(ms0, max(lane - Jp, 0));
  const float lsh = __shfl(ls0, max(lane - Jp, 0));
  const float m0 = lane < Jp ? mp0 : msh;
  const float l0 = lane < Jp ? lp0 : lsh;
  float M = lane < J ? m0 : kNegBig;
  for (int j = lane + kWave; j < J; j += kWave) M = fmaxf(M, ml_of(j)[0]);
  M = group_max<kWave>(M);
  // Lane j holds merge chunk j's weight; chunks past the wave width recompute
  // theirs where they are used.
  float Ls = 0.f, w_own = 0.f;
  if (lane < J) {
    w_own = exp2f(m0 - M);
    Ls += w_own * l0;
  }
  for (int j = lane + kWave; j < J; j += kWave) {
    const float* ml = ml_of(j);
    Ls += exp2f(ml[0] - M) * ml[1];
  }
  Ls = group_sum<kWave>(Ls);
  float o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;
  auto weight = [&](int j) { return j < kWave ? __shfl(w_own, j) : exp2f(ml_of(j)[0] - M); };
  // Chunks [k0, k1) of one pass (merge-order index base + k), NP loads in
  // flight at a time (at clamped slots; unused ones are never summed).
  auto accum = [&](auto acc_of, int jmax, int k0, int k1, int base) {
    for (int kb = k0; kb < k1; kb += NP) {
      float v[NP][DPL];
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        const float* src = acc_of(min(kb + q, jmax - 1));
#pragma unroll
        for (int e = 0; e < DPL; ++e) v[q][e] = src[e];
      }
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        if (kb + q < k1) {
          const float wgt = weight(base + kb + q);
#pragma unroll
          for (int e = 0; e < DPL; ++e) o[e] = fmaf(wgt, v[q][e], o[e]);
        }
      }
    }
  };
  // Prefix chunks, then suffix chunks, each in index order; the first NP of
  // each pass come from the up-front loads.
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    if (k < Jp) {
      const float wgt = weight(k);
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] = fmaf(wgt, pre_p[k][e], o[e]);
    }
  }
  accum(acc_p, a.jmax_p, NP, Jp, 0);
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    if (k < Js) {
      const float wgt = weight(Jp + k);
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] = fmaf(wgt, pre_s[k][e], o[e]);
    }
  }
  accum(acc_s, a.jmax_s, NP, Js, Jp);
  const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) a.out[(int64_t)bh * D + lane * DPL + e] = o[e] * inv;
  if (a.lse != nullptr && lane == 0) a.lse[bh] = Ls > 0.f ? (M + log2f(Ls)) * kLn2 : -INFINITY;
}

size_t a256(size_t v) { return (v + 255) & ~(size_t)255; }

// Workspace layout of both passes (prefix then suffix: acc, ml, counts).
struct SharedLayout {
  int jmax_p, rmin_p, rows_p;
  DecodePlan ps;
  size_t acc_p, ml_p, cnt_p, acc_s, ml_s, cnt_s, total;
};

SharedLayout shared_layout(const CacheView& c, int group_size) {
  SharedLayout l;
  const int64_t units_p = (int64_t)(c.batch / group_size) * c.hkv;
  stream_plan(units_p, c.max_pages, &l.jmax_p, &l.rmin_p);
  l.rows_p = c.group * group_size;
  l.ps = decode_plan(c, 0);
  const size_t slots_p = (size_t)units_p * l.jmax_p * l.rows_p;
  const size_t slots_s = (size_t)c.batch * c.hkv * l.ps.jmax * c.group;
  size_t off = 0;
  l.acc_p = off; off += a256(slots_p * c.head_dim * sizeof(float));
  l.ml_p = off;  off += a256(slots_p * 2 * sizeof(float));
  l.cnt_p = off; off += a256((size_t)units_p * sizeof(int));
  l.acc_s = off; off += a256(slots_s * c.head_dim * sizeof(float));
  l.ml_s = off;  off += a256(slots_s * 2 * sizeof(float));
  l.cnt_s = off; off += a256((size_t)c.batch * c.hkv * sizeof(int));
  l.total = off;
  return l;
}

}  // namespace

bool shared_supported(const CacheView& c, int group_size) {
  return c.dtype == SPDEC_BF16 && group_size >= 1 && c.batch % group_size == 0 && c.group * group_size <= 64 &&
         (int64_t)c.batch * c.hkv <= kMaxStreamUnits;
}

size_t shared_workspace_bytes(const CacheView& c, int group_size) { return shared_layout(c, group_size).total; }

hipError_t launch_dense_shared(const CacheView& c, const void* q, int group_size, const int32_t* shared_pages,
                               float scale, float* out, float* lse, void* ws, hipStream_t s) {
  const SharedLayout l = shared_layout(c, group_size);
  char* base = reinterpret_cast<char*>(ws);
  SharedMergeArgs m;
  m.c = c;
  m.group_size = group_size;
  m.shared = shared_pages;
  m.jmax_p = l.jmax_p;
  m.rows_p = l.rows_p;
  m.acc_p = reinterpret_cast<float*>(base + l.acc_p);
  m.ml_p = reinterpret_cast<float*>(base + l.ml_p);
  m.count_p = reinterpret_cast<int*>(base + l.cnt_p);
  m.jmax_s = l.ps.jmax;
  m.acc_s = reinterpret_cast<float*>(base + l.acc_s);
  m.ml_s = reinterpret_cast<float*>(base + l.ml_s);
  m.count_s = reinterpret_cast<int*>(base + l.cnt_s);
  m.out = out;
  m.lse = lse;
  hipError_t e = launch_prefix_partials(c, q, group_size, shared_pages, l.jmax_p, l.rmin_p, scale,
                                        const_cast<float*>(m.acc_p), const_cast<float*>(m.ml_p),
                                        const_cast<int*>(m.count_p), s);
  if (e != hipSuccess) return e;
  e = launch_dense_stream_partials(c, l.ps, q, shared_pages, group_size, scale, const_cast<float*>(m.acc_s),
                                   const_cast<float*>(m.ml_s), const_cast<int*>(m.count_s), s);
  if (e != hipSuccess) return e;
  if (c.head_dim == 64) {
    hipLaunchKernelGGL((shared_merge_kernel<64>), dim3(c.batch * c.hq), dim3(kWave), 0, s, m);
  } else {
    hipLaunchKernelGGL((shared_merge_kernel<128>), dim3(c.batch * c.hq), dim3(kWave), 0, s, m);
  }
  return hipGetLastError();
}

}  // namespace spdec
