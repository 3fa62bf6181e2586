// Split-KV decode attention over a page list (sparse) or over every page (dense).
//
// Block-sparse decode attention reads only the budgeted pages (Sparrow project
// page, "Insights" and the "Control Study 2" cost model, whose memory term is
// the KV budget read per generated token); the dense verifier reads the
// complete KV (S3R abstract). Both run the same kernel; only the page-list
// iterator differs.
//
// Two decompositions share the plan and the merge order:
//   * bf16 caches (the workloads measured here): a persistent stream-K kernel
//     (decode_stream_kernel, below) in which every wave owns one contiguous
//     range of the flattened (sequence x KV head, page-list entry) pairs, with
//     q.K^T on the matrix cores (and P.V too for eight query heads per KV
//     head, decode_stream_g8_kernel); a second kernel merges each unit's chunks;
//   * fp32 caches and batches too large for the stream plan: one workgroup per
//     (split, sequence, KV head) (decode_split_kernel), a split being a run of
//     `pages_per_split` list entries, merged by decode_merge_kernel.
// Either way all G query heads of a KV head are served together, so every K/V
// byte is read from HBM once, and every merge runs in a fixed order, so the
// result is deterministic.
//
// Split kernel lane layout: a token row of D channels is spread over LPT = D/VEC lanes
// that each hold one 16-byte chunk; one wave load instruction covers TPI =
// 64/LPT tokens (1 KiB for bf16 D=128). Scores are LPT-lane butterfly sums.
// Each group of LPT lanes keeps its own fp32 online softmax (running max m,
// sum l, accumulator acc[G][VEC]) in the log2 domain; the groups, then the
// four waves, are merged by log-sum-exp at the end of the split, and the
// per-split partials are merged by a second kernel in a fixed order, so the
// result is deterministic.
#include <limits.h>

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "stream_window.h"

namespace spdec {

namespace {

constexpr int kDecodeThreads = 256;
constexpr int kDecodeWaves = kDecodeThreads / kWave;
constexpr int kChunk = 4;           // load instructions per wave per step
constexpr int kMaxPagesPerSplit = 256;
constexpr int kMaxSplits = 2048;     // per (sequence, KV head); bounded by the page-table length

struct DecodeArgs {
  CacheView c;
  const void* q;
  const int32_t* sel_idx;
  const int32_t* sel_cnt;
  int list_cap;         // row stride of sel_idx
  int pages_per_split;
  int nsplit;
  float qk_scale;       // softmax scale * log2(e)
  float* part_acc;      // [B][Hq][nsplit][D]
  float* part_ml;       // [B][Hq][nsplit][2]  (running max in log2 units, sum)
  float* out;           // [B][Hq][D]
  float* lse;           // [B][Hq] or null
};

template <bool SPARSE>
__device__ __forceinline__ int list_length(const DecodeArgs& a, int unit, int P) {
  if constexpr (SPARSE) return min(max(a.sel_cnt[unit], 0), a.list_cap);
  return P;
}

template <typename T, int D, int G, bool SPARSE>
__global__ __launch_bounds__(kDecodeThreads) void decode_split_kernel(DecodeArgs a) {
  constexpr int VEC = T::VEC;
  constexpr int LPT = D / VEC;
  constexpr int TPI = kWave / LPT;
  using S = typename T::storage;
  const CacheView& c = a.c;
  const int unit = blockIdx.y;
  const int b = unit / c.hkv;
  const int g = unit % c.hkv;
  const int L = max(c.seq_lens[b], 0);
  const int P = min((L + c.page_size - 1) >> c.ps_log2, c.max_pages);
  const int n = list_length<SPARSE>(a, unit, P);
  const int e0 = blockIdx.x * a.pages_per_split;
  if (e0 >= n) return;
  const int ne = min(a.pages_per_split, n - e0);

  __shared__ int s_phys[kMaxPagesPerSplit];
  __shared__ int s_valid[kMaxPagesPerSplit];  // tokens of the page present in the cache
  for (int i = threadIdx.x; i < ne; i += kDecodeThreads) {
    int logical = SPARSE ? a.sel_idx[(int64_t)unit * a.list_cap + e0 + i] : e0 + i;
    int phys = -1;
    if (logical >= 0 && logical < P) phys = c.page_table[(int64_t)b * c.max_pages + logical];
    const bool ok = phys >= 0 && phys < c.num_phys;
    s_phys[i] = ok ? phys : 0;
    s_valid[i] = ok ? min(c.page_size, L - logical * c.page_size) : 0;
  }

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int sub = lane % LPT;
  const int tslot = lane / LPT;
  const int d0 = sub * VEC;

  float qf[G][VEC];
  const S* q = reinterpret_cast<const S*>(a.q);
#pragma unroll
  for (int h = 0; h < G; ++h) unpack<T>(load16(q + ((int64_t)b * c.hq + g * G + h) * D + d0), qf[h]);

  float m[G], l[G], acc[G][VEC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[h][e] = 0.f;
  }
  __syncthreads();

  const S* kp = reinterpret_cast<const S*>(c.k_pool);
  const S* vp = reinterpret_cast<const S*>(c.v_pool);
  const int ninstr = (ne << c.ps_log2) / TPI;  // TPI divides every supported page size
  const int nchunks = (ninstr + kChunk - 1) / kChunk;

  auto load_chunk = [&](int chunk, u32x4* kr, u32x4* vr, bool* ok) {
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const int ins = chunk * kChunk + i;
      const int s = ins * TPI + tslot;
      const int e = min(s >> c.ps_log2, ne - 1);
      const int slot = s & (c.page_size - 1);
      ok[i] = ins < ninstr && slot < s_valid[e];
      const int64_t off = ((((int64_t)s_phys[e] * c.hkv + g) << c.ps_log2) + (ok[i] ? slot : 0)) * D + d0;
      kr[i] = load16_stream(kp + off);
      vr[i] = load16_stream(vp + off);
    }
  };

  u32x4 kA[kChunk], vA[kChunk], kB[kChunk], vB[kChunk];
  bool okA[kChunk], okB[kChunk];
  int chunk = wave;
  if (chunk < nchunks) load_chunk(chunk, kA, vA, okA);
  for (; chunk < nchunks; chunk += kDecodeWaves) {
    const int next = chunk + kDecodeWaves;
    if (next < nchunks) load_chunk(next, kB, vB, okB);

    float sc[kChunk][G];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      float kf[VEC];
      unpack<T>(kA[i], kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) d = fmaf(qf[h][e], kf[e], d);
        d = group_sum<LPT>(d);
        sc[i][h] = okA[i] ? d * a.qk_scale : -INFINITY;
      }
    }
    float p[kChunk][G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = sc[0][h];
#pragma unroll
      for (int i = 1; i < kChunk; ++i) mx = fmaxf(mx, sc[i][h]);
      const float mn = fmaxf(m[h], mx);
      const float alpha = exp2f(m[h] - mn);
      m[h] = mn;
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < kChunk; ++i) {
        p[i][h] = exp2f(sc[i][h] - mn);
        ps += p[i][h];
      }
      l[h] = l[h] * alpha + ps;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[h][e] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      float vf[VEC];
      unpack<T>(vA[i], vf);
#pragma unroll
      for (int e = 0; e < VEC; ++e) vf[e] = okA[i] ? vf[e] : 0.f;  // never multiply unread slots
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[h][e] = fmaf(p[i][h], vf[e], acc[h][e]);
    }
#pragma unroll
    for (int i = 0; i < kChunk; ++i) { kA[i] = kB[i]; vA[i] = vB[i]; okA[i] = okB[i]; }
  }

  // Merge the TPI token groups of the wave (butterfly over lanes LPT apart).
#pragma unroll
  for (int off = LPT; off < kWave; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], off);
      const float lo = __shfl_xor(l[h], off);
      const float M = fmaxf(m[h], mo);
      const float f1 = exp2f(m[h] - M), f2 = exp2f(mo - M);
      l[h] = l[h] * f1 + lo * f2;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float ao = __shfl_xor(acc[h][e], off);
        acc[h][e] = acc[h][e] * f1 + ao * f2;
      }
      m[h] = M;
    }
  }

  // Merge the waves through LDS and write this split's partial.
  __shared__ float s_acc[kDecodeWaves][G][D];
  __shared__ float s_m[kDecodeWaves][G], s_l[kDecodeWaves][G];
  if (tslot == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) s_acc[wave][h][d0 + e] = acc[h][e];
      if (sub == 0) { s_m[wave][h] = m[h]; s_l[wave][h] = l[h]; }
    }
  }
  __syncthreads();
  const int64_t row0 = ((int64_t)b * c.hq + g * G) * a.nsplit + blockIdx.x;  // head g*G, this split
  for (int idx = threadIdx.x; idx < G * D; idx += kDecodeThreads) {
    const int h = idx / D, d = idx % D;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < kDecodeWaves; ++w) M = fmaxf(M, s_m[w][h]);
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) o += exp2f(s_m[w][h] - M) * s_acc[w][h][d];
    a.part_acc[(row0 + (int64_t)h * a.nsplit) * D + d] = o;
    if (d == 0) {
      float Ls = 0.f;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) Ls += exp2f(s_m[w][h] - M) * s_l[w][h];
      a.part_ml[(row0 + (int64_t)h * a.nsplit) * 2 + 0] = M;
      a.part_ml[(row0 + (int64_t)h * a.nsplit) * 2 + 1] = Ls;
    }
  }
}

// bf16 variant with q.K^T on the matrix cores (v_mfma_f32_16x16x32_bf16).
//
// A tile is 16 consecutive tokens of the split's page list. One MFMA contracts
// 32 channels: A = the group's queries (the 16 rows hold query heads h % G, so
// every row group of the output sees every head), B = 16 tokens x 32 channels
// of K loaded straight from the page (lane l: token l%16, channels
// 32j+8(l/16)..+8), D = 16 rows x 16 tokens in four fp32 registers per lane:
// lane l holds token l%16 and rows 4(l/16)..+3, i.e. every head once (G <= 4;
// eight heads take the transposed form further below). Softmax
// state is kept per head and is uniform across the wave; the running maximum
// is only raised when a tile exceeds it by more than 2^8, so the O(G*D)
// rescale of the accumulator is rare. P.V stays on the VALU with V rows read
// as 1 KiB contiguous wave loads; each lane fetches its token's probability
// from the lane that owns that token (ds_bpermute).



constexpr int kDecodeMinRange = 4;  // entries: the shortest wave range worth its start-up

struct StreamArgs {
  CacheView c;
  const void* q;
  const int32_t* sel_idx;
  const int32_t* sel_cnt;
  int list_cap;      // row stride of sel_idx
  int jmax;          // partial slots per unit
  int rmin;          // minimum entries per wave range (bounds the chunks per unit by jmax)
  float qk_scale;    // softmax scale * log2(e)
  float* part_acc;   // [units][jmax][G][D]
  float* part_ml;    // [units][jmax][G][2]
  int* count;        // [units] chunks written for the unit
  float* out;
  float* lse;
  // Dense lists only: sequence b's list starts at logical page
  // first_page[b / group_size] (the pages before it are attended elsewhere);
  // null means page 0.
  const int32_t* first_page;
  int group_size;
};

template <bool SPARSE>
__device__ __forceinline__ int list_first(const StreamArgs& a, int b) {
  if constexpr (SPARSE) return 0;
  return a.first_page != nullptr ? max(a.first_page[b / a.group_size], 0) : 0;
}

template <bool SPARSE>
__device__ __forceinline__ int unit_entries(const StreamArgs& a, int u) {
  const CacheView& c = a.c;
  if constexpr (SPARSE) return min(max(a.sel_cnt[u], 0), a.list_cap);
  const int b = u / c.hkv;
  const int L = max(c.seq_lens[b], 0);
  const int P = min((L + c.page_size - 1) >> c.ps_log2, c.max_pages);
  return max(P - list_first<SPARSE>(a, b), 0);
}

// Persistent split-KV decode. The (unit, page-list entry) pairs of all
// sequences and KV heads are laid end to end and every wave owns one
// contiguous range of R entries: it streams its range once, emitting one
// partial (m, l, acc) per unit segment it covers, so every wave works until
// the end and no workgroup is launched for an empty split. The wave that
// finishes a unit records how many chunks the unit has for the merge.
template <int D, int G, bool SPARSE>
__global__ __launch_bounds__(kDecodeThreads, (D == 64 && G <= 2) ? 4 : 1) void decode_stream_kernel(StreamArgs a) {
  static_assert(G <= 4, "eight heads per KV head use decode_stream_g8_kernel");
  constexpr int NJ = D / 32;             // MFMAs per tile
  constexpr int LPT = D / 8;             // lanes per V row
  const CacheView& c = a.c;
  extern __shared__ int s_pre[];         // units + 1
  __shared__ int s_tmp[kDecodeWaves];
  __shared__ int s_emax[kDecodeWaves];
  const int units = c.batch * c.hkv;
  int emax = 0;
  for (int u = threadIdx.x; u < units; u += kDecodeThreads) {
    const int e = unit_entries<SPARSE>(a, u);
    s_pre[u] = e;
    emax = max(emax, e);
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) emax = max(emax, __shfl_xor(emax, off));
  if (threadIdx.x % kWave == 0) s_emax[threadIdx.x / kWave] = emax;
  __syncthreads();
  block_exclusive_scan(s_pre, units, s_tmp);
#pragma unroll
  for (int i = 0; i < kDecodeWaves; ++i) emax = max(emax, s_emax[i]);
  const int total = s_pre[units];
  const int lane = threadIdx.x % kWave;
  const int64_t nw = (int64_t)gridDim.x * kDecodeWaves;
  const int64_t w = (int64_t)blockIdx.x * kDecodeWaves + threadIdx.x / kWave;
  // Ranges of at least ceil(longest list / (jmax - 1)) entries keep every
  // unit within jmax chunks; the longest list is measured here, so short
  // lists under a large capacity still spread over every wave.
  const int64_t rmin = min<int64_t>(a.rmin, max((emax + a.jmax - 2) / (a.jmax - 1), kDecodeMinRange));
  const int64_t R = max<int64_t>((total + nw - 1) / nw, rmin);
  if (w * R >= total) return;
  int pos = (int)(w * R);
  const int end = (int)min<int64_t>(pos + R, total);
  int u = find_unit(s_pre, units, pos);

  const int r16 = lane % 16;   // token of the tile this lane scores
  const int q4 = lane / 16;    // row group
  const int vsub = lane % LPT; // V channel chunk
  const int vtok = lane / LPT; // V row within a load instruction
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q);

  while (pos < end) {
    while (s_pre[u + 1] <= pos) ++u;  // units with no entry have no segment
    const int b = u / c.hkv, g = u % c.hkv;
    const int ubase = s_pre[u];
    const int seg_end = min(end, s_pre[u + 1]);
    const int j = (int)(w - ubase / R);  // this wave's chunk of the unit
    int L = c.seq_lens[b];
    const int first = list_first<SPARSE>(a, b);
    // List entries come 64 at a time, one per lane, read at clamped indices
    // (entry < the unit's segment end) so that no load waits on a branch.
    auto list_raw = [&](int wb) -> int {
      const int e = min(wb + lane, seg_end - ubase - 1);
      return SPARSE ? a.sel_idx[(int64_t)u * a.list_cap + e] : first + e;
    };
    int raw = list_raw(pos - ubase);

    // A operands: row r16 holds query head r16 % G.
    u32x4 qa[NJ];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj)
      qa[jj] = load16(qp + ((int64_t)b * c.hq + g * G + r16 % G) * D + 32 * jj + 8 * q4);
    // Length, queries and the first list window share one wait.
    hold(L);
    hold(raw);
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) hold(qa[jj]);
    L = max(L, 0);
    const int P = min((L + c.page_size - 1) >> c.ps_log2, c.max_pages);
    float m[G], lsum[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = kNegBig;
      lsum[h] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }

    for (int wb = pos - ubase; wb < seg_end - ubase; wb += kWave) {
      // Window of up to 64 entries: lane i holds entry wb+i's physical page and valid tokens.
      const int nwin = min(kWave, seg_end - ubase - wb);
      if (wb != pos - ubase) raw = list_raw(wb);
      const int logical = raw;
      const int ph = c.page_table[(int64_t)b * c.max_pages + min(max(logical, 0), c.max_pages - 1)];
      const bool ok = lane < nwin && logical >= 0 && logical < P && ph >= 0 && ph < c.num_phys;
      const int phys_w = ok ? ph : 0;
      const int valid_w = ok ? min(c.page_size, L - logical * c.page_size) : 0;
      stream_window<D, G>(c, g, nwin, phys_w, valid_w, qa, a.qk_scale, lane, m, lsum, acc);
    }

    close_segment<D, G>(lsum, acc);
    if (j < a.jmax) {
      const int64_t slot0 = ((int64_t)u * a.jmax + j) * G;
      if (vtok == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float* dst = a.part_acc + (slot0 + h) * D + 8 * vsub;
#pragma unroll
          for (int e = 0; e < 8; ++e) dst[e] = acc[h][e];
        }
      }
      if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          a.part_ml[(slot0 + h) * 2 + 0] = m[h];
          a.part_ml[(slot0 + h) * 2 + 1] = lsum[h];
        }
        if (seg_end == s_pre[u + 1]) a.count[u] = j + 1;
      }
    }
    pos = seg_end;
    ++u;
  }
}

// G = 8 variant: heads on the MFMA rows and P.V on the matrix cores.
//
// With eight heads the VALU form spends 256 FMAs and 32 lane fetches per lane
// on P.V for every 16-token tile, which caps the dense pass near 5.4 TB/s.
// Here the scores are computed transposed, S^T = K Q^T
// (v_mfma_f32_16x16x32_bf16: K rows as they lie in the page are the A
// operand, the eight heads, repeated on rows 8..15, the B operand), which
// leaves lane l holding head l % 8 for tokens 4(l/16) .. +3: the A layout of
// v_mfma_f32_16x16x16_bf16, so the weights feed P.V without a lane exchange.
// For the B operand each lane loads, for its own four tokens, the chunk of
// DPC = D/16 channels starting at DPC (l % 16): column n of block jb then
// stands for channel DPC n + jb (no transpose). Each fp32 weight enters P.V
// as the sum of three bf16 values that add up to it exactly (hi: the weight
// with its low 16 bits cleared; mid: the same of the exact remainder; lo: the
// rest, at most 8 significant bits), so the products and fp32 sums match the
// VALU form up to summation order.
template <int DPC> struct VChunk;
template <> struct VChunk<8> { using type = u32x4; };
template <> struct VChunk<4> { typedef uint32_t type __attribute__((ext_vector_type(2))); };

__device__ __forceinline__ u32x4 load_vchunk(const uint16_t* p, u32x4*) { return load16_stream(p); }
__device__ __forceinline__ VChunk<4>::type load_vchunk(const uint16_t* p, VChunk<4>::type*) {
  return __builtin_nontemporal_load(reinterpret_cast<const VChunk<4>::type*>(p));
}


typedef short s16x4_t __attribute__((ext_vector_type(4)));

template <int D, bool SPARSE>
__global__ __launch_bounds__(kDecodeThreads, 2) void decode_stream_g8_kernel(StreamArgs a) {
  constexpr int G = 8;
  constexpr int NJ = D / 32;   // S^T MFMA steps (16x16x32)
  constexpr int NB = D / 16;   // P.V column blocks (16x16x16)
  constexpr int DPC = D / 16;  // V channels per lane and token
  using VC = typename VChunk<DPC>::type;
  const CacheView& c = a.c;
  extern __shared__ int s_pre[];  // units + 1
  __shared__ int s_tmp[kDecodeWaves];
  __shared__ int s_emax[kDecodeWaves];
  const int units = c.batch * c.hkv;
  int emax = 0;
  for (int u = threadIdx.x; u < units; u += kDecodeThreads) {
    const int e = unit_entries<SPARSE>(a, u);
    s_pre[u] = e;
    emax = max(emax, e);
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) emax = max(emax, __shfl_xor(emax, off));
  if (threadIdx.x % kWave == 0) s_emax[threadIdx.x / kWave] = emax;
  __syncthreads();
  block_exclusive_scan(s_pre, units, s_tmp);
#pragma unroll
  for (int i = 0; i < kDecodeWaves; ++i) emax = max(emax, s_emax[i]);
  const int total = s_pre[units];
  const int lane = threadIdx.x % kWave;
  const int64_t nw = (int64_t)gridDim.x * kDecodeWaves;
  const int64_t w = (int64_t)blockIdx.x * kDecodeWaves + threadIdx.x / kWave;
  const int64_t rmin = min<int64_t>(a.rmin, max((emax + a.jmax - 2) / (a.jmax - 1), kDecodeMinRange));
  const int64_t R = max<int64_t>((total + nw - 1) / nw, rmin);
  if (w * R >= total) return;
  int pos = (int)(w * R);
  const int end = (int)min<int64_t>(pos + R, total);
  int u = find_unit(s_pre, units, pos);

  const int r16 = lane % 16;  // K: token of the tile; scores, P and V: head row / V column
  const int q4 = lane / 16;   // K: channel group; scores: tokens 4 q4 .. +3
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q);
  const uint16_t* kp = reinterpret_cast<const uint16_t*>(c.k_pool);
  const uint16_t* vp = reinterpret_cast<const uint16_t*>(c.v_pool);

  while (pos < end) {
    while (s_pre[u + 1] <= pos) ++u;  // units with no entry have no segment
    const int b = u / c.hkv, g = u % c.hkv;
    const int ubase = s_pre[u];
    const int seg_end = min(end, s_pre[u + 1]);
    const int j = (int)(w - ubase / R);
    int L = c.seq_lens[b];
    const int first = list_first<SPARSE>(a, b);
    auto list_raw = [&](int wb) -> int {
      const int e = min(wb + lane, seg_end - ubase - 1);
      return SPARSE ? a.sel_idx[(int64_t)u * a.list_cap + e] : first + e;
    };
    int raw = list_raw(pos - ubase);
    // B operands of S^T: head r16 % 8, channels 32 jj + 8 q4 .. +8.
    u32x4 qb[NJ];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj)
      qb[jj] = load16(qp + ((int64_t)b * c.hq + g * G + (r16 & 7)) * D + 32 * jj + 8 * q4);
    hold(L);
    hold(raw);
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) hold(qb[jj]);
    L = max(L, 0);
    const int P = min((L + c.page_size - 1) >> c.ps_log2, c.max_pages);
    // Softmax state of row r16 (uniform over its four lanes; lsum is this
    // lane's share). o[jb]: rows 4 q4 .. +3, channel DPC r16 + jb.
    float m = kNegBig, lsum = 0.f;
    f32x4_t o[NB];
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) o[jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int wb = pos - ubase; wb < seg_end - ubase; wb += kWave) {
      const int nwin = min(kWave, seg_end - ubase - wb);
      if (wb != pos - ubase) raw = list_raw(wb);
      const int logical = raw;
      const int ph = c.page_table[(int64_t)b * c.max_pages + min(max(logical, 0), c.max_pages - 1)];
      const bool ok = lane < nwin && logical >= 0 && logical < P && ph >= 0 && ph < c.num_phys;
      const int phys_w = ok ? ph : 0;
      const int valid_w = ok ? min(c.page_size, L - logical * c.page_size) : 0;
      const int ntiles = ((nwin << c.ps_log2) + 15) >> 4;

      auto page_base = [&](int e, int& valid) -> int64_t {
        const int ee = min(e, kWave - 1);
        const int phs = __builtin_amdgcn_readlane(phys_w, ee);
        valid = e < nwin ? __builtin_amdgcn_readlane(valid_w, ee) : 0;
        return (((int64_t)phs * c.hkv + g) << c.ps_log2) * D;
      };
      // kv0 / kv1: valid tokens of the tile's one or two entries (two when ps = 8).
      struct TileValid { int kv0, kv1; };
      auto load_tile = [&](int t, u32x4* kr, VC* vr, TileValid& tv) {
        const int e0 = (t * 16) >> c.ps_log2;
        const int64_t base0 = page_base(e0, tv.kv0);
        int64_t base1 = base0;
        tv.kv1 = 0;
        if (c.page_size < 16) base1 = page_base(e0 + 1, tv.kv1);
        {
          const int slot = (t * 16 + r16) & (c.page_size - 1);
          const bool second = c.page_size < 16 && r16 >= c.page_size;
          const int va = second ? tv.kv1 : tv.kv0;
          const uint16_t* src = kp + (second ? base1 : base0) + (slot < va ? slot : 0) * D + 8 * q4;
#pragma unroll
          for (int jj = 0; jj < NJ; ++jj) kr[jj] = load16_stream(src + 32 * jj);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = 4 * q4 + e;
          const int slot = (t * 16 + k) & (c.page_size - 1);
          const bool second = c.page_size < 16 && k >= c.page_size;
          const int va = second ? tv.kv1 : tv.kv0;
          vr[e] = load_vchunk(vp + (second ? base1 : base0) + (slot < va ? slot : 0) * D + DPC * r16,
                              static_cast<VC*>(nullptr));
        }
      };

      // K double-buffered; V chunks become B operands at the top of each
      // iteration, after which the next tile's loads may overwrite them.
      u32x4 kA[NJ], kB[NJ];
      VC vR[4];
      TileValid tA, tB;
      load_tile(0, kA, vR, tA);
      for (int t = 0; t < ntiles; ++t) {
        bool tok_ok[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = 4 * q4 + e;
          const int slot = (t * 16 + k) & (c.page_size - 1);
          const int va = (c.page_size < 16 && k >= c.page_size) ? tA.kv1 : tA.kv0;
          tok_ok[e] = slot < va;
        }
        s16x4_t vb[NB];
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) {
          short h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t wd = vR[e][jb >> 1];
            h[e] = tok_ok[e] ? (short)((jb & 1) ? (wd >> 16) : (wd & 0xFFFFu)) : (short)0;
          }
          vb[jb] = s16x4_t{h[0], h[1], h[2], h[3]};
        }
        if (t + 1 < ntiles) load_tile(t + 1, kB, vR, tB);
        f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kA[jj]), as_bf16x8(qb[jj]), d, 0, 0, 0);
        float sv[4];
        float tmax = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sv[e] = tok_ok[e] ? d[e] * a.qk_scale : -INFINITY;
          tmax = fmaxf(tmax, sv[e]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const bool up = tmax > m + kLazyRescale;
        if (__ballot(up) != 0ull) {  // some row raises its maximum
          const float mnew = up ? tmax : m;
          const float alpha = fast_exp2(m - mnew);
          m = mnew;
          lsum *= alpha;
          float ar[4];  // factors of the accumulator rows 4 q4 + r
#pragma unroll
          for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * q4 + r);
#pragma unroll
          for (int jb = 0; jb < NB; ++jb)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[jb][r] *= ar[r];
        }
        s16x4_t p1, p2, p3;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pe = fast_exp2(sv[e] - m);
          lsum += pe;
          const uint32_t u1 = __float_as_uint(pe) & 0xFFFF0000u;
          const float r1 = pe - __uint_as_float(u1);
          const uint32_t u2 = __float_as_uint(r1) & 0xFFFF0000u;
          const float r2 = r1 - __uint_as_float(u2);
          p1[e] = (short)(u1 >> 16);
          p2[e] = (short)(u2 >> 16);
          p3[e] = (short)(__float_as_uint(r2) >> 16);
        }
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) {
          o[jb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p1, vb[jb], o[jb], 0, 0, 0);
          o[jb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p2, vb[jb], o[jb], 0, 0, 0);
          o[jb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p3, vb[jb], o[jb], 0, 0, 0);
        }
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) kA[jj] = kB[jj];
        tA = tB;
      }
    }

    // Close the segment: each row's l over its four token groups.
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if (j < a.jmax) {
      const int64_t slot0 = ((int64_t)u * a.jmax + j) * G;
      if (q4 < 2) {  // rows 4 q4 + r < 8 are the heads; rows 8..15 repeat them
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float* dst = a.part_acc + (slot0 + 4 * q4 + r) * D + DPC * r16;
#pragma unroll
          for (int jb = 0; jb < NB; ++jb) dst[jb] = o[jb][r];
        }
      }
      if (q4 == 0 && r16 < G) {
        a.part_ml[(slot0 + r16) * 2 + 0] = m;
        a.part_ml[(slot0 + r16) * 2 + 1] = lsum;
      }
      if (lane == 0 && seg_end == s_pre[u + 1]) a.count[u] = j + 1;
    }
    pos = seg_end;
    ++u;
  }
}

// Merge of the stream partials of one (sequence, query head):
// o = sum_j w_j acc_j / sum_j w_j l_j with w_j = 2^(m_j - M), M = max_j m_j,
// and lse = ln2 (M + log2 sum_j w_j l_j). The workgroup's threads split the
// partials by channel group (four channels, one 16-byte load) and chunk
// subset (chunks s, s + NS, ...), so all of a unit's chunks are requested at
// once (up to kMergeBatch per thread, at clamped slots: slots below jmax lie
// inside the workspace), together with the chunk count and the (m, l) pairs:
// a unit of up to kMergeBatch * NS chunks costs one round trip to memory.
// Weights go through LDS; subset sums are added in subset order, so the
// result is fixed for a given chunking.
// The launch takes the smallest form (64 threads x 4 loads, 128 x 8 or
// 256 x 8) whose first batch covers the chunks a unit is expected to have
// (waves / units + 2, at most jmax); units with more take further batches.
constexpr int kMaxMergeChunks = 1024;  // stream_plan caps the chunks per unit here

template <int D, int NT, int kMergeBatch, bool SPARSE>
__global__ __launch_bounds__(NT) void stream_merge_kernel(StreamArgs a) {
  constexpr int kMergeThreads = NT;
  constexpr int CG = D / 4;               // channel groups
  constexpr int NS = kMergeThreads / CG;  // chunk subsets
  constexpr int NWV = kMergeThreads / kWave;
  __shared__ float s_w[kMaxMergeChunks];
  __shared__ float s_red[2][NWV];
  __shared__ float4 s_o[NS][CG];
  const CacheView& c = a.c;
  const int bh = blockIdx.x;
  const int b = bh / c.hq, h = bh % c.hq;
  const int u = b * c.hkv + h / c.group;
  const int hh = h % c.group;
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int cg = tid % CG, sub = tid / CG;
  auto ml_of = [&](int jj) { return a.part_ml + (((int64_t)u * a.jmax + jj) * c.group + hh) * 2; };
  auto acc_of = [&](int jj) {
    return reinterpret_cast<const float4*>(a.part_acc + (((int64_t)u * a.jmax + jj) * c.group + hh) * D) + cg;
  };
  const float* ml0 = ml_of(min(tid, a.jmax - 1));
  const float m0 = ml0[0], l0 = ml0[1];
  float4 pre[kMergeBatch];
#pragma unroll
  for (int q = 0; q < kMergeBatch; ++q) {
    pre[q] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (q * NS < a.jmax) pre[q] = *acc_of(min(sub + q * NS, a.jmax - 1));
  }
  const int n = unit_entries<SPARSE>(a, u);
  const int J = n > 0 ? min(max(a.count[u], 0), a.jmax) : 0;
  float M = tid < J ? m0 : kNegBig;
  for (int jj = tid + kMergeThreads; jj < J; jj += kMergeThreads) M = fmaxf(M, ml_of(jj)[0]);
  M = group_max<kWave>(M);
  if (lane == 0) s_red[0][wv] = M;
  __syncthreads();
  M = s_red[0][0];
#pragma unroll
  for (int i = 1; i < NWV; ++i) M = fmaxf(M, s_red[0][i]);
  float Ls = 0.f;
  if (tid < J) {
    const float w = exp2f(m0 - M);
    s_w[tid] = w;
    Ls = w * l0;
  }
  for (int jj = tid + kMergeThreads; jj < J; jj += kMergeThreads) {
    const float* ml = ml_of(jj);
    const float w = exp2f(ml[0] - M);
    s_w[jj] = w;
    Ls = fmaf(w, ml[1], Ls);
  }
  Ls = group_sum<kWave>(Ls);
  if (lane == 0) s_red[1][wv] = Ls;
  __syncthreads();  // also publishes s_w
  Ls = s_red[1][0];
#pragma unroll
  for (int i = 1; i < NWV; ++i) Ls += s_red[1][i];
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add = [&](float w, const float4& v) {
    o.x = fmaf(w, v.x, o.x);
    o.y = fmaf(w, v.y, o.y);
    o.z = fmaf(w, v.z, o.z);
    o.w = fmaf(w, v.w, o.w);
  };
#pragma unroll
  for (int q = 0; q < kMergeBatch; ++q) {
    const int jj = sub + q * NS;
    if (jj < J) add(s_w[jj], pre[q]);
  }
  // Units of more chunks (long lists over few units): further batches.
  for (int jb = kMergeBatch * NS; jb < J; jb += kMergeBatch * NS) {
    float4 v[kMergeBatch];
#pragma unroll
    for (int q = 0; q < kMergeBatch; ++q) v[q] = *acc_of(min(jb + sub + q * NS, a.jmax - 1));
#pragma unroll
    for (int q = 0; q < kMergeBatch; ++q) {
      const int jj = jb + sub + q * NS;
      if (jj < J) add(s_w[jj], v[q]);
    }
  }
  s_o[sub][cg] = o;
  __syncthreads();
  if (sub == 0) {
    float4 t = s_o[0][cg];
#pragma unroll
    for (int i = 1; i < NS; ++i) {
      t.x += s_o[i][cg].x;
      t.y += s_o[i][cg].y;
      t.z += s_o[i][cg].z;
      t.w += s_o[i][cg].w;
    }
    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
    float* dst = a.out + (int64_t)bh * D + 4 * cg;
    dst[0] = t.x * inv;
    dst[1] = t.y * inv;
    dst[2] = t.z * inv;
    dst[3] = t.w * inv;
  }
  if (a.lse != nullptr && tid == 0) a.lse[bh] = Ls > 0.f ? (M + log2f(Ls)) * kLn2 : -INFINITY;
}

// out_h = sum_j 2^{m_j-M} acc_j / sum_j 2^{m_j-M} l_j, lse_h = ln2 (M + log2 sum_j 2^{m_j-M} l_j),
// splits taken in index order.
template <int D, bool SPARSE>
__global__ __launch_bounds__(kWave) void decode_merge_kernel(DecodeArgs a) {
  constexpr int DPL = D / kWave;  // channels per lane
  __shared__ float s_w[kMaxSplits];
  const CacheView& c = a.c;
  const int bh = blockIdx.x;
  const int b = bh / c.hq;
  const int h = bh % c.hq;
  const int unit = b * c.hkv + h / c.group;
  const int L = max(c.seq_lens[b], 0);
  const int P = min((L + c.page_size - 1) >> c.ps_log2, c.max_pages);
  const int n = list_length<SPARSE>(a, unit, P);
  const int ns = (n + a.pages_per_split - 1) / a.pages_per_split;
  const int lane = threadIdx.x;
  const float* ml = a.part_ml + (int64_t)bh * a.nsplit * 2;
  const float* pa = a.part_acc + (int64_t)bh * a.nsplit * D;
  float M = kNegBig;
  for (int j = lane; j < ns; j += kWave) M = fmaxf(M, ml[2 * j]);
  M = group_max<kWave>(M);
  float Ls = 0.f;
  for (int j = lane; j < ns; j += kWave) {
    const float w = exp2f(ml[2 * j] - M);
    s_w[j] = w;
    Ls += w * ml[2 * j + 1];
  }
  Ls = group_sum<kWave>(Ls);
  __syncthreads();
  float o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;
#pragma unroll 8
  for (int j = 0; j < ns; ++j) {
    const float w = s_w[j];
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] = fmaf(w, pa[(int64_t)j * D + lane * DPL + e], o[e]);
  }
  const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) a.out[(int64_t)bh * D + lane * DPL + e] = o[e] * inv;
  if (a.lse != nullptr && lane == 0) a.lse[bh] = Ls > 0.f ? (M + log2f(Ls)) * kLn2 : -INFINITY;
}

template <typename T, int D, int G, bool SPARSE>
hipError_t decode_impl(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.nsplit, a.c.batch * a.c.hkv);
  hipLaunchKernelGGL((decode_split_kernel<T, D, G, SPARSE>), grid, dim3(kDecodeThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D, SPARSE>), dim3(a.c.batch * a.c.hq), dim3(kWave), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D, bool SPARSE>
hipError_t decode_g(const DecodeArgs& a, hipStream_t s) {
  switch (a.c.group) {
    case 1: return decode_impl<T, D, 1, SPARSE>(a, s);
    case 2: return decode_impl<T, D, 2, SPARSE>(a, s);
    case 4: return decode_impl<T, D, 4, SPARSE>(a, s);
    default: return decode_impl<T, D, 8, SPARSE>(a, s);
  }
}

template <bool SPARSE>
hipError_t decode_dispatch(const DecodeArgs& a, hipStream_t s) {
  if (a.c.dtype == SPDEC_BF16)
    return a.c.head_dim == 64 ? decode_g<BF16, 64, SPARSE>(a, s) : decode_g<BF16, 128, SPARSE>(a, s);
  return a.c.head_dim == 64 ? decode_g<F32, 64, SPARSE>(a, s) : decode_g<F32, 128, SPARSE>(a, s);
}


// The stream kernel for group size G (G = 8: the matrix-core P.V form);
// `waves` (nullable) receives the waves launched.
template <int D, int G, bool SPARSE>
hipError_t stream_kernel_launch(const StreamArgs& a, hipStream_t s, int64_t* waves = nullptr) {
  const int units = a.c.batch * a.c.hkv;
  const size_t lds = (size_t)(units + 1) * sizeof(int);
  const void* fn;
  if constexpr (G == 8)
    fn = reinterpret_cast<const void*>(&decode_stream_g8_kernel<D, SPARSE>);
  else
    fn = reinterpret_cast<const void*>(&decode_stream_kernel<D, G, SPARSE>);
  int grid = 0;
  hipError_t e = persistent_grid(fn, kDecodeThreads, lds, &grid);
  if (e != hipSuccess) return e;
  if (waves != nullptr) *waves = (int64_t)grid * kDecodeWaves;
  if constexpr (G == 8)
    hipLaunchKernelGGL((decode_stream_g8_kernel<D, SPARSE>), dim3(grid), dim3(kDecodeThreads), lds, s, a);
  else
    hipLaunchKernelGGL((decode_stream_kernel<D, G, SPARSE>), dim3(grid), dim3(kDecodeThreads), lds, s, a);
  return hipGetLastError();
}

// The dense stream kernel alone (partials and per-unit chunk counts, no merge).
template <int D, int G>
hipError_t stream_partials_impl(const StreamArgs& a, hipStream_t s) {
  return stream_kernel_launch<D, G, false>(a, s);
}

template <int D, int G, bool SPARSE>
hipError_t stream_impl(const StreamArgs& a, hipStream_t s) {
  int64_t waves = 0;
  hipError_t e = stream_kernel_launch<D, G, SPARSE>(a, s, &waves);
  if (e != hipSuccess) return e;
  const int64_t units = (int64_t)a.c.batch * a.c.hkv;
  const int64_t expect = std::min<int64_t>(a.jmax, (waves + units - 1) / units + 2);
  const dim3 grid(a.c.batch * a.c.hq);
  if (expect <= 4 * (64 / (D / 4)))
    hipLaunchKernelGGL((stream_merge_kernel<D, 64, 4, SPARSE>), grid, dim3(64), 0, s, a);
  else if (expect <= 8 * (128 / (D / 4)))
    hipLaunchKernelGGL((stream_merge_kernel<D, 128, 8, SPARSE>), grid, dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL((stream_merge_kernel<D, 256, 8, SPARSE>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D, bool SPARSE>
hipError_t stream_g(const StreamArgs& a, hipStream_t s) {
  switch (a.c.group) {
    case 1: return stream_impl<D, 1, SPARSE>(a, s);
    case 2: return stream_impl<D, 2, SPARSE>(a, s);
    case 4: return stream_impl<D, 4, SPARSE>(a, s);
    default: return stream_impl<D, 8, SPARSE>(a, s);
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Waves the stream plan is sized for (a few per SIMD on a 256-CU part); more
// resident waves only lengthen each range.
constexpr int kStreamWaveTarget = 8192;

}  // namespace

void stream_plan(int64_t units, int list_pages, int* jmax, int* rmin) {
  *jmax = (int)std::min<int64_t>(std::max<int64_t>((kStreamWaveTarget + units - 1) / units + 2, 3), kMaxMergeChunks);
  *rmin = (list_pages + *jmax - 2) / (*jmax - 1);
}

DecodePlan decode_plan(const CacheView& c, int max_budget_pages) {
  DecodePlan p;
  p.list_pages = max_budget_pages > 0 ? max_budget_pages : c.max_pages;
  const int64_t units = (int64_t)c.batch * c.hkv;
  p.stream = c.dtype == SPDEC_BF16 && units <= kMaxStreamUnits;
  // Stream plan: at most jmax partials per unit, so every wave range holds at
  // least rmin = ceil(cap / (jmax - 1)) entries.
  stream_plan(units, p.list_pages, &p.jmax, &p.rmin);
  // Split plan (fp32 caches and very large batches): about 512 tokens per
  // split, fewer when the grid would leave compute units idle. The plan
  // depends only on the list capacity, so a sparse call whose capacity is
  // every page splits exactly like the dense one.
  constexpr int kTargetTokens = 512;
  int pps = max(1, kTargetTokens / c.page_size);
  while (pps > 1 && units * ((p.list_pages + pps - 1) / pps) < 2048) pps >>= 1;
  pps = max(pps, (p.list_pages + kMaxSplits - 1) / kMaxSplits);
  p.pages_per_split = min(pps, kMaxPagesPerSplit);
  p.nsplit = (p.list_pages + p.pages_per_split - 1) / p.pages_per_split;
  return p;
}

size_t decode_workspace_bytes(const CacheView& c, const DecodePlan& p) {
  if (p.stream) {
    const size_t slots = (size_t)c.batch * c.hkv * p.jmax * c.group;
    return align256(slots * c.head_dim * sizeof(float)) + align256(slots * 2 * sizeof(float)) +
           align256((size_t)c.batch * c.hkv * sizeof(int));
  }
  const size_t rows = (size_t)c.batch * c.hq * p.nsplit;
  return align256(rows * c.head_dim * sizeof(float)) + align256(rows * 2 * sizeof(float));
}

hipError_t launch_decode(const CacheView& c, const DecodePlan& p, const void* q, const int32_t* sel_idx,
                         const int32_t* sel_cnt, float scale, float* out, float* lse, void* ws, hipStream_t s) {
  const bool sparse = sel_idx != nullptr;
  char* base = reinterpret_cast<char*>(ws);
  if (p.stream) {
    StreamArgs a;
    a.c = c;
    a.q = q;
    a.sel_idx = sel_idx;
    a.sel_cnt = sel_cnt;
    a.list_cap = p.list_pages;
    a.jmax = p.jmax;
    a.rmin = p.rmin;
    a.qk_scale = scale * kLog2e;
    const size_t slots = (size_t)c.batch * c.hkv * p.jmax * c.group;
    a.part_acc = reinterpret_cast<float*>(base);
    a.part_ml = reinterpret_cast<float*>(base + align256(slots * c.head_dim * sizeof(float)));
    a.count = reinterpret_cast<int*>(base + align256(slots * c.head_dim * sizeof(float)) +
                                     align256(slots * 2 * sizeof(float)));
    a.out = out;
    a.lse = lse;
    a.first_page = nullptr;
    a.group_size = 1;
    if (c.head_dim == 64) return sparse ? stream_g<64, true>(a, s) : stream_g<64, false>(a, s);
    return sparse ? stream_g<128, true>(a, s) : stream_g<128, false>(a, s);
  }
  DecodeArgs a;
  a.c = c;
  a.q = q;
  a.sel_idx = sel_idx;
  a.sel_cnt = sel_cnt;
  a.list_cap = p.list_pages;
  a.pages_per_split = p.pages_per_split;
  a.nsplit = p.nsplit;
  a.qk_scale = scale * kLog2e;
  const size_t rows = (size_t)c.batch * c.hq * p.nsplit;
  a.part_acc = reinterpret_cast<float*>(base);
  a.part_ml = reinterpret_cast<float*>(base + align256(rows * c.head_dim * sizeof(float)));
  a.out = out;
  a.lse = lse;
  return sparse ? decode_dispatch<true>(a, s) : decode_dispatch<false>(a, s);
}

hipError_t launch_stream_merge(const CacheView& c, const int32_t* sel_cnt, int list_cap, int jmax,
                               const float* part_acc, const float* part_ml, const int* count, float* out, float* lse,
                               hipStream_t s) {
  StreamArgs a;
  a.c = c;
  a.q = nullptr;
  a.sel_idx = nullptr;
  a.sel_cnt = sel_cnt;
  a.list_cap = list_cap;
  a.jmax = jmax;
  a.rmin = 1;
  a.qk_scale = 0.f;
  a.part_acc = const_cast<float*>(part_acc);
  a.part_ml = const_cast<float*>(part_ml);
  a.count = const_cast<int*>(count);
  a.out = out;
  a.lse = lse;
  a.first_page = nullptr;
  a.group_size = 1;
  const dim3 grid(c.batch * c.hq);
  const int D = c.head_dim;
  if (jmax <= 4 * (64 / (D / 4))) {
    if (D == 64) hipLaunchKernelGGL((stream_merge_kernel<64, 64, 4, true>), grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL((stream_merge_kernel<128, 64, 4, true>), grid, dim3(64), 0, s, a);
  } else {
    if (D == 64) hipLaunchKernelGGL((stream_merge_kernel<64, 128, 8, true>), grid, dim3(128), 0, s, a);
    else hipLaunchKernelGGL((stream_merge_kernel<128, 128, 8, true>), grid, dim3(128), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_dense_stream_partials(const CacheView& c, const DecodePlan& p, const void* q,
                                        const int32_t* first_page, int group_size, float scale, float* part_acc,
                                        float* part_ml, int* count, hipStream_t s) {
  StreamArgs a;
  a.c = c;
  a.q = q;
  a.sel_idx = nullptr;
  a.sel_cnt = nullptr;
  a.list_cap = p.list_pages;
  a.jmax = p.jmax;
  a.rmin = p.rmin;
  a.qk_scale = scale * kLog2e;
  a.part_acc = part_acc;
  a.part_ml = part_ml;
  a.count = count;
  a.out = nullptr;
  a.lse = nullptr;
  a.first_page = first_page;
  a.group_size = group_size;
  const int D = c.head_dim;
  switch (c.group) {
    case 1: return D == 64 ? stream_partials_impl<64, 1>(a, s) : stream_partials_impl<128, 1>(a, s);
    case 2: return D == 64 ? stream_partials_impl<64, 2>(a, s) : stream_partials_impl<128, 2>(a, s);
    case 4: return D == 64 ? stream_partials_impl<64, 4>(a, s) : stream_partials_impl<128, 4>(a, s);
    default: return D == 64 ? stream_partials_impl<64, 8>(a, s) : stream_partials_impl<128, 8>(a, s);
  }
}

}  // namespace spdec
