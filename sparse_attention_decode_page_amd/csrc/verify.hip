// Dense verification of a sparse draft: causal multi-query decode attention.
//
// After k tokens are drafted with sparse attention, one full-attention pass
// verifies the k + 1 positions over the complete KV cache (S3R page, abstract
// and Tables 6-7; k = 6 there). Query t of the T verified positions sits at
// cache position L - T + t (the drafted tokens are already appended) and
// attends to positions 0 .. L - T + t.
//
// With T positions and G query heads per KV head, every K/V tile meets
// R = G * T query rows (28 for Qwen3-8B at k = 6), so both products are real
// contractions and both run on MFMA:
//   * scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_16x16x32_bf16: K rows as they lie in the page are the A
//     operand (lane l: token l % 16, channels 32j + 8(l / 16) .. +8) and the
//     query rows are the B operand; the result leaves lane l holding query row
//     l % 16 for tokens 4(l / 16) .. +3;
//   * that is exactly the A-operand layout of v_mfma_f32_16x16x16_bf16, so
//     P feeds P.V directly, each fp32 weight as three bf16 terms (its whole
//     significand, so the verified outputs match the single-query dense
//     decode up to summation order). For the B operand each lane
//     loads, for its own four tokens, the chunk of D/16 channels starting at
//     (D/16)(l % 16): column n of block j then stands for channel
//     (D/16) n + j, so V needs no transpose and no LDS.
// Query rows are padded to 16 * NSETS (NSETS <= 2, 32 rows per pass; 33 to 64
// rows take two passes over the cache) and parked in
// LDS (each lane reads back what it wrote) to keep two waves per SIMD. The softmax is
// online in fp32 (log2 domain) with the running maximum raised only when a
// tile exceeds it by 2^8. The (unit, page) pairs are streamed persistently
// exactly like the single-query dense decode; partials are merged per output
// row by a second kernel, chunks in index order.
#include <limits.h>

#include "common.h"
#include "launch.h"

namespace spdec {

namespace {

constexpr int kVerifyThreads = 256;
constexpr int kVerifyWaves = kVerifyThreads / kWave;
constexpr float kVerifyLazyRescale = 8.0f;  // log2 units

typedef __bf16 vbf16x8_t __attribute__((ext_vector_type(8)));
typedef short vs16x4_t __attribute__((ext_vector_type(4)));
typedef float vf32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ vbf16x8_t vas_bf16x8(const u32x4& v) { return __builtin_bit_cast(vbf16x8_t, v); }

// A non-negative finite fp32 weight as three bf16 terms that sum to it
// exactly: hi is the weight with its low 16 bits cleared, mid the same of
// the remainder (w - hi has at most 16 significant bits, and the subtraction
// is exact), lo the remainder after that (at most 8 significant bits, so it
// is a bf16 value).
__device__ __forceinline__ void split3_bf16(float w, short& hi, short& mid, short& lo) {
  const uint32_t u1 = __float_as_uint(w) & 0xFFFF0000u;
  const float r1 = w - __uint_as_float(u1);
  const uint32_t u2 = __float_as_uint(r1) & 0xFFFF0000u;
  const float r2 = r1 - __uint_as_float(u2);
  hi = (short)(u1 >> 16);
  mid = (short)(u2 >> 16);
  lo = (short)(__float_as_uint(r2) >> 16);
}

// A lane's V chunk of one token: DPC bf16 channels (16 bytes for D = 128,
// 8 bytes for D = 64), loaded with the non-temporal hint.
template <int DPC> struct VChunkOf;
template <> struct VChunkOf<8> { using type = u32x4; };
template <> struct VChunkOf<4> { typedef uint32_t type __attribute__((ext_vector_type(2))); };

__device__ __forceinline__ u32x4 load_vchunk_impl(const uint16_t* p, u32x4*) { return load16_stream(p); }
__device__ __forceinline__ VChunkOf<4>::type load_vchunk_impl(const uint16_t* p, VChunkOf<4>::type*) {
  return __builtin_nontemporal_load(reinterpret_cast<const VChunkOf<4>::type*>(p));
}

// bf16 element i of a chunk, as the low 16 bits of a word.
template <typename C>
__device__ __forceinline__ uint32_t vchunk_half(const C& v, int i) {
  const uint32_t w = v[i >> 1];
  return (i & 1) ? (w >> 16) : (w & 0xFFFFu);
}

struct VerifyArgs {
  CacheView c;
  const void* q;     // verify: [B][T][Hq][D]; shared prefix: [B][Hq][D]
  int T;             // verify: positions per sequence; shared prefix: sequences per group
  const int32_t* shared;  // shared prefix: leading pages of each group (read once for the group)
  int rows;          // G * T query rows per unit
  int row0;          // first of the (at most 16 * NSETS) rows this launch computes
  int jmax, rmin;    // stream plan of the dense decode
  float qk_scale;    // softmax scale * log2(e)
  float* part_acc;   // [units][jmax][rows][D]
  float* part_ml;    // [units][jmax][rows][2]
  int* count;        // [units] chunks written for the unit
  float* out;        // [B][T][Hq][D]
  float* lse;        // [B][T][Hq] or null
};

// Two waves per SIMD: with the query rows parked in LDS the 32-row form fits
// the 256 registers that occupancy needs.
//
// PREFIX = true is the same stream over the pages a group of T consecutive
// sequences shares (their prompt): a unit is (group, KV head), its list is the
// group's shared pages (page table and lengths of the group's first
// sequence), and its query rows are the G heads of each of the T members,
// with no causal limit. Each shared page is then read once for the group.
template <int D, int NSETS, bool PREFIX>
__global__ __launch_bounds__(kVerifyThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void verify_stream_kernel(VerifyArgs a) {
  constexpr int NJ = D / 32;        // q.K^T MFMA steps (16x16x32)
  constexpr int NB = D / 16;        // P.V MFMA column blocks (16x16x16)
  constexpr int DPC = D / 16;       // V channels per lane and token
  using VChunk = typename VChunkOf<DPC>::type;
  const CacheView& c = a.c;
  extern __shared__ int s_pre[];    // units + 1
  __shared__ int s_tmp[kVerifyWaves];
  __shared__ __attribute__((aligned(16))) uint16_t s_q[kVerifyWaves][16 * NSETS * D];  // query rows per wave
  const int units = (PREFIX ? c.batch / a.T : c.batch) * c.hkv;
  for (int u = threadIdx.x; u < units; u += kVerifyThreads) {
    const int b = PREFIX ? (u / c.hkv) * a.T : u / c.hkv;
    const int L = max(c.seq_lens[b], 0);
    const int P = min((L + c.page_size - 1) >> c.ps_log2, c.max_pages);
    s_pre[u] = PREFIX ? min(max(a.shared[u / c.hkv], 0), P) : P;
  }
  __syncthreads();
  block_exclusive_scan(s_pre, units, s_tmp);
  const int total = s_pre[units];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int64_t nw = (int64_t)gridDim.x * kVerifyWaves;
  const int64_t w = (int64_t)blockIdx.x * kVerifyWaves + wave;
  const int64_t R = max<int64_t>((total + nw - 1) / nw, a.rmin);
  if (w * R >= total) return;
  int pos = (int)(w * R);
  const int end = (int)min<int64_t>(pos + R, total);
  int u = find_unit(s_pre, units, pos);

  const int r16 = lane % 16;   // K: token of the tile; scores and P: query row of the set
  const int q4 = lane / 16;    // K: channel group; scores: token group 4*q4 .. +3
  const int G = c.group;
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q);
  const uint16_t* kp = reinterpret_cast<const uint16_t*>(c.k_pool);
  const uint16_t* vp = reinterpret_cast<const uint16_t*>(c.v_pool);
  uint16_t* qs = s_q[wave];

  while (pos < end) {
    while (s_pre[u + 1] <= pos) ++u;  // units with no entry have no segment
    while (s_pre[u + 1] <= pos) ++u;  // units with no entry have no segment
    const int b = PREFIX ? (u / c.hkv) * a.T : u / c.hkv;  // sequence whose page table the list follows
    const int g = u % c.hkv;
    const int ubase = s_pre[u];
    const int seg_end = min(end, s_pre[u + 1]);
    const int j = (int)(w - ubase / R);  // this wave's chunk of the unit
    const int L = max(c.seq_lens[b], 0);
    const int P = min((L + c.page_size - 1) >> c.ps_log2, c.max_pages);

    // B operands of S^T = K Q^T: set st, lane l holds query row
    // row0 + 16 st + l % 16 (position t = row / G, head g G + row % G),
    // channels 32 jj + 8 (l / 16).
    // They are parked in this wave's LDS rows (each lane later reads back
    // exactly what it wrote). lim: last token index the row may attend; -1
    // for padding rows.
    int lim[NSETS];
#pragma unroll
    for (int st = 0; st < NSETS; ++st) {
      const int row = a.row0 + 16 * st + r16;
      lim[st] = -1;
      const uint16_t* src = qp;
      if (row < a.rows) {
        const int t = row / G, h = row % G;
        if constexpr (PREFIX) {  // member t of the group; the shared pages precede every query
          lim[st] = INT_MAX;
          src = qp + ((int64_t)(b + t) * c.hq + g * G + h) * D + 8 * q4;
        } else {
          lim[st] = L - a.T + t;
          src = qp + (((int64_t)b * a.T + t) * c.hq + g * G + h) * D + 8 * q4;
        }
      }
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        const u32x4 v = row < a.rows ? load16(src + 32 * jj) : u32x4{0u, 0u, 0u, 0u};
        __builtin_memcpy(qs + (16 * st + r16) * D + 32 * jj + 8 * q4, &v, sizeof(v));
      }
    }
    // Softmax state of the lane's row (uniform over the four lanes of a row);
    // l is this lane's partial over its tokens. o[st][jb]: rows 4 q4 .. +3 of
    // set st, channels 16 jb + l % 16.
    float m[NSETS], lsum[NSETS];
    vf32x4_t o[NSETS][NB];
#pragma unroll
    for (int st = 0; st < NSETS; ++st) {
      m[st] = kNegBig;
      lsum[st] = 0.f;
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) o[st][jb] = vf32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    for (int wb = pos - ubase; wb < seg_end - ubase; wb += kWave) {
      // Window of up to 64 pages: lane i holds page wb+i's physical page and valid tokens.
      const int nwin = min(kWave, seg_end - ubase - wb);
      int phys_w = 0, valid_w = 0;
      if (lane < nwin) {
        const int logical = wb + lane;
        if (logical < P) {
          const int ph = c.page_table[(int64_t)b * c.max_pages + logical];
          if (ph >= 0 && ph < c.num_phys) {
            phys_w = ph;
            valid_w = min(c.page_size, L - logical * c.page_size);
          }
        }
      }
      const int ntiles = ((nwin << c.ps_log2) + 15) >> 4;
      const int tok0 = wb << c.ps_log2;  // cache position of the window's first token

      // Tiles of 16 tokens; a tile spans pages 2t and 2t+1 when ps = 8 (kv0 /
      // kv1 are their valid-token counts). K: lane l loads token l % 16,
      // channels 32 jj + 8 (l / 16) (the A operand of S^T). V: lane l loads,
      // for its four score tokens 4 (l / 16) + e, the channels
      // DPC (l % 16) .. +DPC: column n of P.V block jb then stands for
      // channel DPC n + jb, and the B operand of block jb is element jb of
      // the lane's four V chunks (no transpose, no LDS).
      struct TileValid { int kv0, kv1; };
      auto page_base = [&](int e, int& valid) -> int64_t {
        const int ee = min(e, kWave - 1);
        const int ph = __builtin_amdgcn_readlane(phys_w, ee);
        valid = e < nwin ? __builtin_amdgcn_readlane(valid_w, ee) : 0;
        return (((int64_t)ph * c.hkv + g) << c.ps_log2) * D;
      };
      auto load_vchunk = [](const uint16_t* p) { return load_vchunk_impl(p, static_cast<VChunk*>(nullptr)); };
      auto load_tile = [&](int t, u32x4* kr, VChunk* vr, TileValid& tv) {
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
          vr[e] = load_vchunk(vp + (second ? base1 : base0) + (slot < va ? slot : 0) * D + DPC * r16);
        }
      };

      // K is double-buffered in registers, V carried in one buffer: tile t's
      // V chunks are turned into B operands at the top of iteration t, after
      // which tile t+1's loads may overwrite them.
      u32x4 kA[NJ], kB[NJ];
      VChunk vR[4];
      TileValid tA, tB;
      load_tile(0, kA, vR, tA);
      for (int t = 0; t < ntiles; ++t) {
        // The lane's four tokens: tile tokens 4 q4 + e; present in their page?
        int tpos[4];
        bool tok_ok[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = 4 * q4 + e;
          const int slot = (t * 16 + k) & (c.page_size - 1);
          const int va = (c.page_size < 16 && k >= c.page_size) ? tA.kv1 : tA.kv0;
          tok_ok[e] = slot < va;
          tpos[e] = tok0 + t * 16 + k;
        }
        // B operands of P.V: block jb takes channel DPC n + jb of the four
        // tokens (unread slots as zeros).
        vs16x4_t vb[NB];
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) {
          uint32_t h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = tok_ok[e] ? vchunk_half(vR[e], jb) : 0u;
          vb[jb] = vs16x4_t{(short)h[0], (short)h[1], (short)h[2], (short)h[3]};
        }
        if (t + 1 < ntiles) load_tile(t + 1, kB, vR, tB);
        // An opaque zero added to the query-row LDS address keeps those reads
        // inside the loop (hoisted, they would pin 16 * NSETS registers).
        int oz;
        asm volatile("v_mov_b32 %0, 0" : "=v"(oz));
#pragma unroll
        for (int st = 0; st < NSETS; ++st) {
          vf32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int jj = 0; jj < NJ; ++jj) {
            u32x4 qv;
            __builtin_memcpy(&qv, qs + oz + (16 * st + r16) * D + 32 * jj + 8 * q4, sizeof(qv));
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vas_bf16x8(kA[jj]), vas_bf16x8(qv), d, 0, 0, 0);
          }
          float s[4];
          float tmax = -INFINITY;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s[e] = (tok_ok[e] && tpos[e] <= lim[st]) ? d[e] * a.qk_scale : -INFINITY;
            tmax = fmaxf(tmax, s[e]);
          }
          tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
          tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
          const bool up = tmax > m[st] + kVerifyLazyRescale;
          if (__ballot(up) != 0ull) {  // some row of the set raises its maximum
            const float mnew = up ? tmax : m[st];
            const float alpha = fast_exp2(m[st] - mnew);
            m[st] = mnew;
            lsum[st] *= alpha;
            float ar[4];  // factors of the accumulator rows 4 q4 + r (held by lanes 0..15)
#pragma unroll
            for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * q4 + r);
#pragma unroll
            for (int jb = 0; jb < NB; ++jb)
#pragma unroll
              for (int r = 0; r < 4; ++r) o[st][jb][r] *= ar[r];
          }
          // Each fp32 weight enters P.V as three bf16 terms that sum to it
          // exactly (split3_bf16): the products match fp32 weights and the
          // result matches the single-query dense decode up to summation order.
          vs16x4_t p1, p2, p3;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pe = fast_exp2(s[e] - m[st]);
            lsum[st] += pe;
            short hi, mid, lo;
            split3_bf16(pe, hi, mid, lo);
            p1[e] = hi;
            p2[e] = mid;
            p3[e] = lo;
          }
#pragma unroll
          for (int jb = 0; jb < NB; ++jb) {
            o[st][jb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p1, vb[jb], o[st][jb], 0, 0, 0);
            o[st][jb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p2, vb[jb], o[st][jb], 0, 0, 0);
            o[st][jb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p3, vb[jb], o[st][jb], 0, 0, 0);
          }
        }
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) kA[jj] = kB[jj];
        tA = tB;
      }
    }

    // Close the segment: each row's l over its four token groups.
#pragma unroll
    for (int st = 0; st < NSETS; ++st) {
      lsum[st] += __shfl_xor(lsum[st], 16);
      lsum[st] += __shfl_xor(lsum[st], 32);
    }
    if (j < a.jmax) {
      const int64_t slot0 = ((int64_t)u * a.jmax + j) * a.rows;
#pragma unroll
      for (int st = 0; st < NSETS; ++st) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = a.row0 + 16 * st + 4 * q4 + r;
          if (row < a.rows) {
            float* dst = a.part_acc + (slot0 + row) * D + DPC * r16;
#pragma unroll
            for (int jb = 0; jb < NB; ++jb) dst[jb] = o[st][jb][r];
          }
        }
        const int row = a.row0 + 16 * st + r16;
        if (q4 == 0 && row < a.rows) {
          a.part_ml[(slot0 + row) * 2 + 0] = m[st];
          a.part_ml[(slot0 + row) * 2 + 1] = lsum[st];
        }
      }
      if (lane == 0 && seg_end == s_pre[u + 1]) a.count[u] = j + 1;
    }
    pos = seg_end;
    ++u;
  }
}

// One wave per output row (sequence, position, query head): chunks in index order.
// The first kVerifyMergePre chunks' partials (slots below jmax lie inside the
// workspace) are requested together with the chunk count: one round trip for
// a unit of that many chunks.
constexpr int kVerifyMergePre = 8;

template <int D>
__global__ __launch_bounds__(kWave) void verify_merge_kernel(VerifyArgs a) {
  constexpr int DPL = D / kWave;
  const CacheView& c = a.c;
  const int orow = blockIdx.x;  // ((b * T + t) * Hq + hq)
  const int hq = orow % c.hq;
  const int bt = orow / c.hq;
  const int b = bt / a.T, t = bt % a.T;
  const int u = b * c.hkv + hq / c.group;
  const int row = t * c.group + hq % c.group;
  const int lane = threadIdx.x;
  auto ml_of = [&](int jj) { return a.part_ml + (((int64_t)u * a.jmax + jj) * a.rows + row) * 2; };
  auto acc_of = [&](int jj) { return a.part_acc + (((int64_t)u * a.jmax + jj) * a.rows + row) * D + lane * DPL; };
  const float* ml0 = ml_of(min(lane, a.jmax - 1));
  const float m0 = ml0[0], l0 = ml0[1];
  float pre[kVerifyMergePre][DPL];
#pragma unroll
  for (int i = 0; i < kVerifyMergePre; ++i) {
    const float* src = acc_of(min(i, a.jmax - 1));
#pragma unroll
    for (int e = 0; e < DPL; ++e) pre[i][e] = src[e];
  }
  const int L = max(c.seq_lens[b], 0);
  const int P = min((L + c.page_size - 1) >> c.ps_log2, c.max_pages);
  const int J = P > 0 ? min(max(a.count[u], 0), a.jmax) : 0;
  float M = lane < J ? m0 : kNegBig;
  for (int jj = lane + kWave; jj < J; jj += kWave) M = fmaxf(M, ml_of(jj)[0]);
  M = group_max<kWave>(M);
  // Lane jj holds chunk jj's weight; chunks past the wave width (long lists
  // only) recompute theirs where they are used.
  float Ls = 0.f, w_own = 0.f;
  if (lane < J) {
    w_own = exp2f(m0 - M);
    Ls += w_own * l0;
  }
  for (int jj = lane + kWave; jj < J; jj += kWave) {
    const float* ml = ml_of(jj);
    Ls += exp2f(ml[0] - M) * ml[1];
  }
  Ls = group_sum<kWave>(Ls);
  float o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;
#pragma unroll
  for (int i = 0; i < kVerifyMergePre; ++i) {
    if (i < J) {
      const float wgt = __shfl(w_own, i);
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] = fmaf(wgt, pre[i][e], o[e]);
    }
  }
  // Later chunks (long lists), kVerifyMergePre loads in flight at a time, at clamped
  // slots (unused ones are never summed).
  for (int jb = kVerifyMergePre; jb < J; jb += kVerifyMergePre) {
    float v[kVerifyMergePre][DPL];
#pragma unroll
    for (int q = 0; q < kVerifyMergePre; ++q) {
      const float* src = acc_of(min(jb + q, a.jmax - 1));
#pragma unroll
      for (int e = 0; e < DPL; ++e) v[q][e] = src[e];
    }
#pragma unroll
    for (int q = 0; q < kVerifyMergePre; ++q) {
      const int jj = jb + q;
      if (jj < J) {
        const float wgt = jj < kWave ? __shfl(w_own, jj) : exp2f(ml_of(jj)[0] - M);
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] = fmaf(wgt, v[q][e], o[e]);
      }
    }
  }
  const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) a.out[(int64_t)orow * D + lane * DPL + e] = o[e] * inv;
  if (a.lse != nullptr && lane == 0) a.lse[orow] = Ls > 0.f ? (M + log2f(Ls)) * kLn2 : -INFINITY;
}

template <int D, int NSETS, bool PREFIX>
hipError_t stream_launch(const VerifyArgs& a, hipStream_t s) {
  const int units = (PREFIX ? a.c.batch / a.T : a.c.batch) * a.c.hkv;
  const size_t lds = (size_t)(units + 1) * sizeof(int);
  int grid = 0;
  hipError_t e = persistent_grid(reinterpret_cast<const void*>(&verify_stream_kernel<D, NSETS, PREFIX>),
                                 kVerifyThreads, lds, &grid);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((verify_stream_kernel<D, NSETS, PREFIX>), dim3(grid), dim3(kVerifyThreads), lds, s, a);
  return hipGetLastError();
}

// Up to 32 rows in one pass; 33 .. 64 rows (eight heads per KV head at
// k >= 4, say) in two passes of 32 rows over the same stream plan, each
// reading the K/V once more, into the same partial slots.
template <int D, int NSETS>
hipError_t verify_impl(const VerifyArgs& a0, hipStream_t s) {
  VerifyArgs a = a0;
  hipError_t e = hipSuccess;
  for (a.row0 = 0; a.row0 < a.rows && e == hipSuccess; a.row0 += 16 * NSETS) e = stream_launch<D, NSETS, false>(a, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((verify_merge_kernel<D>), dim3(a.c.batch * a.T * a.c.hq), dim3(kWave), 0, s, a);
  return hipGetLastError();
}

size_t align256v(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

bool verify_supported(const CacheView& c, int T) {
  return c.dtype == SPDEC_BF16 && T >= 1 && T <= 16 && c.group * T <= 64 &&
         (int64_t)c.batch * c.hkv <= kMaxStreamUnits;
}

size_t verify_workspace_bytes(const CacheView& c, int T) {
  const DecodePlan p = decode_plan(c, 0);
  const size_t slots = (size_t)c.batch * c.hkv * p.jmax * c.group * T;
  return align256v(slots * c.head_dim * sizeof(float)) + align256v(slots * 2 * sizeof(float)) +
         align256v((size_t)c.batch * c.hkv * sizeof(int));
}

hipError_t launch_verify(const CacheView& c, const void* q, int T, float scale, float* out, float* lse, void* ws,
                         hipStream_t s) {
  const DecodePlan p = decode_plan(c, 0);
  VerifyArgs a;
  a.c = c;
  a.q = q;
  a.T = T;
  a.shared = nullptr;
  a.rows = c.group * T;
  a.row0 = 0;
  a.jmax = p.jmax;
  a.rmin = p.rmin;
  a.qk_scale = scale * kLog2e;
  const size_t slots = (size_t)c.batch * c.hkv * p.jmax * a.rows;
  char* base = reinterpret_cast<char*>(ws);
  a.part_acc = reinterpret_cast<float*>(base);
  a.part_ml = reinterpret_cast<float*>(base + align256v(slots * c.head_dim * sizeof(float)));
  a.count = reinterpret_cast<int*>(base + align256v(slots * c.head_dim * sizeof(float)) +
                                   align256v(slots * 2 * sizeof(float)));
  a.out = out;
  a.lse = lse;
  const bool two = a.rows > 16;
  if (c.head_dim == 64) return two ? verify_impl<64, 2>(a, s) : verify_impl<64, 1>(a, s);
  return two ? verify_impl<128, 2>(a, s) : verify_impl<128, 1>(a, s);
}

hipError_t launch_prefix_partials(const CacheView& c, const void* q, int group_size, const int32_t* shared_pages,
                                  int jmax, int rmin, float scale, float* part_acc, float* part_ml, int* count,
                                  hipStream_t s) {
  VerifyArgs a;
  a.c = c;
  a.q = q;
  a.T = group_size;
  a.shared = shared_pages;
  a.rows = c.group * group_size;
  a.row0 = 0;
  a.jmax = jmax;
  a.rmin = rmin;
  a.qk_scale = scale * kLog2e;
  a.part_acc = part_acc;
  a.part_ml = part_ml;
  a.count = count;
  a.out = nullptr;
  a.lse = nullptr;
  if (a.rows <= 16) return c.head_dim == 64 ? stream_launch<64, 1, true>(a, s) : stream_launch<128, 1, true>(a, s);
  // 17 .. 64 rows: passes of 32 rows over the same plan (33 .. 64 rows read the shared pages twice).
  hipError_t e = hipSuccess;
  for (a.row0 = 0; a.row0 < a.rows && e == hipSuccess; a.row0 += 32)
    e = c.head_dim == 64 ? stream_launch<64, 2, true>(a, s) : stream_launch<128, 2, true>(a, s);
  return e;
}

}  // namespace spdec
