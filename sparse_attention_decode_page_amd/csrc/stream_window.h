// One wave's attention over a window of page-list entries (device code shared
// by the stream decode kernels and the fused sparse-path kernel).
//
// A tile is 16 consecutive tokens of the list. One MFMA contracts 32
// channels: A = the group's queries (the 16 rows hold query heads h % G), B =
// 16 tokens x 32 channels of K loaded straight from the page, D = 16 rows x 16
// tokens in four fp32 registers per lane: lane l holds token l%16 and rows
// 4(l/16)..+3, i.e. every head once (G <= 4). Softmax state is per head and
// uniform across the wave; the running maximum is only raised when a tile
// exceeds it by more than 2^8. P.V stays on the VALU with V rows read as
// 1 KiB contiguous wave loads; each lane fetches its token's probability from
// the lane that owns that token (ds_bpermute).
#pragma once

#include "common.h"
#include "launch.h"

namespace spdec {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr float kLazyRescale = 8.0f;  // log2 units

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8_t, v); }

// Streams one window of up to 64 page-list entries of KV head g (lane i holds
// entry i's physical page phys_w and valid-token count valid_w; entries at and
// past nwin hold none) in tiles of 16 tokens into this wave's running softmax
// state: m (log2 units), lsum (per token lane) and acc (per V row group).
// q.K^T runs on v_mfma_f32_16x16x32_bf16 with row r16 of the A operand holding
// query head r16 % G (qa), P.V on the VALU; the next tile is loaded while one
// is used.
template <int D, int G>
__device__ __forceinline__ void stream_window(const CacheView& c, int g, int nwin, int phys_w, int valid_w,
                                              const u32x4 (&qa)[D / 32], float qk_scale, int lane, float (&m)[G],
                                              float (&lsum)[G], float (&acc)[G][8]) {
  constexpr int NJ = D / 32;             // MFMAs per tile
  constexpr int LPT = D / 8;             // lanes per V row
  constexpr int TPI = kWave / LPT;       // V rows per load instruction
  constexpr int NV = 16 / TPI;           // V load instructions per tile
  const int r16 = lane % 16;   // token of the tile this lane scores
  const int q4 = lane / 16;    // row group
  const int vsub = lane % LPT; // V channel chunk
  const int vtok = lane / LPT; // V row within a load instruction
  const uint16_t* kp = reinterpret_cast<const uint16_t*>(c.k_pool);
  const uint16_t* vp = reinterpret_cast<const uint16_t*>(c.v_pool);
  const int ntiles = ((nwin << c.ps_log2) + 15) >> 4;

  // Tiles of 16 stream tokens. For every supported page size the entry of
  // a V load instruction is wave-uniform, and so is a K tile's entry when
  // ps >= 16 (with ps = 8 a K tile spans entries 2t and 2t+1): physical
  // page and valid-token count come from the window with v_readlane into
  // scalar registers, and per-lane addresses are 32-bit offsets from a
  // scalar page base.
  auto page_base = [&](int e, int& valid) -> int64_t {
    const int ee = min(e, kWave - 1);
    const int ph = __builtin_amdgcn_readlane(phys_w, ee);
    valid = e < nwin ? __builtin_amdgcn_readlane(valid_w, ee) : 0;
    return (((int64_t)ph * c.hkv + g) << c.ps_log2) * D;
  };
  // Per tile only wave-uniform valid-token counts are carried (kv0/kv1 for
  // the K tile's one or two entries, vv[i] for V load i); each lane
  // re-derives its own validity from its slot when the data is used.
  struct TileValid { int kv0, kv1, vv[NV]; };
  auto k_slot = [&](int t) { return (t * 16 + r16) & (c.page_size - 1); };
  auto v_slot = [&](int t, int i) { return (t * 16 + i * TPI + vtok) & (c.page_size - 1); };
  auto k_ok = [&](int t, const TileValid& tv) {
    const int va = (c.page_size < 16 && r16 >= c.page_size) ? tv.kv1 : tv.kv0;
    return k_slot(t) < va;
  };
  auto load_tile = [&](int t, u32x4* kr, u32x4* vr, TileValid& tv) {
    {
      const int e0 = (t * 16) >> c.ps_log2;
      int64_t base = page_base(e0, tv.kv0);
      tv.kv1 = 0;
      if (c.page_size < 16) {  // the tile's second half lies on the next entry
        const int64_t base1 = page_base(e0 + 1, tv.kv1);
        if (r16 >= c.page_size) base = base1;
      }
      const int slot = k_slot(t);
      const uint16_t* src = kp + base + (k_ok(t, tv) ? slot : 0) * D + 8 * q4;
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) kr[jj] = load16_stream(src + 32 * jj);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int64_t base = page_base((t * 16 + i * TPI) >> c.ps_log2, tv.vv[i]);
      const int slot = v_slot(t, i);
      vr[i] = load16_stream(vp + base + (slot < tv.vv[i] ? slot : 0) * D + 8 * vsub);
    }
  };

  u32x4 kA[NJ], vA[NV], kB[NJ], vB[NV];
  TileValid tA, tB;
  load_tile(0, kA, vA, tA);
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) load_tile(t + 1, kB, vB, tB);
    // Row 4 q4 + r holds head r % G, so d[h] is head h's score of the lane's token.
    float sc[G];
    {
      f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj)
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[jj]), as_bf16x8(kA[jj]), d, 0, 0, 0);
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h] = d[h];
    }
    const bool kok = k_ok(t, tA);
    float p[G], mnew[G];
    bool grow = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      p[h] = kok ? sc[h] * qk_scale : -INFINITY;
      const float tmax = group_max<16>(p[h]);
      const bool up = tmax > m[h] + kLazyRescale;
      mnew[h] = up ? tmax : m[h];
      grow |= up;
    }
    if (grow) {  // uniform across the wave: every lane sees the same tile maxima
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float alpha = fast_exp2(m[h] - mnew[h]);
        lsum[h] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
        m[h] = mnew[h];
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      p[h] = fast_exp2(p[h] - m[h]);
      lsum[h] += p[h];
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float vf[8];
      unpack<BF16>(vA[i], vf);
      if (v_slot(t, i) >= tA.vv[i]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[e] = 0.f;  // never multiply unread slots
      }
      const int src = (i * TPI + vtok) * 4;       // byte address of the lane owning this token
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ph = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(p[h])));
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(ph, vf[e], acc[h][e]);
      }
    }
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) kA[jj] = kB[jj];
#pragma unroll
    for (int i = 0; i < NV; ++i) vA[i] = vB[i];
    tA = tB;
  }
}

// Closes a wave's segment: lsum summed over the 16 token lanes, acc over the
// V row groups (every lane of a V channel chunk then holds its sums).
template <int D, int G>
__device__ __forceinline__ void close_segment(float (&lsum)[G], float (&acc)[G][8]) {
  constexpr int LPT = D / 8;
#pragma unroll
  for (int h = 0; h < G; ++h) lsum[h] = group_sum<16>(lsum[h]);
#pragma unroll
  for (int off = LPT; off < kWave; off <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);
}

}  // namespace
}  // namespace spdec
