// Page key summaries: per-page, per-channel key minimum and maximum.
//
// The page bound used for selection (Quest-style, cited by title on the
// Sparrow citation-map page) needs, for every page, the elementwise minimum and
// maximum of the keys it holds. They are kept current as tokens are appended
// (append_kv) and can be rebuilt in bulk from a prefilled cache (build_meta).
// min/max select existing values, so the summary is exact in the KV dtype.
#include "common.h"
#include "launch.h"

namespace spdec {

namespace {

template <typename T>
__device__ __forceinline__ void minmax_chunk(const u32x4& k, u32x4& lo, u32x4& hi, bool first);

// Elementwise min/max on decoded values; the stored bits are the winning
// element's own bits, ties keep the value already held.
template <>
__device__ __forceinline__ void minmax_chunk<F32>(const u32x4& k, u32x4& lo, u32x4& hi, bool first) {
  if (first) { lo = k; hi = k; return; }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float kv = __uint_as_float(k[i]);
    if (kv < __uint_as_float(lo[i])) lo[i] = k[i];
    if (kv > __uint_as_float(hi[i])) hi[i] = k[i];
  }
}

__device__ __forceinline__ uint32_t pick_bf16_pair(uint32_t cur, uint32_t k, bool want_min) {
  float c0 = bf16_lo(cur), c1 = bf16_hi(cur);
  float k0 = bf16_lo(k), k1 = bf16_hi(k);
  uint32_t lo_bits = ((want_min ? (k0 < c0) : (k0 > c0)) ? k : cur) & 0x0000ffffu;
  uint32_t hi_bits = ((want_min ? (k1 < c1) : (k1 > c1)) ? k : cur) & 0xffff0000u;
  return lo_bits | hi_bits;
}

template <>
__device__ __forceinline__ void minmax_chunk<BF16>(const u32x4& k, u32x4& lo, u32x4& hi, bool first) {
  if (first) { lo = k; hi = k; return; }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo[i] = pick_bf16_pair(lo[i], k[i], true);
    hi[i] = pick_bf16_pair(hi[i], k[i], false);
  }
}

// One workgroup per sequence; lanes cover (KV head, 16-byte channel chunk).
template <typename T, int D>
__global__ __launch_bounds__(256) void append_kv_kernel(CacheView c, const void* __restrict__ k_new,
                                                        const void* __restrict__ v_new) {
  constexpr int VEC = T::VEC;
  constexpr int CPR = D / VEC;  // 16-byte chunks per head row
  const int b = blockIdx.x;
  const int t = c.seq_lens[b];
  const int page = t >> c.ps_log2;
  const int slot = t & (c.page_size - 1);
  int phys = -1;
  if (t >= 0 && page < c.max_pages) phys = c.page_table[(int64_t)b * c.max_pages + page];
  const bool ok = phys >= 0 && phys < c.num_phys;
  if (ok) {
    using S = typename T::storage;
    const S* kn = reinterpret_cast<const S*>(k_new);
    const S* vn = reinterpret_cast<const S*>(v_new);
    S* kp = reinterpret_cast<S*>(c.k_pool);
    S* vp = reinterpret_cast<S*>(c.v_pool);
    S* mm = reinterpret_cast<S*>(c.kminmax);
    for (int i = threadIdx.x; i < c.hkv * CPR; i += blockDim.x) {
      const int g = i / CPR;
      const int d0 = (i % CPR) * VEC;
      const int64_t src = ((int64_t)b * c.hkv + g) * D + d0;
      const int64_t dst = (((int64_t)phys * c.hkv + g) * c.page_size + slot) * D + d0;
      const int64_t mrow = ((int64_t)phys * c.hkv + g) * 2 * D + d0;
      u32x4 k = load16(kn + src);
      u32x4 v = load16(vn + src);
      store16(kp + dst, k);
      store16(vp + dst, v);
      u32x4 lo, hi;
      if (slot != 0) { lo = load16(mm + mrow); hi = load16(mm + mrow + D); }
      minmax_chunk<T>(k, lo, hi, slot == 0);
      store16(mm + mrow, lo);
      store16(mm + mrow + D, hi);
    }
  }
  __syncthreads();  // every lane has read seq_lens[b] before it moves
  if (threadIdx.x == 0 && ok) c.seq_lens[b] = t + 1;
}

// Workgroup = (a run of kPagesPerBlock logical pages, one sequence).
constexpr int kPagesPerBlock = 8;

template <typename T, int D>
__global__ __launch_bounds__(256) void build_meta_kernel(CacheView c) {
  constexpr int VEC = T::VEC;
  constexpr int CPR = D / VEC;
  using S = typename T::storage;
  const int b = blockIdx.y;
  const int L = c.seq_lens[b];
  const int P = min((L + c.page_size - 1) >> c.ps_log2, c.max_pages);
  const int p0 = blockIdx.x * kPagesPerBlock;
  if (p0 >= P) return;
  const S* kp = reinterpret_cast<const S*>(c.k_pool);
  S* mm = reinterpret_cast<S*>(c.kminmax);
  const int items = kPagesPerBlock * c.hkv * CPR;
  for (int i = threadIdx.x; i < items; i += blockDim.x) {
    const int pl = i / (c.hkv * CPR);
    const int rem = i % (c.hkv * CPR);
    const int g = rem / CPR;
    const int d0 = (rem % CPR) * VEC;
    const int p = p0 + pl;
    if (p >= P) continue;
    const int phys = c.page_table[(int64_t)b * c.max_pages + p];
    if (phys < 0 || phys >= c.num_phys) continue;
    const int valid = min(c.page_size, L - p * c.page_size);
    const S* base = kp + (((int64_t)phys * c.hkv + g) * c.page_size) * D + d0;
    u32x4 lo, hi;
    for (int s = 0; s < valid; ++s) minmax_chunk<T>(load16_stream(base + (int64_t)s * D), lo, hi, s == 0);
    const int64_t mrow = ((int64_t)phys * c.hkv + g) * 2 * D + d0;
    store16(mm + mrow, lo);
    store16(mm + mrow + D, hi);
  }
}

template <typename T, int D>
hipError_t append_impl(const CacheView& c, const void* k, const void* v, hipStream_t s) {
  hipLaunchKernelGGL((append_kv_kernel<T, D>), dim3(c.batch), dim3(256), 0, s, c, k, v);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t build_impl(const CacheView& c, hipStream_t s) {
  dim3 grid((c.max_pages + kPagesPerBlock - 1) / kPagesPerBlock, c.batch);
  hipLaunchKernelGGL((build_meta_kernel<T, D>), grid, dim3(256), 0, s, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append_kv(const CacheView& c, const void* k_new, const void* v_new, hipStream_t s) {
  if (c.dtype == SPDEC_BF16) {
    return c.head_dim == 64 ? append_impl<BF16, 64>(c, k_new, v_new, s) : append_impl<BF16, 128>(c, k_new, v_new, s);
  }
  return c.head_dim == 64 ? append_impl<F32, 64>(c, k_new, v_new, s) : append_impl<F32, 128>(c, k_new, v_new, s);
}

hipError_t launch_build_meta(const CacheView& c, hipStream_t s) {
  if (c.dtype == SPDEC_BF16) return c.head_dim == 64 ? build_impl<BF16, 64>(c, s) : build_impl<BF16, 128>(c, s);
  return c.head_dim == 64 ? build_impl<F32, 64>(c, s) : build_impl<F32, 128>(c, s);
}

}  // namespace spdec
