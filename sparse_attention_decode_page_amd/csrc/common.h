// Device helpers shared by the spdec kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spdec {

constexpr int kWave = 64;

// 16 bytes moved per lane per load: the unit every kernel streams in.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Storage types: float, or bf16 kept as raw uint16 bits.
struct F32 {
  using storage = float;
  static constexpr int VEC = 4;  // elements per 16 bytes
  static constexpr int BYTES = 4;
};
struct BF16 {
  using storage = uint16_t;
  static constexpr int VEC = 8;
  static constexpr int BYTES = 2;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Widen one 16-byte chunk to VEC floats (exact for both storage types).
template <typename T>
__device__ __forceinline__ void unpack(const u32x4& r, float* f);

template <>
__device__ __forceinline__ void unpack<F32>(const u32x4& r, float* f) {
  f[0] = __uint_as_float(r.x);
  f[1] = __uint_as_float(r.y);
  f[2] = __uint_as_float(r.z);
  f[3] = __uint_as_float(r.w);
}

template <>
__device__ __forceinline__ void unpack<BF16>(const u32x4& r, float* f) {
  f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x);
  f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
  f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z);
  f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
}

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Streaming load for data read once per kernel (K/V rows, page summaries):
// the non-temporal hint keeps it from displacing reused lines and lifts
// sustained HBM read bandwidth on this chip (measured 6.1 -> 6.8 TB/s for
// random 4 KiB page gathers).
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void store16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// 2^x on the transcendental unit (v_exp_f32, about 1 ulp) without the
// wrapper that computes results below the smallest normal: in softmax weights
// those are far below what the sums can see, and they flush to zero here.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Marks a loaded value as needed at this point, so that its load is not
// sunk into a later branch: independent loads held together share one wait.
__device__ __forceinline__ void hold(int& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void hold(u32x4& x) { asm volatile("" : "+v"(x)); }

// Data-parallel-primitive lane exchange inside a 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadSwap1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7-i inside each 8-lane half
constexpr int kRowMirror = 0x140;      // lane i <-> 15-i inside each 16-lane row

// Butterfly all-reduce over aligned groups of N lanes (N a power of two <= 64).
// Every lane of a group ends with the bit-identical result.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<kQuadSwap1>(x);
  if constexpr (N >= 4) x += dpp<kQuadSwap2>(x);
  if constexpr (N >= 8) x += dpp<kRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kRowMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

template <int CTRL>
__device__ __forceinline__ double dpp(double x) {
  const uint64_t u = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

template <int N>
__device__ __forceinline__ double group_sum(double x) {
  if constexpr (N >= 2) x += dpp<kQuadSwap1>(x);
  if constexpr (N >= 4) x += dpp<kQuadSwap2>(x);
  if constexpr (N >= 8) x += dpp<kRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kRowMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp<kQuadSwap1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp<kQuadSwap2>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp<kRowHalfMirror>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp<kRowMirror>(x));
  if constexpr (N >= 32) x = fmaxf(x, __shfl_xor(x, 16));
  if constexpr (N >= 64) x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

// Running-max sentinel: finite so that empty partial softmax states merge
// without producing NaN (exp2(sentinel - sentinel) == 1 on zero sums).
constexpr float kNegBig = -1.0e30f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// In-place exclusive prefix sum of s[0..n) by the whole workgroup; s[n] gets
// the total. `tmp` needs one int per wave. Ends with a barrier.
__device__ __forceinline__ void block_exclusive_scan(int* s, int n, int* tmp) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int lane = tid % kWave, wave = tid / kWave, nw = nt / kWave;
  const int per = (n + nt - 1) / nt;
  const int i0 = min(tid * per, n), i1 = min(i0 + per, n);
  int sum = 0;
  for (int i = i0; i < i1; ++i) sum += s[i];
  int incl = sum;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == kWave - 1) tmp[wave] = incl;
  __syncthreads();
  int base = incl - sum;
  for (int w = 0; w < wave; ++w) base += tmp[w];
  int total = 0;
  for (int w = 0; w < nw; ++w) total += tmp[w];
  for (int i = i0; i < i1; ++i) {
    const int v = s[i];
    s[i] = base;
    base += v;
  }
  if (tid == 0) s[n] = total;
  __syncthreads();
}

// Largest u in [0, n) with s[u] <= x for a non-decreasing s[0..n] (s[0] <= x).
__device__ __forceinline__ int find_unit(const int* s, int n, int x) {
  int lo = 0, hi = n;  // invariant: s[lo] <= x < s[hi] (s[n] > x)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Order-preserving map of an fp32 score to uint32 (-0 and +0 share one key).
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The score of a key (the inverse of score_key; a zero score comes back as +0).
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

}  // namespace spdec
