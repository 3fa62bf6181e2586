// Sparsity-schedule controller: one correction of the budget schedule per step
// from the on-device tail statistic, so the budgets of the next step follow
// the monitored acceptance without a host round trip.
//
// The Sparrow project page ("Control Study 1") grows the budget with the
// generated length so the per-token mismatch stays roughly constant, and keeps
// the lower 5th percentile of the per-token acceptance at a threshold; it gives
// no control law. Here the schedule is linear in the cached length,
//   tokens_b = s * (base + slope * L_b),  pages_b = clamp(ceil(tokens_b / ps), 2, cap),
// and the scalar s is corrected once per step by a multiplicative integral
// step s' = clamp(s * (1 + gain * (target - p5)), s_min, s_max).
// Every step is one IEEE fp32 operation with its own rounding (no fused
// multiply-add), so the integer budgets are reproducible bit for bit.
#include "common.h"
#include "launch.h"

namespace spdec {

namespace {

constexpr int kControlThreads = 256;

__global__ __launch_bounds__(kControlThreads) void budget_update_kernel(const float* __restrict__ tail,
                                                                       float* __restrict__ state,
                                                                       const int32_t* __restrict__ seq_lens,
                                                                       int batch, spdec_budget_params p,
                                                                       int32_t* __restrict__ budget) {
  float s = state[0];
  if (!(s > 0.f) || !isfinite(s)) s = p.scale_max;  // lost state: the most lenient schedule
  const float p5 = tail[1];
  if (isfinite(p5)) {
    const float e = __fsub_rn(p.target, p5);
    s = __fmul_rn(s, __fadd_rn(1.0f, __fmul_rn(p.gain, e)));
  }
  s = s < p.scale_min ? p.scale_min : (s > p.scale_max ? p.scale_max : s);
  __syncthreads();  // every thread has read the old state
  if (threadIdx.x == 0) state[0] = s;
  const float ps = (float)p.page_size;
  for (int b = threadIdx.x; b < batch; b += kControlThreads) {
    const float L = (float)max(seq_lens[b], 0);
    const float tok = __fmul_rn(s, __fadd_rn(p.base_tokens, __fmul_rn(p.tokens_per_token, L)));
    const float pages = __fdiv_rn(tok, ps);  // a power of two: exact
    budget[b] = !(pages < (float)p.max_budget_pages) ? p.max_budget_pages : max((int)ceilf(pages), 2);
  }
}

}  // namespace

hipError_t launch_budget_update(const float* tail, float* state, const int32_t* seq_lens, int batch,
                                const spdec_budget_params& p, int32_t* budget, hipStream_t s) {
  hipLaunchKernelGGL(budget_update_kernel, dim3(1), dim3(kControlThreads), 0, s, tail, state, seq_lens, batch, p,
                     budget);
  return hipGetLastError();
}

}  // namespace spdec
