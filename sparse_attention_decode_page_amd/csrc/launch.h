// Host-side launchers behind the C ABI (one per kernel family).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "spdec.h"

namespace spdec {

// Validated, flattened view of a spdec_cache plus derived shape constants.
struct CacheView {
  int batch, hq, hkv, group, head_dim, page_size, ps_log2, max_pages;
  int64_t num_phys;
  int dtype;
  void* k_pool;
  void* v_pool;
  void* kminmax;
  const int32_t* page_table;
  int32_t* seq_lens;
};

// Split-KV plan shared by the workspace query and the decode launch.
struct DecodePlan {
  bool stream;       // persistent stream-K kernel (bf16) instead of fixed splits
  int jmax, rmin;    // stream plan: partial slots per unit, minimum entries per wave
  int pages_per_split;
  int nsplit;        // splits per (sequence, KV head) at the list capacity
  int list_pages;    // capacity of the page list (max_budget_pages or max_pages)
};

DecodePlan decode_plan(const CacheView& c, int max_budget_pages);

// Units (sequence x KV head) up to which the persistent kernels keep the
// per-unit prefix in LDS.
constexpr int kMaxStreamUnits = 8192;

// Workgroups that fill the current device once for `kernel` (resident blocks
// per compute unit x compute units).
hipError_t persistent_grid(const void* kernel, int block, size_t dyn_lds, int* grid);
size_t decode_workspace_bytes(const CacheView& c, const DecodePlan& p);
size_t select_workspace_bytes(const CacheView& c);
size_t acceptance_workspace_bytes(int rows, int vocab);

hipError_t launch_append_kv(const CacheView& c, const void* k_new, const void* v_new, hipStream_t s);
hipError_t launch_build_meta(const CacheView& c, hipStream_t s);
hipError_t launch_select(const CacheView& c, const void* q, const int32_t* budget, int max_budget,
                         int32_t* sel_idx, int32_t* sel_cnt, float* scores, void* ws, hipStream_t s);
hipError_t launch_decode(const CacheView& c, const DecodePlan& p, const void* q, const int32_t* sel_idx,
                         const int32_t* sel_cnt, float scale, float* out, float* lse, void* ws, hipStream_t s);
bool verify_supported(const CacheView& c, int T);
size_t verify_workspace_bytes(const CacheView& c, int T);
hipError_t launch_verify(const CacheView& c, const void* q, int T, float scale, float* out, float* lse, void* ws,
                         hipStream_t s);
size_t spec_accept_workspace_bytes(int batch, int k, int vocab);
hipError_t launch_spec_accept(const float* p, const float* q, int batch, int k, int vocab, int64_t stride,
                              const int32_t* draft, const float* u_accept, const float* u_sample, float temperature,
                              int32_t* n_accepted, int32_t* token, void* ws, hipStream_t s);
hipError_t launch_acceptance(const float* a, const float* b, int rows, int vocab, int64_t stride, float temperature,
                             float* alpha, void* ws, hipStream_t s);

}  // namespace spdec
