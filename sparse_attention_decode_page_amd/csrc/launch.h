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

// Stream plan for `units` lists of at most `list_pages` entries: partial slots
// per unit (jmax) and the minimum entries per wave range (rmin) that bound the
// chunks of a unit by jmax.
void stream_plan(int64_t units, int list_pages, int* jmax, int* rmin);

// Units (sequence x KV head) up to which the persistent kernels keep the
// per-unit prefix in LDS.
constexpr int kMaxStreamUnits = 8192;

// Workgroups that fill the current device once for `kernel` (resident blocks
// per compute unit x compute units).
hipError_t persistent_grid(const void* kernel, int block, size_t dyn_lds, int* grid);
// Compute units of the current device (0 if the runtime cannot say).
int device_compute_units();
size_t decode_workspace_bytes(const CacheView& c, const DecodePlan& p);
size_t select_workspace_bytes(const CacheView& c);
size_t acceptance_workspace_bytes(int rows, int vocab);

hipError_t launch_append_kv(const CacheView& c, const void* k_new, const void* v_new, hipStream_t s);
hipError_t launch_build_meta(const CacheView& c, hipStream_t s);
hipError_t launch_select(const CacheView& c, const void* q, const int32_t* budget, int max_budget,
                         int32_t* sel_idx, int32_t* sel_cnt, float* scores, void* ws, hipStream_t s);
// Page scores of every (sequence, KV head) into scores[unit][max_pages].
hipError_t launch_score(const CacheView& c, const void* q, float* scores, hipStream_t s);
// Score-mass (top-p) selection: scoring, then the kept set per unit.
hipError_t launch_select_top_p(const CacheView& c, const void* q, float top_p, float score_scale,
                               const int32_t* budget, int max_budget, int32_t* sel_idx, int32_t* sel_cnt,
                               float* scores, void* ws, hipStream_t s);
// Selection with the shared leading pages of each group of group_size
// sequences scored once per (group, KV head); same outputs as launch_select.
bool select_shared_supported(const CacheView& c, int group_size);
hipError_t launch_select_shared(const CacheView& c, const void* q, const int32_t* budget, int max_budget,
                                int group_size, const int32_t* shared_pages, int32_t* sel_idx, int32_t* sel_cnt,
                                float* scores, void* ws, hipStream_t s);
// The whole sparse path (scores, Top-B select, attention over the kept pages,
// merge) in one launch, one workgroup per (sequence, KV head): bf16 caches
// with G <= 4, at most kPathMaxPages pages per sequence and in the list, at
// most kPathMaxSeqs sequences, and at least one unit per compute unit.
constexpr int kPathMaxPages = 4096;
constexpr int kPathMaxSeqs = 512;
bool path_fused_supported(const CacheView& c, int max_budget);
// The sliced sparse path for batches of few units: each unit's pages cut into
// S slices scored by S workgroups (slice candidates, then the unit's Top-B
// from them) and its kept list streamed by the same S workgroups, partials
// merged by the stream merge. slice_count gives S for this shape on a device
// of `cus` compute units, 0 where the form does not apply (bf16, G <= 4, at
// least two slices per unit, at most kSliceMaxUnits units and kSliceMaxPages pages per slice,
// S * (max_budget - 2) <= kSliceMaxCand candidates, max_budget <= kSliceMaxList).
constexpr int kSliceMaxS = 16;
constexpr int kSliceMaxUnits = 128;
constexpr int kSliceMaxPages = 4096;
constexpr int kSliceMaxCand = 4096;
constexpr int kSliceMaxList = 4096;
int slice_count(const CacheView& c, int max_budget, int cus);
size_t slice_workspace_bytes(const CacheView& c, int max_budget);
// out == nullptr: the selection only (sel_idx, sel_cnt, scores).
hipError_t launch_slice_path(const CacheView& c, const void* q, const int32_t* budget, int max_budget, int S,
                             float scale, int32_t* sel_idx, int32_t* sel_cnt, float* scores, float* out, float* lse,
                             void* ws, hipStream_t s);
// The stream merge alone over partials in the decode's layout ([units][jmax]
// slots, count[u] of them written); units with sel_cnt 0 get zeros, lse -inf.
hipError_t launch_stream_merge(const CacheView& c, const int32_t* sel_cnt, int list_cap, int jmax,
                               const float* part_acc, const float* part_ml, const int* count, float* out, float* lse,
                               hipStream_t s);
hipError_t launch_sparse_path_fused(const CacheView& c, const void* q, const int32_t* budget, int max_budget,
                                    float scale, int32_t* sel_idx, int32_t* sel_cnt, float* scores, float* out,
                                    float* lse, hipStream_t s);
// spdec_select_pages_top_p in one kernel (the shapes path_fused_supported takes):
// scores in LDS, the top-p cut there.
hipError_t launch_select_topp_fused(const CacheView& c, const void* q, float top_p, float score_scale,
                                    const int32_t* budget, int max_budget, int32_t* sel_idx, int32_t* sel_cnt,
                                    float* scores, hipStream_t s);
hipError_t launch_decode(const CacheView& c, const DecodePlan& p, const void* q, const int32_t* sel_idx,
                         const int32_t* sel_cnt, float scale, float* out, float* lse, void* ws, hipStream_t s);
// Dense stream partials over each sequence's pages from first_page[b / group_size]
// on (the shared-prefix decode's suffix pass); no merge.
hipError_t launch_dense_stream_partials(const CacheView& c, const DecodePlan& p, const void* q,
                                        const int32_t* first_page, int group_size, float scale, float* part_acc,
                                        float* part_ml, int* count, hipStream_t s);
// Multi-row partials over the pages a group of group_size sequences shares
// (shared_pages[n] leading pages of group n, read once for the group's
// group_size * G query rows); no merge.
hipError_t launch_prefix_partials(const CacheView& c, const void* q, int group_size, const int32_t* shared_pages,
                                  int jmax, int rmin, float scale, float* part_acc, float* part_ml, int* count,
                                  hipStream_t s);
bool shared_supported(const CacheView& c, int group_size);
size_t shared_workspace_bytes(const CacheView& c, int group_size);
hipError_t launch_dense_shared(const CacheView& c, const void* q, int group_size, const int32_t* shared_pages,
                               float scale, float* out, float* lse, void* ws, hipStream_t s);
bool verify_supported(const CacheView& c, int T);
size_t verify_workspace_bytes(const CacheView& c, int T);
hipError_t launch_verify(const CacheView& c, const void* q, int T, float scale, float* out, float* lse, void* ws,
                         hipStream_t s);
size_t spec_accept_workspace_bytes(int batch, int k, int vocab);
hipError_t launch_spec_accept(const float* p, const float* q, int batch, int k, int vocab, int64_t stride,
                              const int32_t* draft, const float* u_accept, const float* u_sample, float temperature,
                              int32_t* n_accepted, int32_t* token, void* ws, hipStream_t s);
constexpr int kTailMaxRows = 8192;  // values the tail statistics sort in LDS
hipError_t launch_tail_stats(const float* alpha, int n, float* out, hipStream_t s);
// Streaming tail monitor (ring of per-token acceptance values; capacity <= kMonitorMaxCapacity).
constexpr int kMonitorMaxCapacity = 1 << 28;
size_t monitor_workspace_bytes(int capacity);
hipError_t launch_monitor_reset(void* ws, int capacity, hipStream_t s);
hipError_t launch_monitor_append(void* ws, int capacity, const float* alpha, int n, hipStream_t s);
hipError_t launch_monitor_stats(void* ws, int capacity, float* out, hipStream_t s);
hipError_t launch_budget_update(const float* tail, float* state, const int32_t* seq_lens, int batch,
                                const spdec_budget_params& p, int32_t* budget, hipStream_t s);
// Precondition counts of spdec_check_inputs into report[SPDEC_CHECK_WORDS].
hipError_t launch_check(const CacheView& c, const void* q, const int32_t* sel_idx, const int32_t* sel_cnt,
                        int max_budget, int group_size, const int32_t* shared_pages, int32_t* report, hipStream_t s);
// Bytes at the start of an acceptance workspace that must be zero before its
// first call; every call leaves them zero.
size_t acceptance_sync_bytes();
// Polls of a row's chunk pairs before a single-read workgroup reads the row itself.
constexpr int kAcceptanceSpinLimit = 1 << 14;
// Options of the acceptance launch (null: automatic path, default wait).
struct AcceptanceDiag {
  int force_path;   // -1 automatic, 1 single read, 2 two passes
  int spin_limit;   // -1 default
  int* fallbacks;   // device int32, nullable: single-read workgroups that stopped waiting
  int* path;        // host, nullable: the path taken (1 or 2)
};
hipError_t launch_acceptance(const float* a, const float* b, int rows, int vocab, int64_t stride, float temperature,
                             float* alpha, void* ws, hipStream_t s, const AcceptanceDiag* diag);
// Host-side argument checks shared by the acceptance entry points.
spdec_status acceptance_args(const float* logits_a, const float* logits_b, int rows, int vocab, int64_t row_stride,
                             float temperature, float* alpha);

}  // namespace spdec
