// C ABI of libspdec: argument checks, workspace queries and stream-ordered launches.
//
// Every entry point validates its host-side arguments before touching the HIP
// runtime, so a rejected call launches nothing and needs no GPU.
#include <math.h>

#include "launch.h"
#include "spdec.h"

using spdec::CacheView;

namespace {

constexpr int kMaxPagesPerSeq = 32768;

int log2_exact(int v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return (1 << s) == v ? s : -1;
}

// Checks the descriptor's shape fields; fills `v` on success.
spdec_status view_of(const spdec_cache* c, CacheView* v) {
  if (c == nullptr) return SPDEC_ERR_INVALID;
  if (c->batch < 1 || c->num_q_heads < 1 || c->num_kv_heads < 1 || c->max_pages_per_seq < 1 ||
      c->num_phys_pages < 1 || c->head_dim < 1 || c->page_size < 1)
    return SPDEC_ERR_INVALID;
  if (c->num_q_heads % c->num_kv_heads != 0) return SPDEC_ERR_INVALID;
  if ((int64_t)c->batch * c->num_kv_heads > 65535) return SPDEC_ERR_UNSUPPORTED;  // grid.y limit
  if (c->max_pages_per_seq > kMaxPagesPerSeq) return SPDEC_ERR_UNSUPPORTED;
  const int group = c->num_q_heads / c->num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8) return SPDEC_ERR_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return SPDEC_ERR_UNSUPPORTED;
  if (c->page_size != 8 && c->page_size != 16 && c->page_size != 32 && c->page_size != 64) return SPDEC_ERR_UNSUPPORTED;
  if (c->dtype != SPDEC_F32 && c->dtype != SPDEC_BF16) return SPDEC_ERR_UNSUPPORTED;
  if (c->page_table == nullptr || c->seq_lens == nullptr) return SPDEC_ERR_INVALID;
  v->batch = c->batch;
  v->hq = c->num_q_heads;
  v->hkv = c->num_kv_heads;
  v->group = group;
  v->head_dim = c->head_dim;
  v->page_size = c->page_size;
  v->ps_log2 = log2_exact(c->page_size);
  v->max_pages = c->max_pages_per_seq;
  v->num_phys = c->num_phys_pages;
  v->dtype = c->dtype;
  v->k_pool = c->k_pool;
  v->v_pool = c->v_pool;
  v->kminmax = c->kminmax;
  v->page_table = c->page_table;
  v->seq_lens = c->seq_lens;
  return SPDEC_OK;
}

spdec_status from_hip(hipError_t e) { return e == hipSuccess ? SPDEC_OK : SPDEC_ERR_HIP; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

const char* spdec_status_string(spdec_status status) {
  switch (status) {
    case SPDEC_OK: return "SPDEC_OK";
    case SPDEC_ERR_INVALID: return "SPDEC_ERR_INVALID: invalid argument";
    case SPDEC_ERR_UNSUPPORTED: return "SPDEC_ERR_UNSUPPORTED: shape or dtype not supported";
    case SPDEC_ERR_WORKSPACE: return "SPDEC_ERR_WORKSPACE: workspace missing or too small";
    case SPDEC_ERR_HIP: return "SPDEC_ERR_HIP: HIP runtime error";
    default: return "unknown spdec status";
  }
}

int spdec_version(void) { return 100; }

float spdec_default_scale(const spdec_cache* cache) {
  CacheView v;
  if (view_of(cache, &v) != SPDEC_OK) return 0.f;
  return (float)(1.0 / sqrt((double)v.head_dim));  // rounded once
}

float spdec_default_score_scale(const spdec_cache* cache) {
  CacheView v;
  if (view_of(cache, &v) != SPDEC_OK) return 0.f;
  return (float)(1.0 / ((double)v.group * sqrt((double)v.head_dim)));  // rounded once
}

spdec_status spdec_append_kv(const spdec_cache* cache, const void* k_new, const void* v_new, hipStream_t stream) {
  CacheView v;
  spdec_status st = view_of(cache, &v);
  if (st != SPDEC_OK) return st;
  if (!v.k_pool || !v.v_pool || !v.kminmax || !k_new || !v_new) return SPDEC_ERR_INVALID;
  if (!aligned16(v.k_pool) || !aligned16(v.v_pool) || !aligned16(v.kminmax) || !aligned16(k_new) || !aligned16(v_new))
    return SPDEC_ERR_INVALID;
  return from_hip(spdec::launch_append_kv(v, k_new, v_new, stream));
}

spdec_status spdec_build_meta(const spdec_cache* cache, hipStream_t stream) {
  CacheView v;
  spdec_status st = view_of(cache, &v);
  if (st != SPDEC_OK) return st;
  if (!v.k_pool || !v.kminmax || !aligned16(v.k_pool) || !aligned16(v.kminmax)) return SPDEC_ERR_INVALID;
  return from_hip(spdec::launch_build_meta(v, stream));
}

size_t spdec_select_workspace_bytes(const spdec_cache* cache, int max_budget_pages) {
  CacheView v;
  if (view_of(cache, &v) != SPDEC_OK || max_budget_pages < 2) return 0;
  const size_t scores = spdec::select_workspace_bytes(v);
  const size_t sliced = spdec::slice_workspace_bytes(v, max_budget_pages);
  return scores > sliced ? scores : sliced;
}

// The form spdec_select_pages takes for a validated shape on the current
// device, given workspace_bytes of workspace: the one-kernel selection needs
// none, the sliced one its candidate slots, the two kernels the scores
// (unless they go to scores_out).
static int select_form(const CacheView& v, int max_budget_pages, size_t workspace_bytes, int* slices) {
  *slices = 0;
  if (spdec::path_fused_supported(v, max_budget_pages)) return SPDEC_PATH_ONE_KERNEL;
  const int S = spdec::slice_count(v, max_budget_pages, spdec::device_compute_units());
  if (S > 0 && workspace_bytes >= spdec::slice_workspace_bytes(v, max_budget_pages)) {
    *slices = S;
    return SPDEC_PATH_SLICED;
  }
  return SPDEC_PATH_TWO_CALLS;
}

int spdec_select_pages_form(const spdec_cache* cache, int max_budget_pages) {
  CacheView v;
  const spdec_status st = view_of(cache, &v);
  if (st != SPDEC_OK) return st;
  if (max_budget_pages < 2) return SPDEC_ERR_INVALID;
  int slices;
  return select_form(v, max_budget_pages, spdec_select_workspace_bytes(cache, max_budget_pages), &slices);
}

spdec_status spdec_select_pages(const spdec_cache* cache, const void* q, const int32_t* budget_pages,
                                int max_budget_pages, int32_t* sel_idx, int32_t* sel_cnt, float* scores_out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  CacheView v;
  spdec_status st = view_of(cache, &v);
  if (st != SPDEC_OK) return st;
  if (!v.kminmax || !q || !budget_pages || !sel_idx || !sel_cnt) return SPDEC_ERR_INVALID;
  if (!aligned16(v.kminmax) || !aligned16(q)) return SPDEC_ERR_INVALID;
  if (max_budget_pages < 2) return SPDEC_ERR_INVALID;
  if (scores_out == nullptr &&
      (workspace == nullptr || workspace_bytes < spdec_select_workspace_bytes(cache, max_budget_pages)))
    return SPDEC_ERR_WORKSPACE;
  int slices;
  const int form = select_form(v, max_budget_pages, workspace == nullptr ? 0 : workspace_bytes, &slices);
  if (form == SPDEC_PATH_ONE_KERNEL)
    return from_hip(spdec::launch_sparse_path_fused(v, q, budget_pages, max_budget_pages, 1.f, sel_idx, sel_cnt,
                                                    scores_out, nullptr, nullptr, stream));
  if (form == SPDEC_PATH_SLICED)
    return from_hip(spdec::launch_slice_path(v, q, budget_pages, max_budget_pages, slices, 1.f, sel_idx, sel_cnt,
                                             scores_out, nullptr, nullptr, workspace, stream));
  return from_hip(spdec::launch_select(v, q, budget_pages, max_budget_pages, sel_idx, sel_cnt, scores_out, workspace,
                                       stream));
}

spdec_status spdec_select_pages_top_p(const spdec_cache* cache, const void* q, float top_p, float score_scale,
                                      const int32_t* budget_pages, int max_budget_pages, int32_t* sel_idx,
                                      int32_t* sel_cnt, float* scores_out, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  CacheView v;
  spdec_status st = view_of(cache, &v);
  if (st != SPDEC_OK) return st;
  if (!v.kminmax || !q || !sel_idx || !sel_cnt) return SPDEC_ERR_INVALID;
  if (!aligned16(v.kminmax) || !aligned16(q)) return SPDEC_ERR_INVALID;
  if (max_budget_pages < 2) return SPDEC_ERR_INVALID;
  if (!isfinite(top_p) || !(top_p > 0.f) || !(top_p <= 1.f)) return SPDEC_ERR_INVALID;
  if (!isfinite(score_scale) || !(score_scale >= 0.f)) return SPDEC_ERR_INVALID;
  if (scores_out == nullptr &&
      (workspace == nullptr || workspace_bytes < spdec_select_workspace_bytes(cache, max_budget_pages)))
    return SPDEC_ERR_WORKSPACE;
  return from_hip(spdec::launch_select_top_p(v, q, top_p, score_scale, budget_pages, max_budget_pages, sel_idx,
                                             sel_cnt, scores_out, workspace, stream));
}

spdec_status spdec_select_pages_shared(const spdec_cache* cache, const void* q, int group_size,
                                       const int32_t* shared_pages, const int32_t* budget_pages,
                                       int max_budget_pages, int32_t* sel_idx, int32_t* sel_cnt, float* scores_out,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  CacheView v;
  spdec_status st = view_of(cache, &v);
  if (st != SPDEC_OK) return st;
  if (!v.kminmax || !q || !budget_pages || !sel_idx || !sel_cnt || !shared_pages) return SPDEC_ERR_INVALID;
  if (!aligned16(v.kminmax) || !aligned16(q)) return SPDEC_ERR_INVALID;
  if (max_budget_pages < 2) return SPDEC_ERR_INVALID;
  if (group_size < 1 || v.batch % group_size != 0) return SPDEC_ERR_INVALID;
  if (!spdec::select_shared_supported(v, group_size)) return SPDEC_ERR_UNSUPPORTED;
  if (scores_out == nullptr &&
      (workspace == nullptr || workspace_bytes < spdec_select_workspace_bytes(cache, max_budget_pages)))
    return SPDEC_ERR_WORKSPACE;
  return from_hip(spdec::launch_select_shared(v, q, budget_pages, max_budget_pages, group_size, shared_pages, sel_idx,
                                              sel_cnt, scores_out, workspace, stream));
}

size_t spdec_decode_workspace_bytes(const spdec_cache* cache, int max_budget_pages) {
  CacheView v;
  if (view_of(cache, &v) != SPDEC_OK || max_budget_pages < 0) return 0;
  return spdec::decode_workspace_bytes(v, spdec::decode_plan(v, max_budget_pages));
}

static spdec_status decode_common(const spdec_cache* cache, const void* q, const int32_t* sel_idx,
                                  const int32_t* sel_cnt, int max_budget_pages, float scale, float* out, float* lse,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  CacheView v;
  spdec_status st = view_of(cache, &v);
  if (st != SPDEC_OK) return st;
  if (!v.k_pool || !v.v_pool || !q || !out) return SPDEC_ERR_INVALID;
  if (!aligned16(v.k_pool) || !aligned16(v.v_pool) || !aligned16(q)) return SPDEC_ERR_INVALID;
  if (!(scale > 0.f) || !isfinite(scale)) return SPDEC_ERR_INVALID;
  const spdec::DecodePlan plan = spdec::decode_plan(v, max_budget_pages);
  if (workspace == nullptr || workspace_bytes < spdec::decode_workspace_bytes(v, plan)) return SPDEC_ERR_WORKSPACE;
  return from_hip(spdec::launch_decode(v, plan, q, sel_idx, sel_cnt, scale, out, lse, workspace,
                                       stream));
}

spdec_status spdec_sparse_decode(const spdec_cache* cache, const void* q, const int32_t* sel_idx,
                                 const int32_t* sel_cnt, int max_budget_pages, float scale, float* out, float* lse,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!sel_idx || !sel_cnt || max_budget_pages < 1) return SPDEC_ERR_INVALID;
  return decode_common(cache, q, sel_idx, sel_cnt, max_budget_pages, scale, out, lse, workspace, workspace_bytes,
                       stream);
}

spdec_status spdec_dense_decode(const spdec_cache* cache, const void* q, float scale, float* out, float* lse,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_common(cache, q, nullptr, nullptr, 0, scale, out, lse, workspace, workspace_bytes, stream);
}

static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// The form spdec_sparse_path takes for a validated shape on the current device.
static int path_form(const CacheView& v, int max_budget_pages, int* slices) {
  *slices = 0;
  if (spdec::path_fused_supported(v, max_budget_pages)) return SPDEC_PATH_ONE_KERNEL;
  *slices = spdec::slice_count(v, max_budget_pages, spdec::device_compute_units());
  return *slices > 0 ? SPDEC_PATH_SLICED : SPDEC_PATH_TWO_CALLS;
}

static size_t two_call_bytes(const CacheView& v, int max_budget_pages) {
  return align256(spdec::select_workspace_bytes(v)) +
         spdec::decode_workspace_bytes(v, spdec::decode_plan(v, max_budget_pages));
}

size_t spdec_sparse_path_workspace_bytes(const spdec_cache* cache, int max_budget_pages) {
  CacheView v;
  if (view_of(cache, &v) != SPDEC_OK || max_budget_pages < 2) return 0;
  const size_t two = two_call_bytes(v, max_budget_pages);
  const size_t sliced = spdec::slice_workspace_bytes(v, max_budget_pages);
  return two > sliced ? two : sliced;
}

int spdec_sparse_path_form(const spdec_cache* cache, int max_budget_pages) {
  CacheView v;
  const spdec_status st = view_of(cache, &v);
  if (st != SPDEC_OK) return st;
  if (max_budget_pages < 2) return SPDEC_ERR_INVALID;
  int slices;
  return path_form(v, max_budget_pages, &slices);
}

spdec_status spdec_sparse_path(const spdec_cache* cache, const void* q, const int32_t* budget_pages,
                               int max_budget_pages, float scale, int32_t* sel_idx, int32_t* sel_cnt,
                               float* scores_out, float* out, float* lse, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  CacheView v;
  spdec_status st = view_of(cache, &v);
  if (st != SPDEC_OK) return st;
  if (!v.k_pool || !v.v_pool || !v.kminmax || !q || !budget_pages || !sel_idx || !sel_cnt || !out)
    return SPDEC_ERR_INVALID;
  if (!aligned16(v.k_pool) || !aligned16(v.v_pool) || !aligned16(v.kminmax) || !aligned16(q))
    return SPDEC_ERR_INVALID;
  if (max_budget_pages < 2) return SPDEC_ERR_INVALID;
  if (!(scale > 0.f) || !isfinite(scale)) return SPDEC_ERR_INVALID;
  if (workspace == nullptr || workspace_bytes < spdec_sparse_path_workspace_bytes(cache, max_budget_pages))
    return SPDEC_ERR_WORKSPACE;
  int slices;
  const int form = path_form(v, max_budget_pages, &slices);
  if (form == SPDEC_PATH_ONE_KERNEL)
    return from_hip(spdec::launch_sparse_path_fused(v, q, budget_pages, max_budget_pages, scale, sel_idx, sel_cnt,
                                                    scores_out, out, lse, stream));
  if (form == SPDEC_PATH_SLICED)
    return from_hip(spdec::launch_slice_path(v, q, budget_pages, max_budget_pages, slices, scale, sel_idx, sel_cnt,
                                             scores_out, out, lse, workspace, stream));
  char* ws = static_cast<char*>(workspace);
  const size_t score_bytes = align256(spdec::select_workspace_bytes(v));
  hipError_t e = spdec::launch_select(v, q, budget_pages, max_budget_pages, sel_idx, sel_cnt, scores_out, ws, stream);
  if (e != hipSuccess) return from_hip(e);
  return from_hip(spdec::launch_decode(v, spdec::decode_plan(v, max_budget_pages), q, sel_idx, sel_cnt, scale, out,
                                       lse, ws + score_bytes, stream));
}

size_t spdec_shared_workspace_bytes(const spdec_cache* cache, int group_size) {
  CacheView v;
  if (view_of(cache, &v) != SPDEC_OK || !spdec::shared_supported(v, group_size)) return 0;
  return spdec::shared_workspace_bytes(v, group_size);
}

spdec_status spdec_dense_decode_shared(const spdec_cache* cache, const void* q, int group_size,
                                       const int32_t* shared_pages, float scale, float* out, float* lse,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  CacheView v;
  spdec_status st = view_of(cache, &v);
  if (st != SPDEC_OK) return st;
  if (!v.k_pool || !v.v_pool || !q || !out || !shared_pages) return SPDEC_ERR_INVALID;
  if (!aligned16(v.k_pool) || !aligned16(v.v_pool) || !aligned16(q)) return SPDEC_ERR_INVALID;
  if (!(scale > 0.f) || !isfinite(scale)) return SPDEC_ERR_INVALID;
  if (group_size < 1 || v.batch % group_size != 0) return SPDEC_ERR_INVALID;
  if (!spdec::shared_supported(v, group_size)) return SPDEC_ERR_UNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < spdec::shared_workspace_bytes(v, group_size))
    return SPDEC_ERR_WORKSPACE;
  return from_hip(spdec::launch_dense_shared(v, q, group_size, shared_pages, scale, out, lse, workspace,
                                             stream));
}

size_t spdec_verify_workspace_bytes(const spdec_cache* cache, int num_positions) {
  CacheView v;
  if (view_of(cache, &v) != SPDEC_OK || !spdec::verify_supported(v, num_positions)) return 0;
  return spdec::verify_workspace_bytes(v, num_positions);
}

spdec_status spdec_verify_decode(const spdec_cache* cache, const void* q, int num_positions, float scale,
                                 float* out, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  CacheView v;
  spdec_status st = view_of(cache, &v);
  if (st != SPDEC_OK) return st;
  if (!v.k_pool || !v.v_pool || !q || !out) return SPDEC_ERR_INVALID;
  if (!aligned16(v.k_pool) || !aligned16(v.v_pool) || !aligned16(q)) return SPDEC_ERR_INVALID;
  if (!(scale > 0.f) || !isfinite(scale)) return SPDEC_ERR_INVALID;
  if (num_positions < 1) return SPDEC_ERR_INVALID;
  if (!spdec::verify_supported(v, num_positions)) return SPDEC_ERR_UNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < spdec::verify_workspace_bytes(v, num_positions))
    return SPDEC_ERR_WORKSPACE;
  return from_hip(spdec::launch_verify(v, q, num_positions, scale, out, lse, workspace,
                                       stream));
}

size_t spdec_spec_accept_workspace_bytes(int batch, int num_draft, int vocab) {
  if (batch < 1 || batch > 65535 || num_draft < 0 || num_draft > 64 || vocab < 1 || vocab > (1 << 28)) return 0;
  return spdec::spec_accept_workspace_bytes(batch, num_draft, vocab);
}

spdec_status spdec_spec_accept(const float* p_logits, const float* q_logits, int batch, int num_draft, int vocab,
                               int64_t row_stride, const int32_t* draft, const float* u_accept,
                               const float* u_sample, float temperature, int32_t* num_accepted,
                               int32_t* next_token, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!p_logits || !u_sample || !num_accepted || !next_token) return SPDEC_ERR_INVALID;
  if (num_draft > 0 && (!q_logits || !draft || !u_accept)) return SPDEC_ERR_INVALID;
  if (batch < 1 || num_draft < 0 || vocab < 1 || vocab > (1 << 28) || row_stride < vocab) return SPDEC_ERR_INVALID;
  if (batch > 65535 || num_draft > 64 || (int64_t)batch * (2 * num_draft + 1) > 65535) return SPDEC_ERR_UNSUPPORTED;
  if (!(temperature > 0.f) || !isfinite(temperature)) return SPDEC_ERR_INVALID;
  if (workspace == nullptr || workspace_bytes < spdec::spec_accept_workspace_bytes(batch, num_draft, vocab))
    return SPDEC_ERR_WORKSPACE;
  return from_hip(spdec::launch_spec_accept(p_logits, num_draft > 0 ? q_logits : p_logits, batch, num_draft, vocab,
                                            row_stride, draft, u_accept, u_sample, temperature, num_accepted,
                                            next_token, workspace, stream));
}

size_t spdec_acceptance_workspace_bytes(int rows, int vocab) {
  if (rows < 1 || vocab < 1 || vocab > (1 << 28)) return 0;
  return spdec::acceptance_workspace_bytes(rows, vocab);
}

}  // extern "C"

spdec_status spdec::acceptance_args(const float* logits_a, const float* logits_b, int rows, int vocab,
                                    int64_t row_stride, float temperature, float* alpha) {
  if (!logits_a || !logits_b || !alpha) return SPDEC_ERR_INVALID;
  if (rows < 1 || vocab < 1 || vocab > (1 << 28) || row_stride < vocab) return SPDEC_ERR_INVALID;
  if (rows > 65535) return SPDEC_ERR_UNSUPPORTED;
  if (!(temperature > 0.f) || !isfinite(temperature)) return SPDEC_ERR_INVALID;
  return SPDEC_OK;
}

extern "C" {

spdec_status spdec_acceptance(const float* logits_a, const float* logits_b, int rows, int vocab, int64_t row_stride,
                              float temperature, float* alpha, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  const spdec_status st = spdec::acceptance_args(logits_a, logits_b, rows, vocab, row_stride, temperature, alpha);
  if (st != SPDEC_OK) return st;
  if (workspace == nullptr || workspace_bytes < spdec::acceptance_workspace_bytes(rows, vocab))
    return SPDEC_ERR_WORKSPACE;
  return from_hip(spdec::launch_acceptance(logits_a, logits_b, rows, vocab, row_stride, temperature, alpha, workspace,
                                           stream, nullptr));
}

spdec_status spdec_acceptance_ex(const float* logits_a, const float* logits_b, int rows, int vocab,
                                 int64_t row_stride, float temperature, float* alpha, void* workspace,
                                 size_t workspace_bytes, int force_path, int spin_limit, int32_t* fallbacks,
                                 int32_t* path_taken, hipStream_t stream) {
  const spdec_status st = spdec::acceptance_args(logits_a, logits_b, rows, vocab, row_stride, temperature, alpha);
  if (st != SPDEC_OK) return st;
  if (force_path != -1 && force_path != 1 && force_path != 2) return SPDEC_ERR_INVALID;
  if (spin_limit < -1) return SPDEC_ERR_INVALID;
  if (workspace == nullptr || workspace_bytes < spdec::acceptance_workspace_bytes(rows, vocab))
    return SPDEC_ERR_WORKSPACE;
  spdec::AcceptanceDiag diag{force_path, spin_limit, fallbacks, path_taken};
  const hipError_t e = spdec::launch_acceptance(logits_a, logits_b, rows, vocab, row_stride, temperature, alpha,
                                                workspace, stream, &diag);
  if (e == hipErrorInvalidValue && force_path == 1) return SPDEC_ERR_UNSUPPORTED;
  return from_hip(e);
}

spdec_status spdec_budget_update(const float* tail, float* scale, const int32_t* seq_lens, int batch,
                                 const spdec_budget_params* params, int32_t* budget_pages, hipStream_t stream) {
  if (!tail || !scale || !seq_lens || !params || !budget_pages) return SPDEC_ERR_INVALID;
  const spdec_budget_params& p = *params;
  auto fin = [](float x) { return isfinite(x); };
  if (!fin(p.target) || !(p.target > 0.f) || !(p.target <= 1.f)) return SPDEC_ERR_INVALID;
  if (!fin(p.gain) || !(p.gain >= 0.f)) return SPDEC_ERR_INVALID;
  if (!fin(p.scale_min) || !fin(p.scale_max) || !(p.scale_min > 0.f) || !(p.scale_min <= p.scale_max))
    return SPDEC_ERR_INVALID;
  if (!fin(p.base_tokens) || !(p.base_tokens >= 0.f) || !fin(p.tokens_per_token) || !(p.tokens_per_token >= 0.f))
    return SPDEC_ERR_INVALID;
  if (p.page_size < 1 || p.page_size > (1 << 15) || (p.page_size & (p.page_size - 1)) != 0) return SPDEC_ERR_INVALID;
  if (p.max_budget_pages < 2 || p.max_budget_pages > 32768) return SPDEC_ERR_INVALID;
  if (batch < 1 || batch > 65536) return SPDEC_ERR_INVALID;
  return from_hip(spdec::launch_budget_update(tail, scale, seq_lens, batch, p, budget_pages,
                                              stream));
}

spdec_status spdec_check_inputs(const spdec_cache* cache, const void* q, const int32_t* sel_idx,
                                const int32_t* sel_cnt, int max_budget_pages, int group_size,
                                const int32_t* shared_pages, int32_t* report, hipStream_t stream) {
  CacheView v;
  spdec_status st = view_of(cache, &v);
  if (st != SPDEC_OK) return st;
  if (report == nullptr) return SPDEC_ERR_INVALID;
  if ((sel_idx == nullptr) != (sel_cnt == nullptr)) return SPDEC_ERR_INVALID;
  if (sel_idx != nullptr && max_budget_pages < 1) return SPDEC_ERR_INVALID;
  if (shared_pages != nullptr && (group_size < 1 || v.batch % group_size != 0)) return SPDEC_ERR_INVALID;
  return from_hip(spdec::launch_check(v, q, sel_idx, sel_cnt, sel_idx ? max_budget_pages : 0,
                                      shared_pages ? group_size : 1, shared_pages, report,
                                      stream));
}

size_t spdec_monitor_workspace_bytes(int capacity) {
  if (capacity < 1 || capacity > spdec::kMonitorMaxCapacity) return 0;
  return spdec::monitor_workspace_bytes(capacity);
}

spdec_status spdec_monitor_reset(void* monitor, int capacity, hipStream_t stream) {
  if (!monitor) return SPDEC_ERR_INVALID;
  if (capacity < 1 || capacity > spdec::kMonitorMaxCapacity) return SPDEC_ERR_INVALID;
  return from_hip(spdec::launch_monitor_reset(monitor, capacity, stream));
}

spdec_status spdec_monitor_append(void* monitor, int capacity, const float* alpha, int n, hipStream_t stream) {
  if (!monitor || (n > 0 && !alpha) || n < 0) return SPDEC_ERR_INVALID;
  if (capacity < 1 || capacity > spdec::kMonitorMaxCapacity) return SPDEC_ERR_INVALID;
  if (n == 0) return SPDEC_OK;
  return from_hip(spdec::launch_monitor_append(monitor, capacity, alpha, n, stream));
}

spdec_status spdec_monitor_stats(void* monitor, int capacity, float* out, hipStream_t stream) {
  if (!monitor || !out) return SPDEC_ERR_INVALID;
  if (capacity < 1 || capacity > spdec::kMonitorMaxCapacity) return SPDEC_ERR_INVALID;
  return from_hip(spdec::launch_monitor_stats(monitor, capacity, out, stream));
}

spdec_status spdec_tail_stats(const float* alpha, int rows, float* out, hipStream_t stream) {
  if (!alpha || !out || rows < 1) return SPDEC_ERR_INVALID;
  if (rows > spdec::kTailMaxRows) return SPDEC_ERR_UNSUPPORTED;
  return from_hip(spdec::launch_tail_stats(alpha, rows, out, stream));
}

}  // extern "C"
