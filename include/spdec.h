/*
 * spdec.h - query-aware page-sparse decode attention for AMD Instinct MI355X (gfx950).
 *
 * One decode step of block-sparse (page) attention over a paged KV cache, the
 * dense attention it is checked against, and the per-token sparse-vs-dense
 * acceptance measure. Sources (web pages, cited by title and section):
 *   - Sparrow project page ("Sparrow: Sparse Rollout for Stable and Efficient
 *     Long-context RL of Large Language Models"): "Insights" (block-sparse
 *     attention; per-token mismatch against the dense model; lower 5th
 *     percentile), "Control Study 1" (budget grows with generation length),
 *     "Control Study 2" (cost model: KV budget B, page size, Top-k page
 *     selection; page size 16).
 *   - S3R page ("S3R: Fast and Faithful RL Rollouts via Self-Sparse
 *     Speculative Decoding"): abstract (dense verification needs the complete
 *     KV cache), Table 3 (KV capacity fixed per rollout; graph replay).
 *   - Sparrow citation-map page: Quest (query-aware page bound) and
 *     StreamingLLM (attention sinks) cited by title only.
 *
 * Conventions shared by every call
 * --------------------------------
 * Ownership: every pointer is a device pointer owned by the caller, unless a
 *   parameter says "host". The library never allocates, frees or synchronises;
 *   scratch memory is a caller-provided workspace whose size comes from the
 *   matching *_workspace_bytes query. Workspaces must be zero-filled once
 *   after allocation; every call leaves the parts it relies on zeroed again.
 * Streams: `stream` is a hipStream_t (NULL = the default stream). All work is
 *   enqueued on it in order; calls return before the GPU finishes. No call
 *   syncs the host, so every call can be captured into a HIP graph.
 * Errors: host-side arguments are checked before anything is launched; a
 *   failed check returns a negative status and launches nothing. A launch
 *   failure reported by the HIP runtime returns SPDEC_ERR_HIP.
 * Device-data preconditions (not checked on the host, which cannot read device
 *   memory without a sync): 0 <= seq_lens[b] <= max_pages_per_seq*page_size;
 *   page-table entries of pages in use are in [0, num_phys_pages); inputs are
 *   finite. Kernels never dereference an out-of-range physical page or page
 *   index: such a page is treated as holding no token. spdec_check_inputs
 *   counts violations of these preconditions on the device.
 * Threading: calls keep no global state; concurrent calls on different
 *   streams must not share a workspace.
 */
#ifndef SPDEC_H
#define SPDEC_H

#include <stddef.h>
#include <stdint.h>

/* The HIP runtime's stream handle, declared as the HIP headers declare it
 * (an identical typedef), so this header needs no HIP include and may come
 * before or after them. NULL is the default stream. */
typedef struct ihipStream_t* hipStream_t;

#ifdef __cplusplus
extern "C" {
#endif

typedef enum spdec_status {
  SPDEC_OK = 0,
  SPDEC_ERR_INVALID = -1,     /* null pointer, bad shape or out-of-range scalar            */
  SPDEC_ERR_UNSUPPORTED = -2, /* valid but not built: head_dim, page_size, group size, ... */
  SPDEC_ERR_WORKSPACE = -3,   /* workspace missing or smaller than the query returned      */
  SPDEC_ERR_HIP = -4          /* the HIP runtime reported a launch error                   */
} spdec_status;

/* Element type of queries, keys, values and the key min/max summaries. */
typedef enum spdec_dtype { SPDEC_F32 = 0, SPDEC_BF16 = 1 } spdec_dtype;

/*
 * Paged KV cache descriptor (plain data, read by every call; host memory).
 *
 *  batch                sequences (>= 1)
 *  num_q_heads (Hq)     query heads; query head h reads KV head h / G, G = Hq/Hkv
 *  num_kv_heads (Hkv)   KV heads; Hq % Hkv == 0 and G in {1, 2, 4, 8}
 *  head_dim (D)         64 or 128
 *  page_size (ps)       tokens per page: 8, 16, 32 or 64
 *  max_pages_per_seq    row length of page_table (1 .. 32768)
 *  num_phys_pages       physical pages in each pool
 *  dtype                spdec_dtype of k_pool, v_pool, kminmax and all queries
 *  k_pool, v_pool       [num_phys_pages][Hkv][ps][D]: one (page, KV head) is a
 *                       contiguous ps*D block
 *  kminmax              [num_phys_pages][Hkv][2][D]: per-channel minimum (row 0)
 *                       and maximum (row 1) of the page's valid keys
 *  page_table           int32 [batch][max_pages_per_seq]: logical page -> physical
 *  seq_lens             int32 [batch]: tokens in the cache, the current one included
 */
typedef struct spdec_cache {
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t max_pages_per_seq;
  int64_t num_phys_pages;
  int32_t dtype;
  int32_t reserved;
  void* k_pool;
  void* v_pool;
  void* kminmax;
  const int32_t* page_table;
  int32_t* seq_lens;
} spdec_cache;

/* Human-readable name of a status code (static string, never NULL). */
const char* spdec_status_string(spdec_status status);

/* Version of this ABI: major*10000 + minor*100 + patch. */
int spdec_version(void);

/*
 * Default scales (host computation, no GPU work): spdec_default_scale is the
 * softmax scale 1/sqrt(head_dim) for the decode and verify calls (the pages
 * leave the scale unstated; the standard attention scale is taken);
 * spdec_default_score_scale is 1/(G*sqrt(head_dim)), the logit scale of a
 * page bound in spdec_select_pages_top_p (the bound sums the G query heads'
 * per-head bounds, each a logit at scale 1/sqrt(head_dim)). Both return 0
 * for an invalid descriptor.
 */
float spdec_default_scale(const spdec_cache* cache);
float spdec_default_score_scale(const spdec_cache* cache);

/*
 * spdec_append_kv - write the new token's key and value into the paged cache
 * and keep its page's key summary current.
 *
 * Definition: the budgeted pages are chosen from per-page key summaries that
 * must cover every token in the cache (page scoring as in Quest, cited on the
 * Sparrow citation-map page; pages of `page_size` tokens per the Sparrow
 * project page, "Control Study 2"). For each sequence b and KV head g, with
 * t = seq_lens[b]: slot t % ps of logical page t / ps receives k_new[b][g] and
 * v_new[b][g]; if the slot is the page's first, the page's minimum and maximum
 * become that key, otherwise they widen to include it (elementwise). Then
 * seq_lens[b] becomes t + 1.
 *
 * k_new, v_new: [batch][Hkv][D] in the cache dtype. A sequence whose next slot
 * falls outside its page table or maps to an out-of-range physical page is
 * left unchanged (no write, no increment).
 */
spdec_status spdec_append_kv(const spdec_cache* cache, const void* k_new, const void* v_new, hipStream_t stream);

/*
 * spdec_build_meta - recompute every in-use page's key minimum and maximum
 * from the keys in the cache (bulk form of the upkeep in spdec_append_kv, for
 * a prefilled cache). Only the page's valid tokens t < seq_lens[b] count.
 */
spdec_status spdec_build_meta(const spdec_cache* cache, hipStream_t stream);

/*
 * spdec_select_pages - score every page of every (sequence, KV head) and keep
 * the budgeted Top-k (Sparrow project page, "Control Study 2": a KV budget of
 * B tokens in pages of `page_size`, chosen by Top-k; budget schedule per
 * sequence, "Control Study 1").
 *
 * Score of page p for KV head g (Quest-style bound, computed in fp32):
 *   s_p = sum over the G query heads h of g, sum over channels d, of
 *         max(q_hd * kmax_pd, q_hd * kmin_pd)
 * Selection with P = ceil(seq_lens[b]/ps) pages and
 * K = min(max(budget_pages[b], 2), max_budget_pages, P):
 *   K >= P -> all pages; otherwise page 0 (sink) and page P-1 (local, holds
 *   the current token) plus the K-2 highest-scoring pages of 1..P-2, equal
 *   scores going to the lower page index.
 *
 * q:            [batch][Hq][D], cache dtype
 * budget_pages: int32 [batch], budget in pages (sink and local included)
 * sel_idx:      int32 [batch][Hkv][max_budget_pages] out: logical page indices,
 *               ascending; entries past sel_cnt are left untouched
 * sel_cnt:      int32 [batch][Hkv] out: K
 * scores_out:   nullable fp32 [batch][Hkv][max_pages_per_seq] out: s_p for p < P
 * Forms (SPDEC_PATH_* below; the same scores and cut in each, so the same
 * selection), bf16 cache and G <= 4 for the fused ones, on the current device:
 *   SPDEC_PATH_ONE_KERNEL: the shapes of spdec_sparse_path's one-kernel form:
 *     one workgroup per (sequence, KV head) scores its pages into LDS and
 *     takes the Top-k there (no workspace used);
 *   SPDEC_PATH_SLICED: the shapes of spdec_sparse_path's sliced form, when
 *     the workspace holds spdec_select_workspace_bytes(): each slice's own
 *     Top-k candidates, then the unit's Top-k from them (two kernels);
 *   SPDEC_PATH_TWO_CALLS: otherwise: a scoring kernel writes every score to
 *     scores_out or the workspace, a Top-k kernel reads them.
 * max_budget_pages >= 2. Workspace: spdec_select_workspace_bytes() (enough
 * for every form; may be null when scores_out is given, which rules out the
 * sliced form). No part of it needs to be cleared.
 */
#define SPDEC_PATH_TWO_CALLS 0
#define SPDEC_PATH_ONE_KERNEL 1
#define SPDEC_PATH_SLICED 2
size_t spdec_select_workspace_bytes(const spdec_cache* cache, int max_budget_pages);
/* The form (SPDEC_PATH_*) spdec_select_pages takes for this cache shape on the
 * current device with the full workspace, or a negative spdec_status for an
 * invalid descriptor or max_budget_pages < 2. */
int spdec_select_pages_form(const spdec_cache* cache, int max_budget_pages);
spdec_status spdec_select_pages(const spdec_cache* cache, const void* q, const int32_t* budget_pages,
                                int max_budget_pages, int32_t* sel_idx, int32_t* sel_cnt, float* scores_out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * spdec_select_pages_top_p - score-mass (top-p) page selection: the budget
 * follows the query instead of being fixed (the RTPurbo abstract on the first
 * page of the source set argues for dynamic top-p over fixed top-k; the
 * page-level form is a stated reading).
 *
 * Scores s_p as in spdec_select_pages. Page masses w_p = exp(score_scale *
 * (s_p - max_q s_q)) (fp64). Pages 0 and P-1 are always kept; the pages
 * 1 .. P-2 are taken in the Top-B order (score descending, lower index first
 * on equal scores) while the kept mass is below top_p * sum_p w_p and fewer
 * than K_cap pages are kept, K_cap = min(max(budget_pages[b], 2),
 * max_budget_pages, P) (budget_pages nullable: then min(max_budget_pages, P)).
 * P <= 2 keeps every page. Masses are summed as 2^-48 fixed-point integers
 * (order-independent, so the result is deterministic); the target is
 * ceil(top_p * total) in those units.
 *
 * 0 < top_p <= 1, score_scale >= 0 (finite; 1/(G*sqrt(D)) reads the bound,
 * which sums the G query heads, as a per-head logit). Outputs and workspace
 * as spdec_select_pages. Forms: in the shapes of spdec_select_pages'
 * SPDEC_PATH_ONE_KERNEL form, one kernel (scores in LDS, the same cut);
 * otherwise a scoring kernel and a top-p kernel (no sliced form).
 */
spdec_status spdec_select_pages_top_p(const spdec_cache* cache, const void* q, float top_p, float score_scale,
                                      const int32_t* budget_pages, int max_budget_pages, int32_t* sel_idx,
                                      int32_t* sel_cnt, float* scores_out, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/*
 * spdec_select_pages_shared - spdec_select_pages for groups of sequences that
 * share their leading pages (a prompt sampled several times; the Sparrow
 * project page's cost model, "Control Study 2", charges the prompt once per
 * group rather than once per sample).
 *
 * Groups as in spdec_dense_decode_shared: sequences n*N .. n*N + N - 1 (N =
 * group_size) map logical pages 0 .. shared_pages[n] - 1 to the same physical
 * pages, all full (device preconditions; those pages' summaries are read once
 * per (group, KV head) through the first member's page table and bounded
 * against each member's query). Scores, selection, outputs and workspace are
 * those of spdec_select_pages: every score is the same fp32 value up to the
 * fp64 summation order inside it.
 *
 * shared_pages: int32 [batch / N]. Requires a bf16 cache, batch % N == 0,
 * 1 <= N <= 8 and (batch / N + batch) * Hkv <= 8192 (SPDEC_ERR_UNSUPPORTED otherwise).
 */
spdec_status spdec_select_pages_shared(const spdec_cache* cache, const void* q, int group_size,
                                       const int32_t* shared_pages, const int32_t* budget_pages,
                                       int max_budget_pages, int32_t* sel_idx, int32_t* sel_cnt, float* scores_out,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * spdec_sparse_decode - block-sparse decode attention over the selected pages
 * (Sparrow project page, "Insights": block-sparse attention; "Control Study
 * 2": reads only the budgeted KV).
 *
 * For query head h of sequence b with group g = h / G, over the tokens t of the
 * pages sel_idx[b][g][0 .. sel_cnt[b][g]) with t < seq_lens[b]:
 *   z_t = scale * q_h . k_t,  out_h = sum_t e^{z_t} v_t / sum_t e^{z_t},
 *   lse_h = ln sum_t e^{z_t}
 * computed in fp32 as split-KV partials with an online softmax, merged by
 * log-sum-exp in a fixed order (deterministic, no float atomics). A sequence
 * with seq_lens[b] == 0 attends over no token: its rows of out are zeros and
 * its lse is -inf (an empty softmax sum is 0; the pages do not cover it).
 *
 * q: [batch][Hq][D] cache dtype; out: fp32 [batch][Hq][D]; lse: nullable fp32
 * [batch][Hq]. sel_idx/sel_cnt as written by spdec_select_pages with the same
 * max_budget_pages. Workspace: spdec_decode_workspace_bytes(cache, max_budget_pages).
 */
size_t spdec_decode_workspace_bytes(const spdec_cache* cache, int max_budget_pages);
spdec_status spdec_sparse_decode(const spdec_cache* cache, const void* q, const int32_t* sel_idx,
                                 const int32_t* sel_cnt, int max_budget_pages, float scale, float* out,
                                 float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * spdec_dense_decode - the same attention over every page of the cache: the
 * dense verifier over the complete KV (S3R abstract: dense verification needs
 * the complete historical KV cache). Workspace: spdec_decode_workspace_bytes(cache, 0).
 */
spdec_status spdec_dense_decode(const spdec_cache* cache, const void* q, float scale, float* out, float* lse,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * spdec_sparse_path - one decode step of the sparse path: spdec_select_pages
 * then spdec_sparse_decode over the pages it kept (Sparrow project page,
 * "Control Study 2": score the pages, keep the budgeted Top-k, attend over
 * the kept KV only).
 *
 * Arguments and outputs are those of the two calls: sel_idx, sel_cnt and
 * scores_out (nullable) as spdec_select_pages writes them, out and lse
 * (nullable) as spdec_sparse_decode writes them for that selection. The
 * selection is always the same, page indices and scores bit for bit; out and
 * lse may differ from the two calls by the order in which the kept tokens'
 * partial sums are added (fp32 rounding). Forms, by shape (bf16 cache and
 * G <= 4 for both fused forms), on the current device:
 *   SPDEC_PATH_ONE_KERNEL: at least one (sequence, KV head) per compute unit,
 *     max_pages_per_seq and max_budget_pages <= 4096, batch <= 512: one
 *     kernel, one workgroup per (sequence, KV head) with scores, kept list
 *     and page-table row in LDS;
 *   SPDEC_PATH_SLICED: at most half as many (sequence, KV head) as compute
 *     units (and at most 128), max_budget_pages <= 4096: each unit's pages cut
 *     into S slices (S = compute units / units, at most 16, raised until a
 *     slice holds at most 4096 pages), S * (max_budget_pages - 2) <= 4096:
 *     each slice's own Top-k candidates, the unit's Top-k from them, the kept
 *     pages streamed by the S workgroups and their partials merged (three
 *     kernels);
 *   SPDEC_PATH_TWO_CALLS: any other shape.
 * max_budget_pages >= 2, scale > 0. Workspace:
 * spdec_sparse_path_workspace_bytes(cache, max_budget_pages) (enough for any
 * form; no part of it needs to be cleared). Calls that share a workspace must
 * not overlap.
 */
size_t spdec_sparse_path_workspace_bytes(const spdec_cache* cache, int max_budget_pages);
/* The form (SPDEC_PATH_*) spdec_sparse_path takes for this cache shape on the
 * current device, or a negative spdec_status for an invalid descriptor or
 * max_budget_pages < 2. Queries the current device. */
int spdec_sparse_path_form(const spdec_cache* cache, int max_budget_pages);
spdec_status spdec_sparse_path(const spdec_cache* cache, const void* q, const int32_t* budget_pages,
                               int max_budget_pages, float scale, int32_t* sel_idx, int32_t* sel_cnt,
                               float* scores_out, float* out, float* lse, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * spdec_dense_decode_shared - spdec_dense_decode for groups of sequences that
 * share their leading pages (a prompt sampled several times; the Sparrow
 * project page's cost model, "Control Study 2", charges the prompt once per
 * group rather than once per sample).
 *
 * Sequences n*N .. n*N + N - 1 (N = group_size) form group n; their page
 * tables map logical pages 0 .. shared_pages[n] - 1 to the same physical
 * pages, all full (device preconditions; the kernel reads those pages through
 * the first member's page table). The result is the dense decode of every
 * sequence up to rounding: the shared pages are read once per (group, KV
 * head) for the group's N * G query rows, each sequence's remaining pages once,
 * and the two partials are merged by log-sum-exp in a fixed order.
 *
 * q: [batch][Hq][D] bf16; shared_pages: int32 [batch / N]; out, lse as for
 * spdec_dense_decode. Requires a bf16 cache, batch % N == 0 and N * G <= 64
 * (SPDEC_ERR_UNSUPPORTED otherwise; above 32 query rows per (group, KV head)
 * the shared pages are read twice, once per 32 rows). Workspace:
 * spdec_shared_workspace_bytes(cache, N), zero-filled once.
 */
size_t spdec_shared_workspace_bytes(const spdec_cache* cache, int group_size);
spdec_status spdec_dense_decode_shared(const spdec_cache* cache, const void* q, int group_size,
                                       const int32_t* shared_pages, float scale, float* out, float* lse,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * spdec_verify_decode - dense verification of a sparse draft: causal
 * multi-query attention over the complete KV (S3R page, abstract and Tables
 * 6-7: k tokens drafted with sparse attention are verified by one
 * full-attention pass over the k + 1 positions).
 *
 * The T verified positions of sequence b are the last T tokens of its cache
 * (append them first): position t sits at L - T + t with L = seq_lens[b] and
 * attends to tokens 0 .. L - T + t. For query head h (group g = h / G):
 *   z_s = scale * q_{b,t,h} . k_s,  out = sum_s e^{z_s} v_s / sum_s e^{z_s},
 *   lse = ln sum_s e^{z_s}
 * in fp32 (scores and the attention weights pass through bf16 for the matrix
 * cores), merged by log-sum-exp in a fixed order.
 *
 * q: [batch][T][Hq][D] bf16; out: fp32 [batch][T][Hq][D]; lse: nullable fp32
 * [batch][T][Hq]. Requires a bf16 cache, 1 <= T <= 16 and G * T <= 64
 * (SPDEC_ERR_UNSUPPORTED otherwise; above 32 query rows per KV head the
 * cache is read twice, once per 32 rows); seq_lens[b] >= T is a device
 * precondition (a row with no visible token returns zeros and lse = -inf).
 * Workspace: spdec_verify_workspace_bytes(cache, T), zero-filled once.
 */
size_t spdec_verify_workspace_bytes(const spdec_cache* cache, int num_positions);
spdec_status spdec_verify_decode(const spdec_cache* cache, const void* q, int num_positions, float scale,
                                 float* out, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * spdec_spec_accept - exact speculative sampling of the drafted tokens (S3R
 * page, abstract: drafts proposed with sparse attention are accepted by exact
 * speculative sampling against the full-attention pass, so the emitted tokens
 * follow the dense policy; the method is that of the speculative-decoding
 * papers the citation-map page lists by title).
 *
 * For sequence b with k = num_draft drafted tokens x_i = draft[b][i]:
 *   p_i = softmax(p_logits row (b, i) / T), i = 0..k (the verifier's logits at
 *         the k + 1 verified positions), q_i = softmax(q_logits row (b, i) / T),
 *         i = 0..k-1 (the drafter's logits the drafts were sampled from);
 *   draft i is kept while u_accept[b][i] * q_i(x_i) < p_i(x_i), in order;
 *   at the first rejection j, next_token[b] is drawn from max(0, p_j - q_j)
 *   (from p_j itself when that residual has no weight at any token, i.e.
 *   p_j = q_j up to rounding), and when all k are kept from p_k. A draw with
 *   uniform u = u_sample[b] takes the first token whose running weight sum
 *   exceeds u times the total.
 * num_accepted[b] = number of kept drafts. Everything in fp32 with fixed
 * reduction orders; decisions whose margin is within fp32 rounding may differ
 * from an exact computation.
 *
 * p_logits: fp32, row (b, i) at (b * (k + 1) + i) * row_stride elements;
 * q_logits: fp32, row (b, i) at (b * k + i) * row_stride (unused when k = 0);
 * draft: int32 [batch][k]; u_accept: fp32 [batch][k] in [0, 1); u_sample:
 * fp32 [batch] in [0, 1); num_accepted, next_token: int32 [batch] out.
 * 0 <= k <= 64, batch * (2k + 1) <= 65535, 1 <= vocab <= 2^28, row_stride >= vocab,
 * temperature > 0. Workspace: spdec_spec_accept_workspace_bytes(batch, k, vocab).
 */
size_t spdec_spec_accept_workspace_bytes(int batch, int num_draft, int vocab);
spdec_status spdec_spec_accept(const float* p_logits, const float* q_logits, int batch, int num_draft, int vocab,
                               int64_t row_stride, const int32_t* draft, const float* u_accept,
                               const float* u_sample, float temperature, int32_t* num_accepted,
                               int32_t* next_token, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * spdec_acceptance - per-token sparse-vs-dense acceptance (Sparrow project
 * page, "Insights": per-token mismatch against the dense model; wispaper blog:
 * "acceptance rate"):
 *   alpha_r = sum_v min(softmax(a_r / T)_v, softmax(b_r / T)_v) = 1 - TV,
 * computed in fp32 with a fixed reduction order and clamped to [0, 1].
 *
 * logits_a, logits_b: fp32 rows of `vocab` entries, row r at r*row_stride
 * (elements); alpha: fp32 [rows] out. temperature > 0. 1 <= rows <= 65535,
 * 1 <= vocab <= 2^28. Workspace: spdec_acceptance_workspace_bytes(rows, vocab);
 * its first 96 KiB must be zero before the first call (every call leaves them
 * zero, whatever its shape), so one zero-filled workspace serves any sequence
 * of shapes.
 *
 * When all rows' 10240-entry chunks fit on the device at once (rows *
 * ceil(vocab / 10240) at most the resident workgroups of its kernel, e.g. 64
 * rows of 151936 on 256 compute units), every logit is read once: the chunks
 * of a row exchange their partial normalisers through the workspace and wait
 * for each other with a bounded wait (a chunk that stops waiting reads its
 * row again, with identical results). Otherwise two passes read the logits
 * twice. Either way the result is run-to-run identical; the two forms may
 * differ in the last bits.
 * The mean and lower 5th percentile of alpha: spdec_tail_stats.
 */
size_t spdec_acceptance_workspace_bytes(int rows, int vocab);
spdec_status spdec_acceptance(const float* logits_a, const float* logits_b, int rows, int vocab,
                              int64_t row_stride, float temperature, float* alpha, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * spdec_acceptance_noalloc - spdec_acceptance for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): same arguments and results, no workspace.
 *
 * Its workspace is a SPDEC_NOALLOC_SCRATCH_BYTES device array inside the
 * library, one per GPU, held until the process ends; its address is looked
 * up on the first call on each device (with that device current). The call
 * allocates nothing. Shapes whose spdec_acceptance_workspace_bytes exceeds
 * the array (above 1332 rows of 151936 entries) return
 * SPDEC_ERR_UNSUPPORTED without launching. Every call on one GPU uses the same
 * array: calls that overlap on one GPU (other streams, other host threads)
 * race and give undefined results; calls on one stream are ordered and safe.
 */
#define SPDEC_NOALLOC_SCRATCH_BYTES (2u << 20)
spdec_status spdec_acceptance_noalloc(const float* logits_a, const float* logits_b, int rows, int vocab,
                                      int64_t row_stride, float temperature, float* alpha, hipStream_t stream);

/*
 * spdec_acceptance_ex - spdec_acceptance with its form and wait made explicit
 * (for tests and diagnostics; same arguments, results and workspace otherwise).
 *
 * force_path: -1 automatic (as spdec_acceptance), 1 single read
 *   (SPDEC_ERR_UNSUPPORTED if the rows' chunks do not fit the device at once),
 *   2 two passes.
 * spin_limit: polls of a row's partial normalisers before a waiting chunk
 *   reads the row itself; -1 = the default (16384), 0 = never wait.
 * fallbacks: device int32 [1], nullable: incremented by every single-read
 *   chunk that stopped waiting (the caller clears it).
 * path_taken: host int32, nullable: set to the form launched (1 or 2).
 */
spdec_status spdec_acceptance_ex(const float* logits_a, const float* logits_b, int rows, int vocab,
                                 int64_t row_stride, float temperature, float* alpha, void* workspace,
                                 size_t workspace_bytes, int force_path, int spin_limit, int32_t* fallbacks,
                                 int32_t* path_taken, hipStream_t stream);

/*
 * spdec_tail_stats - on-device tail statistics of the per-token acceptance
 * (Sparrow project page, "Control Study 1": training stays stable while the
 * lower 5th percentile of the per-token mismatch stays above a threshold,
 * 0.86 in its takeaway), so a budget schedule can read them without a host
 * round trip.
 *
 * out[0] = mean of alpha[0 .. rows), out[1] = its 5th percentile by linear
 * interpolation between the order statistics at rank 0.05 * (rows - 1) (the
 * numpy default). Computed in fp64 and rounded once to fp32.
 * alpha: fp32 [rows] (device); out: fp32 [2] (device). 1 <= rows <= 8192
 * (SPDEC_ERR_UNSUPPORTED above). No workspace.
 */
spdec_status spdec_tail_stats(const float* alpha, int rows, float* out, hipStream_t stream);

/*
 * spdec_monitor_* - streaming tail monitor of the per-token acceptance over a
 * rollout's tokens (Sparrow project page, "Control Study 1": training stays
 * stable while the lower 5th percentile of the per-token mismatch stays above
 * a threshold, 0.86 in its takeaway), kept entirely on the device so a budget
 * schedule reads it every step without a host round trip.
 *
 * monitor: device workspace of spdec_monitor_workspace_bytes(capacity) bytes
 *   holding a ring of the `capacity` most recent values and a 64-bit count of
 *   values appended; it must be zero-filled before its first use (a fresh
 *   window) or reset with spdec_monitor_reset. 1 <= capacity <= 2^28 (the
 *   query returns 0 outside). Calls on one monitor must be stream-ordered.
 * spdec_monitor_reset: starts a new window (count = 0).
 * spdec_monitor_append: appends alpha[0 .. n) (device fp32, n >= 0; of a batch
 *   longer than capacity only its last capacity values are kept).
 * spdec_monitor_stats: out[0] = mean and out[1] = lower 5th percentile (linear
 *   interpolation between the order statistics at rank 0.05 * (m - 1), the
 *   numpy default) of the m = min(count, capacity) values in the window,
 *   exact up to one rounding of each to fp32 (the mean sums in fp64 in a fixed
 *   order). out is the layout spdec_budget_update reads. An empty window
 *   gives NaN for both (the controller then keeps its state).
 */
size_t spdec_monitor_workspace_bytes(int capacity);
spdec_status spdec_monitor_reset(void* monitor, int capacity, hipStream_t stream);
spdec_status spdec_monitor_append(void* monitor, int capacity, const float* alpha, int n, hipStream_t stream);
spdec_status spdec_monitor_stats(void* monitor, int capacity, float* out, hipStream_t stream);

/*
 * spdec_budget_update - sparsity-schedule controller: one correction of the
 * per-sequence budgets from the on-device tail statistic (Sparrow project
 * page, "Control Study 1": the budget grows with the generated length so the
 * per-token mismatch stays roughly constant, and the lower 5th percentile of
 * the per-token acceptance is held at a threshold, 0.86 in its takeaway; the
 * page gives no control law, so this one is a stated reading).
 *
 * With p5 = tail[1] (as written by spdec_tail_stats) and s = *scale:
 *   s' = clamp(s * (1 + gain * (target - p5)), scale_min, scale_max)
 *   budget_pages[b] = clamp(ceil(s' * (base_tokens + tokens_per_token * L_b) / page_size), 2, max_budget_pages)
 * with L_b = seq_lens[b], every operation one fp32 rounding in that order (no
 * fused multiply-add). A tail below the target raises every budget, one above
 * it lowers them, one on target leaves them. A non-finite p5 leaves s
 * unchanged; a non-finite or non-positive *scale restarts from scale_max.
 * *scale is overwritten with s'.
 *
 * tail: fp32 [2] (device); scale: fp32 [1] (device, caller-owned state,
 * e.g. 1.0 at the start); seq_lens: int32 [batch]; budget_pages: int32 [batch]
 * out (may be the budget array spdec_select_pages reads next). Host checks:
 * 0 < target <= 1, gain >= 0, 0 < scale_min <= scale_max, base_tokens >= 0,
 * tokens_per_token >= 0 (all finite), page_size a power of two in 1 .. 2^15,
 * 2 <= max_budget_pages <= 32768, 1 <= batch <= 65536 (SPDEC_ERR_INVALID
 * otherwise). No workspace.
 */
typedef struct spdec_budget_params {
  float target;            /* held 5th percentile of the acceptance */
  float gain;              /* relative scale change per unit of (target - p5) */
  float scale_min, scale_max;
  float base_tokens;       /* schedule at length 0, in tokens */
  float tokens_per_token;  /* schedule growth per cached token */
  int32_t page_size;       /* tokens per page */
  int32_t max_budget_pages;
} spdec_budget_params;

spdec_status spdec_budget_update(const float* tail, float* scale, const int32_t* seq_lens, int batch,
                                 const spdec_budget_params* params, int32_t* budget_pages, hipStream_t stream);

/*
 * spdec_check_inputs - counts, on the device, violations of the data
 * preconditions that the other calls assume without checking (a debug aid:
 * it reads the page table, the lengths and, when given, the selection, the
 * query and the shared-page counts once; the hot calls skip that read).
 *
 * report: int32 [SPDEC_CHECK_WORDS], overwritten (stream-ordered) with
 *   [0] sequences whose seq_lens[b] is outside [0, max_pages_per_seq*page_size];
 *   [1] page-table entries of live pages (logical page < P_b = ceil(L_b/ps),
 *       L_b clamped to that range) outside [0, num_phys_pages);
 *   [2] (sequence, KV head) rows of a selection that spdec_select_pages with
 *       this max_budget_pages could not have written: sel_cnt outside
 *       [0, min(max_budget_pages, P_b)], or an entry among the first sel_cnt
 *       outside [0, P_b) or not above the entry before it (entries ascend
 *       strictly; repeated pages would be counted twice);
 *   [3] non-finite values of q [batch][Hq][D] (cache dtype);
 *   [4] groups n of group_size sequences (the shared-prefix calls' layout)
 *       whose shared_pages[n] is outside [0, max_pages_per_seq], exceeds the
 *       full pages floor(L/ps) of a member, or whose first shared_pages[n]
 *       page-table entries differ between members;
 *   [5] SPDEC_CHECK_FIRST: the lowest sequence with a violation in [0]..[4]
 *       (a group's first sequence for [4]), or batch if there is none;
 *   [6], [7] zero.
 * Layouts: q [batch][Hq][D] (cache dtype); sel_idx int32
 * [batch][Hkv][max_budget_pages]; sel_cnt int32 [batch][Hkv]; shared_pages
 * int32 [batch / group_size]. q, sel_idx/sel_cnt (both or neither;
 * max_budget_pages >= 1 with them) and shared_pages (then group_size >= 1
 * divides batch) are nullable: a null pointer skips its check. Only the descriptor's sizes index the arrays, so
 * any values in them are safe to check; the pools and summaries are not read.
 */
#define SPDEC_CHECK_WORDS 8
#define SPDEC_CHECK_FIRST 5
spdec_status spdec_check_inputs(const spdec_cache* cache, const void* q, const int32_t* sel_idx,
                                const int32_t* sel_cnt, int max_budget_pages, int group_size,
                                const int32_t* shared_pages, int32_t* report, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPDEC_H */
