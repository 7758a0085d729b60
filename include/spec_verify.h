/*
 * spec_verify.h -- C ABI of the batched draft-verify rejection sampler for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (zwjcode.cn, "生成 4 个 Token 为何不一定要跑 4 次大模型？
 * Speculative Decoding 的提议、验证与接受", sections 02-07; pinghaoyang.com.cn,
 * "vLLM 源码完全拆解（十）：投机解码——草稿模型、批量验证与 token 接受流水线",
 * section "拒绝采样：RejectionSampler 的两个分支" and its greedy / random kernel
 * subsections):
 *
 *   For each request i with gamma_i draft tokens y_0..y_{gamma_i-1}:
 *   1. gamma_i is the index of the first negative entry of draft_ids[i, :]
 *      (gmax if none); later entries are ignored.
 *   2. Greedy requests (temperature 0): t_j = argmax of target row j (lowest
 *      id on ties); accept while y_j == t_j; A = first mismatch (or gamma_i);
 *      the output is y_0..y_{A-1}, t_A.
 *   3. Sampled requests (temperature T > 0): p'_j = softmax(l_j / T) restricted
 *      to the top-k / top-p kept set and renormalised; q'_j = q_j^(1/T)
 *      restricted by the same rule (own thresholds) and renormalised, or the
 *      one-hot of y_j when draft_probs is NULL.  Top-k keeps every value tied
 *      with the k-th largest; top-p keeps the smallest set of whole tie groups,
 *      largest values first, whose mass reaches top_p of the top-k mass.
 *      Position j is accepted iff u_accept[i,j] * q'_j(y_j) < p'_j(y_j).
 *      A = first rejected position (or gamma_i).  If A < gamma_i the token at
 *      A is drawn from w = max(0, p'_A - q'_A) (p'_A when that is all zero);
 *      otherwise the bonus token is drawn from w = p'_{gamma_i}.  The draw is
 *      z = min{x : C_x > u_sample[i] * S} with C the running sum of w over
 *      ascending token id and S = sum(w) (if rounding leaves no such x, the
 *      largest x with w_x > 0).
 *   4. out_tokens[i, :] = y_0..y_{A-1}, z, then -1 up to gmax + 1 entries;
 *      out_num_accepted[i] = A.
 *
 * Data faults are reported per request, never by aborting the launch: the
 * request's out_tokens row is all -1 and out_num_accepted[i] = -1.  Faults:
 * a draft id >= V before the first negative id; a temperature that is NaN,
 * negative, infinite or subnormal; on a sampled request a top_p that is NaN or
 * <= 0; a read target row (rows 0..gamma_i) holding NaN or +inf or no finite
 * value; on a sampled request with draft_probs, a read draft row (rows
 * 0..gamma_i-1) holding NaN, +-inf or an entry with its sign bit set, or
 * whose kept mass is zero.  Rows beyond those are never read (they may hold
 * anything, including NaN).  top_k <= 0 or >= V and top_p >= 1 switch the
 * filter off.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* target_logits element types */
#define SPEC_VERIFY_F32 0  /* IEEE binary32                          */
#define SPEC_VERIFY_BF16 1 /* bfloat16 bit patterns (uint16 storage) */

/* return codes (nothing is enqueued unless SPEC_VERIFY_OK is returned) */
#define SPEC_VERIFY_OK 0
#define SPEC_VERIFY_ERR_NULL 1      /* a required pointer is NULL                        */
#define SPEC_VERIFY_ERR_SHAPE 2     /* N < 0, gmax outside [0, 64], V < 1, or too large  */
/* "Too large": V * (gmax + 1) above 2^40, V above 2^31 - 4097, or either
 * launch grid reaching 2^32 work-items: 256 * N * (gmax + 1) (row pass; in
 * the padded layout 256 * N * (gmax + 2) when gmax is a positive multiple of
 * 8, and 256 * N in the synthetic mode) or 256 * N * ceil(ceil(V / 2048) / 4)
 * (draw pass). */
#define SPEC_VERIFY_ERR_DTYPE 3     /* unknown logits_dtype                              */
#define SPEC_VERIFY_ERR_WORKSPACE 4 /* workspace_bytes below spec_verify_workspace_size  */
#define SPEC_VERIFY_ERR_HIP 5       /* a HIP runtime call failed (launch, copy, wait)      */
#define SPEC_VERIFY_ERR_SCRATCH 6   /* spec_verify_static: sizes need more workspace than its scratch */

/* fault bits of the diagnostic fault output */
#define SPEC_VERIFY_FAULT_DRAFT_ID 1
#define SPEC_VERIFY_FAULT_TEMPERATURE 2
#define SPEC_VERIFY_FAULT_TOP_P 4
#define SPEC_VERIFY_FAULT_TARGET_ROW 8
#define SPEC_VERIFY_FAULT_DRAFT_ROW 16
#define SPEC_VERIFY_FAULT_DRAFT_MASS 32
#define SPEC_VERIFY_FAULT_DRAFT_COUNT 64 /* flattened layout: gamma_i outside [0, gmax] or past num_drafts */
#define SPEC_VERIFY_FAULT_BAN_LIST 128   /* banned-token list longer than 512, not ascending, or an id outside [0, V) */
#define SPEC_VERIFY_FAULT_ROW_INDEX 256  /* a target_logits row index outside [0, logits_rows) */
#define SPEC_VERIFY_FAULT_PENALTY 512    /* a penalty list or penalty value breaks the rules of spec_verify_flat_ex */

/*
 * Bytes of device workspace one call with these sizes needs.  The layout is
 * private to the library; its contents do not need initialising.  After a
 * call it holds that call's count of faulted requests, read by
 * spec_verify_device_errors; the rest is not meaningful.
 */
size_t spec_verify_workspace_size(int N, int gmax, int V);

/*
 * Verify a batch.  All array arguments are DEVICE pointers owned by the
 * caller, row-major with the vocabulary contiguous:
 *   draft_ids         int32   [N, gmax]        -1 (any negative) pads
 *   draft_probs       float32 [N, gmax, V]     or NULL: draft-free (n-gram) drafts
 *   target_logits     f32/bf16 [N, gmax+1, V]  row gamma_i is the bonus position
 *   temperature       float32 [N]              or NULL: 1.0 for every request
 *   top_k             int32   [N]              or NULL: off
 *   top_p             float32 [N]              or NULL: off
 *   u_accept          float32 [N, gmax]        uniforms in [0, 1) (may be NULL if gmax == 0)
 *   u_sample          float32 [N]              uniforms in [0, 1)
 *   out_tokens        int32   [N, gmax+1]      written
 *   out_num_accepted  int32   [N]              written
 * workspace: device memory of at least spec_verify_workspace_size(N, gmax, V)
 * bytes, owned by the caller (SPEC_VERIFY_ERR_NULL if NULL and N > 0): the
 * library allocates nothing and keeps no state between calls.  stream: a
 * hipStream_t, or NULL for the default stream.  The call only enqueues kernels
 * on the stream and returns; it never waits for the device.  Calls that share
 * a workspace must be ordered on one stream.  N == 0 is a valid empty batch.
 * Inputs are read only; outputs must not alias inputs or the workspace.
 */
int spec_verify(int N, int gmax, int V, const int32_t *draft_ids, const float *draft_probs,
                const void *target_logits, int logits_dtype, const float *temperature,
                const int32_t *top_k, const float *top_p, const float *u_accept,
                const float *u_sample, int32_t *out_tokens, int32_t *out_num_accepted,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * spec_verify plus diagnostic outputs, each an optional DEVICE pointer:
 *   p_y         float64 [N, gmax]  p'_j(y_j) for j < gamma_i of sampled requests
 *   q_y         float64 [N, gmax]  q'_j(y_j) (1 for draft-free requests)
 *   resid_mass  float64 [N]        S of the final draw (sampled requests)
 *   fault       int32   [N]        fault bits (0: none)
 * Entries that do not apply are written as NaN (p_y, q_y, resid_mass).
 */
int spec_verify_diag(int N, int gmax, int V, const int32_t *draft_ids, const float *draft_probs,
                     const void *target_logits, int logits_dtype, const float *temperature,
                     const int32_t *top_k, const float *top_p, const float *u_accept,
                     const float *u_sample, int32_t *out_tokens, int32_t *out_num_accepted,
                     double *p_y, double *q_y, double *resid_mass, int32_t *fault,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * spec_verify_diag plus three optional hipEvent_t handles (created by the
 * caller, may be NULL) that are recorded on `stream`: ev_start at the start
 * of the row pass (every row's statistics and accept flag, and the draw of a
 * row that may be drawn from and kept its top-k set on chip) and ev_mid at
 * its end, both taken by the row pass's own dispatch (hipExtLaunchKernel),
 * so they add no packets around it; ev_end after the draw pass (each
 * request's first rejection and outputs, and the draw for requests whose
 * draw row made none).  For timing the two phases; results are identical to
 * spec_verify_diag.
 */
int spec_verify_timed(int N, int gmax, int V, const int32_t *draft_ids, const float *draft_probs,
                      const void *target_logits, int logits_dtype, const float *temperature,
                      const int32_t *top_k, const float *top_p, const float *u_accept,
                      const float *u_sample, int32_t *out_tokens, int32_t *out_num_accepted,
                      double *p_y, double *q_y, double *resid_mass, int32_t *fault,
                      void *workspace, size_t workspace_bytes, void *stream,
                      void *ev_start, void *ev_mid, void *ev_end);

/*
 * Verify a batch in the flattened (ragged) layout, with no padding rows.
 * vLLM page, section "SpecDecodeMetadata：验证阶段的「索引地图」": the drafts of
 * all requests are concatenated in request order and a prefix sum of the
 * draft counts locates each request's span.  Request i has gamma_i =
 * cu_num_draft_tokens[i] - cu_num_draft_tokens[i-1] drafts (the term for
 * i = 0 is 0), 0 <= gamma_i <= gmax, and num_drafts = cu_num_draft_tokens[N-1].
 * All array arguments are DEVICE pointers owned by the caller:
 *   cu_num_draft_tokens  int32    [N]                inclusive prefix sums of gamma_i
 *   draft_ids            int32    [num_drafts]       request i's at cu[i-1] .. cu[i]-1
 *   draft_probs          float32  [Q, V] or NULL     the draft rows of the requests that carry
 *                                                    them, in request order (Q = sum of their gamma_i)
 *   has_draft_probs      uint8    [N] or NULL        request i carries draft rows iff nonzero
 *                                                    (NULL: all do; ignored when draft_probs is NULL);
 *                                                    the others are draft-free (n-gram) requests
 *   target_logits        f32/bf16 [num_drafts + N, V] request i's gamma_i draft positions, then its
 *                                                    bonus position: rows cu[i-1] + i .. cu[i] + i
 *   temperature, top_k, top_p, u_sample  [N]  as for spec_verify
 *   u_accept             float32  [num_drafts]       aligned with draft_ids
 *   out_tokens           int32    [N, gmax+1]        written, -1 padded as for spec_verify
 *   out_num_accepted     int32    [N]                written
 * The method, the outputs, the faults, the workspace (spec_verify_workspace_size
 * with the same N, gmax, V) and the stream behave as for spec_verify; a
 * request whose count is out of range gets SPEC_VERIFY_FAULT_DRAFT_COUNT and
 * its inputs are not read.  Returns SPEC_VERIFY_ERR_NULL for a NULL
 * cu_num_draft_tokens (N > 0), or NULL draft_ids / u_accept when num_drafts
 * > 0; SPEC_VERIFY_ERR_SHAPE for num_drafts outside [0, N * gmax].
 */
int spec_verify_flat(int N, int gmax, int V, int num_drafts, const int32_t *cu_num_draft_tokens,
                     const int32_t *draft_ids, const float *draft_probs,
                     const uint8_t *has_draft_probs, const void *target_logits, int logits_dtype,
                     const float *temperature, const int32_t *top_k, const float *top_p,
                     const float *u_accept, const float *u_sample, int32_t *out_tokens,
                     int32_t *out_num_accepted, void *workspace, size_t workspace_bytes,
                     void *stream);

/*
 * spec_verify_flat with the diagnostic outputs of spec_verify_diag (p_y and
 * q_y are [N, gmax], position j of request i at [i, j]) and the three
 * optional events of spec_verify_timed.
 */
int spec_verify_flat_timed(int N, int gmax, int V, int num_drafts, const int32_t *cu_num_draft_tokens,
                           const int32_t *draft_ids, const float *draft_probs,
                           const uint8_t *has_draft_probs, const void *target_logits,
                           int logits_dtype, const float *temperature, const int32_t *top_k,
                           const float *top_p, const float *u_accept, const float *u_sample,
                           int32_t *out_tokens, int32_t *out_num_accepted, double *p_y,
                           double *q_y, double *resid_mass, int32_t *fault, void *workspace,
                           size_t workspace_bytes, void *stream, void *ev_start, void *ev_mid,
                           void *ev_end);

/*
 * spec_verify_flat_timed with the three options of the flattened call as vLLM
 * feeds it; each may be left out (NULL).
 *
 * Row indices (vLLM page, section "SpecDecodeMetadata：验证阶段的「索引地图」",
 * fields target_logits_indices and bonus_logits_indices; the sampler's second
 * step gathers the rows it verifies with them): the target model's logits
 * tensor holds rows for other positions too, and these say which row holds
 * each position, so that no gather copy is needed.
 *   target_logits          f32/bf16 [logits_rows, V]
 *   target_logits_indices  int32    [num_drafts]  row of flattened draft position t
 *   bonus_logits_indices   int32    [N]           row of request i's bonus position
 * bonus_logits_indices selects the option; target_logits_indices may then be
 * NULL only when num_drafts is 0.  Without the option the rows are in request
 * order as for spec_verify_flat and logits_rows must be at least
 * num_drafts + N.  Rows
 * no index names are never read.  An index outside [0, logits_rows) gives its
 * request SPEC_VERIFY_FAULT_ROW_INDEX; an index is read only for a request
 * whose count and parameters are valid.
 *
 * Banned tokens (zwjcode.cn page, section 06: p and q must go through
 * identical transforms, banned tokens among them): a banned token of request i
 * has logit -inf in every target row of the request and probability 0 in every
 * draft row, before temperature, top-k and top-p.  It can therefore never be
 * committed, and a draft of it is always rejected.
 *   banned_offsets  int32 [N + 1]   request i's list is banned_ids[off[i] .. off[i+1]-1]
 *   banned_ids      int32           strictly ascending per request, each in [0, V),
 *                                   at most 512 per request
 * banned_offsets selects the option; banned_ids may then be NULL when every
 * list is empty.  A request whose list breaks those rules (a nonempty list
 * with NULL banned_ids among them) gets SPEC_VERIFY_FAULT_BAN_LIST.
 *
 * Repetition penalties (zwjcode.cn page, section 06: the same transforms at
 * the same position in p and q, repetition penalties among them; vLLM page,
 * the sampler's second step: "penalty" logits processors): each position
 * carries its own list, the tokens of the context it continues (the draft
 * tokens before it included) with their counts in the generated output.
 *   penalty_offsets     int32 [num_drafts + N + 1]  position j of request i
 *                       (j = 0 .. gamma_i) has index cu[i-1] + i + j and its list
 *                       is penalty_ids[off[p] .. off[p+1]-1]
 *   penalty_ids         int32   strictly ascending per position, each in [0, V),
 *                               at most 1024 per position
 *   penalty_counts      int32   aligned with penalty_ids, >= 0 (0: the token is
 *                               only in the prompt)
 *   repetition_penalty  float32 [N] or NULL (1)    theta_i: positive and finite
 *   presence_penalty    float32 [N] or NULL (0)    finite
 *   frequency_penalty   float32 [N] or NULL (0)    finite
 * A listed token with logit l reads as (l > 0 ? l / theta : l * theta) - d,
 * with d = frequency * count + presence when count > 0, else 0: float32
 * arithmetic, each operation rounded, and a bf16 result rounded back to bf16
 * to nearest even.  Its draft probability reads as q * exp(-d) (d shifts the
 * draft's logits alike; the draft rows are renormalised as always).  Both
 * happen before temperature, top-k and top-p, and a banned token stays
 * banned.  A repetition penalty other than 1 on a request that carries draft
 * rows (has_draft_probs) and a nonzero temperature is a fault: draft
 * probabilities fix the draft's logits only up to a constant, so the
 * multiplicative change has no counterpart on them.  A list or value that
 * breaks these rules gives its request SPEC_VERIFY_FAULT_PENALTY; the lists
 * of a request with SPEC_VERIFY_FAULT_DRAFT_COUNT are not read.
 * penalty_offsets selects the option; penalty_ids and penalty_counts are
 * given together, and may both be NULL when every list is empty.
 *
 * Returns SPEC_VERIFY_ERR_NULL (N > 0) for target_logits_indices without
 * bonus_logits_indices, bonus_logits_indices without target_logits_indices
 * when num_drafts > 0, banned_ids without banned_offsets, any penalty
 * argument without penalty_offsets, or only one of penalty_ids and
 * penalty_counts; and
 * SPEC_VERIFY_ERR_SHAPE for logits_rows below 1, or below num_drafts + N
 * without indices (N > 0).
 */
int spec_verify_flat_ex(int N, int gmax, int V, int num_drafts, const int32_t *cu_num_draft_tokens,
                        const int32_t *draft_ids, const float *draft_probs,
                        const uint8_t *has_draft_probs, const void *target_logits, int logits_rows,
                        const int32_t *target_logits_indices, const int32_t *bonus_logits_indices,
                        int logits_dtype, const float *temperature, const int32_t *top_k,
                        const float *top_p, const int32_t *banned_offsets, const int32_t *banned_ids,
                        const int32_t *penalty_offsets, const int32_t *penalty_ids,
                        const int32_t *penalty_counts, const float *repetition_penalty,
                        const float *presence_penalty, const float *frequency_penalty,
                        const float *u_accept, const float *u_sample, int32_t *out_tokens,
                        int32_t *out_num_accepted, double *p_y, double *q_y, double *resid_mass,
                        int32_t *fault, void *workspace, size_t workspace_bytes, void *stream,
                        void *ev_start, void *ev_mid, void *ev_end);

/*
 * The synthetic acceptance mode (vLLM page, section "关于 synthetic / block
 * 验证模式"), for exercising a drafter without real target probabilities:
 * draft j of every request is accepted iff u_accept < synthetic_rates[j]
 * (DEVICE float32 [gmax], expected non-increasing in j; the rule is applied
 * as given), so the first rejection A_i is known before any row is read and
 * the row pass streams only row A_i of each request.  The token at A_i is
 * drawn as in spec_verify: the argmax of row A_i for a greedy request, else
 * the replacement from max(0, p' - q') (p' if that is zero) at a rejection, or
 * the bonus from p' when every draft was accepted.  Faults come from the
 * request's parameters and from row A_i (the other rows are not read).
 * Arguments as for spec_verify_flat, plus `fault` (DEVICE int32 [N] or NULL)
 * and the three optional events of spec_verify_timed.  Returns
 * SPEC_VERIFY_ERR_NULL for a NULL synthetic_rates when N > 0 and gmax > 0.
 */
int spec_verify_flat_synthetic(int N, int gmax, int V, int num_drafts,
                               const int32_t *cu_num_draft_tokens, const int32_t *draft_ids,
                               const float *draft_probs, const uint8_t *has_draft_probs,
                               const void *target_logits, int logits_dtype,
                               const float *temperature, const int32_t *top_k, const float *top_p,
                               const float *synthetic_rates, const float *u_accept,
                               const float *u_sample, int32_t *out_tokens,
                               int32_t *out_num_accepted, int32_t *fault, void *workspace,
                               size_t workspace_bytes, void *stream, void *ev_start, void *ev_mid,
                               void *ev_end);

/*
 * KV bookkeeping after a verify call, enqueued on `stream` after it (KV page
 * "投机解码如何与 KV Cache 交互：Placeholder、回滚与草稿 KV", sections 3.1 and 3.2;
 * vLLM page, the padded drafter batch paragraph: rejected draft slots become
 * PADDING_SLOT_ID).  For request i with A_i = num_accepted[i] accepted of its
 * gamma_i drafts, the gamma_i - A_i rejected ones are rolled back:
 *   num_computed_tokens[i]      -= gamma_i - A_i   if it is positive
 *   num_output_placeholders[i]  -= gamma_i - A_i   if it is positive
 *   slot_mapping at draft positions A_i .. gamma_i - 1 = -1
 * gamma_i comes from exactly one of cu_num_draft_tokens [N] (flattened
 * layout; slot_mapping [num_drafts] aligned with the flattened drafts) or
 * draft_ids [N, gmax] (padded layout, gamma_i = index of the first negative
 * id; slot_mapping [N, gmax]).  All arrays are DEVICE int32 arrays; the three
 * updated ones may each be NULL (not updated).  A request whose A_i is outside
 * [0, gamma_i] (num_accepted = -1 after a fault) or whose count exceeds gmax
 * is left unchanged.  Returns SPEC_VERIFY_ERR_SHAPE for N < 0 or gmax outside
 * [0, 64]; SPEC_VERIFY_ERR_NULL for a NULL num_accepted (N > 0) or unless
 * exactly one of cu_num_draft_tokens / draft_ids is given (gmax > 0).
 */
int spec_verify_rollback(int N, int gmax, const int32_t *cu_num_draft_tokens,
                         const int32_t *draft_ids, const int32_t *num_accepted,
                         int32_t *num_computed_tokens, int32_t *num_output_placeholders,
                         int32_t *slot_mapping, void *stream);

/*
 * The number of requests that the most recent call using `workspace` reported
 * as faulted (out_num_accepted = -1; the plain entry points have no other
 * fault output).  The call's first kernel sets the count to zero and its last
 * kernel adds one per faulted request, so it is the count of that call alone.
 * Enqueues a copy of the count on `stream` (the stream of that call) and waits
 * for the stream to finish, then stores the count in *count (host memory).
 * Returns SPEC_VERIFY_ERR_NULL for a NULL workspace or count,
 * SPEC_VERIFY_ERR_WORKSPACE for workspace_bytes below 256, SPEC_VERIFY_ERR_HIP
 * if the copy or the wait fails.  The count belongs to one call rather than
 * accumulating over calls: the workspace is caller memory that no call
 * requires to be initialised, so a count carried from call to call would start
 * from whatever the memory held.
 */
int spec_verify_device_errors(const void *workspace, size_t workspace_bytes, void *stream, int32_t *count);

/*
 * spec_verify for callers that cannot allocate device memory: code under HIP
 * graph capture, serving loops and harnesses that forbid hipMalloc.  The
 * arguments and the method are those of spec_verify, without the workspace:
 * the library's own scratch array in device memory (a file-scope array of
 * spec_verify_static_scratch_bytes() = 16 MiB, 256-byte aligned; each GPU the
 * library runs on holds its own copy until the process ends) serves as the
 * workspace.  The call allocates nothing and calls no allocating routine; its
 * first call on a device looks up that device's address of the array, with
 * the device current.  Sizes whose spec_verify_workspace_size exceeds the
 * scratch are refused with SPEC_VERIFY_ERR_SCRATCH (N = 4096, gmax = 8,
 * V = 151936 needs 11.9 MiB).  Every call on a GPU shares that GPU's
 * array: calls that overlap on one GPU (different streams, or host threads
 * without ordering) race and their results are undefined; calls ordered on
 * one stream are safe, since each call resets what it reads from the array.
 * Faults show as out_num_accepted = -1 (spec_verify_device_errors needs the
 * caller's workspace and does not apply).
 */
int spec_verify_static(int N, int gmax, int V, const int32_t *draft_ids, const float *draft_probs,
                       const void *target_logits, int logits_dtype, const float *temperature,
                       const int32_t *top_k, const float *top_p, const float *u_accept,
                       const float *u_sample, int32_t *out_tokens, int32_t *out_num_accepted,
                       void *stream);

/* Bytes of the scratch array spec_verify_static uses as its workspace. */
size_t spec_verify_static_scratch_bytes(void);

/* Human-readable text of a return code (static storage). */
const char *spec_verify_status_string(int status);

/* ABI version of this header: 1. */
int spec_verify_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
