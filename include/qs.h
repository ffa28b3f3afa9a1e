/* qs.h — C ABI of the exact top-k / top-p filter-and-sample library for MI355X.
 *
 * One call processes a batch of B rows of vocabulary logits z[B][V] on the
 * caller's HIP stream. Per row r it applies, in this order (page
 * "Attention算完，还没有选出下一个token", section 02, reference convention):
 *   temperature T[r]  ->  legal-token bitmask (illegal -> -inf)  ->  top-k with
 *   renormalisation  ->  top-p (shortest descending-mass prefix whose
 *   cumulative mass reaches p)  ->  renormalisation  ->  (qs_sample) one draw
 *   by inverse CDF in token-id order.
 * The kept set is exactly the one a full stable sort by (-z, token id) gives;
 * boundary duplicates keep the earliest token ids (page "Qrita", key design 3).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every array argument is a DEVICE pointer owned by the caller, scratch
 *   included (the `workspace` argument). The library allocates nothing, keeps
 *   no state between calls and never synchronises:
 *   work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *   default stream). Row outputs are valid once the caller has synchronised
 *   with that stream. Concurrent calls on different streams are safe.
 * - Sizes: 0 <= B <= 4194303 rows (2^22 - 1: one workgroup per row in a
 *   single launch grid) and 1 <= V <= 2^30 tokens; other sizes are
 *   QS_ERR_INVALID_ARG (entry points with a smaller V limit state it).
 * - Logits are row-major, `row_stride` elements apart (row_stride >= V).
 *   `logits` must be 16-byte aligned and row_stride * element size must be a
 *   multiple of 16 bytes.
 * - The legal-token bitmask is packed LSB-first: token i is bit (i & 31) of
 *   32-bit word (i >> 5); W = ceil(V/32) words per row, rows `bitmask_stride`
 *   words apart (>= W). Bits at positions >= V are ignored. NULL = all legal.
 * - Return value: QS_OK, or QS_ERR_INVALID_ARG when a pointer, size, stride or
 *   alignment check fails, or QS_ERR_WORKSPACE when the workspace is missing,
 *   misaligned or smaller than qs_workspace_bytes (both reported before any
 *   HIP call, nothing is enqueued), or QS_ERR_HIP when a launch fails. Row
 *   errors are reported per row in `row_status` (qs_row_status), never by
 *   the return value.
 * - Parameter semantics (page "Sampling 系统设计", temperature section: T = 0 is
 *   greedy, and T < 0, p > 1, k < 0 must be rejected): T finite and >= 0,
 *   T == 0 selects the greedy argmax path; k == 0 disables top-k and k >= the
 *   number of finite legal tokens keeps them all; p == 1 disables top-p;
 *   any other value (T < 0 or not finite, k < 0, p <= 0, p > 1, NaN) makes the
 *   row QS_ROW_BAD_PARAM.
 * - Row errors (page "Attention算完，还没有选出下一个token", sections 03 and 07: an
 *   empty candidate set, NaN and all -inf rows are explicit errors, never a
 *   substituted token) are checked in this order: EMPTY, NONFINITE, ALL_NEG_INF.
 *   An error row gets token -1, an all-zero keep-mask row, cand_count 0,
 *   all-zero dense probabilities and an unchanged RNG offset.
 */
#ifndef QS_H
#define QS_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define QS_API __attribute__((visibility("default")))
#else
#define QS_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QS_OK = 0,
  QS_ERR_INVALID_ARG = 1,
  QS_ERR_WORKSPACE = 2,      /* workspace missing, misaligned or too small  */
  QS_ERR_HIP = 3
} qs_status;

typedef enum {
  QS_ROW_OK = 0,
  QS_ROW_EMPTY = 1,          /* no legal token (all masked)                         */
  QS_ROW_ALL_NEG_INF = 2,    /* legal tokens exist, every legal logit is -inf       */
  QS_ROW_NONFINITE = 3,      /* NaN or +inf at a legal position                     */
  QS_ROW_BAD_PARAM = 4,      /* invalid T, k or p                                   */
  QS_ROW_CAND_OVERFLOW = 5,  /* |P| > cand_cap: candidate lists truncated to
                                cand_cap entries; mask, probs and token complete    */
  QS_ROW_INTERNAL = 6        /* pivot search did not converge (never expected)      */
} qs_row_status;

typedef enum { QS_F32 = 0, QS_BF16 = 1 } qs_dtype;

/* Path switches for ablations and path-invariance tests; outputs are identical
 * with or without them (page "Qrita", ablation table: forced fallback and no
 * truncation). 0 is the normal path, in which bf16 rows held in registers are
 * settled by a value histogram of the whole row; any switch sends every row
 * through the truncation-and-search path, which the switches then vary. */
#define QS_FLAG_FORCE_MISS     1u  /* run every search over the full row        */
#define QS_FLAG_NO_TRUNCATION  2u  /* skip the sigma-truncation compaction      */
#define QS_FLAG_PIVOT_SEARCH   4u  /* quaternary pivot search also on bf16 pools
                                      (instead of their key-histogram scan)     */
#define QS_FLAG_STREAM         8u  /* stream the row even when it fits in
                                      registers                                 */
#define QS_FLAG_BINARY_PIVOT  16u  /* one pivot per search round (the interval's
                                      midpoint) instead of three (ablation)     */
#define QS_FLAG_SORT_SUBSET   32u  /* on a truncation hit, sort the candidate
                                      subset (up to 8192 candidates) and read the
                                      boundaries off the sorted order instead of
                                      searching (the ablation's run I)          */

/* Device scratch a qs_filter_mask / qs_sample call on B rows of V tokens of
 * `dtype` needs, in bytes (0: none). The caller owns it and passes it as
 * `workspace` / `workspace_bytes`; the library never allocates.
 *
 * It holds the candidate set compacted from each row before the selection
 * (page "Qrita", overall framework: the truncation pass writes a small
 * candidate set that the pivot searches then work on; its closing section
 * names full-vocabulary temporaries as a cost, so the buffer is capped:
 * at most 896 entries of every 4096-token segment of a row, plus 32 bytes
 * per segment and 32 per 16384-token chunk). Only bf16 rows longer than
 * the per-row kernel holds in registers (V > 155648) and of at most 2^20
 * tokens take that chunked pass; with S = ceil(V / 16384) chunks a row, they
 * need
 *   align256(B * 4S * 32) + align256(B * S * 32) + B * 4S * 896 * 4 bytes;
 * other calls (fp32, bf16 rows of up to 155648 tokens, longer than 2^20)
 * need none. cand_cap does not change it (the caller's candidate
 * lists are outputs, not scratch). Pure function of its arguments; 0 for
 * invalid ones.
 *
 * The workspace must be 256-byte aligned. Its contents on entry do not
 * matter and are left undefined; two calls that may run at the same time
 * (different streams) need different workspaces. */
QS_API size_t qs_workspace_bytes(int64_t B, int64_t V, int dtype, int64_t cand_cap);

/* Filter a batch: kept-candidate mask and renormalised probabilities.
 *
 * Defines the candidate set O of page "Qrita" (overall framework: strict
 * top-k / top-p mask and candidate set) under the contract order above.
 *
 * logits       [B][row_stride] float32 or bfloat16 (dtype)
 * temperature  [B] float32; top_k [B] int32; top_p [B] float32
 * bitmask      [B][bitmask_stride] uint32, or NULL
 * keep_mask    [B][ceil(V/32)] uint32 out, required: bit i set iff token i is
 *              in the final set P (packed like the bitmask; every word written)
 * cand_ids     [B][cand_cap] int32 out, optional: ids of P in ascending order
 * cand_probs   [B][cand_cap] float32 out, optional: their probabilities
 * cand_count   [B] int32 out, required if cand_ids or cand_probs is given:
 *              |P| (the true size, also when it exceeds cand_cap)
 * dense_probs  [B][V] float32 out, optional: probability of every token
 *              (0 outside P)
 * row_status   [B] int32 out, required (qs_row_status)
 * debug_stats  [B][4] int32 out, optional: {path (0 candidate pool, 1 full
 *              row, 2 candidates of the chunked first pass, 3 full row for
 *              the top-k search, then its top-k set), search rounds,
 *              |Z_t| (candidates above the truncation threshold), |P|}; bf16
 *              rows settled by a value histogram report 0 rounds (path 0 with
 *              |Z_t| = the tokens at or above the final boundary value when
 *              the row was held in registers)
 * flags        QS_FLAG_* bits, 0 normally
 * workspace, workspace_bytes
 *              device scratch of at least qs_workspace_bytes(B, V, dtype,
 *              cand_cap) bytes, 256-byte aligned (NULL / 0 when that is 0);
 *              otherwise QS_ERR_WORKSPACE is returned before any HIP call.
 */
QS_API int qs_filter_mask(const void* logits, int dtype, int64_t B, int64_t V,
                   int64_t row_stride, const float* temperature,
                   const int32_t* top_k, const float* top_p,
                   const uint32_t* bitmask, int64_t bitmask_stride,
                   uint32_t* keep_mask, int32_t* cand_ids, float* cand_probs,
                   int32_t* cand_count, int64_t cand_cap, float* dense_probs,
                   int32_t* row_status, int32_t* debug_stats, uint32_t flags,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Filter and draw one token per row.
 *
 * Same inputs, optional outputs and workspace as qs_filter_mask (keep_mask
 * is optional here). The draw walks P in ascending token id and returns the first id whose
 * cumulative probability exceeds u (page "Attention算完，还没有选出下一个token",
 * section 02 widget: CDF by token id; right-open intervals).
 *
 * seed, offset [B] uint64: per-row RNG state (page above, section 06: explicit
 *              seed/offset advanced by actual consumption). A sampled row
 *              draws u from Philox4x32-10 (Salmon et al., SC'11) with
 *              counter (offset lo, offset hi, 0, 0) and key (seed lo, seed hi),
 *              u = (x0 >> 8) * 2^-24, and then offset += 1. Greedy rows and
 *              error rows consume nothing and leave offset unchanged.
 *              Required unless `uniforms` is given.
 * uniforms     [B] float64 in [0,1), optional: when given, row r uses
 *              u = uniforms[r] and offsets are neither read nor written.
 * tokens       [B] int32 out, required: the token, -1 on an error row.
 * logprobs     [B] float32 out, optional: natural log of the drawn token's
 *              probability under the distribution it was drawn from (after
 *              temperature, mask, top-k, top-p and renormalisation; page
 *              "Sampling 系统设计：从 logits 到可控生成", logprobs section: the
 *              sampler may return it and must state which distribution it
 *              refers to). 0 on greedy rows (a point mass), NaN on error rows.
 */
QS_API int qs_sample(const void* logits, int dtype, int64_t B, int64_t V,
              int64_t row_stride, const float* temperature,
              const int32_t* top_k, const float* top_p,
              const uint32_t* bitmask, int64_t bitmask_stride,
              const uint64_t* seed, uint64_t* offset, const double* uniforms,
              int32_t* tokens, float* logprobs, uint32_t* keep_mask, int32_t* cand_ids,
              float* cand_probs, int32_t* cand_count, int64_t cand_cap,
              float* dense_probs, int32_t* row_status, int32_t* debug_stats,
              uint32_t flags, void* workspace, size_t workspace_bytes, void* stream);

/* qs_sample without a caller workspace, for callers that cannot allocate
 * device memory around the call: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation. Same arguments, outputs and
 * results as qs_sample, minus workspace / workspace_bytes: the scratch of the
 * chunked pass is a fixed array inside the library, QS_SCRATCH_BYTES per GPU
 * (held by each GPU the library runs on until the process ends; its address
 * is taken once per device on the first call there). Calls whose
 * qs_workspace_bytes(B, V, dtype, cand_cap) exceeds QS_SCRATCH_BYTES return
 * QS_ERR_WORKSPACE before any HIP call (64 MiB: e.g. 256 rows of up to
 * 262144 bf16 tokens). Calls on one GPU share its array: calls that overlap
 * in time on one GPU (other streams, other threads) race and must not be
 * issued; calls in order on one stream are safe. Nothing is allocated, and
 * the array needs no clearing between calls. */
#define QS_SCRATCH_BYTES ((size_t)64 << 20)
QS_API int qs_sample_noalloc(const void* logits, int dtype, int64_t B, int64_t V,
              int64_t row_stride, const float* temperature,
              const int32_t* top_k, const float* top_p,
              const uint32_t* bitmask, int64_t bitmask_stride,
              const uint64_t* seed, uint64_t* offset, const double* uniforms,
              int32_t* tokens, float* logprobs, uint32_t* keep_mask, int32_t* cand_ids,
              float* cand_probs, int32_t* cand_count, int64_t cand_cap,
              float* dense_probs, int32_t* row_status, int32_t* debug_stats,
              uint32_t flags, void* stream);

/* Greedy selection: tokens[r] = lowest token id holding the largest finite
 * legal logit. No softmax and no random number (page "第 9 讲 · 生成与推测解码",
 * section 1: argmax needs no normalisation; exercise 1: ties by vocabulary
 * order). tokens and row_status are required; row statuses as above
 * (QS_ROW_EMPTY, QS_ROW_NONFINITE, QS_ROW_ALL_NEG_INF, else QS_ROW_OK). */
QS_API int qs_argmax(const void* logits, int dtype, int64_t B, int64_t V,
              int64_t row_stride, const uint32_t* bitmask,
              int64_t bitmask_stride, int32_t* tokens, int32_t* row_status,
              void* stream);

/* Exact speculative-decoding verification of one draft token per row
 * (page "第 9 讲 · 生成与推测解码", section 5.2: accept the draft token x with
 * probability min(1, p(x)/q(x)); on rejection draw from max(0, p - q)
 * renormalised, so that the output is distributed exactly as p).
 *
 * p (target) and q (draft) are candidate lists as qs_filter_mask / qs_sample
 * write them: ids ascending and unique, float32 probabilities; a token outside
 * a list has probability 0 in it. A row may be one position of a draft run;
 * the caller keeps the accepted prefix.
 *
 * target_ids, target_probs [B][target_cap]; target_count [B] int32
 * draft_ids, draft_probs   [B][draft_cap];  draft_count [B] int32
 * draft_tokens [B] int32: x, drawn from the draft list
 * u_accept, u_resample [B] float64 in [0,1): the row's two uniforms.
 *              Accept iff u_accept * q(x) < p(x) (float64 on the widened list
 *              values). Else the residual r(y) = max(0, p(y) - q(y)) over the
 *              target list, R its sum, and the first y in id order whose
 *              cumulative residual exceeds u_resample * R (the last y with
 *              r(y) > 0 if rounding leaves none). If R == 0 (only through
 *              the lists' rounding) the draw uses p itself.
 * tokens, accepted, row_status [B] int32 out: the output token, 1 if it is
 *              the accepted draft token else 0, and the row status:
 *              QS_ROW_BAD_PARAM for a negative count, x missing from the
 *              draft list or a uniform outside [0,1); QS_ROW_EMPTY for an
 *              empty list (or a target list of zero mass); QS_ROW_CAND_OVERFLOW
 *              when a count exceeds its capacity (the list is truncated). An
 *              error row gets token -1 and accepted 0.
 * Every pointer is required. Lists that are not ascending give unspecified
 * tokens (every read stays within the counts and capacities). One kernel
 * launch on `stream`; nothing is allocated. */
QS_API int qs_spec_verify(int64_t B, const int32_t* target_ids, const float* target_probs,
                   const int32_t* target_count, int64_t target_cap,
                   const int32_t* draft_ids, const float* draft_probs,
                   const int32_t* draft_count, int64_t draft_cap,
                   const int32_t* draft_tokens, const double* u_accept,
                   const double* u_resample, int32_t* tokens, int32_t* accepted,
                   int32_t* row_status, void* stream);

/* qs_sample that also writes each row's n most probable tokens and their
 * log-probabilities, as qs_top_logprobs would read them off the candidate
 * lists this call writes (page "Sampling 系统设计：从 logits 到可控生成",
 * logprobs section: top tokens with their log-probabilities besides the
 * chosen one's), in the same launch: each row's workgroup reads its own list
 * back once it is written. Arguments and outputs are qs_sample's, plus
 *   top_n        1 <= top_n <= 64 (QS_ERR_INVALID_ARG otherwise)
 *   top_ids      [B][top_n] int32 out: the ids, probability descending
 *                (float32 values compared exactly), ties by ascending id; -1
 *                past the list's length
 *   top_logprobs [B][top_n] float32 out: ln q (ln 2 (e + log2 m) from frexp and
 *                the hardware log2, within about 1e-7); -inf past the list's
 *                length and for q = 0
 * cand_ids and cand_probs are required (the source of the top tokens); a row
 * whose status is not QS_ROW_OK (a row error, or QS_ROW_CAND_OVERFLOW: the
 * list was truncated to cand_cap, so its top tokens are not known) gets every
 * slot empty. */
QS_API int qs_sample_top_logprobs(const void* logits, int dtype, int64_t B, int64_t V,
              int64_t row_stride, const float* temperature,
              const int32_t* top_k, const float* top_p,
              const uint32_t* bitmask, int64_t bitmask_stride,
              const uint64_t* seed, uint64_t* offset, const double* uniforms,
              int32_t* tokens, float* logprobs, uint32_t* keep_mask, int32_t* cand_ids,
              float* cand_probs, int32_t* cand_count, int64_t cand_cap,
              float* dense_probs, int32_t* row_status, int32_t* debug_stats,
              uint32_t flags, int64_t top_n, int32_t* top_ids, float* top_logprobs,
              void* workspace, size_t workspace_bytes, void* stream);

/* Logit processors applied inside qs_sample_processed / qs_filter_mask_processed
 * (page "Sampling 系统设计：从 logits 到可控生成", repetition-penalty and
 * LogitsProcessor sections: history-dependent processors edit the logits
 * before the selection). Per row r the logits the selection sees are those
 * qs_apply_penalties and then qs_apply_logit_bias would leave (same formulas,
 * float32 operations and dtype rounding), but the caller's logits are only
 * read: the edited values exist only inside the kernel.
 *
 * Penalties (all four pointers NULL: none): history [B][history_cap] int32
 *   token ids, history_count [B] int32, repetition_penalty and
 *   presence_penalty [B] float32, frequency_penalty [B] float32 or NULL (0).
 * Bias (all three pointers NULL: none): bias_ids [B][bias_cap] int32,
 *   bias_values [B][bias_cap] float32, bias_count [B] int32.
 * A row whose processor arguments qs_apply_penalties or qs_apply_logit_bias
 * would flag (a frequency penalty with more than 4096 history entries among
 * them), or whose bias list holds more than 4096 entries, gets
 * QS_ROW_BAD_PARAM and no outputs (no token, no draw). Histories without a
 * frequency penalty may be of any length. */
typedef struct QsProcessors {
  const int32_t* history;
  int64_t history_cap;
  const int32_t* history_count;
  const float* repetition_penalty;
  const float* presence_penalty;
  const float* frequency_penalty;
  const int32_t* bias_ids;
  const float* bias_values;
  int64_t bias_cap;
  const int32_t* bias_count;
} QsProcessors;

/* Bytes of caller workspace a processed call needs: B rows of
 * align256(V * element size) (a row that the kernel cannot settle from its
 * registers is rewritten there with its processors applied, and selected
 * from that copy); V at most 155648. 0 for invalid arguments. */
QS_API size_t qs_processors_workspace_bytes(int64_t B, int64_t V, int dtype);

/* qs_sample / qs_filter_mask with logit processors `proc` (non-NULL) applied
 * to every row first, in the same launch. Arguments, outputs and statuses are
 * those of qs_sample / qs_filter_mask, with `workspace` sized by
 * qs_processors_workspace_bytes (256-byte aligned; QS_ERR_WORKSPACE before
 * any HIP call otherwise) and V <= 155648 (QS_ERR_INVALID_ARG otherwise). */
QS_API int qs_sample_processed(const void* logits, int dtype, int64_t B, int64_t V,
              int64_t row_stride, const float* temperature,
              const int32_t* top_k, const float* top_p,
              const uint32_t* bitmask, int64_t bitmask_stride,
              const uint64_t* seed, uint64_t* offset, const double* uniforms,
              int32_t* tokens, float* logprobs, uint32_t* keep_mask, int32_t* cand_ids,
              float* cand_probs, int32_t* cand_count, int64_t cand_cap,
              float* dense_probs, int32_t* row_status, int32_t* debug_stats,
              uint32_t flags, const QsProcessors* proc, void* workspace,
              size_t workspace_bytes, void* stream);
QS_API int qs_filter_mask_processed(const void* logits, int dtype, int64_t B, int64_t V,
                   int64_t row_stride, const float* temperature,
                   const int32_t* top_k, const float* top_p,
                   const uint32_t* bitmask, int64_t bitmask_stride,
                   uint32_t* keep_mask, int32_t* cand_ids, float* cand_probs,
                   int32_t* cand_count, int64_t cand_cap, float* dense_probs,
                   int32_t* row_status, int32_t* debug_stats, uint32_t flags,
                   const QsProcessors* proc, void* workspace, size_t workspace_bytes,
                   void* stream);

/* Repetition and presence penalties over each row's history, applied in place
 * to the logits before qs_filter_mask / qs_sample (page "Sampling 系统设计：从
 * logits 到可控生成", repetition-penalty section: a history-dependent logits
 * processor; the page leaves the formula open). For each distinct token t of
 * row r's history with 0 <= t < V:
 *   z[r][t] <- (z > 0 ? z / rep[r] : z * rep[r]) - pres[r]
 * in float32, each operation rounded, stored in the logits' dtype (bfloat16:
 * round to nearest even). A token repeated in the history is penalised once;
 * ids outside [0, V) are ignored; every other logit is untouched (the work is
 * proportional to the history, not to V). rep = 1 and pres = 0 change nothing.
 *
 * logits            [B][row_stride] float32 or bfloat16 (dtype), modified in
 *                   place; aligned to its element size; V <= 2^20
 * history           [B][history_cap] int32 token ids; history_count [B] int32
 * repetition_penalty, presence_penalty [B] float32
 * frequency_penalty [B] float32, optional (NULL: 0): then also
 *                   z[r][t] <- z - f[r] * n_t (both in float32), n_t the
 *                   number of times t occurs in the history; a row with
 *                   f != 0 may hold at most 4096 history entries
 * row_status        [B] int32 out: QS_ROW_OK, or QS_ROW_BAD_PARAM (row left
 *                   unchanged) when rep is not finite or <= 0, pres or f is
 *                   not finite, the count lies outside [0, history_cap], or
 *                   f != 0 with more than 4096 entries.
 * Every pointer but frequency_penalty is required. One kernel launch on `stream`; nothing is
 * allocated. */
QS_API int qs_apply_penalties(void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                       const int32_t* history, int64_t history_cap,
                       const int32_t* history_count, const float* repetition_penalty,
                       const float* presence_penalty, const float* frequency_penalty,
                       int32_t* row_status, void* stream);

/* Additive logit bias, applied in place to the logits before qs_filter_mask /
 * qs_sample (page "Sampling 系统设计：从 logits 到可控生成", logits-processor
 * section: processors edit the logits before the softmax; a per-row list of
 * token biases is the plain additive one). For each (t, b) of row r's first
 * bias_count[r] entries with 0 <= t < V:  z[r][t] <- z[r][t] + b  in float32,
 * stored in the logits' dtype (bfloat16: round to nearest even); ids outside
 * [0, V) are ignored. A bias of -inf is not accepted: use the legal-token
 * bitmask to exclude tokens.
 *
 * logits       [B][row_stride] float32 or bfloat16 (dtype), modified in place;
 *              aligned to its element size; V <= 2^20
 * bias_ids     [B][bias_cap] int32; bias_values [B][bias_cap] float32;
 *              bias_count [B] int32
 * row_status   [B] int32 out: QS_ROW_OK, or QS_ROW_BAD_PARAM (row left
 *              unchanged) when the count lies outside [0, bias_cap], a value
 *              is not finite, or a token in [0, V) is listed twice.
 * Every pointer is required. One kernel launch on `stream`; nothing is
 * allocated. */
QS_API int qs_apply_logit_bias(void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                        const int32_t* bias_ids, const float* bias_values, int64_t bias_cap,
                        const int32_t* bias_count, int32_t* row_status, void* stream);

/* The n most probable tokens of each row's candidate list and their natural
 * log-probabilities under the final distribution (page "Sampling 系统设计：从
 * logits 到可控生成", logprobs section: top tokens with their log-probabilities
 * besides the chosen one's). The lists are those qs_filter_mask / qs_sample
 * write (the final, renormalised distribution). Order: probability descending
 * (float32 values compared exactly), ties by ascending id.
 *
 * cand_ids, cand_probs [B][cand_cap]; cand_count [B] int32
 * n            slots per row, 1 <= n <= 4096
 * top_ids      [B][n] int32 out: the ids, -1 past the list's length
 * top_logprobs [B][n] float32 out: their log-probabilities (ln 2 (e + log2 m)
 *              from frexp and the hardware log2, within about 1e-7), -inf past
 *              the list's length (and for a probability of 0)
 * row_status   [B] int32 out: QS_ROW_OK; QS_ROW_BAD_PARAM (every slot
 *              empty) for a negative count; QS_ROW_CAND_OVERFLOW (every slot
 *              empty) for a count above cand_cap, which is how the filter
 *              reports a list it truncated: the filter's cand_cap must be at
 *              least |P| for the top tokens of a row to be known
 * Every pointer is required. One kernel launch on `stream`; nothing is
 * allocated. */
QS_API int qs_top_logprobs(int64_t B, const int32_t* cand_ids, const float* cand_probs,
                    const int32_t* cand_count, int64_t cand_cap, int64_t n,
                    int32_t* top_ids, float* top_logprobs, int32_t* row_status,
                    void* stream);

/* Library version string (static storage). */
QS_API const char* qs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QS_H */
