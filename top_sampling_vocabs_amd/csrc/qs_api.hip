// C-ABI entry points: argument validation (before any HIP call), launch
// geometry, and error mapping. Every entry point enqueues its kernels on the
// caller's stream (one launch; two for filter calls on bf16 rows longer than
// the per-row kernel holds in registers: the chunk pass and the per-row
// filter) and returns without synchronising.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/qs.h"

#include "qs_aux.hpp"
#include "qs_chunk.hpp"
#include "qs_launch.hpp"
#include "qs_proc.hpp"
#include "qs_topn.hpp"

namespace {

constexpr int64_t kMaxV = (int64_t)1 << 30;
// one workgroup of up to 1024 threads per row: B * 1024 threads must fit one
// launch grid (fewer than 2^32)
constexpr int64_t kMaxB = ((int64_t)1 << 22) - 1;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Workspace of the chunked first pass, which takes bf16 rows longer than the
// per-row kernel holds in registers (those stream there, one workgroup per
// row) and of at most kMaxChunks chunks. Rows held in registers fill the GPU
// with one workgroup each and need no workspace.
bool chunked_rows(int64_t V, int dtype) {
  return dtype == QS_BF16 && !qs::filter_row_resident(QS_BF16, (int)V) &&
         qs::chunk::chunks_for(V) <= qs::chunk::kMaxChunks;
}
size_t ws_bytes(int64_t B, int64_t V, int dtype) {
  if (B == 0 || !chunked_rows(V, dtype)) return 0;
  return qs::chunk::workspace_bytes(B, V);
}
// a processed call: one 256-byte aligned workspace row per row
size_t proc_row_bytes(int64_t V, int dtype) {
  return ((size_t)V * (dtype == QS_F32 ? 4 : 2) + 255) & ~(size_t)255;
}
size_t proc_ws_bytes(int64_t B, int64_t V, int dtype) {
  return (size_t)B * proc_row_bytes(V, dtype);
}

// Shared checks of the logits / bitmask description.
int check_input(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                const uint32_t* bitmask, int64_t bitmask_stride) {
  if (dtype != QS_F32 && dtype != QS_BF16) return QS_ERR_INVALID_ARG;
  if (B < 0 || B > kMaxB || V < 1 || V > kMaxV) return QS_ERR_INVALID_ARG;
  if (B == 0) return QS_OK;
  if (!logits || !aligned(logits, 16)) return QS_ERR_INVALID_ARG;
  const int64_t es = dtype == QS_F32 ? 4 : 2;
  if (row_stride < V || (row_stride * es) % 16 != 0) return QS_ERR_INVALID_ARG;
  if (bitmask) {
    if (!aligned(bitmask, 4)) return QS_ERR_INVALID_ARG;
    if (bitmask_stride < (V + 31) / 32) return QS_ERR_INVALID_ARG;
  }
  return QS_OK;
}

int filter_common(bool sample, const void* logits, int dtype, int64_t B, int64_t V,
                  int64_t row_stride, const float* temperature, const int32_t* top_k,
                  const float* top_p, const uint32_t* bitmask, int64_t bitmask_stride,
                  const uint64_t* seed, uint64_t* offset, const double* uniforms,
                  int32_t* tokens, float* logprobs, uint32_t* keep_mask, int32_t* cand_ids,
                  float* cand_probs,
                  int32_t* cand_count, int64_t cand_cap, float* dense_probs,
                  int32_t* row_status, int32_t* debug_stats, uint32_t flags, void* workspace,
                  size_t workspace_bytes, void* stream, const QsProcessors* proc = nullptr,
                  int64_t top_n = 0, int32_t* top_ids = nullptr, float* top_logprobs = nullptr) {
  int rc = check_input(logits, dtype, B, V, row_stride, bitmask, bitmask_stride);
  if (rc != QS_OK) return rc;
  if (flags & ~(QS_FLAG_FORCE_MISS | QS_FLAG_NO_TRUNCATION | QS_FLAG_PIVOT_SEARCH |
                QS_FLAG_STREAM | QS_FLAG_BINARY_PIVOT | QS_FLAG_SORT_SUBSET))
    return QS_ERR_INVALID_ARG;
  if (B == 0) return QS_OK;
  if (!temperature || !top_k || !top_p || !row_status) return QS_ERR_INVALID_ARG;
  if (!sample && !keep_mask) return QS_ERR_INVALID_ARG;
  if (sample) {
    if (!tokens) return QS_ERR_INVALID_ARG;
    if (!uniforms && (!seed || !offset)) return QS_ERR_INVALID_ARG;
  }
  if (cand_ids || cand_probs) {
    if (!cand_count || cand_cap < 1 || cand_cap > kMaxV) return QS_ERR_INVALID_ARG;
  }
  if (!aligned(temperature, 4) || !aligned(top_k, 4) || !aligned(top_p, 4) ||
      !aligned(row_status, 4) || !aligned(keep_mask, 4) || !aligned(cand_ids, 4) ||
      !aligned(cand_probs, 4) || !aligned(cand_count, 4) || !aligned(dense_probs, 4) ||
      !aligned(debug_stats, 4) || !aligned(tokens, 4) || !aligned(logprobs, 4) ||
      !aligned(seed, 8) || !aligned(offset, 8) || !aligned(uniforms, 8))
    return QS_ERR_INVALID_ARG;
  if (proc) {
    // every pointer of a group or none; V within the in-kernel table
    const bool hist_any = proc->history || proc->history_count || proc->repetition_penalty ||
                          proc->presence_penalty || proc->frequency_penalty;
    const bool hist_all = proc->history && proc->history_count && proc->repetition_penalty &&
                          proc->presence_penalty;
    const bool bias_any = proc->bias_ids || proc->bias_values || proc->bias_count;
    const bool bias_all = proc->bias_ids && proc->bias_values && proc->bias_count;
    if (V > qs::proc::kMaxV || (hist_any && !hist_all) || (bias_any && !bias_all))
      return QS_ERR_INVALID_ARG;
    if (hist_all && (proc->history_cap < 0 || proc->history_cap > kMaxV * 64)) return QS_ERR_INVALID_ARG;
    if (bias_all && (proc->bias_cap < 0 || proc->bias_cap > kMaxV * 64)) return QS_ERR_INVALID_ARG;
    if (!aligned(proc->history, 4) || !aligned(proc->history_count, 4) ||
        !aligned(proc->repetition_penalty, 4) || !aligned(proc->presence_penalty, 4) ||
        !aligned(proc->frequency_penalty, 4) || !aligned(proc->bias_ids, 4) ||
        !aligned(proc->bias_values, 4) || !aligned(proc->bias_count, 4))
      return QS_ERR_INVALID_ARG;
  }
  if (top_n != 0) {
    // the top tokens are read off the candidate lists the call writes
    if (top_n < 1 || top_n > qs::kTopNMax || !top_ids || !top_logprobs || !cand_ids ||
        !cand_probs || proc || !aligned(top_ids, 4) || !aligned(top_logprobs, 4))
      return QS_ERR_INVALID_ARG;
  }
  const size_t need = proc ? proc_ws_bytes(B, V, dtype) : ws_bytes(B, V, dtype);
  if (need > 0) {
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < need) return QS_ERR_WORKSPACE;
  }

  qs::FilterArgs a;
  a.logits = static_cast<const uint8_t*>(logits);
  a.row_bytes = row_stride * (dtype == QS_F32 ? 4 : 2);
  a.V = (int)V;
  a.seg = qs::seg_for((int)V);  // the launcher sets the slice length of its tier
  a.T = temperature;
  a.k = top_k;
  a.p = top_p;
  a.bitmask = bitmask;
  a.bm_stride = bitmask_stride;
  a.seed = seed;
  a.offset = offset;
  a.uniforms = uniforms;
  a.tokens = tokens;
  a.logprobs = logprobs;
  a.keep_mask = keep_mask;
  a.cand_ids = cand_ids;
  a.cand_probs = cand_probs;
  a.cand_count = cand_count;
  a.cand_cap = (cand_ids || cand_probs) ? cand_cap : 0;
  a.dense = dense_probs;
  a.status = row_status;
  a.dbg = debug_stats;
  a.flags = flags;
  a.ws_segs = nullptr;
  a.ws_mass = nullptr;
  a.ws_cands = nullptr;
  a.S = 0;
  a.p_on = 0;
  a.p_hist = nullptr; a.p_hist_cap = 0; a.p_hist_count = nullptr;
  a.p_rep = nullptr; a.p_pres = nullptr; a.p_freq = nullptr;
  a.p_bias_ids = nullptr; a.p_bias_vals = nullptr; a.p_bias_cap = 0; a.p_bias_count = nullptr;
  a.p_copy = nullptr; a.p_copy_bytes = 0;
  a.top_n = (int)top_n;
  a.top_ids = top_ids;
  a.top_lp = top_logprobs;
  if (proc) {
    a.p_on = 1;
    if (proc->history) {
      a.p_hist = proc->history; a.p_hist_cap = proc->history_cap;
      a.p_hist_count = proc->history_count;
      a.p_rep = proc->repetition_penalty; a.p_pres = proc->presence_penalty;
      a.p_freq = proc->frequency_penalty;
    }
    if (proc->bias_ids) {
      a.p_bias_ids = proc->bias_ids; a.p_bias_vals = proc->bias_values;
      a.p_bias_cap = proc->bias_cap; a.p_bias_count = proc->bias_count;
    }
    a.p_copy = static_cast<uint8_t*>(workspace);
    a.p_copy_bytes = (int64_t)proc_row_bytes(V, dtype);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!proc && need > 0 && flags == 0u) {
    // long bf16 rows: the chunk kernel streams every row first, the filter
    // kernel then settles each row from the chunks' candidates (path switches
    // skip it)
    qs::chunk::Args ca;
    ca.logits = a.logits;
    ca.row_bytes = a.row_bytes;
    ca.V = a.V;
    ca.B = (int)B;
    ca.S = qs::chunk::chunks_for(V);
    ca.stride = qs::chunk::sample_stride(V);
    ca.T = temperature;
    ca.k = top_k;
    ca.p = top_p;
    ca.bitmask = bitmask;
    ca.bm_stride = bitmask_stride;
    uint8_t* const ws = static_cast<uint8_t*>(workspace);
    ca.segs = reinterpret_cast<qs::chunk::SegSummary*>(ws);
    ca.mass = reinterpret_cast<qs::chunk::ChunkMass*>(ws + qs::chunk::seg_bytes(B, V));
    ca.cands = reinterpret_cast<uint32_t*>(ws + qs::chunk::seg_bytes(B, V) +
                                           qs::chunk::mass_bytes(B, V));
    if (qs::chunk::launch_scan_bf16(ca, st) != hipSuccess) return QS_ERR_HIP;
    a.ws_segs = ca.segs;
    a.ws_mass = ca.mass;
    a.ws_cands = ca.cands;
    a.S = ca.S;
  }
  hipError_t e = qs::launch_filter(a, dtype, sample, (int)B, st);
  return e == hipSuccess ? QS_OK : QS_ERR_HIP;
}

// The chunked pass's scratch for qs_sample_noalloc, one copy per GPU. In
// host code `scratch` names a host-side stand-in: kernels and copies get the
// device address from hipGetSymbolAddress (taken once per device, with that
// device current), never the array's name.
static __device__ __align__(256) uint8_t scratch[QS_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The device address of this device's `scratch` (nullptr on a HIP error).
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

size_t qs_processors_workspace_bytes(int64_t B, int64_t V, int dtype) {
  if (B < 0 || B > kMaxB || V < 1 || V > qs::proc::kMaxV || (dtype != QS_F32 && dtype != QS_BF16))
    return 0;
  return proc_ws_bytes(B, V, dtype);
}

int qs_sample_processed(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                        const float* temperature, const int32_t* top_k, const float* top_p,
                        const uint32_t* bitmask, int64_t bitmask_stride, const uint64_t* seed,
                        uint64_t* offset, const double* uniforms, int32_t* tokens,
                        float* logprobs, uint32_t* keep_mask, int32_t* cand_ids,
                        float* cand_probs, int32_t* cand_count, int64_t cand_cap,
                        float* dense_probs, int32_t* row_status, int32_t* debug_stats,
                        uint32_t flags, const QsProcessors* proc, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (!proc) return QS_ERR_INVALID_ARG;
  return filter_common(true, logits, dtype, B, V, row_stride, temperature, top_k, top_p,
                       bitmask, bitmask_stride, seed, offset, uniforms, tokens, logprobs,
                       keep_mask, cand_ids, cand_probs, cand_count, cand_cap, dense_probs,
                       row_status, debug_stats, flags, workspace, workspace_bytes, stream, proc);
}

int qs_filter_mask_processed(const void* logits, int dtype, int64_t B, int64_t V,
                             int64_t row_stride, const float* temperature, const int32_t* top_k,
                             const float* top_p, const uint32_t* bitmask, int64_t bitmask_stride,
                             uint32_t* keep_mask, int32_t* cand_ids, float* cand_probs,
                             int32_t* cand_count, int64_t cand_cap, float* dense_probs,
                             int32_t* row_status, int32_t* debug_stats, uint32_t flags,
                             const QsProcessors* proc, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (!proc) return QS_ERR_INVALID_ARG;
  return filter_common(false, logits, dtype, B, V, row_stride, temperature, top_k, top_p,
                       bitmask, bitmask_stride, nullptr, nullptr, nullptr, nullptr, nullptr,
                       keep_mask, cand_ids, cand_probs, cand_count, cand_cap, dense_probs,
                       row_status, debug_stats, flags, workspace, workspace_bytes, stream, proc);
}

size_t qs_workspace_bytes(int64_t B, int64_t V, int dtype, int64_t cand_cap) {
  (void)cand_cap;
  if (B < 0 || B > kMaxB || V < 1 || V > kMaxV || (dtype != QS_F32 && dtype != QS_BF16))
    return 0;
  return ws_bytes(B, V, dtype);
}

int qs_filter_mask(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                   const float* temperature, const int32_t* top_k, const float* top_p,
                   const uint32_t* bitmask, int64_t bitmask_stride, uint32_t* keep_mask,
                   int32_t* cand_ids, float* cand_probs, int32_t* cand_count, int64_t cand_cap,
                   float* dense_probs, int32_t* row_status, int32_t* debug_stats,
                   uint32_t flags, void* workspace, size_t workspace_bytes, void* stream) {
  return filter_common(false, logits, dtype, B, V, row_stride, temperature, top_k, top_p,
                       bitmask, bitmask_stride, nullptr, nullptr, nullptr, nullptr, nullptr, keep_mask,
                       cand_ids, cand_probs, cand_count, cand_cap, dense_probs, row_status,
                       debug_stats, flags, workspace, workspace_bytes, stream);
}

int qs_sample(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
              const float* temperature, const int32_t* top_k, const float* top_p,
              const uint32_t* bitmask, int64_t bitmask_stride, const uint64_t* seed,
              uint64_t* offset, const double* uniforms, int32_t* tokens, float* logprobs,
              uint32_t* keep_mask, int32_t* cand_ids, float* cand_probs, int32_t* cand_count, int64_t cand_cap,
              float* dense_probs, int32_t* row_status, int32_t* debug_stats, uint32_t flags,
              void* workspace, size_t workspace_bytes, void* stream) {
  return filter_common(true, logits, dtype, B, V, row_stride, temperature, top_k, top_p,
                       bitmask, bitmask_stride, seed, offset, uniforms, tokens, logprobs,
                       keep_mask, cand_ids, cand_probs, cand_count, cand_cap, dense_probs, row_status,
                       debug_stats, flags, workspace, workspace_bytes, stream);
}

int qs_sample_top_logprobs(const void* logits, int dtype, int64_t B, int64_t V,
                           int64_t row_stride, const float* temperature, const int32_t* top_k,
                           const float* top_p, const uint32_t* bitmask, int64_t bitmask_stride,
                           const uint64_t* seed, uint64_t* offset, const double* uniforms,
                           int32_t* tokens, float* logprobs, uint32_t* keep_mask,
                           int32_t* cand_ids, float* cand_probs, int32_t* cand_count,
                           int64_t cand_cap, float* dense_probs, int32_t* row_status,
                           int32_t* debug_stats, uint32_t flags, int64_t top_n, int32_t* top_ids,
                           float* top_logprobs, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (top_n == 0) return QS_ERR_INVALID_ARG;
  return filter_common(true, logits, dtype, B, V, row_stride, temperature, top_k, top_p,
                       bitmask, bitmask_stride, seed, offset, uniforms, tokens, logprobs,
                       keep_mask, cand_ids, cand_probs, cand_count, cand_cap, dense_probs,
                       row_status, debug_stats, flags, workspace, workspace_bytes, stream,
                       nullptr, top_n, top_ids, top_logprobs);
}

int qs_sample_noalloc(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                      const float* temperature, const int32_t* top_k, const float* top_p,
                      const uint32_t* bitmask, int64_t bitmask_stride, const uint64_t* seed,
                      uint64_t* offset, const double* uniforms, int32_t* tokens,
                      float* logprobs, uint32_t* keep_mask, int32_t* cand_ids,
                      float* cand_probs, int32_t* cand_count, int64_t cand_cap,
                      float* dense_probs, int32_t* row_status, int32_t* debug_stats,
                      uint32_t flags, void* stream) {
  // the size check first, as qs_sample's (before any HIP call)
  int rc = check_input(logits, dtype, B, V, row_stride, bitmask, bitmask_stride);
  if (rc != QS_OK) return rc;
  if (B == 0) return QS_OK;
  if (ws_bytes(B, V, dtype) > QS_SCRATCH_BYTES) return QS_ERR_WORKSPACE;
  void* const ws = scratch_address();
  if (ws == nullptr) return QS_ERR_HIP;
  return filter_common(true, logits, dtype, B, V, row_stride, temperature, top_k, top_p,
                       bitmask, bitmask_stride, seed, offset, uniforms, tokens, logprobs,
                       keep_mask, cand_ids, cand_probs, cand_count, cand_cap, dense_probs,
                       row_status, debug_stats, flags, ws, QS_SCRATCH_BYTES, stream);
}

int qs_argmax(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
              const uint32_t* bitmask, int64_t bitmask_stride, int32_t* tokens,
              int32_t* row_status, void* stream) {
  int rc = check_input(logits, dtype, B, V, row_stride, bitmask, bitmask_stride);
  if (rc != QS_OK) return rc;
  if (B == 0) return QS_OK;
  if (!tokens || !row_status || !aligned(tokens, 4) || !aligned(row_status, 4))
    return QS_ERR_INVALID_ARG;
  qs::ArgmaxArgs a;
  a.logits = static_cast<const uint8_t*>(logits);
  a.row_bytes = row_stride * (dtype == QS_F32 ? 4 : 2);
  a.V = (int)V;
  a.seg = qs::seg_for((int)V);
  a.bitmask = bitmask;
  a.bm_stride = bitmask_stride;
  a.tokens = tokens;
  a.status = row_status;
  hipError_t e = qs::launch_argmax(a, dtype, (int)B, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? QS_OK : QS_ERR_HIP;
}

int qs_spec_verify(int64_t B, const int32_t* target_ids, const float* target_probs,
                   const int32_t* target_count, int64_t target_cap, const int32_t* draft_ids,
                   const float* draft_probs, const int32_t* draft_count, int64_t draft_cap,
                   const int32_t* draft_tokens, const double* u_accept,
                   const double* u_resample, int32_t* tokens, int32_t* accepted,
                   int32_t* row_status, void* stream) {
  if (B < 0 || B > kMaxB) return QS_ERR_INVALID_ARG;
  if (B == 0) return QS_OK;
  if (target_cap < 1 || target_cap > kMaxV || draft_cap < 1 || draft_cap > kMaxV)
    return QS_ERR_INVALID_ARG;
  const void* req4[] = {target_ids, target_probs, target_count, draft_ids, draft_probs,
                        draft_count, draft_tokens, tokens, accepted, row_status};
  for (const void* p : req4)
    if (!p || !aligned(p, 4)) return QS_ERR_INVALID_ARG;
  if (!u_accept || !u_resample || !aligned(u_accept, 8) || !aligned(u_resample, 8))
    return QS_ERR_INVALID_ARG;
  qs::SpecArgs a;
  a.t_ids = target_ids;
  a.t_probs = target_probs;
  a.t_count = target_count;
  a.t_cap = target_cap;
  a.d_ids = draft_ids;
  a.d_probs = draft_probs;
  a.d_count = draft_count;
  a.d_cap = draft_cap;
  a.x = draft_tokens;
  a.u_accept = u_accept;
  a.u_resample = u_resample;
  a.tokens = tokens;
  a.accepted = accepted;
  a.status = row_status;
  hipError_t e = qs::launch_spec(a, (int)B, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? QS_OK : QS_ERR_HIP;
}

int qs_apply_penalties(void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                       const int32_t* history, int64_t history_cap,
                       const int32_t* history_count, const float* repetition_penalty,
                       const float* presence_penalty, const float* frequency_penalty,
                       int32_t* row_status, void* stream) {
  if (dtype != QS_F32 && dtype != QS_BF16) return QS_ERR_INVALID_ARG;
  if (B < 0 || B > kMaxB || V < 1 || V > qs::kPenaltyMaxV) return QS_ERR_INVALID_ARG;
  if (B == 0) return QS_OK;
  const int64_t es = dtype == QS_F32 ? 4 : 2;
  if (!logits || !aligned(logits, (uintptr_t)es) || row_stride < V) return QS_ERR_INVALID_ARG;
  if (history_cap < 1 || history_cap > kMaxV) return QS_ERR_INVALID_ARG;
  const void* req4[] = {history, history_count, repetition_penalty, presence_penalty, row_status};
  for (const void* p : req4)
    if (!p || !aligned(p, 4)) return QS_ERR_INVALID_ARG;
  if (!aligned(frequency_penalty, 4)) return QS_ERR_INVALID_ARG;
  qs::PenaltyArgs a;
  a.logits = static_cast<uint8_t*>(logits);
  a.row_bytes = row_stride * es;
  a.V = (int)V;
  a.dtype = dtype;
  a.hist = history;
  a.hist_cap = history_cap;
  a.count = history_count;
  a.rep = repetition_penalty;
  a.pres = presence_penalty;
  a.freq = frequency_penalty;
  a.status = row_status;
  hipError_t e = qs::launch_penalty(a, (int)B, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? QS_OK : QS_ERR_HIP;
}

int qs_apply_logit_bias(void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                        const int32_t* bias_ids, const float* bias_values, int64_t bias_cap,
                        const int32_t* bias_count, int32_t* row_status, void* stream) {
  if (dtype != QS_F32 && dtype != QS_BF16) return QS_ERR_INVALID_ARG;
  if (B < 0 || B > kMaxB || V < 1 || V > qs::kPenaltyMaxV) return QS_ERR_INVALID_ARG;
  if (B == 0) return QS_OK;
  const int64_t es = dtype == QS_F32 ? 4 : 2;
  if (!logits || !aligned(logits, (uintptr_t)es) || row_stride < V) return QS_ERR_INVALID_ARG;
  if (bias_cap < 1 || bias_cap > kMaxV) return QS_ERR_INVALID_ARG;
  const void* req4[] = {bias_ids, bias_values, bias_count, row_status};
  for (const void* p : req4)
    if (!p || !aligned(p, 4)) return QS_ERR_INVALID_ARG;
  qs::BiasArgs a;
  a.logits = static_cast<uint8_t*>(logits);
  a.row_bytes = row_stride * es;
  a.V = (int)V;
  a.dtype = dtype;
  a.ids = bias_ids;
  a.vals = bias_values;
  a.cap = bias_cap;
  a.count = bias_count;
  a.status = row_status;
  hipError_t e = qs::launch_bias(a, (int)B, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? QS_OK : QS_ERR_HIP;
}

int qs_top_logprobs(int64_t B, const int32_t* cand_ids, const float* cand_probs,
                    const int32_t* cand_count, int64_t cand_cap, int64_t n, int32_t* top_ids,
                    float* top_logprobs, int32_t* row_status, void* stream) {
  if (B < 0 || B > kMaxB) return QS_ERR_INVALID_ARG;
  if (B == 0) return QS_OK;
  if (cand_cap < 1 || cand_cap > kMaxV || n < 1 || n > 4096) return QS_ERR_INVALID_ARG;
  const void* req4[] = {cand_ids, cand_probs, cand_count, top_ids, top_logprobs, row_status};
  for (const void* p : req4)
    if (!p || !aligned(p, 4)) return QS_ERR_INVALID_ARG;
  qs::TopArgs a;
  a.ids = cand_ids;
  a.probs = cand_probs;
  a.count = cand_count;
  a.cap = cand_cap;
  a.n = (int)n;
  a.out_ids = top_ids;
  a.out_lp = top_logprobs;
  a.status = row_status;
  hipError_t e = qs::launch_top(a, (int)B, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? QS_OK : QS_ERR_HIP;
}

const char* qs_version(void) { return "qs 0.1.0 gfx950"; }

}  // extern "C"
