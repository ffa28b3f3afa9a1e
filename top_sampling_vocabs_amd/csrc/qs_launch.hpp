// Kernel argument blocks and launchers shared by the C-ABI layer and the
// kernels' translation unit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qs_chunk.hpp"

namespace qs {

struct FilterArgs {
  const uint8_t* logits;
  int64_t row_bytes;      // distance between rows in bytes
  int V;
  int seg;                // tokens per wave slice (multiple of 32)
  const float* T;
  const int32_t* k;
  const float* p;
  const uint32_t* bitmask;
  int64_t bm_stride;      // words
  const uint64_t* seed;
  uint64_t* offset;
  const double* uniforms;
  int32_t* tokens;
  uint32_t* keep_mask;
  int32_t* cand_ids;
  float* cand_probs;
  int32_t* cand_count;
  int64_t cand_cap;
  float* dense;
  int32_t* status;
  int32_t* dbg;
  uint32_t flags;
  // optional: log q of the drawn token. Last, so that the fields above keep
  // their offsets: moving them changed how the compiler keeps the arguments
  // in scalar registers and cost the filter kernel about 1 us.
  float* logprobs;
  // the chunked first pass's results in the caller's workspace (bf16 rows),
  // or null: the filter kernel then reads every row itself
  const chunk::SegSummary* ws_segs;
  const chunk::ChunkMass* ws_mass;
  const uint32_t* ws_cands;
  int S;                  // chunks per row
  // logit processors applied in the kernel (p_on = 0: none); p_copy holds one
  // workspace row of p_copy_bytes per row for rows selected from an edited copy
  int p_on;
  const int32_t* p_hist;
  int64_t p_hist_cap;
  const int32_t* p_hist_count;
  const float* p_rep;
  const float* p_pres;
  const float* p_freq;
  const int32_t* p_bias_ids;
  const float* p_bias_vals;
  int64_t p_bias_cap;
  const int32_t* p_bias_count;
  uint8_t* p_copy;
  int64_t p_copy_bytes;
  // the n most probable tokens of each row written after the row (top_n = 0:
  // none): ids and log-probabilities, [B][top_n]
  int top_n;
  int32_t* top_ids;
  float* top_lp;
};

struct ArgmaxArgs {
  const uint8_t* logits;
  int64_t row_bytes;
  int V;
  int seg;
  const uint32_t* bitmask;
  int64_t bm_stride;
  int32_t* tokens;
  int32_t* status;
};

int seg_for(int V);
hipError_t launch_filter(const FilterArgs& a, int dtype, bool sample, int B, hipStream_t st);
// Whether the per-row filter kernel holds a row of V tokens of this dtype in
// registers (its resident tiers); longer rows stream.
bool filter_row_resident(int dtype, int V);
hipError_t launch_argmax(const ArgmaxArgs& a, int dtype, int B, hipStream_t st);

}  // namespace qs
