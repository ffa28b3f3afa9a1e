// Kernel argument blocks and launchers shared by the C-ABI layer and the
// kernels' translation unit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

struct SpecArgs {
  const int32_t* t_ids;    // [B][t_cap] target list ids, ascending
  const float* t_probs;
  const int32_t* t_count;
  int64_t t_cap;
  const int32_t* d_ids;    // [B][d_cap] draft list
  const float* d_probs;
  const int32_t* d_count;
  int64_t d_cap;
  const int32_t* x;        // [B] draft tokens
  const double* u_accept;
  const double* u_resample;
  int32_t* tokens;
  int32_t* accepted;
  int32_t* status;
};

constexpr int kPenaltyMaxV = 1 << 20;  // vocabulary bitmap held in LDS

struct PenaltyArgs {
  uint8_t* logits;         // modified in place
  int64_t row_bytes;
  int V;
  int dtype;
  const int32_t* hist;     // [B][hist_cap] token ids
  int64_t hist_cap;
  const int32_t* count;
  const float* rep;
  const float* pres;
  const float* freq;       // optional (NULL: 0)
  int32_t* status;
};

struct BiasArgs {
  uint8_t* logits;         // modified in place
  int64_t row_bytes;
  int V;
  int dtype;
  const int32_t* ids;      // [B][cap] token ids
  const float* vals;       // [B][cap] biases
  int64_t cap;
  const int32_t* count;
  int32_t* status;
};

int seg_for(int V);
hipError_t launch_filter(const FilterArgs& a, int dtype, bool sample, int B, hipStream_t st);
hipError_t launch_argmax(const ArgmaxArgs& a, int dtype, int B, hipStream_t st);
hipError_t launch_spec(const SpecArgs& a, int B, hipStream_t st);
hipError_t launch_penalty(const PenaltyArgs& a, int B, hipStream_t st);
hipError_t launch_bias(const BiasArgs& a, int B, hipStream_t st);

}  // namespace qs
