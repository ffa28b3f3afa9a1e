// Argument blocks and launchers of the kernels that work around the filter:
// the speculative verifier and the in-place logit processors. Kept apart from
// the filter's own header so that the filter kernel's sources do not change
// with them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qs {

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

struct TopArgs {
  const int32_t* ids;      // [B][cap] candidate lists
  const float* probs;
  const int32_t* count;
  int64_t cap;
  int n;                   // slots per row
  int32_t* out_ids;        // [B][n]
  float* out_lp;           // [B][n]
  int32_t* status;
};

hipError_t launch_spec(const SpecArgs& a, int B, hipStream_t st);
hipError_t launch_top(const TopArgs& a, int B, hipStream_t st);
hipError_t launch_penalty(const PenaltyArgs& a, int B, hipStream_t st);
hipError_t launch_bias(const BiasArgs& a, int B, hipStream_t st);

}  // namespace qs
