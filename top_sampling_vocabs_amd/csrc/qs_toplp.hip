// The n most probable tokens of each row's candidate list, with their
// log-probabilities under the final distribution.
//
// Page "Sampling 系统设计：从 logits 到可控生成", logprobs section: besides the
// chosen token's log-probability a sampler may return the top tokens with
// theirs. The candidate lists the filter writes hold the final distribution
// (ids ascending, float32 probabilities), so the top n are read off them.
//
// One workgroup of 256 threads per row and n rounds. Each entry has the key
// (probability bits << 32 | ~id): probabilities are non-negative floats, whose
// bits order like their values, and ~id makes the lower id win a tie. Round j
// takes the largest key below round j-1's winner: a block-wide maximum (wave
// reductions, then the 4 waves' results through LDS), so no entry is marked
// or moved. The log is ln 2 (e + log2 m) from frexp and the hardware log2.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qs.h"
#include "qs_aux.hpp"
#include "qs_device.hpp"

namespace qs {
namespace {

constexpr int kTopThreads = 256;
constexpr int kTopWaves = kTopThreads / 64;

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t o = (uint64_t)__shfl_xor((long long)v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

__global__ void __launch_bounds__(kTopThreads) top_logprobs_kernel(TopArgs a) {
  __shared__ uint64_t s_best[kTopWaves];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = tid >> 6;
  const int cnt = a.count[r];
  int32_t* const out_id = a.out_ids + (size_t)r * a.n;
  float* const out_lp = a.out_lp + (size_t)r * a.n;
  if (cnt < 0 || (int64_t)cnt > a.cap) {
    for (int j = tid; j < a.n; j += kTopThreads) {
      out_id[j] = -1;
      out_lp[j] = -INFINITY;
    }
    if (tid == 0) a.status[r] = QS_ROW_BAD_PARAM;
    return;
  }
  const int32_t* ids = a.ids + (size_t)r * a.cap;
  const float* pr = a.probs + (size_t)r * a.cap;
  uint64_t prev = ~0ull;  // every key lies below it
  for (int j = 0; j < a.n; ++j) {
    uint64_t best = 0u;  // below every key (a key's low half is ~id != 0)
    for (int i = tid; i < cnt; i += kTopThreads) {
      const uint64_t key = ((uint64_t)__float_as_uint(pr[i]) << 32) | (uint32_t)~ids[i];
      if (key < prev && key > best) best = key;
    }
    best = wave_max_u64(best);
    if (lane == 0) s_best[w] = best;
    __syncthreads();
    uint64_t b = s_best[0];
#pragma unroll
    for (int k = 1; k < kTopWaves; ++k) b = s_best[k] > b ? s_best[k] : b;
    __syncthreads();  // s_best is rewritten next round
    if (tid == 0) {
      if (b == 0u) {  // fewer entries than n
        out_id[j] = -1;
        out_lp[j] = -INFINITY;
      } else {
        const float q = __uint_as_float((uint32_t)(b >> 32));
        out_id[j] = (int32_t)~(uint32_t)b;
        int e;
        const float m = frexpf(q, &e);
        out_lp[j] = q > 0.0f ? (float)(((double)e + (double)__log2f(m)) * 0.6931471805599453)
                             : -INFINITY;
      }
    }
    prev = b;
    if (b == 0u) {  // the rest of the slots stay empty
      for (int k = j + 1 + tid; k < a.n; k += kTopThreads) {
        out_id[k] = -1;
        out_lp[k] = -INFINITY;
      }
      break;
    }
  }
  if (tid == 0) a.status[r] = QS_ROW_OK;
}

}  // namespace

hipError_t launch_top(const TopArgs& a, int B, hipStream_t st) {
  hipLaunchKernelGGL(top_logprobs_kernel, dim3((unsigned)B), dim3(kTopThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace qs
