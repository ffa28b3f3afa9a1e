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
//
// For n <= 64 over lists of at most 16,384 entries a second kernel keeps each
// thread's 16 keys in registers and never waits on the block per round: each
// of its 16 waves finds the top n of its own keys by wave-wide maxima, writes
// them to LDS, and after the one barrier wave 0 takes the top n of those
// 16 n survivors the same way. The global top n lie among the survivors,
// since a key beaten by n larger keys of its own wave is beaten overall.

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

constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / 64;
constexpr int kSmallPer = 16;   // keys a thread holds: lists up to 16,384 entries
constexpr int kSmallN = 64;     // largest n of the register path
constexpr int kSortFromN = 16;  // from this n on, lanes sort their keys first

__device__ __forceinline__ float key_logprob(uint64_t b) {
  const float q = __uint_as_float((uint32_t)(b >> 32));
  int e;
  const float m = frexpf(q, &e);
  return q > 0.0f ? (float)(((double)e + (double)__log2f(m)) * 0.6931471805599453)
                  : -INFINITY;
}

// One step of a wave maximum: the value of the lane the DPP pattern names
// (both halves moved with the same pattern), kept if larger.
template <int Ctrl>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, Ctrl, 0xF, 0xF, true);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), Ctrl, 0xF, 0xF, true);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > v ? o : v;
}

// Wave maximum: within each row of 16 lanes by DPP moves (swap neighbours,
// swap pairs, mirror each half row, mirror the row: after each step every
// lane holds the maximum of a group twice as large), then across the four
// rows by two lane shuffles. Every lane of the wave must be active.
__device__ __forceinline__ uint64_t wave_max_u64_dpp(uint64_t v) {
  v = dpp_max_step<0xB1>(v);   // quad_perm(1,0,3,2)
  v = dpp_max_step<0x4E>(v);   // quad_perm(2,3,0,1)
  v = dpp_max_step<0x141>(v);  // row_half_mirror
  v = dpp_max_step<0x140>(v);  // row_mirror
#pragma unroll
  for (int off = 16; off < 64; off <<= 1) {
    const uint64_t o = (uint64_t)__shfl_xor((long long)v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

// Sorts a lane's keys into descending order (bitonic network; every index is
// a compile-time constant, so the keys stay in registers).
template <int N>
__device__ __forceinline__ void sort_desc(uint64_t (&key)[N]) {
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int l = i ^ j;
        if (l > i) {
          const bool desc = (i & k) == 0;
          const uint64_t x = key[i], y = key[l];
          const bool sw = desc ? x < y : x > y;
          key[i] = sw ? y : x;
          key[l] = sw ? x : y;
        }
      }
    }
  }
}

// Takes the wave's largest head key; the lane that held it (keys are
// distinct) moves its next key up. Returns 0 once every lane is empty.
template <int N>
__device__ __forceinline__ uint64_t wave_pop_max(uint64_t (&key)[N]) {
  const uint64_t b = wave_max_u64_dpp(key[0]);
  if (b != 0u && key[0] == b) {
#pragma unroll
    for (int t = 0; t + 1 < N; ++t) key[t] = key[t + 1];
    key[N - 1] = 0u;
  }
  return b;
}

// Largest key below `prev` among this lane's keys, then across the wave.
template <int N>
__device__ __forceinline__ uint64_t wave_next_below(const uint64_t (&key)[N], uint64_t prev) {
  uint64_t best = 0u;
#pragma unroll
  for (int t = 0; t < N; ++t) best = (key[t] < prev && key[t] > best) ? key[t] : best;
  return wave_max_u64_dpp(best);
}

// Sorted: each lane sorts its keys once and a round looks at heads only (pays
// off from about 16 rounds on); else every round scans all of a lane's keys.
template <bool kSorted>
__global__ void __launch_bounds__(kSmallThreads) top_logprobs_small_kernel(TopArgs a) {
  __shared__ uint64_t s_cand[kSmallWaves * kSmallN];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = tid >> 6;
  const int cnt = a.count[r];
  int32_t* const out_id = a.out_ids + (size_t)r * a.n;
  float* const out_lp = a.out_lp + (size_t)r * a.n;
  if (cnt < 0 || (int64_t)cnt > a.cap) {
    for (int j = tid; j < a.n; j += kSmallThreads) {
      out_id[j] = -1;
      out_lp[j] = -INFINITY;
    }
    // a count above the capacity is a list the filter truncated (its overflow
    // status); a negative count is bad input
    if (tid == 0) a.status[r] = cnt < 0 ? QS_ROW_BAD_PARAM : QS_ROW_CAND_OVERFLOW;
    return;
  }
  const int32_t* ids = a.ids + (size_t)r * a.cap;
  const float* pr = a.probs + (size_t)r * a.cap;
  uint64_t key[kSmallPer];
#pragma unroll
  for (int t = 0; t < kSmallPer; ++t) {
    const int i = tid + t * kSmallThreads;
    key[t] = i < cnt ? ((uint64_t)__float_as_uint(pr[i]) << 32) | (uint32_t)~ids[i] : 0u;
  }
  s_cand[tid] = 0u;  // slots a wave leaves unused read as "no key"
  __syncthreads();
  if (kSorted) sort_desc(key);
  uint64_t prev = ~0ull;
  for (int j = 0; j < a.n; ++j) {
    const uint64_t b = kSorted ? wave_pop_max(key) : wave_next_below(key, prev);
    if (b == 0u) break;  // wave-uniform: this wave has no more keys
    if (lane == 0) s_cand[w * kSmallN + j] = b;
    prev = b;
  }
  __syncthreads();
  if (w != 0) return;
  uint64_t cand[kSmallWaves];
#pragma unroll
  for (int t = 0; t < kSmallWaves; ++t) cand[t] = s_cand[t * kSmallN + lane];
  if (kSorted) sort_desc(cand);
  prev = ~0ull;
  int j = 0;
  for (; j < a.n; ++j) {
    const uint64_t b = kSorted ? wave_pop_max(cand) : wave_next_below(cand, prev);
    if (b == 0u) break;
    if (lane == 0) {
      out_id[j] = (int32_t)~(uint32_t)b;
      out_lp[j] = key_logprob(b);
    }
    prev = b;
  }
  for (int k = j + lane; k < a.n; k += 64) {  // fewer entries than n
    out_id[k] = -1;
    out_lp[k] = -INFINITY;
  }
  if (lane == 0) a.status[r] = QS_ROW_OK;
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
    // a count above the capacity is a list the filter truncated (its overflow
    // status); a negative count is bad input
    if (tid == 0) a.status[r] = cnt < 0 ? QS_ROW_BAD_PARAM : QS_ROW_CAND_OVERFLOW;
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
        out_id[j] = (int32_t)~(uint32_t)b;
        out_lp[j] = key_logprob(b);
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
  if (a.n <= kSmallN && a.cap <= (int64_t)kSmallThreads * kSmallPer) {
    if (a.n >= kSortFromN)
      hipLaunchKernelGGL(top_logprobs_small_kernel<true>, dim3((unsigned)B), dim3(kSmallThreads),
                         0, st, a);
    else
      hipLaunchKernelGGL(top_logprobs_small_kernel<false>, dim3((unsigned)B), dim3(kSmallThreads),
                         0, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(top_logprobs_kernel, dim3((unsigned)B), dim3(kTopThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace qs
