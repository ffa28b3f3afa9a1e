// Repetition and presence penalties over each row's history, in place.
//
// Page "Sampling 系统设计：从 logits 到可控生成", repetition-penalty section: the
// penalty depends on the tokens the sequence produced before and belongs in a
// logits processor fed by that history; the page leaves the formula open.
// Taken here: for each distinct token t of the row's history (0 <= t < V),
//   z_t <- (z_t > 0 ? z_t / r : z_t * r) - a
// in float32, each operation rounded (contraction is off in these kernels: no
// multiply is fused with the subtraction after it), stored back in the logits' dtype
// (bfloat16 round to nearest even). Every other logit is untouched, so the
// work is O(history), not O(V): the sampling kernels then read the modified
// row as they read any other.
//
// One workgroup of 1024 threads per row, 4 history entries per thread per
// round with their loads issued together (a history of up to 4096 ids is
// read once and held in registers). A token repeated in the history is
// penalised once: every history entry clears its token's bit in an LDS bitmap
// of the vocabulary, then sets it with an atomic OR; the entry that finds the
// bit clear owns the token and alone rewrites its logit, so no two threads
// write the same element.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qs.h"
#include "qs_aux.hpp"
#include "qs_launch.hpp"

namespace qs {
namespace {

constexpr int kPenThreads = 1024;
constexpr int kPenU = 4;  // history entries per thread per round, their loads issued together
__shared__ uint32_t s_seen[kPenaltyMaxV / 32];  // 128 KB

constexpr int kFreqMax = 4096;  // history length with a frequency penalty (sorted in LDS)
__shared__ int32_t s_sort[kFreqMax];  // 16 KB

__device__ __forceinline__ uint16_t to_bf16_rne(float v) {
  const uint32_t b = __float_as_uint(v);
  if (v != v) return (uint16_t)((b >> 16) | 0x40u);  // NaN stays NaN (quiet)
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

__global__ void __launch_bounds__(kPenThreads) penalty_kernel(PenaltyArgs a) {
#pragma clang fp contract(off)
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int cnt = a.count[r];
  const float rep = a.rep[r], pres = a.pres[r];
  const float freq = a.freq ? a.freq[r] : 0.0f;
  const bool ok = isfinite(rep) && rep > 0.0f && isfinite(pres) && isfinite(freq) &&
                  cnt >= 0 && (int64_t)cnt <= a.hist_cap && (freq == 0.0f || cnt <= kFreqMax);
  if (!ok) {
    if (tid == 0) a.status[r] = QS_ROW_BAD_PARAM;
    return;
  }
  const int32_t* h = a.hist + (size_t)r * a.hist_cap;
  uint8_t* row = a.logits + (size_t)r * a.row_bytes;
  if (freq != 0.0f) {
    // counts: the history sorted ascending in LDS (bitonic; ids outside [0, V)
    // and the padding sort last as INT_MAX); the first entry of each run of
    // equal ids owns its token, and the run's length is its count
    for (int i = tid; i < kFreqMax; i += kPenThreads) {
      const int x = i < cnt ? h[i] : -1;
      s_sort[i] = x >= 0 && x < a.V ? x : INT32_MAX;
    }
    __syncthreads();
    for (int k = 2; k <= kFreqMax; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < kFreqMax; i += kPenThreads) {
          const int l = i ^ j;
          if (l > i) {
            const int x = s_sort[i], y = s_sort[l];
            if ((x > y) == ((i & k) == 0)) {
              s_sort[i] = y;
              s_sort[l] = x;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int i = tid; i < kFreqMax; i += kPenThreads) {
      const int t = s_sort[i];
      if (t == INT32_MAX || (i > 0 && s_sort[i - 1] == t)) continue;
      int lo = i + 1, len = kFreqMax - lo;  // first index past the run of t
      while (len > 0) {
        const int half = len >> 1;
        if (s_sort[lo + half] <= t) {
          lo += half + 1;
          len -= half + 1;
        } else {
          len = half;
        }
      }
      const float n = (float)(lo - i);
      float v;
      if (a.dtype == QS_F32) v = reinterpret_cast<float*>(row)[t];
      else v = __uint_as_float((uint32_t)reinterpret_cast<uint16_t*>(row)[t] << 16);
      v = v > 0.0f ? v / rep : v * rep;
      v = v - pres;
      v = v - freq * n;
      if (a.dtype == QS_F32) reinterpret_cast<float*>(row)[t] = v;
      else reinterpret_cast<uint16_t*>(row)[t] = to_bf16_rne(v);
    }
    if (tid == 0) a.status[r] = QS_ROW_OK;
    return;
  }
  auto load_ids = [&](int i0, int (&t)[kPenU]) {
#pragma unroll
    for (int u = 0; u < kPenU; ++u) {
      const int i = i0 + u * kPenThreads;
      const int x = i < cnt ? h[i] : -1;
      t[u] = x >= 0 && x < a.V ? x : -1;  // -1: nothing to do
    }
  };
  auto clear_bits = [&](const int (&t)[kPenU]) {
#pragma unroll
    for (int u = 0; u < kPenU; ++u)
      if (t[u] >= 0) s_seen[t[u] >> 5] = 0u;
  };
  // claim each id's bit; the owners read, penalise and write back their logits
  auto penalise = [&](int (&t)[kPenU]) {
#pragma unroll
    for (int u = 0; u < kPenU; ++u) {
      if (t[u] >= 0) {
        const uint32_t bit = 1u << (t[u] & 31);
        const uint32_t old = __hip_atomic_fetch_or(&s_seen[t[u] >> 5], bit, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_WORKGROUP);
        if (old & bit) t[u] = -1;  // an earlier entry of the same token owns it
      }
    }
    float v[kPenU];
#pragma unroll
    for (int u = 0; u < kPenU; ++u) {
      v[u] = 0.0f;
      if (t[u] >= 0) {
        if (a.dtype == QS_F32) v[u] = reinterpret_cast<float*>(row)[t[u]];
        else v[u] = __uint_as_float((uint32_t)reinterpret_cast<uint16_t*>(row)[t[u]] << 16);
      }
    }
#pragma unroll
    for (int u = 0; u < kPenU; ++u) {
      if (t[u] >= 0) {
        float x = v[u] > 0.0f ? v[u] / rep : v[u] * rep;
        x = x - pres;
        if (a.dtype == QS_F32) reinterpret_cast<float*>(row)[t[u]] = x;
        else reinterpret_cast<uint16_t*>(row)[t[u]] = to_bf16_rne(x);
      }
    }
  };
  if (cnt <= kPenU * kPenThreads) {  // one round: the ids stay in registers
    int t[kPenU];
    load_ids(tid, t);
    clear_bits(t);
    __syncthreads();
    penalise(t);
  } else {
    for (int i0 = tid; i0 < cnt; i0 += kPenU * kPenThreads) {
      int t[kPenU];
      load_ids(i0, t);
      clear_bits(t);
    }
    __syncthreads();
    for (int i0 = tid; i0 < cnt; i0 += kPenU * kPenThreads) {
      int t[kPenU];
      load_ids(i0, t);
      penalise(t);
    }
  }
  if (tid == 0) a.status[r] = QS_ROW_OK;
}

// Additive logit bias: z_t <- z_t + b for each (t, b) of the row's list with
// 0 <= t < V, in float32, stored in the logits' dtype. The list must name each
// token once: the first phase checks that (bitmap as above; any entry that
// finds its bit already set flags the row) and that every value is finite,
// and only a clean row is modified, so a flagged row is left untouched. A list
// of up to 4096 entries is read once and held in registers, its logit loads
// issued together.
__global__ void __launch_bounds__(kPenThreads) bias_kernel(BiasArgs a) {
#pragma clang fp contract(off)
  __shared__ int s_bad;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int cnt = a.count[r];
  if (cnt < 0 || (int64_t)cnt > a.cap) {
    if (tid == 0) a.status[r] = QS_ROW_BAD_PARAM;
    return;
  }
  const int32_t* ids = a.ids + (size_t)r * a.cap;
  const float* vals = a.vals + (size_t)r * a.cap;
  uint8_t* row = a.logits + (size_t)r * a.row_bytes;
  if (tid == 0) s_bad = 0;
  if (cnt <= kPenU * kPenThreads) {  // one round: ids and values stay in registers
    int t[kPenU];
    float b[kPenU];
#pragma unroll
    for (int u = 0; u < kPenU; ++u) {
      const int i = tid + u * kPenThreads;
      const bool in = i < cnt;
      const int x = in ? ids[i] : -1;
      b[u] = in ? vals[i] : 0.0f;
      t[u] = x >= 0 && x < a.V ? x : -1;
    }
#pragma unroll
    for (int u = 0; u < kPenU; ++u)
      if (t[u] >= 0) s_seen[t[u] >> 5] = 0u;
    __syncthreads();
    bool bad1 = false;
#pragma unroll
    for (int u = 0; u < kPenU; ++u) {
      bad1 = bad1 || !isfinite(b[u]);
      if (t[u] >= 0) {
        const uint32_t bit = 1u << (t[u] & 31);
        const uint32_t old = __hip_atomic_fetch_or(&s_seen[t[u] >> 5], bit, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_WORKGROUP);
        bad1 = bad1 || (old & bit) != 0u;
      }
    }
    if (bad1) s_bad = 1;
    __syncthreads();
    if (s_bad) {
      if (tid == 0) a.status[r] = QS_ROW_BAD_PARAM;
      return;
    }
    float v[kPenU];
#pragma unroll
    for (int u = 0; u < kPenU; ++u) {
      v[u] = 0.0f;
      if (t[u] >= 0) {
        if (a.dtype == QS_F32) v[u] = reinterpret_cast<float*>(row)[t[u]];
        else v[u] = __uint_as_float((uint32_t)reinterpret_cast<uint16_t*>(row)[t[u]] << 16);
      }
    }
#pragma unroll
    for (int u = 0; u < kPenU; ++u) {
      if (t[u] >= 0) {
        const float x = v[u] + b[u];
        if (a.dtype == QS_F32) reinterpret_cast<float*>(row)[t[u]] = x;
        else reinterpret_cast<uint16_t*>(row)[t[u]] = to_bf16_rne(x);
      }
    }
    if (tid == 0) a.status[r] = QS_ROW_OK;
    return;
  }
  for (int i = tid; i < cnt; i += kPenThreads) {
    const int t = ids[i];
    if (t >= 0 && t < a.V) s_seen[t >> 5] = 0u;
  }
  __syncthreads();
  bool bad = false;
  for (int i = tid; i < cnt; i += kPenThreads) {
    const int t = ids[i];
    bad = bad || !isfinite(vals[i]);
    if (t >= 0 && t < a.V) {
      const uint32_t bit = 1u << (t & 31);
      const uint32_t old = __hip_atomic_fetch_or(&s_seen[t >> 5], bit, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_WORKGROUP);
      bad = bad || (old & bit) != 0u;
    }
  }
  if (bad) s_bad = 1;
  __syncthreads();
  if (s_bad) {
    if (tid == 0) a.status[r] = QS_ROW_BAD_PARAM;
    return;
  }
  for (int i = tid; i < cnt; i += kPenThreads) {
    const int t = ids[i];
    if (t < 0 || t >= a.V) continue;
    if (a.dtype == QS_F32) {
      float* const p = reinterpret_cast<float*>(row) + t;
      *p = *p + vals[i];
    } else {
      uint16_t* const p = reinterpret_cast<uint16_t*>(row) + t;
      *p = to_bf16_rne(__uint_as_float((uint32_t)*p << 16) + vals[i]);
    }
  }
  if (tid == 0) a.status[r] = QS_ROW_OK;
}

}  // namespace

hipError_t launch_bias(const BiasArgs& a, int B, hipStream_t st) {
  hipLaunchKernelGGL(bias_kernel, dim3((unsigned)B), dim3(kPenThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_penalty(const PenaltyArgs& a, int B, hipStream_t st) {
  hipLaunchKernelGGL(penalty_kernel, dim3((unsigned)B), dim3(kPenThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace qs
