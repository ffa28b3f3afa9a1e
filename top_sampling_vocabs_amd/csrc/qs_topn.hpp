// The n most probable tokens of a row, written by the filter/sample kernel
// after the row (page "Sampling 系统设计：从 logits 到可控生成", logprobs
// section: besides the chosen token's log-probability a sampler may return the
// top tokens with theirs). The row's candidate list, just written by the same
// workgroup (ids ascending, float32 probabilities: the final distribution), is
// read back; the order is probability descending with float32 values compared
// exactly, ties by ascending id, as qs_top_logprobs orders it.
//
// The n-th largest probability is found by a radix select over the list (11,
// 11 and 10 bits of the probability's bits, which order like the values: the
// probabilities are not negative), so each level reads the list once; then
// the entries above it and the first of its ties by id (the list is in id
// order) are gathered, at most n <= 64, and wave 0 sorts them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qs_device.hpp"
#include "qs_launch.hpp"
#include "../../include/qs.h"

namespace qs {

constexpr int kTopNMax = 64;

// natural log of a probability as ln 2 (e + log2 m) from frexp and the
// hardware log2 (the formula qs_top_logprobs uses); -inf for 0
__device__ __forceinline__ float topn_logprob(float q) {
  int e;
  const float m = frexpf(q, &e);
  return q > 0.0f ? (float)(((double)e + (double)__log2f(m)) * 0.6931471805599453) : -INFINITY;
}

// All 1024 threads call it after the row; lds: 8,832 bytes of the
// workgroup's LDS, free by then.
__device__ __forceinline__ void top_n_tail(const FilterArgs& a, uint8_t* lds) {
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = a.top_n;
  int32_t* const oi = a.top_ids + (size_t)r * n;
  float* const ol = a.top_lp + (size_t)r * n;
  uint32_t* const hist = reinterpret_cast<uint32_t*>(lds);  // 2048 bins
  uint32_t* const ctl = hist + 2048;                        // 32 words
  uint64_t* const g = reinterpret_cast<uint64_t*>(ctl + 32);  // kTopNMax keys
  // the list's stores (from every wave) have completed before it is read: a
  // workgroup-scope release and a wait for them, then the barrier (the
  // readers are this workgroup's, on this compute unit)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int st = a.status[r];
  const uint32_t L = st == QS_ROW_OK ? (uint32_t)a.cand_count[r] : 0u;  // else no entries
  const int32_t* const ids = a.cand_ids + (size_t)r * a.cand_cap;
  const uint32_t* const qb = reinterpret_cast<const uint32_t*>(a.cand_probs + (size_t)r * a.cand_cap);
  const uint32_t m = L < (uint32_t)n ? L : (uint32_t)n;  // slots filled
  auto key_of = [&](uint32_t i) -> uint64_t {  // probability bits above, ~id below
    return ((uint64_t)qb[i] << 32) | (uint32_t)~ids[i];
  };
  // lists of up to kHeld entries: each thread's probability bits (entries
  // tid + 1024 j) are read once into registers; longer lists are read again
  // at every level
  constexpr int kPer = 16;
  constexpr uint32_t kHeld = (uint32_t)kPer * kThreads;
  const bool held = L <= kHeld;
  uint32_t qv[kPer];
  if (held) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t i = (uint32_t)tid + (uint32_t)kThreads * (uint32_t)j;
      qv[j] = i < L ? qb[i] : 0u;
    }
  }
  if (L <= (uint32_t)n) {
    for (uint32_t i = (uint32_t)tid; i < L; i += kThreads) g[i] = key_of(i);
  } else {
    // radix select: the bits tau of the n-th largest probability, and how
    // many of its ties belong to the top n
    // A level whose boundary bin leaves at most kTopNMax entries at or above
    // it ends the search: those are gathered whole and sorted (held lists)
    uint32_t prefix = 0u, need = (uint32_t)n, thr = 0u, n_ge = 0u;
#pragma unroll 1
    for (int lvl = 0; lvl < 3; ++lvl) {
      const int shift = lvl == 0 ? 21 : (lvl == 1 ? 10 : 0);
      const int width = lvl == 2 ? 10 : 11;
      const uint32_t nb = 1u << width;
      for (uint32_t i = (uint32_t)tid; i < nb; i += kThreads) hist[i] = 0u;
      __syncthreads();
      const int hs = shift + width;  // bits above this level's digit
      auto count = [&](uint32_t b) __attribute__((always_inline)) {
        if (hs >= 32 || (b >> hs) == (prefix >> hs))
          __hip_atomic_fetch_add(hist + ((b >> shift) & (nb - 1u)), 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
      };
      if (held) {
#pragma unroll
        for (int j = 0; j < kPer; ++j)
          if ((uint32_t)tid + (uint32_t)kThreads * (uint32_t)j < L) count(qv[j]);
      } else {
        for (uint32_t i = (uint32_t)tid; i < L; i += kThreads) count(qb[i]);
      }
      __syncthreads();
      if (w == 0) {
        // lane l holds bins nb-1-l*c .. nb-c-l*c (c = nb / 64), from the top
        const uint32_t c = nb >> 6;
        const uint32_t top = nb - 1u - (uint32_t)lane * c;
        uint32_t s = 0u;
        for (uint32_t j = 0; j < c; ++j) s += hist[top - j];
        const uint32_t incl = scan_incl_u32(s);
        const uint32_t excl = incl - s;
        if (excl < need && incl >= need) {  // the crossing lies in this lane's bins
          uint32_t cum = excl, bin = top;
          for (uint32_t j = 0; j < c; ++j) {
            const uint32_t h = hist[top - j];
            if (cum + h >= need) { bin = top - j; break; }
            cum += h;
          }
          ctl[0] = bin;
          ctl[1] = cum;  // entries of this level above the bin
          ctl[3] = hist[bin];  // and in it
        }
      }
      __syncthreads();
      prefix |= uni(ctl[0]) << shift;
      need -= uni(ctl[1]);
      thr = prefix;                              // the bin's lowest bits
      n_ge = (uint32_t)n - need + uni(ctl[3]);   // entries with bits >= thr
      __syncthreads();  // ctl and hist are written again
      if (held && n_ge <= (uint32_t)kTopNMax) break;
    }
    const uint32_t above = (uint32_t)n - need;
    if (tid == 0) ctl[2] = 0u;
    __syncthreads();
    if (held && n_ge <= (uint32_t)kTopNMax) {
      // every entry at or above thr fits: gathered in any order (the sort
      // below puts the lower ids of a tie first, and keeps the first n)
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const uint32_t i = (uint32_t)tid + (uint32_t)kThreads * (uint32_t)j;
        if (i < L && qv[j] >= thr) {
          const uint32_t at = __hip_atomic_fetch_add(ctl + 2, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_WORKGROUP);
          g[at] = ((uint64_t)qv[j] << 32) | (uint32_t)~ids[i];
        }
      }
    } else {
      // the entries above tau, and the first `need` of its ties by list
      // position: each thread a run of consecutive positions
      const uint32_t per = (L + kThreads - 1u) / kThreads;
      const uint32_t p0 = min((uint32_t)tid * per, L), p1 = min(p0 + per, L);
      uint32_t tc = 0u;
      for (uint32_t i = p0; i < p1; ++i) tc += qb[i] == prefix ? 1u : 0u;
      const uint32_t incl = scan_incl_u32(tc);
      if (lane == 63) ctl[4 + w] = incl;  // ctl[4..19]: the 16 waves' tie counts
      __syncthreads();
      uint32_t rank = incl - tc;
      for (int ww = 0; ww < w; ++ww) rank += ctl[4 + ww];
      for (uint32_t i = p0; i < p1; ++i) {
        const uint32_t b = qb[i];
        if (b > prefix) {
          const uint32_t at = __hip_atomic_fetch_add(ctl + 2, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_WORKGROUP);
          g[at] = key_of(i);
        } else if (b == prefix) {
          if (rank < need) g[above + rank] = key_of(i);
          ++rank;
        }
      }
    }
  }
  __syncthreads();
  // wave 0: sort the gathered keys descending (a bitonic network over the 64
  // lanes) and write the first m as the slots
  if (w == 0) {
    const uint32_t ng = L <= (uint32_t)n ? L : max(m, uni(ctl[2]));
    uint64_t k = (uint32_t)lane < ng ? g[lane] : 0ull;
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        const uint64_t o = (uint64_t)__shfl_xor((long long)k, stride, 64);
        const bool lower = (lane & stride) == 0;
        const bool desc = (lane & size) == 0;  // this run ends descending
        const bool take_max = lower == desc;
        k = take_max ? (o > k ? o : k) : (o < k ? o : k);
      }
    }
    if (lane < n) {
      const bool on = (uint32_t)lane < m;
      oi[lane] = on ? (int32_t)~(uint32_t)k : -1;
      ol[lane] = on ? topn_logprob(__uint_as_float((uint32_t)(k >> 32))) : -INFINITY;
    }
  }
}

}  // namespace qs
