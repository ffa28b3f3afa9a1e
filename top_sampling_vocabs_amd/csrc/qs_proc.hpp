// Logit processors applied inside the filter kernel (page "Sampling 系统设计：从
// logits 到可控生成", repetition-penalty and LogitsProcessor sections: the
// history-dependent processors edit the logits before the selection). The
// edited values are those the in-place processor kernels would store: for each
// distinct in-range history token t,
//   z_t <- (z_t > 0 ? z_t / r : z_t * r) - a   [- f * n_t]
// in float32 with every operation rounded, stored in the logits' dtype, then
// for each (t, b) of the bias list z_t <- z_t + b, stored again. Here they are
// never stored to the caller's logits: the kernel patches its own copy of the
// values (registers, or a workspace row).
//
// Per row, a table in LDS answers "is token t edited, and how" in O(1):
//   - a bitmap of the row's tokens with one bit per edited token;
//   - per bitmap word, the count of set bits in the words before it (so the
//     rank of a set bit is that count plus the set bits below it in its word);
//   - per rank: the token's count in the history (0: not in it) and its bias
//     (NaN: none; a bias must be finite).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qs_device.hpp"
#include "qs_launch.hpp"
#include "../../include/qs.h"

namespace qs {
namespace proc {

constexpr int kMaxV = 155648;          // tokens a table covers
constexpr int kWords = kMaxV / 32;      // bitmap words
constexpr int kMaxIds = 4096;           // distinct edited tokens per row
constexpr int kFreqMaxHistory = 4096;   // history length allowed with a frequency penalty
constexpr uint32_t kNoBias = 0x7FC00000u;

// Table bytes: bitmap, 16-bit word prefixes, 32-bit counts (the biases live
// in a separate region of kMaxIds floats).
constexpr int kBytes = kWords * 4 + kWords * 2 + kMaxIds * 4;

struct Table {
  uint32_t* bits;      // [kWords]
  uint16_t* before;    // [kWords]: set bits in the words before
  uint32_t* count;     // [kMaxIds]
  uint32_t* bias;      // [kMaxIds] float bits, kNoBias when none
};

__device__ __forceinline__ Table table_at(uint8_t* base, uint32_t* bias_region) {
  Table t;
  t.bits = reinterpret_cast<uint32_t*>(base);
  t.before = reinterpret_cast<uint16_t*>(base + kWords * 4);
  t.count = reinterpret_cast<uint32_t*>(base + kWords * 6);
  t.bias = bias_region;
  return t;
}

// rank of token id among the edited tokens (the bit must be set)
__device__ __forceinline__ uint32_t rank_of(const Table& t, uint32_t id) {
  const uint32_t wd = t.bits[id >> 5];
  return (uint32_t)t.before[id >> 5] + (uint32_t)__popc(wd & ((1u << (id & 31u)) - 1u));
}

__device__ __forceinline__ uint16_t to_bf16(float v) {
  const uint32_t b = __float_as_uint(v);
  if (v != v) return (uint16_t)((b >> 16) | 0x40u);  // NaN stays NaN (quiet)
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// The edited raw bits (bf16 in the low 16 bits, or fp32) of a token with raw
// bits `raw`, history count n (0: not in the history) and bias bits bb.
template <int DT>
__device__ __forceinline__ uint32_t edit(uint32_t raw, uint32_t n, uint32_t bb, float rep,
                                         float pres, float freq) {
#pragma clang fp contract(off)
  uint32_t out = raw;
  if (n) {
    float v = DT == 1 ? __uint_as_float(raw << 16) : __uint_as_float(raw);
    v = v > 0.0f ? v / rep : v * rep;
    v = v - pres;
    if (freq != 0.0f) v = v - freq * (float)n;
    out = DT == 1 ? (uint32_t)to_bf16(v) : __float_as_uint(v);
  }
  if (bb != kNoBias) {
    const float v = (DT == 1 ? __uint_as_float(out << 16) : __uint_as_float(out)) +
                    __uint_as_float(bb);
    out = DT == 1 ? (uint32_t)to_bf16(v) : __float_as_uint(v);
  }
  return out;
}

// Per-row processor parameters, read by every thread.
struct RowParams {
  int hcnt, bcnt;
  float rep, pres, freq;
  bool ok;
};

__device__ __forceinline__ RowParams row_params(const FilterArgs& a, int r) {
  RowParams p;
  p.hcnt = a.p_hist ? a.p_hist_count[r] : 0;
  p.bcnt = a.p_bias_ids ? a.p_bias_count[r] : 0;
  p.rep = a.p_hist ? a.p_rep[r] : 1.0f;
  p.pres = a.p_hist ? a.p_pres[r] : 0.0f;
  p.freq = (a.p_hist && a.p_freq) ? a.p_freq[r] : 0.0f;
  p.ok = isfinite(p.rep) && p.rep > 0.0f && isfinite(p.pres) && isfinite(p.freq) &&
         p.hcnt >= 0 && (int64_t)p.hcnt <= a.p_hist_cap &&
         (p.freq == 0.0f || p.hcnt <= kFreqMaxHistory) && p.bcnt >= 0 &&
         (int64_t)p.bcnt <= a.p_bias_cap;
  return p;
}

// Build the table of row r with all 1024 threads (every thread must call it;
// it holds barriers). `flag` is one LDS word of scratch. Returns false, the
// same in every thread, when the row's processor arguments are invalid: a
// non-finite bias, a token listed twice in the bias list, or more than
// kMaxIds distinct edited tokens.
__device__ __forceinline__ bool build(const FilterArgs& a, int r, int tid, const RowParams& p,
                                      const Table& t, uint32_t* flag, uint32_t* wsum) {
  const int V = a.V;
  const int W = (V + 31) >> 5;
  const int32_t* const h = a.p_hist ? a.p_hist + (size_t)r * a.p_hist_cap : nullptr;
  const int32_t* const bi = a.p_bias_ids ? a.p_bias_ids + (size_t)r * a.p_bias_cap : nullptr;
  const float* const bv = a.p_bias_ids ? a.p_bias_vals + (size_t)r * a.p_bias_cap : nullptr;
  for (int i = tid; i < W; i += 1024) t.bits[i] = 0u;
  for (int i = tid; i < kMaxIds; i += 1024) {
    t.count[i] = 0u;
    t.bias[i] = kNoBias;
  }
  if (tid == 0) *flag = 0u;
  __syncthreads();
  for (int i = tid; i < p.hcnt; i += 1024) {
    const int x = h[i];
    if (x >= 0 && x < V)
      __hip_atomic_fetch_or(t.bits + (x >> 5), 1u << (x & 31), __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  bool bad = false;
  for (int i = tid; i < p.bcnt; i += 1024) {
    const int x = bi[i];
    bad = bad || !isfinite(bv[i]);
    if (x >= 0 && x < V)
      __hip_atomic_fetch_or(t.bits + (x >> 5), 1u << (x & 31), __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  if (bad) *flag = 1u;
  __syncthreads();
  // word prefixes: each thread sums a run of up to 5 words, a block scan of
  // the runs, then each thread writes its words' prefixes
  constexpr int kPer = (kWords + 1023) / 1024;
  const int w0 = tid * kPer;
  uint32_t mine = 0u;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (w0 + j < W) mine += (uint32_t)__popc(t.bits[w0 + j]);
  const int lane = tid & 63, wv = tid >> 6;
  const uint32_t incl = scan_incl_u32(mine);
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  uint32_t base = 0u, total = 0u;
  for (int k = 0; k < 16; ++k) {
    const uint32_t s = wsum[k];
    base += k < wv ? s : 0u;
    total += s;
  }
  uint32_t run = base + incl - mine;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (w0 + j < W) {
      t.before[w0 + j] = (uint16_t)min(run, 0xFFFFu);
      run += (uint32_t)__popc(t.bits[w0 + j]);
    }
  }
  __syncthreads();
  if (total > (uint32_t)kMaxIds) return false;
  for (int i = tid; i < p.hcnt; i += 1024) {
    const int x = h[i];
    if (x >= 0 && x < V)
      __hip_atomic_fetch_add(t.count + rank_of(t, (uint32_t)x), 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  bad = false;
  for (int i = tid; i < p.bcnt; i += 1024) {
    const int x = bi[i];
    if (x >= 0 && x < V) {
      uint32_t expect = kNoBias;
      const bool won = __hip_atomic_compare_exchange_strong(
          t.bias + rank_of(t, (uint32_t)x), &expect, __float_as_uint(bv[i]), __ATOMIC_RELAXED,
          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      bad = bad || !won;  // listed twice
    }
  }
  if (bad) *flag = 1u;
  __syncthreads();
  return *flag == 0u;
}

}  // namespace proc
}  // namespace qs
