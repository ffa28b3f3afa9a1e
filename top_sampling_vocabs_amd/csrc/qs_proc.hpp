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
//   - a bitmap of the history's tokens and one of the bias list's tokens;
//   - only where needed, per 128-token block of a bitmap, the count of set
//     bits in the blocks before it (the rank of a set bit is that count plus
//     the set bits below it in its block), and per rank the history count
//     (with a frequency penalty) or the bias.
// A row with only repetition and presence penalties needs the history bitmap
// alone: its table is two barriers and one atomic OR per history entry.
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
constexpr int kBlocks = kWords / 4;     // 128-token blocks
constexpr int kMaxIds = 4096;           // bias entries per row; history entries with a
                                        // frequency penalty
constexpr uint32_t kNoBias = 0x7FC00000u;

// The two LDS regions of a table: the main one (history and bias bitmaps,
// history block prefixes, history counts) and the side one (biases, bias
// block prefixes). Both 16-byte aligned.
constexpr int kMainBytes = kWords * 4 * 2 + kBlocks * 2 + kMaxIds * 4;
constexpr int kSideBytes = kMaxIds * 4 + kBlocks * 2;

struct Table {
  uint32_t* hbits;   // [kWords] history tokens
  uint32_t* bbits;   // [kWords] bias tokens
  uint16_t* hpre;    // [kBlocks] set history bits in the blocks before
  uint32_t* count;   // [kMaxIds] history count per history rank
  uint32_t* bias;    // [kMaxIds] float bits per bias rank
  uint16_t* bpre;    // [kBlocks] set bias bits in the blocks before
};

__device__ __forceinline__ Table table_at(uint8_t* main, uint8_t* side) {
  Table t;
  t.hbits = reinterpret_cast<uint32_t*>(main);
  t.bbits = reinterpret_cast<uint32_t*>(main + kWords * 4);
  t.hpre = reinterpret_cast<uint16_t*>(main + kWords * 8);
  t.count = reinterpret_cast<uint32_t*>(main + kWords * 8 + kBlocks * 2);
  t.bias = reinterpret_cast<uint32_t*>(side);
  t.bpre = reinterpret_cast<uint16_t*>(side + kMaxIds * 4);
  return t;
}

// rank of token id among the set bits of a bitmap (the bit must be set)
__device__ __forceinline__ uint32_t rank_in(const uint32_t* bits, const uint16_t* pre,
                                            uint32_t id) {
  const uint32_t blk = id >> 7;
  const uint4 q = *reinterpret_cast<const uint4*>(bits + blk * 4u);
  const uint32_t wi = (id >> 5) & 3u;
  const uint32_t below = (1u << (id & 31u)) - 1u;
  uint32_t c = (uint32_t)pre[blk];
  c += (uint32_t)__popc(wi > 0u ? q.x : q.x & below);
  c += wi >= 1u ? (uint32_t)__popc(wi > 1u ? q.y : q.y & below) : 0u;
  c += wi >= 2u ? (uint32_t)__popc(wi > 2u ? q.z : q.z & below) : 0u;
  c += wi >= 3u ? (uint32_t)__popc(q.w & below) : 0u;
  return c;
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

// Per-row processor parameters, read by every thread (uniform).
struct RowParams {
  int hcnt, bcnt;
  float rep, pres, freq;
  bool ok;         // the arguments pass the processors' checks (biases aside)
  bool has_h;      // history entries to apply
  bool has_b;      // bias entries to apply
  bool need_cnt;   // a frequency penalty: history counts per token
};

// (P == 1: the call has no frequency penalties and no bias list, which the
// compiler then knows)
template <int P>
__device__ __forceinline__ RowParams row_params(const FilterArgs& a, int r) {
  RowParams p;
  p.hcnt = a.p_hist ? a.p_hist_count[r] : 0;
  p.bcnt = a.p_bias_ids ? a.p_bias_count[r] : 0;
  p.rep = a.p_hist ? a.p_rep[r] : 1.0f;
  p.pres = a.p_hist ? a.p_pres[r] : 0.0f;
  p.freq = (a.p_hist && a.p_freq) ? a.p_freq[r] : 0.0f;
  p.ok = isfinite(p.rep) && p.rep > 0.0f && isfinite(p.pres) && isfinite(p.freq) &&
         p.hcnt >= 0 && (int64_t)p.hcnt <= a.p_hist_cap &&
         (p.freq == 0.0f || p.hcnt <= kMaxIds) && p.bcnt >= 0 &&
         (int64_t)p.bcnt <= a.p_bias_cap && p.bcnt <= kMaxIds;
  p.has_h = p.ok && p.hcnt > 0;
  p.has_b = p.ok && p.bcnt > 0;
  p.need_cnt = p.has_h && p.freq != 0.0f;
  if constexpr (P == 1) {
    p.freq = 0.0f;
    p.bcnt = 0;
    p.has_b = false;
    p.need_cnt = false;
  }
  return p;
}

// Table build in three parts, each ended by a barrier of the caller's
// (all threads call each part; `flag` is one LDS word that part 1 clears and
// part 2 sets for a bad row).
//   1. clear: both bitmaps;
//   2. mark: the counts cleared, one atomic OR per history / bias entry (a
//      bias token listed twice, or a non-finite bias, flags the row);
//   3. ranks (only with a frequency penalty or a bias list): block prefixes
//      of both bitmaps in one block scan, a barrier, then the counts and
//      biases by rank. Ends with its own barrier.
// (part 1 needs no row parameter, so it does not wait for them)
__device__ __forceinline__ void build_clear(const FilterArgs& a, const Table& t, int tid,
                                            uint32_t* flag) {
  const int Wc = (((a.V + 31) >> 5) + 3) & ~3;  // whole 4-word blocks
  for (int i = tid; i < Wc; i += 1024) {
    t.hbits[i] = 0u;
    t.bbits[i] = 0u;
  }
  if (tid == 0) *flag = 0u;
}

// The first two history entries of a thread (entries tid and tid + 1024 of
// the row, -1 past the history's capacity), requested before the table is
// cleared so that their latency hides behind it.
struct HistIds {
  int32_t v[2];
};

__device__ __forceinline__ HistIds prefetch_ids(const FilterArgs& a, int r, int tid) {
  HistIds q;
  const int32_t* const h = a.p_hist ? a.p_hist + (size_t)r * a.p_hist_cap : nullptr;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t i = tid + 1024 * j;
    q.v[j] = (h && i < a.p_hist_cap) ? h[i] : -1;
  }
  return q;
}

__device__ __forceinline__ void build_mark(const FilterArgs& a, int r, const RowParams& p,
                                           const Table& t, int tid, uint32_t* flag,
                                           const HistIds& pre) {
  const int V = a.V;
  if (p.need_cnt)
    for (int i = tid; i < kMaxIds; i += 1024) t.count[i] = 0u;
  if (p.has_h) {
    const int32_t* const h = a.p_hist + (size_t)r * a.p_hist_cap;
    for (int i = tid; i < p.hcnt; i += 1024) {
      const int x = i < 2048 ? pre.v[i >> 10] : h[i];
      if (x >= 0 && x < V)
        __hip_atomic_fetch_or(t.hbits + (x >> 5), 1u << (x & 31), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  if (p.has_b) {
    const int32_t* const bi = a.p_bias_ids + (size_t)r * a.p_bias_cap;
    const float* const bv = a.p_bias_vals + (size_t)r * a.p_bias_cap;
    bool bad = false;
    for (int i = tid; i < p.bcnt; i += 1024) {
      const int x = bi[i];
      bad = bad || !isfinite(bv[i]);
      if (x >= 0 && x < V) {
        const uint32_t bit = 1u << (x & 31);
        const uint32_t old = __hip_atomic_fetch_or(t.bbits + (x >> 5), bit, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_WORKGROUP);
        bad = bad || (old & bit) != 0u;  // listed twice
      }
    }
    if (bad) *flag = 1u;
  }
}

__device__ __forceinline__ void build_ranks(const FilterArgs& a, int r, const RowParams& p,
                                            const Table& t, int tid, uint32_t* wsum) {
  // thread i covers blocks 2i and 2i + 1; both bitmaps' counts in 16-bit
  // fields (each total is at most kMaxIds)
  const int nb = (((a.V + 31) >> 5) + 3) >> 2;
  const int b0 = 2 * tid;
  uint32_t s0 = 0u, s1 = 0u;
  auto cnt4 = [&](const uint32_t* bits, int b) -> uint32_t {
    const uint4 q = *reinterpret_cast<const uint4*>(bits + 4 * b);
    return (uint32_t)(__popc(q.x) + __popc(q.y) + __popc(q.z) + __popc(q.w));
  };
  if (b0 < nb) {
    if (p.need_cnt) s0 += cnt4(t.hbits, b0);
    if (p.has_b) s0 += cnt4(t.bbits, b0) << 16;
  }
  if (b0 + 1 < nb) {
    if (p.need_cnt) s1 += cnt4(t.hbits, b0 + 1);
    if (p.has_b) s1 += cnt4(t.bbits, b0 + 1) << 16;
  }
  const uint32_t mine = s0 + s1;
  const int lane = tid & 63, wv = tid >> 6;
  const uint32_t incl = scan_incl_u32(mine);
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  uint32_t base = 0u;
  for (int k = 0; k < 16; ++k) base += k < wv ? wsum[k] : 0u;
  const uint32_t e0 = base + incl - mine, e1 = e0 + s0;
  if (b0 < nb) {
    if (p.need_cnt) t.hpre[b0] = (uint16_t)(e0 & 0xFFFFu);
    if (p.has_b) t.bpre[b0] = (uint16_t)(e0 >> 16);
  }
  if (b0 + 1 < nb) {
    if (p.need_cnt) t.hpre[b0 + 1] = (uint16_t)(e1 & 0xFFFFu);
    if (p.has_b) t.bpre[b0 + 1] = (uint16_t)(e1 >> 16);
  }
  __syncthreads();
  const int V = a.V;
  if (p.need_cnt) {
    const int32_t* const h = a.p_hist + (size_t)r * a.p_hist_cap;
    for (int i = tid; i < p.hcnt; i += 1024) {
      const int x = h[i];
      if (x >= 0 && x < V)
        __hip_atomic_fetch_add(t.count + rank_in(t.hbits, t.hpre, (uint32_t)x), 1u,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  if (p.has_b) {
    const int32_t* const bi = a.p_bias_ids + (size_t)r * a.p_bias_cap;
    const float* const bv = a.p_bias_vals + (size_t)r * a.p_bias_cap;
    for (int i = tid; i < p.bcnt; i += 1024) {
      const int x = bi[i];
      if (x >= 0 && x < V) t.bias[rank_in(t.bbits, t.bpre, (uint32_t)x)] = __float_as_uint(bv[i]);
    }
  }
  __syncthreads();
}

// The edited raw bits of token id (raw bits `raw`) whose history bit is hb
// and bias bit bb (at least one set).
template <int DT>
__device__ __forceinline__ uint32_t edit_token(const Table& t, const RowParams& p, uint32_t id,
                                               uint32_t raw, bool hb, bool bb) {
  const uint32_t n = hb ? (p.need_cnt ? t.count[rank_in(t.hbits, t.hpre, id)] : 1u) : 0u;
  const uint32_t bv = bb ? t.bias[rank_in(t.bbits, t.bpre, id)] : kNoBias;
  return edit<DT>(raw, n, bv, p.rep, p.pres, p.freq);
}

}  // namespace proc
}  // namespace qs
