// Row access for the filter kernels: the pipelined single pass over a wave's
// slice (sigma-truncation compaction into the LDS pool, legal counts, NaN
// checks, optional background mass), re-walks of the full row, and walks of
// the candidate pool.
#pragma once

#include "qs_device.hpp"

namespace qs {

// Per-wave view of one row.
struct Slice {
  const uint8_t* row;   // row start (16-byte aligned)
  const uint8_t* mrow;  // packed legal bits of the row, or null (all legal)
  int V;
  int wb, we;           // this wave's token range [wb, we); wb is a multiple of 32
};

// Raw bits of the 8 tokens a lane handles per step.
template <int DT> struct Raw;
template <> struct Raw<0> {  // fp32
  uint32_t r[8];
  __device__ __forceinline__ uint32_t bits(int j) const { return r[j]; }
};
template <> struct Raw<1> {  // bf16: pairs, element 2p in the low half of r[p]
  uint32_t r[4];
  __device__ __forceinline__ uint32_t bits(int j) const {
    return (r[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
  }
};

// 32 zero bytes: what a lane whose chunk is not a full chunk of its slice reads,
// so that every lane issues the same loads from a valid address.
static __constant__ __align__(16) uint4 kZeroChunk[2] = {};

template <int DT>
__device__ __forceinline__ const uint8_t* chunk_ptr(const uint8_t* row, int e) {
  return row + (size_t)e * (DT == 0 ? 4 : 2);
}

template <int DT>
__device__ __forceinline__ void load_vec(const uint8_t* ptr, Raw<DT>& o) {
  if constexpr (DT == 0) {
    const uint4* p = reinterpret_cast<const uint4*>(ptr);
    uint4 a = p[0], b = p[1];
    o.r[0] = a.x; o.r[1] = a.y; o.r[2] = a.z; o.r[3] = a.w;
    o.r[4] = b.x; o.r[5] = b.y; o.r[6] = b.z; o.r[7] = b.w;
  } else {
    uint4 a = *reinterpret_cast<const uint4*>(ptr);
    o.r[0] = a.x; o.r[1] = a.y; o.r[2] = a.z; o.r[3] = a.w;
  }
}

// Tokens e.. of a chunk that ends past V (only the last chunk of a row whose
// length is not a multiple of 8), loaded one by one; missing tokens read 0.
template <int DT>
__device__ __forceinline__ void load_tail(const uint8_t* row, int e, int V, Raw<DT>& o) {
  if constexpr (DT == 0) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(row) + e;
#pragma unroll
    for (int j = 0; j < 8; ++j) o.r[j] = (e + j < V) ? p[j] : 0u;
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(row) + e;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t lo = (e + 2 * j < V) ? (uint32_t)p[2 * j] : 0u;
      uint32_t hi = (e + 2 * j + 1 < V) ? (uint32_t)p[2 * j + 1] : 0u;
      o.r[j] = lo | (hi << 16);
    }
  }
}

// Number of steps (512 tokens) in a slice.
__device__ __forceinline__ int slice_steps(const Slice& s) {
  return s.we > s.wb ? (s.we - s.wb + kStep - 1) / kStep : 0;
}

// Pipelined reader of a wave's slice. Every step issues the same load
// instructions (a lane outside the slice, or on the one ragged chunk at the row
// end, reads a zero chunk instead and its legal bits are clipped), and a slot
// is refilled only after its data has been consumed, so each load writes its
// slot registers directly and the loads of D steps stay in flight.
template <int DT, int D>
struct RowReader {
  const Slice& s;
  int lane, n;
  Raw<DT> ring[D];
  uint32_t mring[D];
  Raw<DT> tail;     // the ragged chunk at the row end (only its lane uses it)
  int tail_e;       // its first token, or -1 (wave-uniform)

  __device__ __forceinline__ RowReader(const Slice& sl, int ln) : s(sl), lane(ln) {
    n = uni(slice_steps(s));
    tail_e = -1;
    if (n > 0 && s.we == s.V && (s.V & 7)) {
      const int e_last = s.V & ~7;
      if (lane == ((e_last - s.wb) & (kStep - 1)) / kChunk) {
        load_tail<DT>(s.row, e_last, s.V, tail);
      }
      tail_e = e_last;
    }
  }
  __device__ __forceinline__ int first(int st) const {
    return s.wb + st * kStep + lane * kChunk;
  }
  // Load step st (any st >= 0; steps past the end read the slice start). The
  // loaded values are not touched here: clipping happens at fetch time.
  __device__ __forceinline__ void issue(int st, int slot) {
    const int e = first(st);
    const uint8_t* dp = chunk_ptr<DT>(s.row, e);
    int em = e;
    if (st >= n - 1) {  // keep every address valid
      if (e + kChunk > s.we) dp = reinterpret_cast<const uint8_t*>(kZeroChunk);
      if (e >= s.we) em = s.wb;  // the mask byte of any token below V is in the row
    }
    load_vec<DT>(dp, ring[slot]);
    mring[slot] = s.mrow ? (uint32_t)s.mrow[em >> 3] : 0xFFu;
  }
  // Data for step st held in slot: legal bits clipped to the slice, and the
  // ragged chunk substituted.
  __device__ __forceinline__ void fetch(int st, int slot, Raw<DT>& raw, uint32_t& mb) const {
    raw = ring[slot];
    mb = mring[slot];
    if (st >= n - 1) {
      const int e = first(st);
      if (e + kChunk > s.we) {
        if (e < s.we) {
          mb &= (1u << (s.we - e)) - 1u;
          if (tail_e >= 0 && e == tail_e) raw = tail;
        } else {
          mb = 0u;
        }
      }
    }
  }
};

// Stand-in for RowReader where the row is held in registers instead.
template <int DT>
struct NoReader {
  int n = 0;
  __device__ __forceinline__ NoReader(const Slice&, int) {}
  __device__ __forceinline__ void issue(int, int) {}
  __device__ __forceinline__ void fetch(int, int, Raw<DT>&, uint32_t& mb) const { mb = 0u; }
  __device__ __forceinline__ int first(int) const { return 0; }
};

// Walk a slice in id order with a D-deep prefetch; f(raw, mb, e) per step.
template <int DT, int D, class F>
__device__ __forceinline__ void stream_slice(const Slice& s, int lane, F&& f) {
  RowReader<DT, D> rd(s, lane);
  const int n = rd.n;
#pragma unroll
  for (int i = 0; i < D; ++i)
    if (i < n) rd.issue(i, i);
  for (int s0 = 0; s0 < n; s0 += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int st = s0 + i;
      if (st < n) {
        Raw<DT> raw;
        uint32_t mb;
        rd.fetch(st, i, raw, mb);
        f(raw, mb, rd.first(st));
        if (st + D < n) rd.issue(st + D, i);
      }
    }
  }
}

// Walk the row in id order: f(key[8], id[8], vm) with vm bit j set iff token
// id[j] is legal and finite (with NEGINF_TOO: legal).
template <int DT, bool NEGINF_TOO = false, int D = 2, class F>
__device__ __forceinline__ void walk_row(const Slice& s, int lane, F&& f) {
  using K = Keys<DT>;
  stream_slice<DT, D>(s, lane, [&](const Raw<DT>& raw, uint32_t mb, int e) {
    uint32_t key[8], id[8];
    uint32_t vm = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      id[j] = (uint32_t)(e + j);
      key[j] = K::of(raw.bits(j));
      bool ok = (mb >> j) & 1u;
      if constexpr (!NEGINF_TOO) ok = ok && key[j] > K::kNegInf && key[j] < K::kPosInf;
      vm |= (ok ? 1u : 0u) << j;
    }
    f(key, id, vm);
  });
}

// Walk this wave's candidate pool in order (which is id order). Entries hold
// raw bits and the id relative to the slice start.
template <int DT, class F>
__device__ __forceinline__ void walk_pool(const typename PoolLayout<DT>::KeyT* pk,
                                          const uint16_t* pid, int cnt, uint32_t base_id,
                                          int lane, F&& f) {
  using K = Keys<DT>;
  for (int base = 0; base < cnt; base += kStep) {
    const int q = base + lane * kChunk;
    uint32_t key[8], id[8];
    uint32_t vm = 0;
    if (q + kChunk <= cnt) {
      if constexpr (DT == 0) {
        uint4 a = *reinterpret_cast<const uint4*>(pk + q);
        uint4 b = *reinterpret_cast<const uint4*>(pk + q + 4);
        key[0] = a.x; key[1] = a.y; key[2] = a.z; key[3] = a.w;
        key[4] = b.x; key[5] = b.y; key[6] = b.z; key[7] = b.w;
      } else {
        uint4 a = *reinterpret_cast<const uint4*>(pk + q);
        key[0] = a.x & 0xFFFFu; key[1] = a.x >> 16; key[2] = a.y & 0xFFFFu; key[3] = a.y >> 16;
        key[4] = a.z & 0xFFFFu; key[5] = a.z >> 16; key[6] = a.w & 0xFFFFu; key[7] = a.w >> 16;
      }
      uint4 c = *reinterpret_cast<const uint4*>(pid + q);
      id[0] = c.x & 0xFFFFu; id[1] = c.x >> 16; id[2] = c.y & 0xFFFFu; id[3] = c.y >> 16;
      id[4] = c.z & 0xFFFFu; id[5] = c.z >> 16; id[6] = c.w & 0xFFFFu; id[7] = c.w >> 16;
      vm = 0xFFu;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bool ok = q + j < cnt;
        key[j] = ok ? (uint32_t)pk[q + j] : 0u;
        id[j] = ok ? (uint32_t)pid[q + j] : 0u;
        vm |= (ok ? 1u : 0u) << j;
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      key[j] = K::of(key[j]);
      id[j] += base_id;
    }
    f(key, id, vm);
  }
}

// ---------------------------------------------------------------------------
// Candidate extraction: lane holds candidate bits cb (bit j = token e + j) and
// the raw bits of its 8 tokens; append them, in id order, to this wave's pool
// at pool_cnt (entries past the capacity are counted, not stored). Returns
// the new count (every lane gets the same value).
template <int DT>
__device__ __forceinline__ uint32_t append_pool(uint32_t cb, const Raw<DT>& raw,
                                                uint32_t e_local, uint32_t pool_cnt,
                                                typename PoolLayout<DT>::KeyT* pk,
                                                uint16_t* pid) {
  using KeyT = typename PoolLayout<DT>::KeyT;
  constexpr uint32_t kCap = (uint32_t)PoolLayout<DT>::kPerWave;
  const uint32_t c = (uint32_t)__popc(cb);
  const uint64_t any = ballot(c != 0u);
  if (!any) return pool_cnt;
  uint32_t excl, total;
  if (!ballot(c > 1u)) {  // at most one candidate per lane: one ballot
    excl = count_below(any);
    total = (uint32_t)__popcll(any);
  } else {                // DPP prefix of the per-lane counts
    const uint32_t incl = scan_incl_u32(c);
    excl = incl - c;
    total = readlane_u32(incl, 63);
  }
  // entries past the capacity overwrite the last slot: an overflowing pool is
  // never read (the row takes the full-row path)
  uint32_t pos = pool_cnt + excl;
  while (ballot(cb != 0u)) {
    if (cb) {
      const uint32_t j = (uint32_t)__builtin_ctz(cb);
      cb &= cb - 1u;
      const uint32_t q = min(pos, kCap - 1u);
      pk[q] = (KeyT)raw_of<DT>(raw, j);
      pid[q] = (uint16_t)(e_local + j);
      ++pos;
    }
  }
  return pool_cnt + total;
}

// Candidate extraction: lane holds candidate bits cb (bit j = token e + j) and
// the raw bits of its 8 tokens; append them, in id order, to this wave's pool
// at pool_cnt. Returns the new count (every lane gets the same value).
template <int DT>
__device__ __forceinline__ uint32_t raw_of(const Raw<DT>& raw, uint32_t j) {
  if constexpr (DT == 1) {
    uint64_t lo = ((uint64_t)raw.r[1] << 32) | raw.r[0];
    uint64_t hi = ((uint64_t)raw.r[3] << 32) | raw.r[2];
    uint64_t v = (j & 4u) ? hi : lo;
    return (uint32_t)(v >> ((j & 3u) * 16u)) & 0xFFFFu;
  } else {
    uint32_t a = (j & 1u) ? raw.r[1] : raw.r[0];
    uint32_t b = (j & 1u) ? raw.r[3] : raw.r[2];
    uint32_t c = (j & 1u) ? raw.r[5] : raw.r[4];
    uint32_t d = (j & 1u) ? raw.r[7] : raw.r[6];
    uint32_t ab = (j & 2u) ? b : a;
    uint32_t cd = (j & 2u) ? d : c;
    return (j & 4u) ? cd : ab;
  }
}

}  // namespace qs
