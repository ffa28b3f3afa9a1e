// Chunked first pass of the filter for bf16 rows: layout of the caller's
// workspace, the pass's arguments, and the constants its launcher and the
// per-row merge share.
//
// A row is cut into segments of kSegTokens tokens (one wave's slice) and
// chunks of four segments, scanned by one workgroup of kThreads threads (page
// "Qrita", overall framework: truncation, then selection on the small
// candidate set; here the truncation runs over the whole GPU, every compute
// unit streaming chunks of many rows). Every wave computes the row's
// sigma-truncation threshold from the same strided sample of the row (page
// "Qrita", key design 1), then writes per segment
//  - its candidates: legal tokens at or above the threshold, in token-id
//    order, as (bf16 bits << 16 | offset in the segment);
//  - a summary: candidate and legal counts, a flag for a negative NaN, and
//    for greedy rows the largest key and the lowest id holding it (a legal
//    +inf or positive NaN shows up among the candidates, or as the greedy
//    maximum);
// and per chunk, for rows whose top-p cut needs it, the exact mass of its
// legal tokens below the threshold (a histogram with one bin per bf16 value).
// The merge then settles each row from its segments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qs {
namespace chunk {

constexpr int kThreads = 256;                    // one chunk workgroup: 4 wave64s
constexpr int kWaves = kThreads / 64;
constexpr int kSteps = 8;                        // 512-token steps per segment
constexpr int kSegTokens = kSteps * 512;         // tokens per segment (one wave's slice)
constexpr int kTokens = kWaves * kSegTokens;     // 16384 tokens per chunk
constexpr int kSegCap = 896;                     // candidate entries per segment
constexpr int kSampleRuns = 16;                  // strided sample: 16 runs of 32 tokens
constexpr int kMaxSegs = 256;                    // segments per row the merge reads at once
constexpr int kMaxChunks = kMaxSegs / kWaves;

// Background histogram (rows whose top-p cut needs the mass below the
// threshold), per sign: bins 0 .. 15 for magnitudes below 2^-12 (a lump), one
// bin per bf16 value of magnitude in [2^-12, 512) (bins 16 .. 16 + kBgExact -
// 1, so that every run of 16 values of a binade starts on a 64-byte line), and
// bin 16 + kBgExact for 512 and above (infinities and NaN among them).
constexpr uint32_t kBgMagLo = 0x3980u;           // magnitude bits of 2^-12
constexpr uint32_t kBgExact = 21u * 128u;        // 21 binades of exact values
constexpr uint32_t kBgTop = 16u + kBgExact;
constexpr uint32_t kBgSide = kBgTop + 16u;       // bins per sign (a multiple of 16)
constexpr int kBgBins = 2 * (int)kBgSide;
static_assert(kBgMagLo + kBgExact == 0x4400u, "the upper lump starts at 512");

// flags of a segment summary / chunk mass
constexpr uint32_t kOverflow = 1u;     // more candidates than kSegCap: none written
constexpr uint32_t kNegNaN = 2u;       // a negative NaN in the segment (legal or not)
constexpr uint32_t kBgInexact = 4u;    // background mass not exact (lumped values)

// Threshold codes besides bf16 bits (the bits field is 16 bits wide).
constexpr uint32_t kThrNone = 0x10000u;  // no candidates (greedy rows, bad parameters)
constexpr uint32_t kThrAll = 0x20000u;   // every legal finite token is a candidate

struct alignas(16) SegSummary {
  uint32_t cand;       // candidate entries written (0 on overflow)
  uint32_t n_legal;    // legal tokens
  uint32_t flags;
  uint32_t pad0;
  int32_t gmax;        // greedy rows: largest order key of a legal token (-32768 if none)
  uint32_t gid;        // greedy rows: lowest id holding gmax (0xFFFFFFFF if none)
  uint32_t thr;        // threshold: bf16 bits of its value, kThrNone or kThrAll
  uint32_t n_cand;     // candidates found (may exceed kSegCap)
};
static_assert(sizeof(SegSummary) == 32, "segment summary layout");

struct alignas(16) ChunkMass {
  double m_bg;         // sum exp((z - v_t) / T) over legal tokens below v_t
  double err;          // bound on its error (lumped values)
  uint32_t flags;      // kBgInexact
  uint32_t pad[3];
};
static_assert(sizeof(ChunkMass) == 32, "chunk mass layout");

inline int chunks_for(int64_t V) { return (int)((V + kTokens - 1) / kTokens); }

// Workspace of B rows: segment summaries [B][4S], chunk masses [B][S],
// candidates [B][4S][kSegCap] (each part 256-byte aligned).
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t seg_bytes(int64_t B, int64_t V) {
  return align256((size_t)B * (size_t)chunks_for(V) * kWaves * sizeof(SegSummary));
}
inline size_t mass_bytes(int64_t B, int64_t V) {
  return align256((size_t)B * (size_t)chunks_for(V) * sizeof(ChunkMass));
}
inline size_t workspace_bytes(int64_t B, int64_t V) {
  return seg_bytes(B, V) + mass_bytes(B, V) +
         (size_t)B * (size_t)chunks_for(V) * kWaves * kSegCap * 4u;
}

// Sample of a row: kSampleRuns runs of 32 tokens, `stride` tokens apart (a
// multiple of 32), starting at token 0; runs at or past V are skipped.
inline int sample_stride(int64_t V) {
  const int64_t s = (V / kSampleRuns) & ~(int64_t)31;
  return (int)(s < 32 ? 32 : s);
}

struct Args {
  const uint8_t* logits;
  int64_t row_bytes;
  int V;
  int B;
  int S;                 // chunks per row
  int stride;            // sample stride
  const float* T;
  const int32_t* k;
  const float* p;
  const uint32_t* bitmask;
  int64_t bm_stride;
  SegSummary* segs;      // [B][4S]
  ChunkMass* mass;       // [B][S]
  uint32_t* cands;       // [B][4S][kSegCap]
};

// Launch over B * S chunks; the grid follows from the device's compute-unit
// count.
hipError_t launch_scan_bf16(Args a, hipStream_t st);

}  // namespace chunk
}  // namespace qs
