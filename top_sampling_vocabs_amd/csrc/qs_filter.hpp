// Exact top-k / top-p filter-and-sample kernels for gfx950 (MI355X). This
// file holds the kernel templates; qs_filter_f32.hip and qs_filter_bf16.hip
// instantiate them per dtype.
//
// One 1024-thread workgroup owns one row. Its 16 wave64s each own a
// contiguous slice of the vocabulary (a multiple of 512 tokens for rows held
// in registers, of 32 tokens otherwise), so every packed-mask word belongs to
// one wave and every per-wave walk runs in token-id order; the outputs are
// deterministic.
//
// Per row (page "Qrita", overall framework and key designs 1-3):
//  1. sigma-truncation (key design 1). Rows of up to 20 loads of 16 bytes per
//     lane are held in VGPRs: every load of the row is issued up front, so the
//     whole row is in flight at once. The first 512-token step of each slice
//     (8192 tokens) is the sample for mean, sigma and the sample maximum; the
//     threshold t = t0 - 0.2|t0| uses the Gaussian quantile of k/V (top-k) or
//     of p under the mass-weighted Gaussian (top-p). Each later step is
//     compacted as soon as it arrives: legal tokens with z >= t go, in id
//     order, to a per-wave LDS pool and (bf16) to a per-key histogram; the pass
//     also counts legal tokens, flags NaN / -inf, and for rows with top-k off
//     sums the mass below t. Longer rows stream through a prefetch ring with
//     the same per-step work.
//  2. hit test: |Z_t| > k (top-k), or mass(Z_t) >= p * W (top-p only);
//     otherwise every later step runs over the full row, re-read from memory
//     (the page's fallback Z_s = Z).
//  3. the k-th largest value and the top-p boundary value. On a bf16 pool the
//     keys above t span a short key range: a suffix scan of the per-key
//     histogram (counts, then fp64 masses) evaluates the page's stop test
//     N_tau >= k > N_tau - N_zm at every key at once. Element sources (fp32
//     pools, the full row) run the quaternary three-pivot search (key design
//     2): pivots at 1/4, 1/2, 3/4 of the key interval, one fused pass counting
//     N_tau, the minimum above tau and its multiplicity for all three pivots.
//  4. duplicate handling (key design 3): at the boundary value only the
//     earliest N_keep token ids are kept; each wave keeps its share of that
//     quota, in id order.
//  5. renormalise, write the packed mask, id-ordered candidate lists and
//     optional dense probabilities, and draw the token by an inverse CDF in
//     id order with Philox4x32-10 (sampling-contract page, sections 02 and 06).

#include <type_traits>

#pragma once

#include "qs_device.hpp"
#include "qs_launch.hpp"
#include "qs_stream.hpp"
#include "qs_bins.hpp"
#include "qs_proc.hpp"
#include "qs_topn.hpp"
#include "../../include/qs.h"

namespace qs {

constexpr int kHistBins = kThreads;   // bf16 pool histogram: one key per thread

// Background histogram of bf16 rows with top-k off: one bin per bf16 value of
// magnitude in [2^-12, 512) and sign, plus a lump below and above that range
// per sign. Bin of a token: i = clamp(mag - (kBgMagLo - 1), 0, kBgExact + 1)
// with mag = bits & 0x7FFF, plus kBgSide for a negative sign.
constexpr uint32_t kBgMagLo = 0x3980u;            // magnitude bits of 2^-12
constexpr uint32_t kBgExact = 21u * 128u;         // exact bins per sign (21 binades)
constexpr uint32_t kBgSide = kBgExact + 2u;       // bins per sign
constexpr int kBgBins = 2 * (int)kBgSide;
static_assert(kBgMagLo + kBgExact == 0x4400u, "the upper lump starts at 512");
// Register-resident tiers (steps of 512 tokens per wave slice), per dtype:
// fp32 rows take two 16-byte loads per step, bf16 rows one.
constexpr int kResidentTier[2][2] = {{5, 10}, {5, 19}};
// Register ring depth (steps in flight per wave) of those tiers.
constexpr int kRingDepth[2] = {5, 10};
constexpr int kStageWords = 320;      // packed-mask words of one slice held in LDS
static_assert(kResidentMaxSteps * (kStep / 32) <= kStageWords, "stage holds a resident slice");

// Natural log of q >= 0 for a float32 output: q = m 2^e with m in [0.5, 1),
// log2 m by the hardware single-precision log2 (about 1e-7 absolute on that
// interval), the sum scaled by ln 2 in float64. A few instructions, where a
// full float64 log would weigh on the code of the kernel it sits in.
__device__ __forceinline__ float log_prob(double q) {
  int e;
  const double m = frexp(q, &e);
  return (float)(((double)e + (double)__log2f((float)m)) * 0.6931471805599453);
}

// The drawn token of row r and, when asked for, the log of its probability
// under the final (renormalised) distribution, the one it was drawn from.
__device__ __forceinline__ void put_token(const FilterArgs& a, int r, int tok, double q) {
  a.tokens[r] = tok;
  if (a.logprobs) a.logprobs[r] = log_prob(q);
}

// Probability of the wave's last kept id with q > 0 (`last_id`, the wave-wide
// maximum of each lane's last such id), read from the lane that holds it.
__device__ __forceinline__ double last_token_q(int my_last_id, double my_last_q, int last_id) {
  const uint64_t at = ballot(last_id >= 0 && my_last_id == last_id);
  return at ? readlane_f64(my_last_q, __ffsll((unsigned long long)at) - 1) : 0.0;
}

#include "qs_select.hpp"
#include "qs_merge.hpp"

// Relative error bound of one hardware exp2 (v_exp_f32), taken as 4 ulp.
constexpr double kExp2Err = 2.384185791015625e-07;  // 2^-22

// fp64 weight of a key relative to the row maximum: exp((z - m) / T).
template <int DT>
__device__ __forceinline__ double weight(uint32_t key, double m, double invT) {
  return exp64(((double)Keys<DT>::value(key) - m) * invT);
}

// ---------------------------------------------------------------------------
// NL > 0: the row is held in registers, NL steps of 512 tokens per wave slice.
// NL == 0: the row streams through a prefetch ring.
// P: logit processors applied in the kernel: 0 none (the instances hold none
// of their code), 1 repetition and presence penalties only, 2 any.
// SRT: the instance holds the sorted-subset ablation switch.
// One row (workgroup blockIdx.x); returns the workgroup's pool LDS, free again
// once every thread has returned.
template <int DT, bool SAMPLE, int NL, int P, bool SRT>
__device__ __forceinline__ uint8_t* filter_row(FilterArgs a) {
  using K = Keys<DT>;
  using PL = PoolLayout<DT>;
  using PKey = typename PL::KeyT;
  constexpr uint32_t kCap = (uint32_t)PL::kPerWave;
  constexpr bool kResident = NL > 0;
  constexpr int kHB = DT == 1 ? kHistBins : 1;
  static_assert(NL <= kResidentMaxSteps, "resident rows are at most 20 steps per slice");
  __shared__ __align__(16) uint8_t pool_raw[kPoolBytes];
  __shared__ __align__(16) uint32_t stage[kWaves][kStageWords];
  __shared__ __align__(16) uint4 lut[DT == 1 ? 256 : 1];
  __shared__ uint32_t hist[kHB];
  __shared__ double binw[kHB];
  // fp32 rows: the radix select's bins, 32 KB (bf16 rows use hist and binw)
  __shared__ __align__(16) uint32_t rb_f32[DT == 0 ? 8192 : 4];
  // the background histogram plus one dump bin per lane (excluded tokens)
  __shared__ __align__(16) uint32_t bgh[DT == 1 ? kBgBins + 64 : 4];
  __shared__ RedScratch red;
  __shared__ RowInfo info;
  __shared__ uint32_t s_proc[P ? 20 : 1];  // logit processors: block-scan totals and a flag
  __shared__ uint32_t s_sort[1];  // the sorted-subset switch: a counter, a claim

  PKey* const pool_key = reinterpret_cast<PKey*>(pool_raw);
  uint16_t* const pool_id = reinterpret_cast<uint16_t*>(pool_raw + sizeof(PKey) * kWaves * kCap);

  const int r = blockIdx.x;
  const int w = uni((int)threadIdx.x >> 6);  // wave index, kept in a scalar register

  // -- bf16 rows scanned by the chunk kernel: settled from its candidates --------
  if constexpr (DT == 1 && !P) {
    if (a.ws_segs != nullptr) {
      const int tid = threadIdx.x;
      if (merge_row<SAMPLE>(a, r, tid, w, tid & 63, pool_raw, &stage[0][0], hist, binw, red,
                            info))
        return pool_raw;
      __syncthreads();  // the other paths reuse the LDS
    }
  }

  // -- bf16 rows held in registers: the value-histogram path ---------------------
  // (rows it cannot settle exactly, and the path switches, take the general
  // path below, which derives its per-lane values again so that none of them
  // is held across this path)
  if constexpr (DT == 1 && kResident) {
    if (a.flags == 0u) {
      const int tid = threadIdx.x;
      const int lane = tid & 63;
      Slice sl;
      sl.row = a.logits + (size_t)r * a.row_bytes;
      sl.mrow = nullptr;
      sl.V = a.V;
      sl.wb = uni(min(a.V, w * a.seg));
      sl.we = uni(min(a.V, (w + 1) * a.seg));
      const int W = (a.V + 31) >> 5;
      const uint32_t* const bmrow = a.bitmask ? a.bitmask + (size_t)r * a.bm_stride : nullptr;
      uint32_t* const mask_row = a.keep_mask ? a.keep_mask + (size_t)r * W : nullptr;
      float* const dense_row = a.dense ? a.dense + (size_t)r * a.V : nullptr;
      if (select_row<SAMPLE, NL, P>(a, sl, r, w, lane, tid, W, bmrow, mask_row, dense_row,
                                 pool_raw, stage, lut, reinterpret_cast<double*>(bgh), red,
                                 info, s_proc))
        return pool_raw;
      __syncthreads();  // the general path reuses the LDS
    }
  }

  const int lane = (int)lane_id();
  const int tid = w * 64 + lane;
  int par = 0;

  const int V = a.V;
  Slice sl;
  sl.row = a.logits + (size_t)r * a.row_bytes;
  sl.mrow = a.bitmask ? reinterpret_cast<const uint8_t*>(a.bitmask + (size_t)r * a.bm_stride)
                      : nullptr;
  sl.V = V;
  sl.wb = uni(min(V, w * a.seg));
  sl.we = uni(min(V, (w + 1) * a.seg));
  const int W = (V + 31) >> 5;
  const uint32_t* const bmrow = a.bitmask ? a.bitmask + (size_t)r * a.bm_stride : nullptr;

  uint32_t* mask_row = a.keep_mask ? a.keep_mask + (size_t)r * W : nullptr;
  float* dense_row = a.dense ? a.dense + (size_t)r * V : nullptr;

  // -- logit processors: the row is selected from an edited copy in the
  //    workspace (its table in the pools' LDS, the side part in the stage) ------
  if constexpr (P) {
    const proc::RowParams prm = proc::row_params<P>(a, r);
    const proc::Table pt = proc::table_at(pool_raw, reinterpret_cast<uint8_t*>(&stage[0][0]));
    static_assert(proc::kMainBytes <= kPoolBytes, "processor table");
    static_assert(proc::kSideBytes <= kWaves * kStageWords * 4, "processor side table");
    const proc::HistIds hids = proc::prefetch_ids(a, r, tid);
    proc::build_clear(a, pt, tid, s_proc + 16);
    __syncthreads();
    proc::build_mark(a, r, prm, pt, tid, s_proc + 16, hids);
    __syncthreads();
    if (!prm.ok || s_proc[16] != 0u) {
      if (mask_row)
        for (int i = tid; i < W; i += kThreads) mask_row[i] = 0u;
      if (dense_row)
        for (int i = tid; i < V; i += kThreads) dense_row[i] = 0.0f;
      if (tid == 0) {
        a.status[r] = QS_ROW_BAD_PARAM;
        if (SAMPLE) {
          a.tokens[r] = -1;
          if (a.logprobs) a.logprobs[r] = __builtin_nanf("");
        }
        if (a.cand_count) a.cand_count[r] = 0;
        if (a.dbg) {
          a.dbg[4 * r + 0] = 0; a.dbg[4 * r + 1] = 0;
          a.dbg[4 * r + 2] = 0; a.dbg[4 * r + 3] = 0;
        }
      }
      return pool_raw;
    }
    if (prm.need_cnt || prm.has_b) proc::build_ranks(a, r, prm, pt, tid, s_proc);
    // copy in 16-byte pieces; the edited tokens of a piece are rewritten first
    constexpr int kPT = 16 / (DT == 0 ? 4 : 2);  // tokens per piece
    constexpr uint32_t kPM = (1u << kPT) - 1u;
    uint8_t* const dst = a.p_copy + (size_t)r * a.p_copy_bytes;
    auto bits_at = [&](int e0, uint32_t m) -> uint32_t {  // history | bias << 8
      const uint32_t sh = (uint32_t)e0 & 31u;
      const uint32_t hw = prm.has_h ? (pt.hbits[e0 >> 5] >> sh) & m : 0u;
      const uint32_t bw = prm.has_b ? (pt.bbits[e0 >> 5] >> sh) & m : 0u;
      return hw | (bw << 8);
    };
    const int npieces = V / kPT;
    for (int c = tid; c < npieces; c += kThreads) {
      uint4 x = *reinterpret_cast<const uint4*>(sl.row + (size_t)c * 16);
      const int e0 = c * kPT;
      const uint32_t pw = bits_at(e0, kPM);
      if (pw) {
        uint32_t r4[4] = {x.x, x.y, x.z, x.w};
        for (int j = 0; j < kPT; ++j) {
          if (!(((pw | (pw >> 8)) >> j) & 1u)) continue;
          const int q = DT == 0 ? j : j >> 1;
          const uint32_t sh = DT == 0 ? 0u : 16u * (uint32_t)(j & 1);
          const uint32_t msk = DT == 0 ? 0xFFFFFFFFu : 0xFFFFu;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            if (qq == q) {
              const uint32_t raw = (r4[qq] >> sh) & msk;
              const uint32_t nv = proc::edit_token<DT>(pt, prm, (uint32_t)(e0 + j), raw,
                                                       (pw >> j) & 1u, (pw >> (8 + j)) & 1u) &
                                  msk;
              r4[qq] = (r4[qq] & ~(msk << sh)) | (nv << sh);
            }
          }
        }
        x = make_uint4(r4[0], r4[1], r4[2], r4[3]);
      }
      *reinterpret_cast<uint4*>(dst + (size_t)c * 16) = x;
    }
    // the tokens past the last whole piece, one by one
    for (int e = npieces * kPT + tid; e < V; e += kThreads) {
      uint32_t raw = DT == 0 ? reinterpret_cast<const uint32_t*>(sl.row)[e]
                             : (uint32_t)reinterpret_cast<const uint16_t*>(sl.row)[e];
      const uint32_t pw = bits_at(e, 1u);
      if (pw) raw = proc::edit_token<DT>(pt, prm, (uint32_t)e, raw, pw & 1u, (pw >> 8) & 1u);
      if (DT == 0) reinterpret_cast<uint32_t*>(dst)[e] = raw;
      else reinterpret_cast<uint16_t*>(dst)[e] = (uint16_t)raw;
    }
    // the copy's stores have completed before this workgroup reads it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // the copy is complete; the LDS is the general path's again
    sl.row = dst;
  }
  // this slice's packed-mask words fit the LDS stage (always for resident rows)
  const bool stage_ok = (sl.we - sl.wb + 31) / 32 <= kStageWords;

  // Zero this wave's share of the mask and dense outputs in memory and wait
  // until the stores have completed, so that a later scatter into the same
  // slice by this wave lands after them.
  auto zero_outputs = [&]() {
    if (mask_row && sl.we > sl.wb) {  // a non-empty slice starts on a word boundary
      int w0 = sl.wb >> 5, w1 = (sl.we + 31) >> 5;
      for (int i = w0 + lane; i < w1; i += 64) mask_row[i] = 0u;
    }
    if (dense_row) {
      for (int i = sl.wb + lane; i < sl.we; i += 64) dense_row[i] = 0.0f;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
  };

  auto finish_error = [&](int code) {
    zero_outputs();
    if (tid == 0) {
      a.status[r] = code;
      if (SAMPLE) {
        a.tokens[r] = -1;
        if (a.logprobs) a.logprobs[r] = __builtin_nanf("");
      }
      if (a.cand_count) a.cand_count[r] = 0;
      if (a.dbg) {
        a.dbg[4 * r + 0] = 0; a.dbg[4 * r + 1] = 0;
        a.dbg[4 * r + 2] = 0; a.dbg[4 * r + 3] = 0;
      }
    }
  };

  // -- the sample: step 0 of every slice ----------------------------------------
  // The first 512 tokens of each of the 16 slices (8192 tokens) are the only
  // request in flight until they have returned, so they come back at unloaded
  // latency; the rest of the row is requested after them. Step 0 stays in the
  // ring for the pass.
  constexpr int kPiece = 16 / (DT == 0 ? 4 : 2);  // tokens per 16-byte piece
  constexpr int kPieces = DT == 0 ? 2 : 1;        // 16-byte loads per lane per step
  constexpr int RD = kResident ? (NL < kRingDepth[DT] ? NL : kRingDepth[DT]) : 1;
  uint4 buf[RD][kPieces];
  // A 16-byte piece that starts below V lies inside the row's stride; pieces
  // past the slice read the slice's last piece instead (their tokens are
  // clipped), so every lane issues the same loads.
  const int last_piece = sl.we > sl.wb ? (sl.we - 1) & ~(kPiece - 1) : 0;
  const int lane_e = sl.wb + lane * kChunk;
  auto res_issue = [&](auto stc) {
    constexpr int st = decltype(stc)::value;
    if constexpr (kResident && st < NL) {
#pragma unroll
      for (int pc = 0; pc < kPieces; ++pc) {
        const int ep = min(lane_e + st * kStep + pc * kPiece, last_piece);
        buf[st % RD][pc] = *reinterpret_cast<const uint4*>(chunk_ptr<DT>(sl.row, ep));
      }
    }
  };
  constexpr int D = DT == 1 ? 8 : 4;
  using Reader = std::conditional_t<kResident, NoReader<DT>, RowReader<DT, D>>;
  Reader rd(sl, lane);
  const int nst = kResident ? NL : rd.n;
  constexpr int kMW = NL * (kStep / 32);  // packed-mask words of a resident slice
  constexpr int kML = kResident ? (kMW + 63) / 64 : 1;
  uint32_t mw[kML];
  if constexpr (kResident) {
    // the slice's packed-mask words come with the sample: the pass needs them
    // from its first step. Without a bitmask the word loads read the row start
    // (16 bytes at least) and are ignored, so that the loads have no branch.
    const uint32_t* const mwsrc = bmrow ? bmrow : reinterpret_cast<const uint32_t*>(sl.row);
    const int w0 = sl.wb >> 5;
    const int wlim = bmrow ? min(W, (sl.we + 31) >> 5) : 0;  // words of this slice
#pragma unroll
    for (int i = 0; i < kML; ++i) {
      const int wi = w0 + lane + 64 * i;
      mw[i] = mwsrc[(lane + 64 * i < kMW && wi < wlim) ? wi : 0];
    }
    res_issue(std::integral_constant<int, 0>{});
  } else {
    if (nst > 0) rd.issue(0, 0);
  }

  // -- parameters ------------------------------------------------------------
  const float Tf = a.T[r];
  const int kk = a.k[r];
  const float pf = a.p[r];
  if (!(isfinite(Tf) && Tf >= 0.0f) || kk < 0 || !(pf > 0.0f && pf <= 1.0f)) {
    finish_error(QS_ROW_BAD_PARAM);
    return pool_raw;
  }
  const bool greedy = (Tf == 0.0f);
  const double invT = greedy ? 0.0 : 1.0 / (double)Tf;
  const double p = (double)pf;
  const bool topp_on = !greedy && pf < 1.0f;
  // top-k is requested for k in [1, V); whether k < |F| is known after the pass
  const bool topk_req = !greedy && kk > 0 && kk < V;
  const bool need_bg = topp_on && !topk_req;
  const bool no_trunc = (a.flags & QS_FLAG_NO_TRUNCATION) != 0u;

  // -- tables ----------------------------------------------------------------------
  // Pair masks of every legal byte (0xFFFF per legal token). Every wave writes
  // the whole table with the same values, so each wave may read it after its
  // own writes without waiting for the others.
  if constexpr (DT == 1) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const uint32_t e = (uint32_t)(lane + 64 * q4);
      uint32_t v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v[q] = (((e >> (2 * q)) & 1u) ? 0x0000FFFFu : 0u) |
               (((e >> (2 * q + 1)) & 1u) ? 0xFFFF0000u : 0u);
      lut[e] = make_uint4(v[0], v[1], v[2], v[3]);
    }
    hist[tid] = 0u;  // used after the pass barrier
    if (need_bg) {   // filled by the pass
      static_assert(kBgBins % 4 == 0, "the background histogram is cleared in 16-byte units");
      uint4* const b4 = reinterpret_cast<uint4*>(bgh);
      for (int i = tid; i < kBgBins / 4; i += kThreads) b4[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  if (tid == 0) info.bsel = -1;

  // -- per-lane sample statistics (legal finite tokens of step 0) ------------------
  double s_n = 0.0, s_sum = 0.0, s_sq = 0.0, s_all = 0.0;
  uint32_t s_maxk = 0u;
  if (sl.we > sl.wb) {
    Raw<DT> raw;
    uint32_t mb;
    if constexpr (kResident) {
      raw.r[0] = buf[0][0].x; raw.r[1] = buf[0][0].y;
      raw.r[2] = buf[0][0].z; raw.r[3] = buf[0][0].w;
      if constexpr (DT == 0) {
        raw.r[4] = buf[0][kPieces - 1].x; raw.r[5] = buf[0][kPieces - 1].y;
        raw.r[6] = buf[0][kPieces - 1].z; raw.r[7] = buf[0][kPieces - 1].w;
      }
      // byte `lane` of the slice's mask words: word lane/4 is held by lane lane/4
      const uint32_t wd = (uint32_t)__shfl((int)mw[0], lane >> 2, 64);
      const uint32_t b0 = bmrow ? (wd >> ((lane & 3) * 8)) & 0xFFu : 0xFFu;
      const int rem = sl.we - lane_e;
      mb = b0 & (rem >= 8 ? 0xFFu : (rem > 0 ? (1u << rem) - 1u : 0u));
    } else {
      rd.fetch(0, 0, raw, mb);
    }
    s_all = (double)max(0, min(8, sl.we - lane_e));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t key = K::of(raw.bits(j));
      if (((mb >> j) & 1u) && key > K::kNegInf && key < K::kPosInf) {
        const double v = (double)K::value(key);
        s_n += 1.0; s_sum += v; s_sq += v * v;
        s_maxk = key > s_maxk ? key : s_maxk;
      }
    }
  }


  // the next ring steps: requested once this wave's sample has returned. A
  // resident ring requests only its first steps before the sample barrier and
  // the rest after it, so that the other waves' samples are not queued behind
  // a full flood
  constexpr int kEarly = RD < 4 ? RD : 4;
  if constexpr (kResident) {
    static_for<1, kEarly>(res_issue);
  } else {
#pragma unroll
    for (int i = 1; i < D; ++i)
      if (i < nst) rd.issue(i, i);
  }

  // -- the row's threshold ------------------------------------------------------------
  // The 16 step-0 samples (8192 tokens) are combined after one barrier; the
  // ring keeps filling meanwhile, so the threshold is computed while data
  // arrives.
  {
    const double st0 = wave_sum_f64(s_n), st1 = wave_sum_f64(s_sum);
    const double st2 = wave_sum_f64(s_sq), st3 = wave_sum_f64(s_all);
    const uint32_t mx = wave_reduce<OpMax>(s_maxk);
    if (lane == 0) {
      const double stv[4] = {st0, st1, st2, st3};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint64_t b = __double_as_longlong(stv[i]);
        red.v[par][w][2 * i] = (uint32_t)b;
        red.v[par][w][2 * i + 1] = (uint32_t)(b >> 32);
      }
      red.v[par][w][8] = mx;
    }
  }
  __syncthreads();  // sample partials, the zeroed histogram, bsel
  if constexpr (kResident) static_for<kEarly, RD>(res_issue);
  {
    // lane i holds wave i's partials; the same combination order in every wave
    const bool act = lane < kWaves;
    double acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc[i] = act ? __longlong_as_double(((uint64_t)red.v[par][lane][2 * i + 1] << 32) |
                                          red.v[par][lane][2 * i])
                   : 0.0;
    const uint32_t mx = act ? red.v[par][lane][8] : 0u;
    s_n = uni(wave_sum_f64(acc[0]));
    s_sum = uni(wave_sum_f64(acc[1]));
    s_sq = uni(wave_sum_f64(acc[2]));
    s_all = uni(wave_sum_f64(acc[3]));
    s_maxk = uni(wave_reduce<OpMax>(mx));
  }
  par ^= 1;
  if constexpr (kResident) {  // stage this slice's packed-mask words
    if (bmrow) {
      const int w0 = sl.wb >> 5;
      const int wlim = min(W, (sl.we + 31) >> 5);
#pragma unroll
      for (int i = 0; i < kML; ++i) {
        const int wi = w0 + lane + 64 * i;
        if (lane + 64 * i < kMW) stage[w][lane + 64 * i] = wi < wlim ? mw[i] : 0u;
      }
    }
  }
  const uint8_t* const stage_bytes = reinterpret_cast<const uint8_t*>(stage[w]) + lane;
  // step ST of a resident slice: raw bits and legal bits (clipped to the slice)
  auto res_fetch = [&](auto stc, Raw<DT>& raw, uint32_t& mb) {
    if constexpr (kResident) {
      constexpr int st = decltype(stc)::value;
      constexpr int sl_ = st % RD;
      raw.r[0] = buf[sl_][0].x; raw.r[1] = buf[sl_][0].y;
      raw.r[2] = buf[sl_][0].z; raw.r[3] = buf[sl_][0].w;
      if constexpr (DT == 0) {
        raw.r[4] = buf[sl_][kPieces - 1].x; raw.r[5] = buf[sl_][kPieces - 1].y;
        raw.r[6] = buf[sl_][kPieces - 1].z; raw.r[7] = buf[sl_][kPieces - 1].w;
      }
      uint32_t m8 = bmrow ? (uint32_t)stage_bytes[st * 64] : 0xFFu;
      if (sl.wb + (st + 1) * kStep > sl.we) {  // a step that ends past the slice
        const int rem = sl.we - (lane_e + st * kStep);
        m8 &= rem >= 8 ? 0xFFu : (rem > 0 ? (1u << rem) - 1u : 0u);
      }
      mb = m8;
    }
  };

  const double ms = s_n >= 1.0 ? (double)K::value(s_maxk) : 0.0;
  // fewer than 32 legal finite sample tokens (a sparse mask): keep every legal
  // finite token
  const double tval = s_n < 32.0 && !greedy
                          ? -__builtin_inf()
                          : truncation_value(s_n, s_sum, s_sq, ms,
                                             s_all > 0.0 ? s_n / s_all : 0.0, V, greedy,
                                             topk_req, kk, topp_on, p, invT);
  // threshold as a key; no_trunc compacts nothing
  const bool t_all = !(tval > -__builtin_inf());
  uint32_t tkey = t_all ? K::kNegInf + 1u : K::of(raw_floor<DT>(tval));
  if (tkey <= K::kNegInf) tkey = K::kNegInf + 1u;
  if (no_trunc) tkey = K::kMax;
  tkey = uni(tkey);
  // the pass compares signed values S = key - 2^(bits-1) (+magnitude / -magnitude)
  const int32_t tS = DT == 1 ? (int32_t)tkey - 0x8000 : (int32_t)(tkey - 0x80000000u);
  // reference point of the background mass (the threshold value itself)
  const float bg_ref = (t_all || no_trunc) ? 0.0f : K::value(tkey);
  const float bg_c = (float)(1.4426950408889634 * invT);

  // -- the pass ------------------------------------------------------------------
  uint32_t anyl = 0u, pcnt = 0u;
  // Non-finite detectors over legal tokens (illegal tokens never trigger them):
  // POS pass: the largest raw bits read as unsigned (> the -inf pattern: a
  // negative NaN; equal: a -inf); NEG pass: the smallest signed value (below
  // -inf: a negative NaN).
  uint32_t ext2 = 0u;                        // bf16, packed per half
  uint32_t ext1 = 0u;                        // fp32
  double bg_sum = 0.0;     // fp32 rows: sum of exp2((z - t) c) over legal finite z < t
  PKey* const my_pk = pool_key + w * kCap;
  uint16_t* const my_pid = pool_id + w * kCap;
  // fp32 background terms: x = z c - t c, excluded tokens read as a large
  // negative finite value so that w = 0
  const float bg_off = -bg_ref * bg_c;
  constexpr uint32_t kSent1 = 0xC47A0000u;   // fp32 -1000

  // One step: 8 tokens per lane. A legal token is a candidate iff its signed
  // value (+magnitude / -magnitude of the raw bits, so that -0 == +0) is >= tS;
  // when t > 0 (POS) that is the raw bits read as a signed integer. Rows with
  // top-k off also sum exp2((z - t) log2(e) / T) over the legal tokens below t
  // (fp32 terms, fp64 accumulation per step).
  auto step = [&](auto pos_c, const Raw<DT>& raw, uint32_t mb, int e) {
    constexpr bool POS = decltype(pos_c)::value;
    anyl |= mb;
    uint32_t cb;
    if constexpr (DT == 1) {
      const uint4 pm4 = lut[mb];
      const uint32_t pm[4] = {pm4.x, pm4.y, pm4.z, pm4.w};
      const uint32_t t2m1 = ((uint32_t)(tS - 1) & 0xFFFFu) * 0x10001u;
      uint32_t dl[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t d = raw.r[q];
        uint32_t rl;
        if constexpr (POS) {
          rl = bfi(pm[q], d, 0x80008000u);  // illegal -> the lowest signed value
          ext2 = bits_of(__builtin_elementwise_max(as_u2(ext2), as_u2(rl)));
        } else {
          const uint32_t sg = bits_of(as_s2(d) >> 15);
          const uint32_t sv = bits_of(as_s2((d & 0x7FFF7FFFu) ^ sg) - as_s2(sg));
          rl = bfi(pm[q], sv, 0x80808080u);  // illegal -> -inf
          ext2 = bits_of(__builtin_elementwise_min(as_s2(ext2), as_s2(rl)));
        }
        dl[q] = bits_of(__builtin_elementwise_sub_sat(as_s2(t2m1), as_s2(rl)));  // <0 iff cand
      }
      // settle the detector here, before the candidate loop below, so that its
      // operands do not stay live across that loop
      __asm__ volatile("" : "+v"(ext2));
      const uint32_t cA = __builtin_amdgcn_perm(dl[1], dl[0], 0x0B0A0908u);
      const uint32_t cB = __builtin_amdgcn_perm(dl[3], dl[2], 0x0B0A0908u);
      cb = __builtin_amdgcn_sad_u8(cB & 0x80402010u, 0u,
                                   __builtin_amdgcn_sad_u8(cA & 0x08040201u, 0u, 0u));
      if (need_bg) {  // count the legal tokens below t in the background histogram
        // excluded tokens (illegal, or candidates) go to this lane's dump bin:
        // no branch per token
        const uint4 nb4 = lut[mb & ~cb];
        const uint32_t nb[4] = {nb4.x, nb4.y, nb4.z, nb4.w};
        const uint32_t dump2 = (uint32_t)(kBgBins + lane) * 0x10001u;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t d = raw.r[q];
          uint32_t bi = bits_of(__builtin_elementwise_sub_sat(
              as_u2(d & 0x7FFF7FFFu), as_u2((kBgMagLo - 1u) * 0x10001u)));
          bi = bits_of(__builtin_elementwise_min(as_u2(bi), as_u2((kBgExact + 1u) * 0x10001u)));
          bi += ((d >> 15) & 0x00010001u) * kBgSide;
          bi = bfi(nb[q], bi, dump2);
          __hip_atomic_fetch_add(bgh + (bi & 0xFFFFu), 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
          __hip_atomic_fetch_add(bgh + (bi >> 16), 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
    } else {
      const int32_t tm1 = tS - 1;
      int32_t dl[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t d = raw.r[j];
        const uint32_t mj = (uint32_t)__builtin_amdgcn_sbfe((int)mb, j, 1);
        uint32_t rl;
        if constexpr (POS) {
          rl = bfi(mj, d, 0x80000000u);
          ext1 = max(ext1, rl);
        } else {
          const uint32_t mag = d & 0x7FFFFFFFu;
          const uint32_t sv = (d & 0x80000000u) ? 0u - mag : mag;
          rl = bfi(mj, sv, 0x80800000u);  // illegal -> -inf
          ext1 = (uint32_t)min((int32_t)ext1, (int32_t)rl);
        }
        dl[j] = (int32_t)rl > tm1 ? -1 : 0;
      }
      __asm__ volatile("" : "+v"(ext1));
      cb = 0u;
#pragma unroll
      for (int j = 0; j < 8; ++j) cb |= (dl[j] & 1u) << j;
      if (need_bg) {
        const uint32_t nb = mb & ~cb;
        float sw = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t zb = ((nb >> j) & 1u) ? raw.r[j] : kSent1;
          sw += __builtin_amdgcn_exp2f(fmaf(__uint_as_float(zb), bg_c, bg_off));
        }
        bg_sum += (double)sw;
      }
    }
    pcnt = append_pool<DT>(cb, raw, (uint32_t)(e - sl.wb), pcnt, my_pk, my_pid);
  };
  auto run_pass = [&](auto pos_c) {
    if constexpr (kResident) {
      static_for<0, NL>([&](auto stc) {
        constexpr int st = decltype(stc)::value;
        Raw<DT> raw;
        uint32_t mb;
        res_fetch(stc, raw, mb);
        res_issue(std::integral_constant<int, st + RD>{});
        step(pos_c, raw, mb, sl.wb + st * kStep + lane * kChunk);
      });
    } else {
      for (int s0 = 0; s0 < nst; s0 += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
          const int st = s0 + i;
          if (st < nst) {
            Raw<DT> raw;
            uint32_t mb;
            rd.fetch(st, i, raw, mb);
            step(pos_c, raw, mb, rd.first(st));
            if (st + D < nst) rd.issue(st + D, i);
          }
        }
      }
    }
  };
  const bool pos_pass = tS > 0;
  if (pos_pass) {
    ext2 = 0u; ext1 = 0u;
    run_pass(std::true_type{});
  } else {
    ext2 = 0x7FFF7FFFu; ext1 = 0x7FFFFFFFu;
    run_pass(std::false_type{});
  }
  // legal negative NaN / legal -inf, from the detectors above
  uint32_t nan_l = 0u, ninf_l = 0u;
  if (pos_pass) {
    const uint32_t hmax = DT == 1 ? max(ext2 & 0xFFFFu, ext2 >> 16) : ext1;
    const uint32_t ninf_raw = DT == 1 ? 0xFF80u : 0xFF800000u;
    nan_l = hmax > ninf_raw ? 1u : 0u;
    ninf_l = hmax == ninf_raw ? 1u : 0u;
  } else {
    int32_t lo;
    if constexpr (DT == 1) {
      const s16x2 v = as_s2(ext2);
      lo = min((int32_t)v.x, (int32_t)v.y);
    } else {
      lo = (int32_t)ext1;
    }
    const int32_t ninf_s = DT == 1 ? -0x7F80 : -0x7F800000;
    nan_l = lo < ninf_s ? 1u : 0u;
    ninf_l = 1u;  // a legal -inf cannot be told from an illegal token here
  }

  // -- reduce the pass -------------------------------------------------------------
  anyl = wave_reduce<OpMax>(anyl);
  nan_l = wave_reduce<OpMax>(nan_l);
  ninf_l = wave_reduce<OpMax>(ninf_l);
  bg_sum = wave_sum_f64(bg_sum);
  if (lane == 0) {
    red.v[par][w][0] = anyl;
    red.v[par][w][1] = nan_l | (ninf_l << 1);
    const uint64_t b0 = __double_as_longlong(bg_sum);
    red.v[par][w][2] = (uint32_t)b0; red.v[par][w][3] = (uint32_t)(b0 >> 32);
    info.cnt[w] = pcnt;
  }
  __syncthreads();  // pools and per-wave results complete
  // the draw's random input: vector loads (a lane-varying address of the same
  // element), so that waits for LDS results do not also wait for them
  double u_in = 0.0;
  uint64_t seed_in = 0u, off_in = 0u;
  if (SAMPLE) {
    const uint32_t z = __builtin_amdgcn_mbcnt_lo(0u, 0u);  // 0 in every lane
    if (a.uniforms) u_in = a.uniforms[r + z];
    else { seed_in = a.seed[r + z]; off_in = a.offset[r + z]; }
  }
  // lane i of every wave reads wave i's results
  const bool act16 = lane < kWaves;
  const int pw = par;  // the per-wave pass results stay in red.v[pw]
  bool overflow, neg_nan, has_neginf, any_legal;
  uint32_t ccount_all, my_wcnt;
  {
    const uint32_t fl = act16 ? red.v[pw][lane][1] : 0u;
    const uint32_t cn = act16 ? info.cnt[lane] : 0u;
    any_legal = uni(wave_reduce<OpMax>(act16 ? red.v[pw][lane][0] : 0u) != 0u);
    neg_nan = uni(wave_reduce<OpMax>(fl & 1u) != 0u);
    has_neginf = uni(wave_reduce<OpMax>((fl >> 1) & 1u) != 0u);
    overflow = uni(wave_reduce<OpMax>(cn > kCap ? 1u : 0u) != 0u);
    ccount_all = uni(wave_reduce<OpSum>(cn));
    my_wcnt = uni(info.cnt[w]);
  }
  (void)has_neginf;
  par ^= 1;

  const PKey* pk = my_pk;
  const uint16_t* pid = my_pid;
  int my_cnt = (int)min(my_wcnt, kCap);
  // pool usable: complete, 16-bit ids fit, not forced off
  const bool pool_ok = !overflow && ccount_all > 0u && !(a.flags & QS_FLAG_FORCE_MISS) &&
                       !no_trunc && a.seg <= 65536;
  // the pool holds every finite legal token (the threshold was -inf)
  const bool pool_all = pool_ok && t_all;

  // -- the pool and the background ---------------------------------------------------
  // Count and histogram (bf16) the pool entries and take their maximum. Rows
  // with top-k off also need the mass of the legal tokens below t, relative
  // to the row maximum, with an error bound: bf16 rows weigh every bin of the
  // background histogram in fp64 (exact bins; the lumps contribute their
  // weight range to the bound); fp32 rows take the pass's fp32 terms.
  uint32_t ccount = 0u, pool_max = 0u;
  bool hist_over = false;
  double bgm = 0.0, bgb = 0.0;
  if (pool_ok) {
    const double tv = (double)K::value(tkey);
    uint32_t ge = 0u, mxk = 0u, hov = 0u;
    walk_pool<DT>(pk, pid, my_cnt, (uint32_t)sl.wb, lane,
                  [&](const uint32_t (&key)[8], const uint32_t (&)[8], uint32_t vm) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if ((vm >> j) & 1u) {
          ++ge;
          mxk = key[j] > mxk ? key[j] : mxk;
          if constexpr (DT == 1) {
            const uint32_t b = key[j] - tkey;
            if (b < (uint32_t)kHistBins) atomicAdd(hist + b, 1u);
            else hov = 1u;
          }
        }
      }
    });
    double bx = 0.0, bb = 0.0;  // background mass relative to w(t) = 1, bound
    if constexpr (DT == 1) {
      if (need_bg) {
        // exact bins in runs of 8 magnitudes: one binade, equal spacing d, so
        // the weights of a run are w0, w0 rho, ..., w0 rho^7 with
        // rho = exp(+-d / T) (Horner over the counts)
        constexpr int kRunsPerSide = (int)kBgExact / 8;
        static_assert(kBgExact % 8 == 0 && (kBgMagLo & 127u) == 0u, "runs stay in one binade");
        if (tid < 2 * kRunsPerSide) {
          const uint32_t side = tid >= kRunsPerSide ? 1u : 0u;
          const uint32_t j0 = 1u + 8u * ((uint32_t)tid - side * (uint32_t)kRunsPerSide);
          const uint32_t* const hb = bgh + side * kBgSide + j0;
          uint32_t c[8], any = 0u;
#pragma unroll
          for (int i = 0; i < 8; ++i) { c[i] = hb[i]; any |= c[i]; }
          if (any) {
            const uint32_t mag0 = kBgMagLo - 1u + j0;
            const double v0 = (double)__uint_as_float(((side << 15) | mag0) << 16);
            const double d = ldexp(1.0, (int)(mag0 >> 7) - 134);  // 2^(e - 127 - 7)
            const double rho = exp64((side ? -d : d) * invT);
            double h = (double)c[7];
#pragma unroll
            for (int i = 6; i >= 0; --i) h = fma(h, rho, (double)c[i]);
            bx = h * exp64((v0 - tv) * invT);
          }
        } else if (tid < 2 * kRunsPerSide + 4) {  // the lumps
          const uint32_t q = (uint32_t)(tid - 2 * kRunsPerSide);
          const uint32_t side = q >> 1;
          const double cd = (double)bgh[side * kBgSide + ((q & 1u) ? kBgExact + 1u : 0u)];
          if (cd > 0.0) {
            if ((q & 1u) == 0u) {   // |z| < 2^-12
              const double e = 0.000244140625;
              bx = cd * exp64(-tv * invT);
              bb = cd * (exp64((e - tv) * invT) - exp64((-e - tv) * invT));
            } else {                // |z| >= 512 (and infinities, NaN)
              bb = cd * (side ? exp64((-512.0 - tv) * invT) : 1.0);
            }
          }
        }
      }
    }
    ge = wave_reduce<OpSum>(ge);
    mxk = wave_reduce<OpMax>(mxk);
    hov = wave_reduce<OpMax>(hov);
    bx = wave_sum_f64(bx);
    bb = wave_sum_f64(bb);
    if (lane == 0) {
      red.v[par][w][0] = ge; red.v[par][w][1] = mxk; red.v[par][w][2] = hov;
      const uint64_t b0 = __double_as_longlong(bx), b1 = __double_as_longlong(bb);
      red.v[par][w][3] = (uint32_t)b0; red.v[par][w][4] = (uint32_t)(b0 >> 32);
      red.v[par][w][5] = (uint32_t)b1; red.v[par][w][6] = (uint32_t)(b1 >> 32);
    }
    __syncthreads();  // the histogram is complete
    ccount = uni(wave_reduce<OpSum>(act16 ? red.v[par][lane][0] : 0u));
    pool_max = uni(wave_reduce<OpMax>(act16 ? red.v[par][lane][1] : 0u));
    hist_over = uni(wave_reduce<OpMax>(act16 ? red.v[par][lane][2] : 0u) != 0u);
    if (need_bg) {
      double bxs, bbs;
      if constexpr (DT == 1) {
        bxs = uni(wave_sum_f64(act16 ? __longlong_as_double(((uint64_t)red.v[par][lane][4] << 32) |
                                                            red.v[par][lane][3])
                                     : 0.0));
        bbs = uni(wave_sum_f64(act16 ? __longlong_as_double(((uint64_t)red.v[par][lane][6] << 32) |
                                                            red.v[par][lane][5])
                                     : 0.0));
        bbs += 1e-12 * bxs;  // fp64 weights and sums
      } else {
        // per wave: the hardware exp2 (4 ulp), the fp32 sums of 8 terms, and
        // the argument's roundings (|dx| <= 2^-24 (|t c| + 2|x|), with
        // w |x| <= 1 / (e ln 2) per term)
        const double bgi = act16 ? __longlong_as_double(((uint64_t)red.v[pw][lane][3] << 32) |
                                                        red.v[pw][lane][2])
                                 : 0.0;
        const double nslice = act16 ? (double)max(0, min(V, (lane + 1) * a.seg) -
                                                     min(V, lane * a.seg))
                                    : 0.0;
        const double cterm = fabs(tv * (double)bg_c) * 4.1315e-8;  // ln2 2^-24 |t c|
        bxs = uni(wave_sum_f64(bgi));
        bbs = uni(wave_sum_f64(bgi * (kExp2Err + 4.2e-7 + cterm) + nslice * 4.4e-8));
      }
      // tv <= the pool maximum: the scale is at most 1
      const double sc = exp64((tv - (double)K::value(pool_max)) * invT);
      bgm = bxs * sc;
      bgb = bbs * sc + 1e-300;
    }
    par ^= 1;
  }

  auto block_sum_f64 = [&](double v) -> double {
    v = wave_sum_f64(v);
    if (lane == 0) {
      uint64_t b = __double_as_longlong(v);
      red.v[par][w][0] = (uint32_t)b;
      red.v[par][w][1] = (uint32_t)(b >> 32);
    }
    __syncthreads();
    double t = 0.0;
    for (int ww = 0; ww < kWaves; ++ww)
      t += __longlong_as_double(((uint64_t)red.v[par][ww][1] << 32) | red.v[par][ww][0]);
    par ^= 1;
    return uni(t);
  };
  auto block_sum_u32 = [&](uint32_t v) -> uint32_t {
    v = wave_reduce<OpSum>(v);
    if (lane == 0) red.v[par][w][0] = v;
    __syncthreads();
    uint32_t t = 0u;
    for (int ww = 0; ww < kWaves; ++ww) t += red.v[par][ww][0];
    par ^= 1;
    return uni(t);
  };

  // -- row maximum, non-finite values, |F| ----------------------------------------
  // With a usable pool the maximum is in it (t never exceeds the sample
  // maximum) and +inf / positive NaNs at legal positions are candidates;
  // otherwise one walk over the row.
  uint32_t maxk = 0u, nfin = 0u;
  bool nonfinite = neg_nan;
  // |F| is known on the row path and when the pool holds all of F
  bool nf_known = true;
  if (pool_ok) {
    maxk = pool_max;
    if (pool_all) nfin = ccount;
    else nf_known = false;  // counted on the row path if needed
  } else {
    uint32_t mk = 0u, mn = 0xFFFFFFFFu, nf = 0u;
    walk_row<DT, true>(sl, lane, [&](const uint32_t (&key)[8], const uint32_t (&)[8],
                                     uint32_t lm) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if ((lm >> j) & 1u) {
          mk = key[j] > mk ? key[j] : mk;
          mn = key[j] < mn ? key[j] : mn;
          nf += key[j] > K::kNegInf ? 1u : 0u;
        }
      }
    });
    mk = wave_reduce<OpMax>(mk);
    mn = wave_reduce<OpMin>(mn);
    nf = wave_reduce<OpSum>(nf);
    if (lane == 0) {
      red.v[par][w][0] = mk; red.v[par][w][1] = mn; red.v[par][w][2] = nf;
    }
    __syncthreads();
    uint32_t gm = 0u, gmn = 0xFFFFFFFFu, gnf = 0u;
    for (int ww = 0; ww < kWaves; ++ww) {
      gm = max(gm, red.v[par][ww][0]);
      gmn = min(gmn, red.v[par][ww][1]);
      gnf += red.v[par][ww][2];
    }
    par ^= 1;
    maxk = uni(gm);
    nfin = uni(gnf);
    nonfinite = nonfinite || uni(gmn < K::kNegInf);
  }
  nonfinite = nonfinite || maxk >= K::kPosInf;

  // -- row status --------------------------------------------------------------
  if (!any_legal) { finish_error(QS_ROW_EMPTY); return pool_raw; }
  if (nonfinite) { finish_error(QS_ROW_NONFINITE); return pool_raw; }
  if (maxk <= K::kNegInf) { finish_error(QS_ROW_ALL_NEG_INF); return pool_raw; }

  const double m = (double)K::value(maxk);

  // -- source selection (hit test) -------------------------------------------
  // top-k hit: k < |Z_t| <= |F|. Top-p only: the pool must hold a mass of at
  // least p * W_F, with the background mass below t only known within +-err.
  bool use_pool = pool_ok;
  bool mass_test = false;
  if (use_pool && !greedy) {
    if (kk > 0 && (uint32_t)kk < ccount) {
      // top-k hit
    } else if (pool_all) {
      // the pool is all of F
    } else if (need_bg) {
      mass_test = true;
    } else {
      use_pool = false;  // k >= |Z_t| with |F| unknown, or everything kept
    }
  }
  // bf16 pools: fp64 weight of every histogram key (one key per thread)
  const bool hist_t = DT == 1 && use_pool && !greedy && !hist_over;
  const int hb = kHistBins - 1 - tid;  // this thread's key (thread 0 holds the top key)
  uint32_t h_own = 0u;
  double w_own = 0.0;
  if constexpr (DT == 1) {
    if (hist_t) {
      h_own = hist[hb];
      const uint32_t key = tkey + (uint32_t)hb;
      if (h_own && key <= maxk) w_own = weight<DT>(key, m, invT);
      binw[hb] = w_own;
    }
  }
  if (hist_t) __syncthreads();  // the weight table is read by every wave below
  double w_f = -1.0, w_f_err = 0.0;
  int rounds = 0;
  bool failed = false;
  // The boundary (pstar, n_keep, w_star): keep key > pstar and the first n_keep
  // ids of key == pstar, whose weight is w_star. `settled` once it is known.
  bool settled = false;
  uint32_t kap = 0u, n_keep_k = 0u;
  uint32_t pstar = K::kNegInf;  // keep-all: every source key is above it
  uint32_t n_keep = 0u;
  double w_star = 0.0;
  // -- single-wave scans of the bf16 pool histogram ---------------------------
  // Wave 0 alone reads the 1024 key bins, 16 per lane from the top key down,
  // and finds the top-k boundary (suffix counts reaching k: the page's stop
  // test N_tau >= k > N_tau - N_zm evaluated at every key) and the top-p
  // boundary (suffix fp64 masses reaching p * W) with DPP prefix sums; the
  // other waves wait at the barrier that publishes the result.
  if (hist_t && !(a.flags & (QS_FLAG_PIVOT_SEARCH | (SRT ? QS_FLAG_SORT_SUBSET : 0u))) &&
      use_pool) {
    const bool tk = kk > 0 && (uint32_t)kk < ccount;
    double bg_mass = bgm;
    double bg_bound = bgb;
    for (int attempt = 0; attempt < 2; ++attempt) {
      if (w == 0) {
        // pass 1: lane l sums bins 1023-16l .. 1008-16l; a DPP prefix over the
        // lanes finds the group of 16 bins holding the boundary; pass 2: lane
        // i < 16 takes bin i of that group and a 16-lane prefix finds the bin.
        const int b0 = kHistBins - 1 - 16 * lane;
        const uint4* const h4 = reinterpret_cast<const uint4*>(hist + (b0 - 15));
        uint32_t kapb = 0u, nkk = 0u;
        if (tk) {
          uint32_t ls = 0u;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint4 v = h4[q];
            ls += v.x + v.y + v.z + v.w;
          }
          const uint32_t incl = scan_incl_u32(ls);
          const int L = __ffsll((unsigned long long)ballot(incl >= (uint32_t)kk)) - 1;
          const uint32_t gex = readlane_u32(incl - ls, L);  // tokens above group L
          const int bi = kHistBins - 1 - 16 * L - (lane & 15);
          const uint32_t hi = lane < 16 ? hist[bi] : 0u;
          const uint32_t gin = gex + scan_incl_u32(hi);  // lanes >= 16 hold junk
          const uint64_t f = ballot(lane < 16 && gin >= (uint32_t)kk) ;
          const int i = __ffsll((unsigned long long)f) - 1;
          kapb = (uint32_t)(kHistBins - 1 - 16 * L - i);
          nkk = (uint32_t)kk - (readlane_u32(gin, i) - readlane_u32(hi, i));
        }
        // restricted count of bin b: inside the top-k set only
        auto hpf = [&](uint32_t b, uint32_t h) -> uint32_t {
          return !tk ? h : (b > kapb ? h : (b == kapb ? nkk : 0u));
        };
        uint32_t ok = 1u, pb = 0xFFFFFFFFu, nk = 0u, refine = 0u, bad = 0u;
        double wz = 0.0, w_ref = 0.0;
        if (topp_on) {
          double ls = 0.0;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint4 v = h4[q];
            const uint32_t hq[4] = {v.x, v.y, v.z, v.w};  // bins b0-15+4q .. b0-12+4q
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int b = b0 - 15 + 4 * q + j;
              ls += (double)hpf((uint32_t)b, hq[j]) * binw[b];
            }
          }
          const double incl = scan_incl_f64(ls);
          const double excl = incl_shift1_f64(incl);
          const double total = readlane_f64(incl, 63);
          double err = 0.0;
          w_ref = total;
          if (mass_test) {
            w_ref = total + bg_mass;
            err = bg_bound;
            ok = total >= p * (w_ref + err) * (1.0 + 1e-9) ? 1u : 0u;
          }
          if (ok) {
            const double target = p * w_ref;
            const uint64_t bal = ballot(incl >= target);
            const int L = bal ? __ffsll((unsigned long long)bal) - 1 : 63;
            const double gex = readlane_f64(excl, L);  // mass above group L
            const int bi = kHistBins - 1 - 16 * L - (lane & 15);
            const uint32_t hp = lane < 16 ? hpf((uint32_t)bi, hist[bi]) : 0u;
            const double wb = lane < 16 ? binw[bi] : 0.0;
            const double Mi = (double)hp * wb;
            const double gin = scan_incl_f64(Mi);
            const double run = gex + gin;  // mass down to and including bin bi
            const uint64_t f = ballot(lane < 16 && Mi > 0.0 && run >= target);
            const uint64_t any = ballot(lane < 16 && Mi > 0.0);
            // the first bin whose inclusive mass reaches the target; if rounding
            // leaves none in the group, its last weighted bin
            const int i = f ? __ffsll((unsigned long long)f) - 1
                            : (any ? 63 - __clzll((long long)any) : -1);
            if (i < 0) {
              bad = 1u;
            } else {
              pb = (uint32_t)(kHistBins - 1 - 16 * L - i);
              const double below = gex + (readlane_f64(gin, i) - readlane_f64(Mi, i));
              wz = readlane_f64(wb, i);
              const uint32_t c = readlane_u32(hp, i);
              // smallest count of boundary tokens that reaches the target
              const double need = (target - below) / wz;
              nk = need <= 1.0 ? 1u : (need >= (double)c ? c : (uint32_t)ceil(need));
              while (nk > 1u && below + (double)(nk - 1u) * wz >= target) --nk;
              while (nk < c && below + (double)nk * wz < target) ++nk;
              const double w_p = below + (double)nk * wz;
              // the same cut for every reference mass in [w_ref - err, w_ref + err]?
              const double lo_t = p * (w_ref - err), hi_t = p * (w_ref + err);
              const double prev = below + (double)(nk - 1u) * wz;
              refine = (err > 0.0 && !(prev < lo_t && hi_t <= w_p)) ? 1u : 0u;
            }
          }
        } else if (tk) {
          pb = kapb;
          nk = nkk;
          wz = binw[kapb];
        }
        if (lane == 0) {
          info.sc_u[0] = ok; info.sc_u[1] = kapb; info.sc_u[2] = nkk; info.sc_u[3] = pb;
          info.sc_u[4] = nk; info.sc_u[5] = refine; info.sc_u[6] = bad;
          info.sc_d[0] = wz; info.sc_d[1] = w_ref;
        }
      }
      __syncthreads();
      const bool ok = uni(info.sc_u[0]) != 0u;
      const bool refine = uni(info.sc_u[5]) != 0u;
      rounds = attempt + 1;
      if (!ok) { use_pool = false; break; }
      if (uni(info.sc_u[6]) != 0u) { failed = true; settled = true; break; }
      if (!refine) {
        settled = true;
        if (tk) { kap = tkey + uni(info.sc_u[1]); n_keep_k = uni(info.sc_u[2]); }
        const uint32_t pbv = uni(info.sc_u[3]);
        if (pbv != 0xFFFFFFFFu) {
          pstar = tkey + pbv;
          n_keep = uni(info.sc_u[4]);
          w_star = uni(info.sc_d[0]);
        }
        w_f = uni(info.sc_d[1]);
        break;
      }
      // exact background mass: fp64 over every finite legal token below t
      double sx = 0.0;
      walk_row<DT, false>(sl, lane, [&](const uint32_t (&key)[8], const uint32_t (&)[8],
                                        uint32_t vm) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (((vm >> j) & 1u) && key[j] < tkey) sx += weight<DT>(key[j], m, invT);
      });
      bg_mass = block_sum_f64(sx);
      bg_bound = 0.0;
    }
  }
  if (mass_test && !settled && use_pool) {
    double sx = 0.0;
    if (hist_t) {
      sx = (double)h_own * w_own;
    } else {
      walk_pool<DT>(pk, pid, my_cnt, (uint32_t)sl.wb, lane,
                    [&](const uint32_t (&key)[8], const uint32_t (&)[8], uint32_t vm) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (((vm >> j) & 1u) && key[j] >= tkey) sx += weight<DT>(key[j], m, invT);
      });
    }
    const double w_pool = block_sum_f64(sx);
    w_f = w_pool + bgm;
    w_f_err = bgb;
    use_pool = w_pool >= p * (w_f + w_f_err) * (1.0 + 1e-9);
  }
  if (!use_pool) {
    w_f = -1.0;
    w_f_err = 0.0;
    if (!nf_known) {  // count the finite legal tokens of the row
      uint32_t nf = 0u;
      walk_row<DT, true>(sl, lane, [&](const uint32_t (&key)[8], const uint32_t (&)[8],
                                       uint32_t lm) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          nf += (((lm >> j) & 1u) && key[j] > K::kNegInf) ? 1u : 0u;
      });
      nfin = block_sum_u32(nf);
    }
  }
  const bool topk_eff = !greedy && kk > 0 && (uint32_t)kk < (use_pool ? ccount : nfin);
  const bool use_hist = hist_t && use_pool;
  uint32_t src_lo = use_pool ? tkey : K::kNegInf + 1u;  // every source key >= src_lo

  // items of the pivot searches: (key, multiplicity) from the histogram, else tokens
  auto for_items = [&](auto&& f) {
    if (DT == 1 && use_hist) {
      if (h_own) f(tkey + (uint32_t)hb, h_own);
    } else {
      auto g = [&](const uint32_t (&key)[8], const uint32_t (&)[8], uint32_t vm) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if ((vm >> j) & 1u) f(key[j], 1u);
      };
      if (use_pool) walk_pool<DT>(pk, pid, my_cnt, (uint32_t)sl.wb, lane, g);
      else walk_row<DT, false>(sl, lane, g);
    }
  };
  // walk the chosen token source (pool or row), in id order per wave
  auto walk = [&](auto&& f) {
    if (use_pool) walk_pool<DT>(pk, pid, my_cnt, (uint32_t)sl.wb, lane, f);
    else walk_row<DT, false>(sl, lane, f);
  };
  // fp64 weight of a source key (histogram keys from the table)
  auto wkey = [&](uint32_t key) -> double {
    if constexpr (DT == 1) {
      if (use_hist) return binw[key - tkey];
    }
    return weight<DT>(key, m, invT);
  };
  // mass of source items with key > lo_excl
  auto mass_above = [&](uint32_t lo_excl) -> double {
    double s = 0.0;
    for_items([&](uint32_t key, uint32_t c) {
      if (key > lo_excl) s += (double)c * wkey(key);
    });
    return block_sum_f64(s);
  };

  // ablation switch: one pivot per round (the midpoint of the key interval)
  // instead of three at its quarters (page "Qrita", ablation table, binary
  // pivot runs); the stop tests are unchanged, only the round count grows
  const bool binary_pivot = (a.flags & QS_FLAG_BINARY_PIVOT) != 0u;

  // Radix select (flags 0; sources other than the bf16 pool histogram, which
  // the scans above settle): the key digits from the top, so that a search
  // walks its items (pool or row) once per level: fp32 keys in three levels
  // (11, 11 and 10 bits, 2048 bins), bf16 keys in two (8 bits, 256 bins),
  // rather than once per pivot round. Bins of counts and fp64 masses for one
  // level are shared by the waves (LDS atomics; the masses only place the
  // boundary, the outputs' probabilities come from the walks below); wave 0
  // scans them from the top digit down. Switched runs keep the page's pivot
  // rounds.
  constexpr int kKeyBits = DT == 1 ? 16 : 32;
  const bool radix = a.flags == 0u && !use_hist;
  bool to_pool = false;  // a full-row source replaced by a key range of it in the pools
  constexpr int kRBins = DT == 1 ? 256 : 2048;
  // digits of a search: 8 bits a level over pools and samples (few items, 256
  // bins), 11 + 11 + 10 over fp32 rows (every token walked once per level)
  auto n_levels = [](bool wide) { return DT == 1 ? 2 : (wide ? 3 : 4); };
  auto lvl_shift = [](bool wide, int l) {
    return (DT == 1 || !wide) ? kKeyBits - 8 - 8 * l : (l == 0 ? 21 : (l == 1 ? 10 : 0));
  };
  auto lvl_width = [](bool wide, int l) { return (DT == 1 || !wide) ? 8 : (l == 2 ? 10 : 11); };
  // counts: 4 interleaved copies (entry 4 b + lane % 4) on levels without
  // masses, so that the lanes of one wave that hit one bin spread over 4 LDS
  // banks; one copy next to the masses otherwise
  uint32_t* const rb_c = DT == 1 ? hist : rb_f32;
  double* const rb_m = DT == 1 ? binw : reinterpret_cast<double*>(rb_f32 + kRBins);
  static_assert(DT == 1 || kRBins + 2 * kRBins <= 8192, "fp32 radix masses");
  static_assert(DT == 1 || 4 * kRBins <= 8192, "fp32 radix bins");
  static_assert(DT == 0 || 4 * kRBins <= kHistBins, "bf16 radix bins");
  // One level: bins of the digit at `shift` (`width` bits) of the source keys
  // that share the digits above it with `prefix` (and, with masses, lie above
  // `excl`), plus an extra bucket of xcnt tokens of key xkey (the top-k
  // boundary tokens inside the top-k set). Returns, through info, the digit b
  // whose bin holds the `need`-th largest key (counts) or where the
  // descending mass from `above` reaches `target` (masses), with the count or
  // mass of the bins above b and b's own count.
  // The bins are clear when a level starts: radix_begin clears them before a
  // search, and wave 0 clears them again once it has scanned a level. The
  // results alternate between two slots of info, so that a level's result is
  // read while the next level's is being written without another barrier.
  int rpar = 0;
  auto radix_begin = [&]() {
    for (int i = tid; i < kRBins; i += kThreads) {
      reinterpret_cast<uint4*>(rb_c)[i] = make_uint4(0u, 0u, 0u, 0u);
      rb_m[i] = 0.0;
    }
    __syncthreads();
  };
  struct RLevel {
    uint32_t b, c_above, c_hit;
    double m_above;
  };
  // (items may pass keys as offsets from kofs: the weights are those of x + kofs)
  auto radix_level = [&](auto&& items, int shift, int width, uint32_t prefix, bool masses,
                         uint32_t excl, double above, uint32_t need, double target,
                         uint32_t xkey, uint32_t xcnt, double xmass,
                         uint32_t kofs = 0u) -> RLevel {
    const int nb = 1 << (width > 8 ? width : 8);  // bins of this level (a multiple of 64)
    const int bpl = nb / 64;                  // bins per lane of the scan
    const int slot = rpar;
    rpar ^= 1;
    const uint32_t hmask = shift + width >= 32 ? 0u : (0xFFFFFFFFu << (shift + width));
    const uint32_t dmask = (1u << width) - 1u;
    const uint32_t hpre = prefix & hmask;
    // masses: consecutive items of one bin are summed in the lane first, one
    // pair of atomics per run of the same bin
    uint32_t run_b = 0xFFFFFFFFu, run_c = 0u;
    double run_m = 0.0;
    items([&](uint32_t x, uint32_t c) {
      if ((x & hmask) == hpre && (!masses || x + kofs > excl)) {
        const uint32_t b = (x >> shift) & dmask;
        if (!masses) {
          __hip_atomic_fetch_add(rb_c + 4u * b + (uint32_t)(lane & 3), c, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
        } else {
          if (b != run_b) {
            if (run_b != 0xFFFFFFFFu) {
              __hip_atomic_fetch_add(rb_c + run_b, run_c, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_WORKGROUP);
              __hip_atomic_fetch_add(rb_m + run_b, run_m, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_WORKGROUP);
            }
            run_b = b;
            run_c = 0u;
            run_m = 0.0;
          }
          run_c += c;
          run_m += (double)c * wkey(x + kofs);
        }
      }
    });
    if (run_b != 0xFFFFFFFFu) {
      __hip_atomic_fetch_add(rb_c + run_b, run_c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      __hip_atomic_fetch_add(rb_m + run_b, run_m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (tid == 0 && xcnt && (xkey & hmask) == hpre) {
      const uint32_t b = (xkey >> shift) & dmask;
      __hip_atomic_fetch_add(rb_c + (masses ? b : 4u * b), xcnt, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_WORKGROUP);
      if (masses)
        __hip_atomic_fetch_add(rb_m + b, xmass, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();
    if (w == 0) {
      // lane l: bins top - bpl l down to top - bpl l - bpl + 1 (descending)
      const int top = nb - 1 - bpl * lane;
      auto cnt_of = [&](int b) -> uint32_t {
        if (masses) return rb_c[b];
        const uint4 v = reinterpret_cast<const uint4*>(rb_c)[b];
        return (v.x + v.y) + (v.z + v.w);
      };
      uint32_t cl = 0u;
      double ml = 0.0;
#pragma unroll 4
      for (int q = 0; q < bpl; ++q) {
        cl += cnt_of(top - q);
        if (masses) ml += rb_m[top - q];
      }
      int b_hit = -1;
      uint32_t c_above = 0u, c_hit = 0u;
      double m_above = 0.0;
      if (!masses) {
        const uint32_t incl = scan_incl_u32(cl);
        uint32_t run = incl - cl;
        if (run < need && need <= incl) {
#pragma unroll 4
          for (int q = 0; q < bpl; ++q) {
            const uint32_t cq = cnt_of(top - q);
            if (b_hit < 0 && run < need && need <= run + cq) {
              b_hit = top - q;
              c_above = run;
              c_hit = cq;
            }
            run += cq;
          }
        }
      } else {
        const double incl = scan_incl_f64(ml);
        double run = above + incl_shift1_f64(incl);
        int b_last = -1;
        double m_last = 0.0;
        uint32_t c_last = 0u;
        if (cl) {
#pragma unroll 4
          for (int q = 0; q < bpl; ++q) {
            const uint32_t cq = rb_c[top - q];
            const double mq = rb_m[top - q];
            if (cq) {
              if (b_hit < 0 && run < target && run + mq >= target) {
                b_hit = top - q;
                m_above = run;
                c_hit = cq;
              }
              if (b_hit < 0) {
                b_last = top - q;
                m_last = run;
                c_last = cq;
              }
            }
            run += mq;
          }
        }
        if (ballot(b_hit >= 0) == 0u) {
          // rounding left the target above every prefix: the lowest weighted bin
          const uint64_t anyb = ballot(b_last >= 0);
          const int L = anyb ? 63 - __clzll((long long)anyb) : -1;
          if (L >= 0 && lane == L) { b_hit = b_last; m_above = m_last; c_hit = c_last; }
        }
      }
      const uint64_t f = ballot(b_hit >= 0);
      const int L = f ? __ffsll((unsigned long long)f) - 1 : -1;
      if (lane == (L < 0 ? 0 : L)) {
        info.sc_u[4 * slot + 0] = L < 0 ? 0xFFFFFFFFu : (uint32_t)b_hit;
        info.sc_u[4 * slot + 1] = c_above;
        info.sc_u[4 * slot + 2] = c_hit;
        info.sc_d[slot] = m_above;
      }
      // clear this level's bins for the next one
      for (int i = lane; i < nb; i += 64) {
        reinterpret_cast<uint4*>(rb_c)[i] = make_uint4(0u, 0u, 0u, 0u);
        if (masses) rb_m[i] = 0.0;
      }
    }
    __syncthreads();
    RLevel res;
    res.b = uni(info.sc_u[4 * slot + 0]);
    res.c_above = uni(info.sc_u[4 * slot + 1]);
    res.c_hit = uni(info.sc_u[4 * slot + 2]);
    res.m_above = uni(info.sc_d[slot]);
    return res;
  };

  // Bucket select over an fp32 pool (flags 0): the pool keys lie in [lo, hi];
  // one level counts them in 1024 buckets of width 2^s spanning that range
  // (s from the span, so the buckets follow the keys actually present rather
  // than fixed digits), and the level's boundary bucket becomes the range of
  // the next. Once that bucket holds at most 64 tokens, its tokens are
  // gathered into one wave, sorted by key and searched directly. Returns the
  // boundary key, the count of its tokens, and what lies above it (the count
  // still needed, or the mass). Masses: only items above excl count; the
  // extra bucket holds xcnt tokens of key xkey (the top-k set's boundary).
  struct RSel {
    bool ok;
    uint32_t key, c_key, need_rest;
    double above;
  };
  // 256 buckets for pools of up to 4096 tokens, 1024 above
  const int kBktBits = ccount_all <= 4096u ? 8 : 10;
  uint32_t* const glist = DT == 0 ? rb_f32 + 4096 : hist;  // 64 (key, count) pairs, a counter
  auto bucket_select = [&](bool masses, uint32_t lo, uint32_t hi, uint32_t excl, uint32_t need,
                           double target, uint32_t xkey, uint32_t xcnt, double xmass) -> RSel {
    RSel out{false, 0u, 0u, need, 0.0};
    double above = 0.0;
    radix_begin();
    for (int it = 0; it < 6; ++it) {
      const uint32_t span = hi - lo;
      const int nbits = span == 0u ? 0 : 32 - __clz(span);
      const int sh = nbits > kBktBits ? nbits - kBktBits : 0;
      const uint32_t blo = lo, bhi = hi;
      auto items = [&](auto&& f) {
        for_items([&](uint32_t x, uint32_t c) {
          if (x >= blo && x <= bhi && (!masses || x > excl)) f(x - blo, c);
        });
      };
      const bool xin = xcnt && xkey >= lo && xkey <= hi;
      const RLevel rl = radix_level(items, sh, kBktBits, 0u, masses, excl, above, need, target,
                                    xin ? xkey - lo : 0u, xin ? xcnt : 0u, xmass, lo);
      ++rounds;
      if (rl.b == 0xFFFFFFFFu) return out;  // (never: the range holds the boundary)
      if (masses) above = rl.m_above;
      else need -= rl.c_above;
      lo = blo + (rl.b << sh);
      hi = min(bhi, lo + ((1u << sh) - 1u));
      if (sh == 0) {  // one key
        out.ok = true;
        out.key = lo;
        out.c_key = rl.c_hit;
        out.need_rest = need;
        out.above = above;
        return out;
      }
      if (rl.c_hit > 64u) continue;
      // gather the bucket's tokens (at most 64 entries) and finish in wave 0
      if (tid == 0) glist[128] = 0u;
      __syncthreads();
      const uint32_t glo = lo, ghi = hi;
      for_items([&](uint32_t x, uint32_t c) {
        if (x >= glo && x <= ghi && (!masses || x > excl)) {
          const uint32_t q = atomicAdd(glist + 128, 1u);
          if (q < 64u) { glist[2 * q] = x; glist[2 * q + 1] = c; }
        }
      });
      if (tid == 0 && xcnt && xkey >= glo && xkey <= ghi) {
        const uint32_t q = atomicAdd(glist + 128, 1u);
        if (q < 64u) { glist[2 * q] = xkey; glist[2 * q + 1] = xcnt; }
      }
      __syncthreads();
      const int slot = rpar;
      rpar ^= 1;
      if (w == 0) {
        const uint32_t n = uni(min(glist[128], 64u));
        uint32_t key = (uint32_t)lane < n ? glist[2 * lane] : 0u;
        uint32_t cnt = (uint32_t)lane < n ? glist[2 * lane + 1] : 0u;
        // every entry against every other (readlane broadcasts, no ordering
        // needed): the tokens, and for masses the mass, of the larger keys
        const double wl = (masses && cnt) ? (double)cnt * wkey(key) : 0.0;
        uint32_t c_gt = 0u, c_eq = 0u;
        double m_gt = 0.0, m_eq = 0.0;
        for (int jj = 0; jj < (int)n; ++jj) {
          const uint32_t kj = readlane_u32(key, jj);
          const uint32_t cj = readlane_u32(cnt, jj);
          c_gt += kj > key ? cj : 0u;
          c_eq += kj == key ? cj : 0u;
          if (masses) {
            const double wj = readlane_f64(wl, jj);
            m_gt += kj > key ? wj : 0.0;
            m_eq += kj == key ? wj : 0.0;
          }
        }
        // the boundary: the largest key whose tokens, with those above, reach
        // the count or the mass
        const bool live = (uint32_t)lane < n && cnt != 0u;
        bool q;
        if (!masses) q = live && c_gt < need && need <= c_gt + c_eq;
        else q = live && above + m_gt < target && above + m_gt + m_eq >= target;
        uint64_t hit = ballot(q);
        if (masses && !hit) {
          // rounding left the target above every prefix: the lowest weighted key
          const uint32_t kmin = wave_reduce<OpMin>(live && wl > 0.0 ? key : 0xFFFFFFFFu);
          hit = ballot(live && key == kmin);
        }
        const int L = hit ? __ffsll((unsigned long long)hit) - 1 : -1;
        const uint32_t kL = L < 0 ? 0u : readlane_u32(key, L < 0 ? 0 : L);
        const uint32_t cgtL = L < 0 ? 0u : readlane_u32(c_gt, L < 0 ? 0 : L);
        const uint32_t ceqL = L < 0 ? 0u : readlane_u32(c_eq, L < 0 ? 0 : L);
        const double mgtL = L < 0 ? 0.0 : readlane_f64(m_gt, L < 0 ? 0 : L);
        if (lane == 0) {
          info.sc_u[4 * slot + 0] = (L < 0 || glist[128] > 64u) ? 0xFFFFFFFFu : kL;
          info.sc_u[4 * slot + 1] = cgtL;
          info.sc_u[4 * slot + 2] = ceqL;
          info.sc_d[slot] = above + mgtL;
        }
      }
      __syncthreads();
      const uint32_t kr = uni(info.sc_u[4 * slot + 0]);
      if (kr == 0xFFFFFFFFu) return out;  // (never: at most 64 entries hold the boundary)
      out.ok = true;
      out.key = kr;
      out.c_key = uni(info.sc_u[4 * slot + 2]);
      out.need_rest = need - uni(info.sc_u[4 * slot + 1]);
      out.above = uni(info.sc_d[slot]);
      return out;
    }
    return out;
  };
  // the bucket select serves fp32 pools; bf16 pools without a value histogram
  // and full rows take the radix levels
  auto use_bucket = [&]() { return DT == 0 && radix && use_pool; };

  // -- a missed truncation with top-k: a second threshold from the sample -----------
  // The source is the whole row. The first step of every slice (the tokens
  // the row statistics came from) estimates the key above which about 2k
  // tokens of the row lie: the sample's R-th largest key, R = 2k n_s / |F| + 8
  // (a radix select over the sample). One walk appends every legal token at
  // or above it to the wave pools; when they hold all of them and at least k,
  // the k-th largest key is among them and the pools become the source of the
  // searches and output walks below. Otherwise the row stays the source.
  if (topk_eff && radix && !use_pool && a.seg <= 65536) {
    Raw<DT> sraw;
    uint32_t smb = 0u;
    {
      RowReader<DT, 1> rd(sl, lane);
      if (rd.n > 0) {
        rd.issue(0, 0);
        rd.fetch(0, 0, sraw, smb);
      }
    }
    uint32_t skey[8], svm = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      skey[j] = K::of(sraw.bits(j));
      const bool ok = ((smb >> j) & 1u) && skey[j] > K::kNegInf && skey[j] < K::kPosInf;
      svm |= (ok ? 1u : 0u) << j;
    }
    const uint32_t ns = uni(block_sum_u32((uint32_t)__popc(svm)));
    if (ns > 0u) {
      const uint64_t r2 = (2ull * (uint64_t)kk * ns + nfin - 1u) / nfin + 8u;
      uint32_t need = (uint32_t)min(r2, (uint64_t)ns);
      auto sample_items = [&](auto&& f) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if ((svm >> j) & 1u) f(skey[j], 1u);
      };
      uint32_t lk = 0u;
      radix_begin();
      for (int l = 0; l < n_levels(false); ++l) {
        const int shift = lvl_shift(false, l);
        const RLevel rl =
            radix_level(sample_items, shift, 8, lk, false, 0u, 0.0, need, 0.0, 0u, 0u, 0.0);
        if (rl.b == 0xFFFFFFFFu) { lk = K::kMax; break; }  // (never: need <= n_s)
        need -= rl.c_above;
        lk |= rl.b << shift;
      }
      if (lk != K::kMax) {
        uint32_t pc = 0u;
        stream_slice<DT, 2>(sl, lane, [&](const Raw<DT>& raw, uint32_t mb, int e) {
          uint32_t cb = 0u;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            cb |= (((mb >> j) & 1u) && K::of(raw.bits(j)) >= lk) ? (1u << j) : 0u;
          pc = append_pool<DT>(cb, raw, (uint32_t)(e - sl.wb), pc, my_pk, my_pid);
        });
        if (lane == 0) info.cnt[w] = pc;
        __syncthreads();
        const uint32_t cn = act16 ? info.cnt[lane] : 0u;
        const bool ovf = uni(wave_reduce<OpMax>(cn > kCap ? 1u : 0u)) != 0u;
        const uint32_t tot = uni(wave_reduce<OpSum>(cn));
        __syncthreads();  // info.cnt is read before it is written again
        if (!ovf && tot >= (uint32_t)kk) {
          use_pool = true;
          to_pool = true;
          my_cnt = (int)pc;
          src_lo = lk;
        }
      }
    }
  }

  // Ablation switch (page "Qrita", ablation table, run I): on a truncation
  // hit the candidate subset is sorted in LDS (keys descending, a bitonic
  // network over the next power of two, at most kSortMax candidates) and the
  // top-k and top-p boundaries are read off the sorted order instead of
  // searched. Larger subsets, and top-p cuts the subset does not reach, take
  // the searches below. The buffer is LDS the searches do not use then: the
  // radix bins (fp32) or the background histogram (bf16, read before).
  // (bf16 keys are 16-bit: 2 bytes an entry)
  constexpr uint32_t kSortMax = 8192u;
  using SKey = typename PL::KeyT;
  SKey* const sbuf = reinterpret_cast<SKey*>(DT == 0 ? rb_f32 : bgh);
  static_assert(sizeof(rb_f32) >= kSortMax * sizeof(SKey) || DT == 1, "fp32 sort buffer");
  static_assert(sizeof(bgh) >= kSortMax * sizeof(SKey) || DT == 0, "bf16 sort buffer");
  if (SRT && (a.flags & QS_FLAG_SORT_SUBSET) && use_pool && !settled && !greedy) {
    if (tid == 0) s_sort[0] = 0u;
    __syncthreads();
    walk_pool<DT>(pk, pid, my_cnt, (uint32_t)sl.wb, lane,
                  [&](const uint32_t (&key)[8], const uint32_t (&)[8], uint32_t vm)
                      __attribute__((always_inline)) {
      if (vm) {
        uint32_t at = __hip_atomic_fetch_add(s_sort, (uint32_t)__popc(vm), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if ((vm >> j) & 1u) {
            if (at < kSortMax) sbuf[at] = (SKey)key[j];
            ++at;
          }
        }
      }
    });
    __syncthreads();
    const uint32_t n = uni(s_sort[0]);
    if (n <= kSortMax) {
      uint32_t N = 2u;
      while (N < n) N <<= 1;
      for (uint32_t i = n + (uint32_t)tid; i < N; i += kThreads) sbuf[i] = (SKey)0;  // below every key
      __syncthreads();
      for (uint32_t size = 2u; size <= N; size <<= 1) {
        for (uint32_t stride = size >> 1; stride > 0u; stride >>= 1) {
          for (uint32_t t = (uint32_t)tid; t < N / 2u; t += kThreads) {
            const uint32_t i = 2u * t - (t & (stride - 1u));
            const uint32_t j = i + stride;
            const SKey x = sbuf[i], y = sbuf[j];
            const bool down = (i & size) == 0u;  // this run of `size` ends descending
            if (down ? x < y : x > y) {
              sbuf[i] = y;
              sbuf[j] = x;
            }
          }
          __syncthreads();
        }
      }
      // entries of the sorted subset's first lim that lie above key x
      auto sorted_above = [&](uint32_t x, uint32_t lim) -> uint32_t {
        double c = 0.0;
        for (uint32_t i = (uint32_t)tid; i < lim; i += kThreads)
          c += (uint32_t)sbuf[i] > x ? 1.0 : 0.0;
        return (uint32_t)block_sum_f64(c);
      };
      // top-k: the k-th entry and the entries above it
      uint32_t skap = 0u, snk = 0u;
      if (topk_eff) {
        skap = uni((uint32_t)sbuf[kk - 1]);
        snk = (uint32_t)kk - sorted_above(skap, (uint32_t)kk);
      }
      if (topp_on) {
        // top-p over the sorted top-k set (every entry without top-k): running
        // fp64 sums, thread t taking a run of consecutive entries; the cut is
        // the first entry whose running sum reaches p W (the smallest index
        // any thread claims). A cut the subset does not reach, or one that the
        // fp32 background's error bound leaves open, goes to the searches.
        const double w_ref = topk_eff ? mass_above(skap) + (double)snk * wkey(skap)
                                      : (w_f >= 0.0 ? w_f : mass_above(0u));
        const double err = topk_eff ? 0.0 : w_f_err;
        const double target = p * w_ref;
        const uint32_t L = topk_eff ? (uint32_t)kk : n;
        const uint32_t c = (L + kThreads - 1u) / kThreads;
        const uint32_t i0 = min((uint32_t)tid * c, L), i1 = min(i0 + c, L);
        double sw = 0.0;
        for (uint32_t i = i0; i < i1; ++i) sw += wkey((uint32_t)sbuf[i]);
        const double incl = scan_incl_f64(sw);
        if (lane == 63) info.mass[w] = incl;
        if (tid == 0) s_sort[0] = 0xFFFFFFFFu;
        __syncthreads();
        double cum = incl - sw;
        for (int ww = 0; ww < kWaves; ++ww) cum += ww < w ? info.mass[ww] : 0.0;
        double prev = 0.0, at = 0.0;
        uint32_t jx = 0xFFFFFFFFu;
        if (cum < target) {
          for (uint32_t i = i0; i < i1; ++i) {
            const double wi = wkey((uint32_t)sbuf[i]);
            if (cum + wi >= target) {
              jx = i;
              prev = cum;
              at = cum + wi;
              break;
            }
            cum += wi;
          }
        }
        if (jx != 0xFFFFFFFFu)
          __hip_atomic_fetch_min(s_sort, jx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __syncthreads();
        const uint32_t jw = uni(s_sort[0]);
        if (jx != 0xFFFFFFFFu && jx == jw) {
          info.sel_d[0] = prev;
          info.sel_d[1] = at;
        }
        __syncthreads();
        if (jw != 0xFFFFFFFFu) {
          const double pv = uni(info.sel_d[0]), w_p = uni(info.sel_d[1]);
          const bool open = err > 0.0 && !(pv < p * (w_ref - err) && p * (w_ref + err) <= w_p);
          if (!open) {
            pstar = uni((uint32_t)sbuf[jw]);
            n_keep = jw + 1u - sorted_above(pstar, jw + 1u);
            w_star = wkey(pstar);
            kap = skap;
            n_keep_k = snk;
            settled = true;
          }
        }
      } else if (topk_eff) {
        kap = skap;
        n_keep_k = snk;
        pstar = skap;
        n_keep = snk;
        w_star = wkey(skap);
        settled = true;
      }
      ++rounds;
    }
  }

  // -- the k-th largest key (top-k) ----------------------------------------------
  if (topk_eff && !settled && radix) {
    uint32_t prefix = 0u, need = (uint32_t)kk, c_kap = 0u;
    const bool wide = !use_pool;
    if (use_bucket()) {
      const RSel rs = bucket_select(false, src_lo, maxk, 0u, need, 0.0, 0u, 0u, 0.0);
      if (!rs.ok) failed = true;
      prefix = rs.key;
      need = rs.need_rest;
      c_kap = rs.c_key;
    } else {
      radix_begin();
    }
    for (int l = 0; l < (use_bucket() ? 0 : n_levels(wide)) && !failed; ++l) {
      const int shift = lvl_shift(wide, l);
      const RLevel rl = radix_level(for_items, shift, lvl_width(wide, l), prefix, false, 0u, 0.0,
                                    need, 0.0, 0u, 0u, 0.0);
      if (rl.b == 0xFFFFFFFFu) { failed = true; break; }  // (never: k <= the finite count)
      need -= rl.c_above;
      c_kap = rl.c_hit;  // at the last level: the tokens of the key itself
      prefix |= rl.b << shift;
      ++rounds;
    }
    kap = prefix;
    n_keep_k = need;
    // A full-row source: every token at or above the k-th largest key (the
    // top-k set and the other ties at its boundary key) is appended, in id
    // order, to the wave pools, which replace the row as the source when they
    // hold it; the top-p search and the output walks then read the pools.
    if (!failed && !use_pool && a.seg <= 65536 &&
        (uint32_t)kk - n_keep_k + c_kap <= (uint32_t)(kWaves * kCap / 2)) {
      uint32_t pc = 0u;
      stream_slice<DT, 2>(sl, lane, [&](const Raw<DT>& raw, uint32_t mb, int e) {
        uint32_t cb = 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          cb |= (((mb >> j) & 1u) && K::of(raw.bits(j)) >= kap) ? (1u << j) : 0u;
        pc = append_pool<DT>(cb, raw, (uint32_t)(e - sl.wb), pc, my_pk, my_pid);
      });
      if (lane == 0) info.cnt[w] = pc;
      __syncthreads();
      const bool ovf = uni(wave_reduce<OpMax>(act16 && info.cnt[lane] > kCap ? 1u : 0u)) != 0u;
      if (!ovf) {
        use_pool = true;
        to_pool = true;
        my_cnt = (int)pc;
      }
    }
  } else if (topk_eff && !settled) {
    // quaternary three-pivot search on counts (page "Qrita", key design 2)
    uint32_t lo = src_lo - 1u, hi = maxk;
    bool found = false;
    while (!found) {
      if (rounds >= 48) { failed = true; break; }
      const uint32_t d = hi - lo;
      uint32_t tau[3];
#pragma unroll
      for (int n = 0; n < 3; ++n)
        tau[n] = binary_pivot ? lo + (d >> 1)
                 : d >= 4u    ? lo + (uint32_t)(((uint64_t)d * (uint64_t)(n + 1)) >> 2)
                              : min(lo + (uint32_t)n, hi - 1u);
      uint32_t N[3] = {0u, 0u, 0u};
      MinCnt mc[3] = {{0xFFFFFFFFu, 0u}, {0xFFFFFFFFu, 0u}, {0xFFFFFFFFu, 0u}};
      for_items([&](uint32_t x, uint32_t c) {
#pragma unroll
        for (int n = 0; n < 3; ++n) {
          if (x > tau[n]) {
            N[n] += c;
            if (x < mc[n].key) { mc[n].key = x; mc[n].cnt = c; }
            else if (x == mc[n].key) { mc[n].cnt += c; }
          }
        }
      });
#pragma unroll
      for (int n = 0; n < 3; ++n) {
        N[n] = wave_reduce<OpSum>(N[n]);
        mc[n] = wave_reduce_mc(mc[n]);
      }
      if (lane == 0) {
#pragma unroll
        for (int n = 0; n < 3; ++n) {
          red.v[par][w][3 * n] = N[n];
          red.v[par][w][3 * n + 1] = mc[n].key;
          red.v[par][w][3 * n + 2] = mc[n].cnt;
        }
      }
      __syncthreads();
#pragma unroll
      for (int n = 0; n < 3; ++n) {
        N[n] = 0u;
        mc[n] = MinCnt{0xFFFFFFFFu, 0u};
        for (int ww = 0; ww < kWaves; ++ww) {
          N[n] += red.v[par][ww][3 * n];
          mc[n] = mc_merge(mc[n], MinCnt{red.v[par][ww][3 * n + 1], red.v[par][ww][3 * n + 2]});
        }
        N[n] = uni(N[n]);
        mc[n].key = uni(mc[n].key);
        mc[n].cnt = uni(mc[n].cnt);
      }
      par ^= 1;
      ++rounds;
      const uint32_t kq = (uint32_t)kk;
#pragma unroll
      for (int n = 0; n < 3; ++n) {
        if (!found && N[n] >= kq && N[n] - mc[n].cnt < kq) {
          found = true;
          kap = mc[n].key;
          n_keep_k = kq - (N[n] - mc[n].cnt);
        }
      }
      if (!found) {
#pragma unroll
        for (int n = 0; n < 3; ++n) {
          if (N[n] >= kq) lo = tau[n] > lo ? tau[n] : lo;
          else hi = tau[n] < hi ? tau[n] : hi;
        }
      }
    }
  }

  // -- top-p over a small top-k set (fp32, flags 0, the pool as source, k <= 64):
  //    the set's keys are gathered, one wave sorts them and cuts at the first
  //    running fp64 mass that reaches p W_K, instead of a bucket select over
  //    the pool ----------------------------------------------------------------
  if constexpr (DT == 0) {
    if (radix && use_pool && topk_eff && topp_on && !settled && !failed && !greedy &&
        kk <= 64) {
      uint32_t* const sk = rb_f32;  // 64 keys, a counter, the result
      if (tid == 0) sk[64] = 0u;
      __syncthreads();
      walk([&](const uint32_t (&key)[8], const uint32_t (&)[8], uint32_t vm)
               __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (((vm >> j) & 1u) && key[j] > kap) {
            const uint32_t at = __hip_atomic_fetch_add(sk + 64, 1u, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            if (at < 64u) sk[at] = key[j];
          }
        }
      });
      __syncthreads();
      if (w == 0) {
        // the set: the keys above kap and n_keep_k copies of kap (kk in all)
        const uint32_t ca = sk[64];
        uint32_t key = (uint32_t)lane < ca ? sk[lane]
                       : ((uint32_t)lane < ca + n_keep_k ? kap : 0u);
#pragma unroll
        for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
          for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const uint32_t o = (uint32_t)__shfl_xor((int)key, stride, 64);
            const bool take_max = ((lane & stride) == 0) == ((lane & size) == 0);
            key = take_max ? max(o, key) : min(o, key);
          }
        }
        const bool on = lane < kk;
        const double wt = on ? wkey(key) : 0.0;
        const double incl = scan_incl_f64(wt);
        const double target = p * readlane_f64(incl, 63);
        const uint64_t hit = ballot(on && incl >= target);  // the last set entry reaches it
        const int j = __ffsll((unsigned long long)hit) - 1;
        const uint32_t ps = (uint32_t)__shfl((int)key, j, 64);
        const int first = __ffsll((unsigned long long)ballot(key == ps)) - 1;
        if (lane == 0) {
          sk[65] = ps;
          sk[66] = (uint32_t)(j + 1 - first);  // its ties needed
        }
      }
      __syncthreads();
      pstar = uni(sk[65]);
      n_keep = uni(sk[66]);
      w_star = wkey(pstar);
      settled = true;
    }
  }

  // -- final boundary (pstar, n_keep): keep key > pstar, and the first n_keep
  //    ids of key == pstar --------------------------------------------------
  if (greedy) {
    pstar = maxk;
    n_keep = 1u;
    w_star = 1.0;
  } else if (!failed && !settled) {
    const double w_kap = topk_eff ? wkey(kap) : 0.0;
    if (topp_on) {
      double w_k;
      if (topk_eff) w_k = mass_above(kap) + (double)n_keep_k * w_kap;
      else if (w_f >= 0.0) w_k = w_f;
      else w_k = mass_above(0u);
      // Quaternary three-pivot search on fp64 mass inside K. When the top-p
      // reference mass is only known within +-err (the background summed with
      // fp32 exp2), the cut must be the same at both ends of that interval;
      // otherwise the background is recomputed in fp64 and the search repeated.
      double err = topk_eff ? 0.0 : w_f_err;
      for (int attempt = 0; attempt < 2 && !failed; ++attempt) {
        const double target = p * w_k;
        uint32_t lo = (topk_eff ? kap : src_lo) - 1u, hi = maxk;
        const uint32_t excl = topk_eff ? kap : 0u;  // per-item terms only for key > excl
        bool found = false, refine = false;
        if (radix) {
          // digits from the top; the top-k boundary key counts n_keep_k tokens
          uint32_t prefix = 0u, c_star = 0u;
          double above = 0.0;
          const bool wide = !use_pool;
          if (use_bucket()) {
            const RSel rs = bucket_select(true, topk_eff ? kap : src_lo, maxk, excl, 0u, target,
                                          kap, topk_eff ? n_keep_k : 0u,
                                          topk_eff ? (double)n_keep_k * w_kap : 0.0);
            if (!rs.ok) failed = true;
            prefix = rs.key;
            c_star = rs.c_key;
            above = rs.above;
          } else {
            radix_begin();
          }
          for (int l = 0; l < (use_bucket() ? 0 : n_levels(wide)) && !failed; ++l) {
            const int shift = lvl_shift(wide, l);
            const RLevel rl = radix_level(
                for_items, shift, lvl_width(wide, l), prefix, true, excl, above, 0u, target, kap,
                topk_eff ? n_keep_k : 0u, topk_eff ? (double)n_keep_k * w_kap : 0.0);
            c_star = rl.c_hit;   // at the last level: the tokens of the key itself
            ++rounds;
            if (rl.b == 0xFFFFFFFFu) { failed = true; break; }  // (never: the top key has weight 1)
            above = rl.m_above;
            prefix |= rl.b << shift;
          }
          if (!failed) {
            // the boundary key, its count and weight, and the smallest count of
            // its tokens that reaches the target
            pstar = prefix;
            const double wz = wkey(pstar);
            const uint32_t c = c_star;   // (n_keep_k when pstar is the top-k boundary)
            const double below = above;
            w_star = wz;
            const double need = (target - below) / wz;
            uint32_t nk = need <= 1.0 ? 1u : (need >= (double)c ? c : (uint32_t)ceil(need));
            while (nk > 1u && below + (double)(nk - 1u) * wz >= target) --nk;
            while (nk < c && below + (double)nk * wz < target) ++nk;
            n_keep = nk;
            const double w_p = below + (double)nk * wz;
            const double lo_t = p * (w_k - err), hi_t = p * (w_k + err);
            const double prev = below + (double)(nk - 1u) * wz;
            refine = err > 0.0 && !(prev < lo_t && hi_t <= w_p);
            found = true;
          }
        }
        while (!found && !failed) {
          if (rounds >= 96) { failed = true; break; }
          const uint32_t d = hi - lo;
          uint32_t tau[3];
#pragma unroll
          for (int n = 0; n < 3; ++n)
            tau[n] = binary_pivot ? lo + (d >> 1)
                     : d >= 4u    ? lo + (uint32_t)(((uint64_t)d * (uint64_t)(n + 1)) >> 2)
                                  : min(lo + (uint32_t)n, hi - 1u);
          double Ms[3] = {0.0, 0.0, 0.0};
          MinCnt mc[3] = {{0xFFFFFFFFu, 0u}, {0xFFFFFFFFu, 0u}, {0xFFFFFFFFu, 0u}};
          for_items([&](uint32_t x, uint32_t c) {
            if (x > excl && x > tau[0]) {
              const double wt = (double)c * wkey(x);
#pragma unroll
              for (int n = 0; n < 3; ++n) {
                if (x > tau[n]) {
                  Ms[n] += wt;
                  if (x < mc[n].key) { mc[n].key = x; mc[n].cnt = c; }
                  else if (x == mc[n].key) { mc[n].cnt += c; }
                }
              }
            }
          });
#pragma unroll
          for (int n = 0; n < 3; ++n) {
            Ms[n] = wave_sum_f64(Ms[n]);
            mc[n] = wave_reduce_mc(mc[n]);
          }
          if (lane == 0) {
#pragma unroll
            for (int n = 0; n < 3; ++n) {
              uint64_t b = __double_as_longlong(Ms[n]);
              red.v[par][w][4 * n] = (uint32_t)b;
              red.v[par][w][4 * n + 1] = (uint32_t)(b >> 32);
              red.v[par][w][4 * n + 2] = mc[n].key;
              red.v[par][w][4 * n + 3] = mc[n].cnt;
            }
          }
          __syncthreads();
#pragma unroll
          for (int n = 0; n < 3; ++n) {
            Ms[n] = 0.0;
            mc[n] = MinCnt{0xFFFFFFFFu, 0u};
            for (int ww = 0; ww < kWaves; ++ww) {
              Ms[n] += __longlong_as_double(((uint64_t)red.v[par][ww][4 * n + 1] << 32) |
                                            red.v[par][ww][4 * n]);
              mc[n] = mc_merge(mc[n], MinCnt{red.v[par][ww][4 * n + 2], red.v[par][ww][4 * n + 3]});
            }
            // the boundary bucket of the top-k set holds only n_keep_k tokens
            if (topk_eff && kap > tau[n]) {
              Ms[n] += (double)n_keep_k * w_kap;
              if (kap < mc[n].key) mc[n] = MinCnt{kap, n_keep_k};
            }
            Ms[n] = uni(Ms[n]);
            mc[n].key = uni(mc[n].key);
            mc[n].cnt = uni(mc[n].cnt);
          }
          par ^= 1;
          ++rounds;
#pragma unroll
          for (int n = 0; n < 3; ++n) {
            if (!found && Ms[n] >= target) {
              const double wz = wkey(mc[n].key);
              const double below = Ms[n] - (double)mc[n].cnt * wz;
              if (below < target) {
                found = true;
                pstar = mc[n].key;
                w_star = wz;
                // smallest count of boundary tokens that reaches the target
                const double need = (target - below) / wz;
                const uint32_t c = mc[n].cnt;
                uint32_t nk = need <= 1.0 ? 1u : (need >= (double)c ? c : (uint32_t)ceil(need));
                while (nk > 1u && below + (double)(nk - 1u) * wz >= target) --nk;
                while (nk < c && below + (double)nk * wz < target) ++nk;
                n_keep = nk;
                const double w_p = below + (double)nk * wz;
                // the same cut for every reference mass in [w_k - err, w_k + err]?
                const double lo_t = p * (w_k - err), hi_t = p * (w_k + err);
                const double prev = below + (double)(nk - 1u) * wz;
                refine = err > 0.0 && !(prev < lo_t && hi_t <= w_p);
              }
            }
          }
          if (!found) {
#pragma unroll
            for (int n = 0; n < 3; ++n) {
              if (Ms[n] >= target) lo = tau[n] > lo ? tau[n] : lo;
              else hi = tau[n] < hi ? tau[n] : hi;
            }
          }
        }
        if (!refine || failed) break;
        // exact background mass: fp64 over every finite legal token below t
        double s = 0.0;
        walk_row<DT, false>(sl, lane, [&](const uint32_t (&key)[8], const uint32_t (&)[8],
                                          uint32_t vm) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (((vm >> j) & 1u) && key[j] < tkey) s += weight<DT>(key[j], m, invT);
        });
        w_k = mass_above(tkey - 1u) + block_sum_f64(s);
        err = 0.0;
      }
    } else if (topk_eff) {
      pstar = kap;
      n_keep = n_keep_k;
      w_star = w_kap;
    } else {
      pstar = K::kNegInf;
      n_keep = 0u;
    }
  }
  if (failed) {
    finish_error(QS_ROW_INTERNAL);
    return pool_raw;
  }
  if (pstar == K::kNegInf) n_keep = 0u;

  // -- walk A: per-wave counts of key > pstar and key == pstar, and their mass ----
  {
    uint32_t gt = 0u, ties = 0u;
    double mgt = 0.0;
    if (!greedy) {
      walk([&](const uint32_t (&key)[8], const uint32_t (&)[8], uint32_t vm) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if ((vm >> j) & 1u) {
            if (key[j] > pstar) {
              ++gt;
              mgt += wkey(key[j]);
            } else if (key[j] == pstar) {
              ++ties;
            }
          }
        }
      });
    } else {
      walk([&](const uint32_t (&key)[8], const uint32_t (&)[8], uint32_t vm) {
#pragma unroll
        for (int j = 0; j < 8; ++j) ties += (((vm >> j) & 1u) && key[j] == pstar) ? 1u : 0u;
      });
    }
    gt = wave_reduce<OpSum>(gt);
    ties = wave_reduce<OpSum>(ties);
    mgt = wave_sum_f64(mgt);
    if (lane == 0) {
      info.gt[w] = gt;
      info.ties[w] = ties;
      info.mass[w] = mgt;
    }
  }
  __syncthreads();

  // per-wave share of the tie quota (earliest ids first), list offsets, masses,
  // W_P and the wave whose cumulative mass holds u
  double u = 0.0;
  const bool sampled = SAMPLE && !greedy;
  if (sampled) {
    if (a.uniforms) u = u_in;
    else u = (double)philox_u24(seed_in, off_in) * (1.0 / 16777216.0);
  }
  u = uni(u);
  // lane i of every wave handles wave i: exclusive prefixes of ties (the
  // quota goes to the earliest ids, i.e. the lowest waves), kept counts and
  // masses; the sampled wave is the first whose cumulative probability passes u
  uint32_t my_off, n_p, my_kt;
  double w_p, my_cumw;
  int sw, last_w;
  {
    const bool act = lane < kWaves;
    const uint32_t t = act ? info.ties[lane] : 0u;
    const uint32_t g = act ? info.gt[lane] : 0u;
    const double mg = act ? info.mass[lane] : 0.0;
    const uint32_t tb = scan_incl_u32(t) - t;
    const uint32_t avail = n_keep > tb ? n_keep - tb : 0u;
    const uint32_t kt = t < avail ? t : avail;
    const uint32_t kept = g + kt;
    const double mw = mg + (double)kt * w_star;
    const uint32_t kincl = scan_incl_u32(kept);
    const double mincl = scan_incl_f64(mw);
    const double mex = incl_shift1_f64(mincl);  // the lane below's inclusive sum
    const int wu = uni(w);
    my_off = readlane_u32(kincl - kept, wu);
    my_kt = readlane_u32(kt, wu);
    my_cumw = readlane_f64(mex, wu);
    n_p = readlane_u32(kincl, kWaves - 1);
    w_p = readlane_f64(mincl, kWaves - 1);
    const uint64_t pos = ballot(act && kept > 0u && mw > 0.0);
    last_w = pos ? 63 - __clzll((long long)pos) : -1;
    sw = -1;
    if (sampled) {
      const uint64_t hit = ballot(act && kept > 0u && u < mincl * (1.0 / w_p));
      sw = hit ? __ffsll((unsigned long long)hit) - 1 : -1;
    }
  }
  my_off = uni(my_off);
  n_p = uni(n_p);
  my_kt = uni(my_kt);
  w_p = uni(w_p);
  my_cumw = uni(my_cumw);
  sw = uni(sw);
  last_w = uni(last_w);
  if (greedy) {
    w_p = 1.0;
    my_cumw = 0.0;
  }
  const double inv_wp = 1.0 / w_p;

  // -- walk D: outputs ------------------------------------------------------------
  int32_t* ids_row = a.cand_ids ? a.cand_ids + (size_t)r * a.cand_cap : nullptr;
  float* probs_row = a.cand_probs ? a.cand_probs + (size_t)r * a.cand_cap : nullptr;
  const uint32_t cap = (uint32_t)a.cand_cap;
  // this slice's mask words (none for an empty slice at the row end, whose
  // start word belongs to the wave before it)
  const int sw0 = sl.wb >> 5, sw1 = sl.we > sl.wb ? (sl.we + 31) >> 5 : sw0;
  uint32_t* const my_stage = stage[w];
  if (mask_row && stage_ok) {
    for (int i = lane; i < sw1 - sw0; i += 64) my_stage[i] = 0u;
  }
  if (dense_row || (mask_row && !stage_ok)) {
    // zero in memory first (the scatter below lands after these stores)
    if (mask_row && !stage_ok && sl.we > sl.wb)
      for (int i = sw0 + lane; i < sw1; i += 64) mask_row[i] = 0u;
    if (dense_row)
      for (int i = sl.wb + lane; i < sl.we; i += 64) dense_row[i] = 0.0f;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
  }
  // set bits of keep-mask word wi: in the LDS stage (workgroup-scope atomic),
  // or directly in memory (device-scope atomic) when the slice does not fit
  auto or_mask_word = [&](int wi, uint32_t bits) {
    if (stage_ok)
      __hip_atomic_fetch_or(my_stage + (wi - sw0), bits, __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_WORKGROUP);
    else
      __hip_atomic_fetch_or(mask_row + wi, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  uint32_t pos_base = my_off;
  uint32_t ties_seen = 0u;
  double cbase = my_cumw * inv_wp;
  int my_token = -1;       // set in wave sw
  double my_q = 0.0;       // its probability
  int last_pos_id = -1;    // last kept id with q > 0 in this wave
  double last_pos_q = 0.0;
  walk([&](const uint32_t (&key)[8], const uint32_t (&id)[8], uint32_t vm) {
    uint32_t tb = 0u, gb = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool v = (vm >> j) & 1u;
      tb |= ((v && key[j] == pstar && n_keep > 0u) ? 1u : 0u) << j;
      gb |= ((v && key[j] > pstar) ? 1u : 0u) << j;
    }
    // ties keep their rank order: the first my_kt ties of this wave are kept
    uint32_t pb = gb;
    if (ballot(tb != 0u)) {
      const uint32_t tc = (uint32_t)__popc(tb);
      const uint32_t tincl = scan_incl_u32(tc);
      uint32_t trank = ties_seen + tincl - tc;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if ((tb >> j) & 1u) {
          if (trank < my_kt) pb |= 1u << j;
          ++trank;
        }
      }
      ties_seen += readlane_u32(tincl, 63);
    }
    const uint32_t pc = (uint32_t)__popc(pb);
    const uint32_t pincl = scan_incl_u32(pc);
    const uint32_t total = readlane_u32(pincl, 63);
    uint32_t pos = pos_base + pincl - pc;
    double qv[8];
    double lane_sum = 0.0;
    int mwi = -1;
    uint32_t mword = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      qv[j] = 0.0;
      if ((pb >> j) & 1u) {
        const double q = greedy ? 1.0 : wkey(key[j]) * inv_wp;
        qv[j] = q;
        lane_sum += q;
        const float qf = (float)q;
        if (ids_row && pos < cap) ids_row[pos] = (int32_t)id[j];
        if (probs_row && pos < cap) probs_row[pos] = qf;
        if (dense_row) dense_row[id[j]] = qf;
        if (q > 0.0) {
          last_pos_id = (int)id[j];
          last_pos_q = q;
        }
        const int wi = (int)(id[j] >> 5);
        if (wi != mwi) {
          if (mwi >= 0 && mask_row) or_mask_word(mwi, mword);
          mwi = wi;
          mword = 0u;
        }
        mword |= 1u << (id[j] & 31u);
        ++pos;
      }
    }
    if (mwi >= 0 && mask_row) or_mask_word(mwi, mword);
    pos_base += total;
    if (w == sw && my_token < 0) {
      const double incl = scan_incl_f64(lane_sum);
      const double wtotal = readlane_f64(incl, 63);
      double c = cbase + (incl - lane_sum);
      int hit = -1;
      double hq = 0.0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        c += qv[j];
        if (hit < 0 && ((pb >> j) & 1u) && u < c) {
          hit = (int)id[j];
          hq = qv[j];
        }
      }
      const uint64_t hbits = ballot(hit >= 0);
      if (hbits) {
        const int fl = __ffsll((unsigned long long)hbits) - 1;
        my_token = __shfl(hit, fl, 64);
        my_q = readlane_f64(hq, fl);
      }
      cbase += wtotal;
    }
  });
  // this wave's mask words
  if (mask_row && stage_ok) {  // streaming stores: on to memory, not held in L2
    for (int i = lane; i < sw1 - sw0; i += 64)
      __builtin_nontemporal_store(my_stage[i], mask_row + sw0 + i);
  }
  // the token: from wave sw; if rounding left u at or above wave sw's last
  // cumulative sum, that wave's last kept id with q > 0; if u lies past every
  // wave, the last kept id with q > 0 of the row
  const int last_id = (int)wave_reduce<OpMax>((uint32_t)(last_pos_id + 1)) - 1;
  if (SAMPLE) {
    const double last_q = a.logprobs ? last_token_q(last_pos_id, last_pos_q, last_id) : 0.0;
    if (lane == 0) {
      if (greedy) {
        if (my_kt > 0u) put_token(a, r, last_id, 1.0);  // the one kept token is in this wave
      } else if (w == sw) {
        if (my_token >= 0) put_token(a, r, my_token, my_q);
        else put_token(a, r, last_id, last_q);
      } else if (sw < 0 && w == last_w) {
        put_token(a, r, last_id, last_q);
      }
    }
  }

  if (tid == 0) {
    const bool over = (a.cand_ids || a.cand_probs) ? n_p > cap : false;
    a.status[r] = over ? QS_ROW_CAND_OVERFLOW : QS_ROW_OK;
    if (a.cand_count) a.cand_count[r] = (int32_t)n_p;
    if (SAMPLE && sampled && !a.uniforms) a.offset[r] = a.offset[r] + 1u;
    if (a.dbg) {
      a.dbg[4 * r + 0] = to_pool ? 3 : (use_pool ? 0 : 1);
      a.dbg[4 * r + 1] = rounds;
      a.dbg[4 * r + 2] = (int32_t)ccount;
      a.dbg[4 * r + 3] = (int32_t)n_p;
    }
  }
  return pool_raw;
}

// ---------------------------------------------------------------------------
// Greedy argmax: one pass, (largest key, lowest id) per row.
template <int DT>
__global__ void __launch_bounds__(kThreads) argmax_rows_kernel(ArgmaxArgs a) {
  using K = Keys<DT>;
  __shared__ RedScratch red;
  const int r = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  Slice sl;
  sl.row = a.logits + (size_t)r * a.row_bytes;
  sl.mrow = a.bitmask ? reinterpret_cast<const uint8_t*>(a.bitmask + (size_t)r * a.bm_stride)
                      : nullptr;
  sl.V = a.V;
  sl.wb = uni(min(a.V, w * a.seg));
  sl.we = uni(min(a.V, (w + 1) * a.seg));
  uint32_t maxk = 0u, mink = 0xFFFFFFFFu, nlegal = 0u, best_id = 0xFFFFFFFFu;
  walk_row<DT, true, DT == 1 ? 8 : 4>(sl, lane, [&](const uint32_t (&key)[8],
                                                    const uint32_t (&id)[8], uint32_t lm) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool legal = (lm >> j) & 1u;
      const uint32_t kx = legal ? key[j] : 0u;
      const uint32_t kn = legal ? key[j] : 0xFFFFFFFFu;
      if (kx > maxk) { maxk = kx; best_id = id[j]; }  // ids ascend along a lane
      mink = kn < mink ? kn : mink;
    }
    nlegal += (uint32_t)__popc(lm);
  });
  const uint32_t wmax = wave_reduce<OpMax>(maxk);
  uint32_t cand = (maxk == wmax) ? best_id : 0xFFFFFFFFu;
  cand = wave_reduce<OpMin>(cand);
  mink = wave_reduce<OpMin>(mink);
  nlegal = wave_reduce<OpSum>(nlegal);
  if (lane == 0) {
    red.v[0][w][0] = wmax;
    red.v[0][w][1] = cand;
    red.v[0][w][2] = mink;
    red.v[0][w][3] = nlegal;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t mx = 0u, bid = 0xFFFFFFFFu, mn = 0xFFFFFFFFu, nl = 0u;
    for (int ww = 0; ww < kWaves; ++ww) {
      const uint32_t x = red.v[0][ww][0], c = red.v[0][ww][1];
      if (x > mx || (x == mx && c < bid)) { mx = x; bid = c; }
      const uint32_t y = red.v[0][ww][2];
      mn = y < mn ? y : mn;
      nl += red.v[0][ww][3];
    }
    int code = QS_ROW_OK;
    if (nl == 0u) code = QS_ROW_EMPTY;
    else if (mx >= K::kPosInf || mn < K::kNegInf) code = QS_ROW_NONFINITE;
    else if (mx <= K::kNegInf) code = QS_ROW_ALL_NEG_INF;
    a.status[r] = code;
    a.tokens[r] = code == QS_ROW_OK ? (int32_t)bid : -1;
  }
}

// ---------------------------------------------------------------------------
// Launch of one dtype's instances (each dtype's translation unit includes this
// file and instantiates its own).

// Steps of 512 tokens per wave slice when the row is held in registers.
inline int resident_steps(int V) {
  const int per_wave = (V + kWaves - 1) / kWaves;
  return (per_wave + kStep - 1) / kStep;
}

// T: the instance also writes each row's top-n tokens (after the row).
template <int DT, bool SAMPLE, int NL, int P, bool SRT, bool T>
__global__ void __launch_bounds__(kThreads) filter_rows_kernel(FilterArgs a) {
  uint8_t* const lds = filter_row<DT, SAMPLE, NL, P, SRT>(a);
  if constexpr (T) top_n_tail(a, lds);
}

template <int DT, bool S, int P, bool SRT, bool T = false>
hipError_t launch_dt(FilterArgs a, int B, hipStream_t st) {
  dim3 grid((unsigned)B), block(kThreads);
  const int n = resident_steps(a.V);
  const bool stream = (a.flags & QS_FLAG_STREAM) != 0u;
  if (!stream && n <= kResidentTier[DT][0]) {
    a.seg = n * kStep;
    hipLaunchKernelGGL((filter_rows_kernel<DT, S, kResidentTier[DT][0], P, SRT, T>), grid, block, 0, st,
                       a);
  } else if (!stream && n <= kResidentTier[DT][1]) {
    a.seg = n * kStep;
    hipLaunchKernelGGL((filter_rows_kernel<DT, S, kResidentTier[DT][1], P, SRT, T>), grid, block, 0, st,
                       a);
  } else {
    a.seg = seg_for(a.V);
    hipLaunchKernelGGL((filter_rows_kernel<DT, S, 0, P, SRT, T>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

template <int DT>
hipError_t launch_argmax_dt(const ArgmaxArgs& a, int B, hipStream_t st) {
  hipLaunchKernelGGL((argmax_rows_kernel<DT>), dim3((unsigned)B), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace qs
