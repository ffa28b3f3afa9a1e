// Exact speculative-decoding verification over candidate lists.
//
// Page "第 9 讲 · 生成与推测解码", section 5.2 (the exact rule of Leviathan et
// al. and Chen et al.): a draft token x, drawn from the draft distribution q,
// is accepted with probability min(1, p(x)/q(x)) under the target
// distribution p; on rejection one token is drawn from max(0, p - q)
// renormalised, which makes the output exactly p-distributed. Both
// distributions arrive as the id-ascending (id, float32 probability) lists the
// filter writes; a token outside a list has probability 0 there.
//
// One workgroup of 16 waves per row:
//   1. wave 0 finds x in the draft list and wave 1 in the target list, each by
//      a 64-ary search (one load per lane per level, 2-3 levels at list
//      lengths in the thousands), while the other 14 waves stage the draft
//      list in LDS (when it fits; an accepted row spends only bandwidth on
//      it, a rejected one finds it there);
//   2. accept iff u_accept * q(x) < p(x) in float64 on the widened list
//      values; an accepted row is finished;
//   3. for a rejected row each wave takes a contiguous sixteenth of the
//      target list, 4 entries per lane per round with the entries of 4 rounds
//      loaded together, looks up q of each id by binary search and sums the
//      residual max(0, p - q) with the same wave scans the draw uses;
//   4. the wave holding u_resample * R (R = the residual mass, summed in wave
//      order) walks its range again and returns the first id whose
//      cumulative residual exceeds it (or its last id with a positive
//      residual, if rounding leaves none). R == 0 (possible only through the
//      rounding of the lists) draws from p itself the same way.
// The target list is read once per pass from memory; nothing is written but
// the three per-row outputs.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qs.h"
#include "qs_device.hpp"
#include "qs_aux.hpp"
#include "qs_launch.hpp"

namespace qs {
namespace {

constexpr int kSpecWaves = 16;
constexpr int kSpecThreads = kSpecWaves * 64;
constexpr int kSpecTile = 16384;  // draft entries staged in LDS (128 KB)
constexpr int kSpecKP = 4;        // target entries per lane per round

// Index of x in the ascending ids[0, n), or -1. Wave-cooperative: each level
// probes 64 evenly spaced entries and keeps the interval the last probe at or
// below x opens. Called by a whole wave; every read stays below n.
__device__ int wave_find(const int32_t* ids, int n, int x) {
  const int lane = lane_id();
  int lo = 0, hi = n;
  while (hi - lo > 64) {
    const int step = (hi - lo + 63) / 64;
    const int i = lo + lane * step;
    const uint64_t le = ballot(i < hi && ids[i] <= x);
    if (!le) return -1;  // x lies below ids[lo]
    lo += (63 - __clzll((long long)le)) * step;
    hi = min(lo + step, hi);
  }
  const int i = lo + lane;
  const uint64_t eq = ballot(i < hi && ids[i] == x);
  return eq ? lo + __ffsll((unsigned long long)eq) - 1 : -1;
}

constexpr int kSpecNR = 4;        // rounds whose entries are loaded together

// The draft list staged in LDS (when it fits).
__shared__ int32_t s_ids[kSpecTile];
__shared__ float s_p[kSpecTile];

// Residual weights max(0, p - q) of one round's KP entries per lane (p itself
// when `use_p`; 0 for absent entries, id < 0), q looked up in the draft list:
// in LDS when STAGED, else in memory. The binary searches take the same
// number of steps in every lane (it depends on the list length only), so the
// KP searches of a lane run interleaved without divergence. Returns the
// lane's sum in k order.
template <bool STAGED>
__device__ double round_weights(const int (&id)[kSpecKP], const float (&p)[kSpecKP], bool use_p,
                                const int32_t* g_ids, const float* g_p, int dc,
                                double (&wv)[kSpecKP]) {
  const int32_t* q_ids = STAGED ? s_ids : g_ids;
  const float* q_p = STAGED ? s_p : g_p;
  double sum = 0.0;
  if (use_p) {
#pragma unroll
    for (int k = 0; k < kSpecKP; ++k) {
      wv[k] = id[k] >= 0 ? (double)p[k] : 0.0;
      sum += wv[k];
    }
    return sum;
  }
  int base[kSpecKP];
#pragma unroll
  for (int k = 0; k < kSpecKP; ++k) base[k] = 0;
  for (int len = dc; len > 1;) {  // reads stay below base + len <= dc
    const int half = len >> 1;
#pragma unroll
    for (int k = 0; k < kSpecKP; ++k) base[k] += q_ids[base[k] + half] < id[k] ? half : 0;
    len -= half;
  }
#pragma unroll
  for (int k = 0; k < kSpecKP; ++k) {
    const int pos = base[k] + (q_ids[base[k]] < id[k] ? 1 : 0);  // lower bound
    const double q = (pos < dc && q_ids[pos] == id[k]) ? (double)q_p[pos] : 0.0;
    const double pk = (double)p[k];
    wv[k] = id[k] >= 0 && pk > q ? pk - q : 0.0;
    sum += wv[k];
  }
  return sum;
}

__global__ void __launch_bounds__(kSpecThreads) spec_verify_kernel(SpecArgs a) {
  __shared__ double s_wsum[kSpecWaves];
  __shared__ double s_px, s_qx;
  __shared__ int s_in_draft;

  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = uni((int)threadIdx.x >> 6);
  const int tc = a.t_count[r], dc = a.d_count[r];
  const int x = a.x[r];
  const double u1 = a.u_accept[r], u2 = a.u_resample[r];

  auto finish = [&](int status, int tok, int acc) {
    if (tid == 0) {
      a.status[r] = status;
      a.tokens[r] = tok;
      a.accepted[r] = acc;
    }
  };
  int status = QS_ROW_OK;
  if (tc < 0 || dc < 0) status = QS_ROW_BAD_PARAM;
  else if (tc == 0 || dc == 0) status = QS_ROW_EMPTY;
  else if ((int64_t)tc > a.t_cap || (int64_t)dc > a.d_cap) status = QS_ROW_CAND_OVERFLOW;
  else if (!(u1 >= 0.0 && u1 < 1.0) || !(u2 >= 0.0 && u2 < 1.0)) status = QS_ROW_BAD_PARAM;
  if (status != QS_ROW_OK) {
    finish(status, -1, 0);
    return;
  }
  const int32_t* t_ids = a.t_ids + (size_t)r * a.t_cap;
  const float* t_p = a.t_probs + (size_t)r * a.t_cap;
  const int32_t* d_ids = a.d_ids + (size_t)r * a.d_cap;
  const float* d_p = a.d_probs + (size_t)r * a.d_cap;

  // -- p(x) and q(x); meanwhile waves 2-15 stage the draft list (before the
  // decision is known: an accepted row spends only bandwidth on it) ---------------
  const bool staged = dc <= kSpecTile;
  if (w >= 2 && staged) {
    constexpr int kStagers = kSpecThreads - 128;
    for (int i0 = tid - 128; i0 < dc; i0 += 4 * kStagers) {
      int32_t iv[4];
      float pv[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {  // the four loads first, then the stores
        const int i = i0 + k * kStagers;
        iv[k] = i < dc ? d_ids[i] : 0;
        pv[k] = i < dc ? d_p[i] : 0.0f;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = i0 + k * kStagers;
        if (i < dc) {
          s_ids[i] = iv[k];
          s_p[i] = pv[k];
        }
      }
    }
  }
  if (w == 0) {
    const int i = wave_find(d_ids, dc, x);
    if (lane == 0) {
      s_in_draft = i >= 0;
      s_qx = i >= 0 ? (double)d_p[i] : 0.0;
    }
  } else if (w == 1) {
    const int i = wave_find(t_ids, tc, x);
    if (lane == 0) s_px = i >= 0 ? (double)t_p[i] : 0.0;
  }
  __syncthreads();
  if (!s_in_draft) {
    finish(QS_ROW_BAD_PARAM, -1, 0);
    return;
  }
  if (u1 * s_qx < s_px) {
    finish(QS_ROW_OK, x, 1);
    return;
  }

  // -- rejected: the residual mass, per wave ------------------------------------------
  const int per = (tc + kSpecWaves - 1) / kSpecWaves;
  const int b0 = min(w * per, tc), b1 = min(b0 + per, tc);

  // the NR rounds' entries i0 + g*64*KP + KP*lane + k of this wave's range,
  // loaded together (one memory latency per NR rounds)
  constexpr int kRound = 64 * kSpecKP;
  auto load_rounds = [&](int i0, int (&id)[kSpecNR][kSpecKP], float (&pv)[kSpecNR][kSpecKP]) {
#pragma unroll
    for (int g = 0; g < kSpecNR; ++g)
#pragma unroll
      for (int k = 0; k < kSpecKP; ++k) {
        const int i = i0 + g * kRound + kSpecKP * lane + k;
        id[g][k] = i < b1 ? t_ids[i] : -1;
        pv[g][k] = i < b1 ? t_p[i] : 0.0f;
      }
  };
  auto weights = [&](const int (&id)[kSpecKP], const float (&pv)[kSpecKP], bool use_p,
                     double (&wv)[kSpecKP]) {
    return staged ? round_weights<true>(id, pv, use_p, d_ids, d_p, dc, wv)
                  : round_weights<false>(id, pv, use_p, d_ids, d_p, dc, wv);
  };
  auto wave_mass = [&](bool use_p) {
    double cb = 0.0;
    for (int i0 = b0; i0 < b1; i0 += kSpecNR * kRound) {
      int id[kSpecNR][kSpecKP];
      float pv[kSpecNR][kSpecKP];
      load_rounds(i0, id, pv);
#pragma unroll
      for (int g = 0; g < kSpecNR; ++g) {
        if (i0 + g * kRound < b1) {
          double wv[kSpecKP];
          const double ls = weights(id[g], pv[g], use_p, wv);
          cb += readlane_f64(scan_incl_f64(ls), 63);
        }
      }
    }
    return cb;
  };
  bool use_p = false;
  double mass = wave_mass(false);
  if (lane == 0) s_wsum[w] = mass;
  __syncthreads();
  double R = 0.0;
  for (int i = 0; i < kSpecWaves; ++i) R += s_wsum[i];
  if (!(R > 0.0)) {  // rounding only: draw from p itself
    __syncthreads();
    use_p = true;
    mass = wave_mass(true);
    if (lane == 0) s_wsum[w] = mass;
    __syncthreads();
    R = 0.0;
    for (int i = 0; i < kSpecWaves; ++i) R += s_wsum[i];
    if (!(R > 0.0)) {  // every listed target probability underflowed
      finish(QS_ROW_EMPTY, -1, 0);
      return;
    }
  }

  // -- the wave holding the target, and the draw inside it -----------------------------
  const double target = u2 * R;
  int cw = -1, last_w = -1;
  double cbase = 0.0, pre = 0.0;
  for (int i = 0; i < kSpecWaves; ++i) {
    const double nxt = pre + s_wsum[i];
    if (cw < 0 && target < nxt) {
      cw = i;
      cbase = pre;
    }
    if (s_wsum[i] > 0.0) last_w = i;
    pre = nxt;
  }
  if (cw < 0) {  // rounding left the target past the total: the last positive wave
    cw = last_w;
    cbase = 0.0;
    for (int i = 0; i < cw; ++i) cbase += s_wsum[i];
  }
  if (w != cw) return;

  int tok = -1, last_pos = -1;
  double cb = cbase;
  for (int i0 = b0; i0 < b1 && tok < 0; i0 += kSpecNR * kRound) {
    int id[kSpecNR][kSpecKP];
    float pv[kSpecNR][kSpecKP];
    load_rounds(i0, id, pv);
#pragma unroll
    for (int g = 0; g < kSpecNR; ++g) {
      if (tok < 0 && i0 + g * kRound < b1) {
        double wv[kSpecKP];
        const double ls = weights(id[g], pv[g], use_p, wv);
        const double incl = scan_incl_f64(ls);
        double cu = cb + (incl - ls);
        int hit = -1;
#pragma unroll
        for (int k = 0; k < kSpecKP; ++k) {
          cu += wv[k];
          if (wv[k] > 0.0) last_pos = id[g][k];
          if (hit < 0 && id[g][k] >= 0 && target < cu) hit = id[g][k];
        }
        const uint64_t hb = ballot(hit >= 0);
        if (hb) tok = __shfl(hit, __ffsll((unsigned long long)hb) - 1, 64);
        cb += readlane_f64(incl, 63);
      }
    }
  }
  if (tok < 0) tok = (int)wave_reduce<OpMax>((uint32_t)(last_pos + 1)) - 1;
  if (lane == 0) {
    a.status[r] = tok >= 0 ? QS_ROW_OK : QS_ROW_INTERNAL;
    a.tokens[r] = tok;
    a.accepted[r] = 0;
  }
}

}  // namespace

hipError_t launch_spec(const SpecArgs& a, int B, hipStream_t st) {
  hipLaunchKernelGGL(spec_verify_kernel, dim3((unsigned)B), dim3(kSpecThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace qs
