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
//      lengths in the thousands);
//   2. accept iff u_accept * q(x) < p(x) in float64 on the widened list
//      values; an accepted row is finished;
//   3. a rejected row stages the draft list in LDS (when it fits), and each
//      wave takes a contiguous sixteenth of the target list, 4 entries per
//      lane per round, looks up q of each id by binary search and sums the
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

struct SpecRow {
  const int32_t* t_ids;
  const float* t_p;
  const int32_t* q_ids;  // the draft list, in LDS or in memory
  const float* q_p;
  int tc, dc;
};

// Weights of the KP entries i0 + KP*lane + k (0 past `end`): the residual
// max(0, p - q), or p itself when `use_p`. Returns the lane's sum in k order.
__device__ double entry_weights(const SpecRow& s, int i0, int end, bool use_p,
                                int (&id)[kSpecKP], double (&wv)[kSpecKP]) {
  const int lane = lane_id();
  int lo[kSpecKP], len[kSpecKP];
  double p[kSpecKP];
#pragma unroll
  for (int k = 0; k < kSpecKP; ++k) {
    const int i = i0 + kSpecKP * lane + k;
    const bool v = i < end;
    id[k] = v ? s.t_ids[i] : -1;
    p[k] = v ? (double)s.t_p[i] : 0.0;
    lo[k] = 0;
    len[k] = v && !use_p ? s.dc : 0;
  }
  // lower bounds of the ids in the draft list, the KP searches interleaved
  bool more = true;
  while (more) {
    more = false;
#pragma unroll
    for (int k = 0; k < kSpecKP; ++k) {
      if (len[k] > 0) {
        const int half = len[k] >> 1;
        if (s.q_ids[lo[k] + half] < id[k]) {
          lo[k] += half + 1;
          len[k] -= half + 1;
        } else {
          len[k] = half;
        }
        more = more || len[k] > 0;
      }
    }
  }
  double sum = 0.0;
#pragma unroll
  for (int k = 0; k < kSpecKP; ++k) {
    double w = p[k];
    if (!use_p && id[k] >= 0) {
      const double q = (lo[k] < s.dc && s.q_ids[lo[k]] == id[k]) ? (double)s.q_p[lo[k]] : 0.0;
      w = p[k] > q ? p[k] - q : 0.0;
    }
    wv[k] = w;
    sum += w;
  }
  return sum;
}

__global__ void __launch_bounds__(kSpecThreads) spec_verify_kernel(SpecArgs a) {
  __shared__ int32_t s_ids[kSpecTile];
  __shared__ float s_p[kSpecTile];
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

  // -- p(x) and q(x) -------------------------------------------------------------------
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
  const bool staged = dc <= kSpecTile;
  if (staged) {
    for (int i = tid; i < dc; i += kSpecThreads) {
      s_ids[i] = d_ids[i];
      s_p[i] = d_p[i];
    }
  }
  __syncthreads();
  const SpecRow s{t_ids, t_p, staged ? s_ids : d_ids, staged ? s_p : d_p, tc, dc};
  const int per = (tc + kSpecWaves - 1) / kSpecWaves;
  const int b0 = min(w * per, tc), b1 = min(b0 + per, tc);

  auto wave_mass = [&](bool use_p) {
    double cb = 0.0;
    for (int i0 = b0; i0 < b1; i0 += 64 * kSpecKP) {
      int id[kSpecKP];
      double wv[kSpecKP];
      const double ls = entry_weights(s, i0, b1, use_p, id, wv);
      cb += readlane_f64(scan_incl_f64(ls), 63);
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
  for (int i0 = b0; i0 < b1; i0 += 64 * kSpecKP) {
    int id[kSpecKP];
    double wv[kSpecKP];
    const double ls = entry_weights(s, i0, b1, use_p, id, wv);
    const double incl = scan_incl_f64(ls);
    double cu = cb + (incl - ls);
    int hit = -1;
#pragma unroll
    for (int k = 0; k < kSpecKP; ++k) {
      cu += wv[k];
      if (wv[k] > 0.0) last_pos = id[k];
      if (hit < 0 && id[k] >= 0 && target < cu) hit = id[k];
    }
    const uint64_t hb = ballot(hit >= 0);
    if (hb) {
      tok = __shfl(hit, __ffsll((unsigned long long)hb) - 1, 64);
      break;
    }
    cb += readlane_f64(incl, 63);
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
