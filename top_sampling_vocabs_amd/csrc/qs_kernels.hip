// Exact top-k / top-p filter-and-sample kernels for gfx950 (MI355X).
//
// One 1024-thread workgroup owns one row. Its 16 wave64s each own a
// contiguous slice of the vocabulary (a multiple of 32 tokens, so every
// packed-mask word belongs to one wave), which keeps every per-wave walk in
// token-id order and makes outputs deterministic.
//
// Per row (page "Qrita", overall framework and key designs 1-3):
//  1. sigma-truncation: the first 512-token step of each wave's slice is a
//     sample (8192 tokens) giving mean, sigma and the sample maximum; the
//     threshold t = t0 - 0.2|t0| comes from the Gaussian quantile of k/V or p
//     (key design 1). One coalesced pass over the row then finds the maximum,
//     the legal count, NaN/+inf, and compacts {z >= t} in id order into a
//     per-wave LDS pool; rows with top-k off also accumulate the fp64 mass
//     below t here.
//  2. hit test: |Z_t| >= k (top-k), or mass(Z_t) >= p * W (top-p only);
//     otherwise every later step runs over the full row (fallback Z_s = Z).
//  3. quaternary three-pivot search (key design 2) for the k-th largest value:
//     pivots at 1/4, 1/2, 3/4 of the current key interval; one fused pass
//     counts N_tau, the minimum above tau and its multiplicity for all three;
//     stop when N_tau >= k and N_tau - N_zm < k. Pivots are taken on
//     order-preserving integer keys, so a search ends in at most 8 (bf16) or
//     16 (fp32) rounds even when values repeat.
//  4. the same search on fp64 mass for the top-p boundary inside the top-k set.
//  5. duplicate handling (key design 3): at the boundary value only the
//     earliest N_keep token ids are kept; the id cut comes from an ordered
//     per-wave count.
//  6. renormalise, write the packed mask, id-ordered candidate lists and
//     optional dense probabilities, and draw the token by an inverse CDF in
//     id order with Philox4x32-10 (sampling-contract page, sections 02 and 06).

#include <type_traits>

#include "qs_device.hpp"
#include "qs_launch.hpp"
#include "../../include/qs.h"

namespace qs {

// ---------------------------------------------------------------------------
// Raw access to 8 consecutive tokens starting at e (e is a multiple of 8).
template <int DT> struct Raw;
template <> struct Raw<0> {
  uint32_t r[8];
  __device__ __forceinline__ uint32_t bits(int j) const { return r[j]; }
};
template <> struct Raw<1> {
  uint32_t r[4];
  __device__ __forceinline__ uint32_t bits(int j) const {
    return (r[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
  }
};

template <int DT>
__device__ __forceinline__ void load_raw(const uint8_t* row, int e, int V, Raw<DT>& o) {
  if (e + kChunk <= V) {
    if constexpr (DT == 0) {
      const uint4* p = reinterpret_cast<const uint4*>(row + (size_t)e * 4);
      uint4 a = p[0], b = p[1];
      o.r[0] = a.x; o.r[1] = a.y; o.r[2] = a.z; o.r[3] = a.w;
      o.r[4] = b.x; o.r[5] = b.y; o.r[6] = b.z; o.r[7] = b.w;
    } else {
      uint4 a = *reinterpret_cast<const uint4*>(row + (size_t)e * 2);
      o.r[0] = a.x; o.r[1] = a.y; o.r[2] = a.z; o.r[3] = a.w;
    }
  } else {
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
}

// Legal bits of tokens e..e+7 restricted to [e, end).
__device__ __forceinline__ uint32_t load_mask_byte(const uint8_t* mrow, int e, int end) {
  int n = end - e;
  if (n <= 0) return 0u;
  uint32_t mb = mrow ? (uint32_t)mrow[e >> 3] : 0xFFu;
  if (n < 8) mb &= (1u << n) - 1u;
  return mb;
}

// Per-wave view of the row.
struct Slice {
  const uint8_t* row;
  const uint8_t* mrow;
  int V;
  int wb, we;  // this wave's token range [wb, we)
};

// Visit this wave's slice in id order, 512 tokens per step. f(key, id, vm):
// vm bit j set iff token id[j] is legal and finite (or, with NEGINF_TOO, legal).
template <int DT, bool NEGINF_TOO = false, class F>
__device__ __forceinline__ void walk_row(const Slice& s, int lane, F&& f) {
  using K = Keys<DT>;
  for (int base = s.wb; base < s.we; base += kStep) {
    int e = base + lane * kChunk;
    uint32_t key[8], id[8];
    uint32_t vm = 0;
    Raw<DT> raw;
    uint32_t mb = load_mask_byte(s.mrow, e, s.we);
    if (mb) load_raw<DT>(s.row, e, s.V, raw);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      id[j] = (uint32_t)(e + j);
      key[j] = mb ? K::of(raw.bits(j)) : 0u;
      bool ok = (mb >> j) & 1u;
      if constexpr (!NEGINF_TOO) ok = ok && key[j] > K::kNegInf && key[j] < K::kPosInf;
      vm |= (ok ? 1u : 0u) << j;
    }
    f(key, id, vm);
  }
}

// Visit this wave's candidate pool in order (which is id order).
template <class F>
__device__ __forceinline__ void walk_pool(const uint32_t* pk, const uint32_t* pid, int cnt,
                                          int lane, F&& f) {
  for (int base = 0; base < cnt; base += kStep) {
    int q = base + lane * kChunk;
    uint32_t key[8], id[8];
    uint32_t vm = 0;
    if (q + kChunk <= cnt) {
      uint4 a = *reinterpret_cast<const uint4*>(pk + q);
      uint4 b = *reinterpret_cast<const uint4*>(pk + q + 4);
      uint4 c = *reinterpret_cast<const uint4*>(pid + q);
      uint4 d = *reinterpret_cast<const uint4*>(pid + q + 4);
      key[0] = a.x; key[1] = a.y; key[2] = a.z; key[3] = a.w;
      key[4] = b.x; key[5] = b.y; key[6] = b.z; key[7] = b.w;
      id[0] = c.x; id[1] = c.y; id[2] = c.z; id[3] = c.w;
      id[4] = d.x; id[5] = d.y; id[6] = d.z; id[7] = d.w;
      vm = 0xFFu;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bool ok = q + j < cnt;
        key[j] = ok ? pk[q + j] : 0u;
        id[j] = ok ? pid[q + j] : 0u;
        vm |= (ok ? 1u : 0u) << j;
      }
    }
    f(key, id, vm);
  }
}

// fp64 weight of a token relative to the row maximum: exp((z - m) / T).
template <int DT>
__device__ __forceinline__ double weight(uint32_t key, double m, double invT) {
  return exp(((double)Keys<DT>::value(key) - m) * invT);
}

// Threshold for the sigma-truncation prefilter. Returns the key below which
// tokens are not compacted (page "Qrita", key design 1 and the lookup table of
// the training-strategy paragraph: delta = Phi^-1(1 - k/V) for top-k; for top-p
// the mass-weighted Gaussian N(mu + sigma^2/T, sigma^2), truncated at the
// sample maximum, gives the value above which a fraction p of the mass lies).
template <int DT>
__device__ __forceinline__ uint32_t truncation_key(double n_s, double sum, double sumsq,
                                                   uint32_t smax_key, double frac_legal,
                                                   int V, bool greedy, bool topk_on, int k,
                                                   bool topp_on, double p, double invT) {
  using K = Keys<DT>;
  const uint32_t lowest = K::kNegInf + 1u;
  if (n_s < 1.0) return lowest;
  double ms = (double)K::value(smax_key);
  if (greedy) return smax_key;
  double mu = sum / n_s;
  double var = sumsq / n_s - mu * mu;
  double sd = var > 0.0 ? sqrt(var) : 0.0;
  double t0;
  if (topk_on) {
    double veff = frac_legal * (double)V;
    double q = (double)k / veff;
    if (!(q < 1.0)) return lowest;
    t0 = mu + sd * (1.4142135623730951 * erfcinv(2.0 * q));
  } else if (topp_on) {
    if (!(sd > 0.0)) return lowest;
    double mp = mu + sd * sd * invT;
    double a = (ms - mp) / sd;
    double c = (1.0 - p) * 0.5 * erfc(-a * 0.7071067811865476);
    if (!(c > 0.0)) return lowest;
    t0 = mp - sd * (1.4142135623730951 * erfcinv(2.0 * c));
  } else {
    return lowest;
  }
  double t = t0 - 0.2 * fabs(t0);
  if (!(t < ms)) t = ms;
  if (!(t > -3.0e38)) return lowest;
  float tf = __double2float_rd(t);
  uint32_t k32 = Keys<0>::of(__float_as_uint(tf));
  uint32_t key = (DT == 0) ? k32 : (k32 >> 16);
  return key < lowest ? lowest : key;
}

// ---------------------------------------------------------------------------
template <int DT, bool SAMPLE>
__global__ void __launch_bounds__(kThreads) filter_rows_kernel(FilterArgs a) {
  using K = Keys<DT>;
  __shared__ __align__(16) uint32_t pool_key[kWaves][kPoolPerWave];
  __shared__ __align__(16) uint32_t pool_id[kWaves][kPoolPerWave];
  __shared__ RedScratch red;
  __shared__ struct {
    uint32_t gt[kWaves];
    uint32_t ties[kWaves];
    double q[kWaves];
  } info;

  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  int par = 0;

  const int V = a.V;
  Slice sl;
  sl.row = a.logits + (size_t)r * a.row_bytes;
  sl.mrow = a.bitmask ? reinterpret_cast<const uint8_t*>(a.bitmask + (size_t)r * a.bm_stride)
                      : nullptr;
  sl.V = V;
  sl.wb = min(V, w * a.seg);
  sl.we = min(V, (w + 1) * a.seg);
  const int W = (V + 31) >> 5;

  uint32_t* mask_row = a.keep_mask ? a.keep_mask + (size_t)r * W : nullptr;
  float* dense_row = a.dense ? a.dense + (size_t)r * V : nullptr;

  // Zero this wave's share of the mask and dense outputs; the fence orders
  // these stores before any later scatter into the same slice by this wave.
  auto zero_outputs = [&]() {
    if (mask_row) {
      int w0 = sl.wb >> 5, w1 = (sl.we + 31) >> 5;
      for (int i = w0 + lane; i < w1; i += 64) mask_row[i] = 0u;
    }
    if (dense_row) {
      for (int i = sl.wb + lane; i < sl.we; i += 64) dense_row[i] = 0.0f;
    }
    __threadfence();
  };

  auto finish_error = [&](int code) {
    zero_outputs();
    if (tid == 0) {
      a.status[r] = code;
      if (SAMPLE) a.tokens[r] = -1;
      if (a.cand_count) a.cand_count[r] = 0;
      if (a.dbg) {
        a.dbg[4 * r + 0] = 0; a.dbg[4 * r + 1] = 0;
        a.dbg[4 * r + 2] = 0; a.dbg[4 * r + 3] = 0;
      }
    }
  };

  // -- parameters ------------------------------------------------------------
  const float Tf = a.T[r];
  const int kk = a.k[r];
  const float pf = a.p[r];
  const bool bad = !(isfinite(Tf) && Tf >= 0.0f) || kk < 0 || !(pf > 0.0f && pf <= 1.0f);
  if (bad) {
    finish_error(QS_ROW_BAD_PARAM);
    return;
  }
  const bool greedy = (Tf == 0.0f);
  const double invT = greedy ? 0.0 : 1.0 / (double)Tf;
  const double p = (double)pf;
  const bool topp_on = !greedy && pf < 1.0f;
  // top-k is on for k in [1, V); whether k >= |F| is only known after the pass
  const bool topk_req = !greedy && kk > 0 && kk < V;
  const bool need_bg = topp_on && !topk_req;
  const bool no_trunc = (a.flags & QS_FLAG_NO_TRUNCATION) != 0u;

  // -- pass 1a: sample statistics from the first step of each slice -------------
  double s_n = 0.0, s_sum = 0.0, s_sq = 0.0, s_all = 0.0;
  uint32_t s_max = 0u;
  {
    int e = sl.wb + lane * kChunk;
    int send = min(sl.we, sl.wb + kStep);
    uint32_t mb = load_mask_byte(sl.mrow, e, send);
    int nin = min(8, max(0, send - e));
    s_all = (double)nin;
    if (mb) {
      Raw<DT> raw;
      load_raw<DT>(sl.row, e, V, raw);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t key = K::of(raw.bits(j));
        if (((mb >> j) & 1u) && key > K::kNegInf && key < K::kPosInf) {
          double v = (double)K::value(key);
          s_n += 1.0; s_sum += v; s_sq += v * v;
          s_max = key > s_max ? key : s_max;
        }
      }
    }
  }
  double st[4] = {s_n, s_sum, s_sq, s_all};
#pragma unroll
  for (int i = 0; i < 4; ++i) st[i] = wave_sum_f64(st[i]);
  s_max = wave_reduce<OpMax>(s_max);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint64_t b = __double_as_longlong(st[i]);
      red.v[par][w][2 * i] = (uint32_t)b;
      red.v[par][w][2 * i + 1] = (uint32_t)(b >> 32);
    }
    red.v[par][w][8] = s_max;
  }
  __syncthreads();
  {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    uint32_t mx = 0u;
    for (int ww = 0; ww < kWaves; ++ww) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[i] += __longlong_as_double(((uint64_t)red.v[par][ww][2 * i + 1] << 32) |
                                       red.v[par][ww][2 * i]);
      uint32_t m2 = red.v[par][ww][8];
      mx = m2 > mx ? m2 : mx;
    }
    s_n = uni(acc[0]); s_sum = uni(acc[1]); s_sq = uni(acc[2]); s_all = uni(acc[3]);
    s_max = uni(mx);
  }
  par ^= 1;

  uint32_t tkey = truncation_key<DT>(s_n, s_sum, s_sq, s_max,
                                     s_all > 0.0 ? s_n / s_all : 0.0, V, greedy,
                                     topk_req, kk, topp_on, p, invT);
  if (no_trunc) tkey = K::kMax;  // nothing is compacted
  tkey = uni(tkey);
  const double m_ref = (s_n >= 1.0) ? (double)K::value(s_max) : 0.0;

  // -- pass 1b: one pass over the row ----------------------------------------
  uint32_t maxk = 0u, mink = 0xFFFFFFFFu, nlegal = 0u;
  uint32_t pcnt = 0u;  // this wave's candidates (may exceed the pool)
  double bg = 0.0;
  auto stream = [&](auto bg_on) {
    constexpr bool BG = decltype(bg_on)::value;
    walk_row<DT, true>(sl, lane, [&](const uint32_t (&key)[8], const uint32_t (&id)[8],
                                     uint32_t lm) {
      uint32_t cb = 0u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bool legal = (lm >> j) & 1u;
        uint32_t kx = legal ? key[j] : 0u;
        uint32_t kn = legal ? key[j] : 0xFFFFFFFFu;
        maxk = kx > maxk ? kx : maxk;
        mink = kn < mink ? kn : mink;
        bool cand = legal && key[j] >= tkey;
        cb |= (cand ? 1u : 0u) << j;
        if constexpr (BG) {
          if (legal && !cand && key[j] > K::kNegInf)
            bg += exp(((double)K::value(key[j]) - m_ref) * invT);
        }
      }
      nlegal += (uint32_t)__popc(lm);
      uint64_t any = ballot(cb != 0u);
      if (any) {
        uint32_t total;
        uint32_t pos = pcnt + wave_excl_small((uint32_t)__popc(cb), total);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if ((cb >> j) & 1u) {
            if (pos < (uint32_t)kPoolPerWave) {
              pool_key[w][pos] = key[j];
              pool_id[w][pos] = id[j];
            }
            ++pos;
          }
        }
        pcnt += total;
      }
    });
  };
  if (need_bg) stream(std::true_type{});
  else stream(std::false_type{});
  maxk = wave_reduce<OpMax>(maxk);
  mink = wave_reduce<OpMin>(mink);
  nlegal = wave_reduce<OpSum>(nlegal);
  bg = wave_sum_f64(bg);
  if (lane == 0) {
    red.v[par][w][0] = maxk;
    red.v[par][w][1] = mink;
    red.v[par][w][2] = nlegal;
    red.v[par][w][3] = pcnt;
    uint64_t b = __double_as_longlong(bg);
    red.v[par][w][4] = (uint32_t)b;
    red.v[par][w][5] = (uint32_t)(b >> 32);
  }
  __syncthreads();
  uint32_t ccount = 0u, my_wcnt = 0u;
  bool overflow = false;
  {
    uint32_t mx = 0u, mn = 0xFFFFFFFFu, nl = 0u;
    double b2 = 0.0;
    for (int ww = 0; ww < kWaves; ++ww) {
      uint32_t x = red.v[par][ww][0], y = red.v[par][ww][1];
      mx = x > mx ? x : mx;
      mn = y < mn ? y : mn;
      nl += red.v[par][ww][2];
      uint32_t c = red.v[par][ww][3];
      if (ww == w) my_wcnt = c;
      ccount += c;
      overflow = overflow || c > (uint32_t)kPoolPerWave;
      b2 += __longlong_as_double(((uint64_t)red.v[par][ww][5] << 32) | red.v[par][ww][4]);
    }
    maxk = uni(mx); mink = uni(mn); nlegal = uni(nl); bg = uni(b2);
  }
  ccount = uni(ccount);
  my_wcnt = uni(my_wcnt);
  overflow = uni(overflow);
  par ^= 1;

  // -- row status --------------------------------------------------------------
  if (nlegal == 0u) { finish_error(QS_ROW_EMPTY); return; }
  if (maxk >= K::kPosInf || mink < K::kNegInf) { finish_error(QS_ROW_NONFINITE); return; }
  if (maxk <= K::kNegInf) { finish_error(QS_ROW_ALL_NEG_INF); return; }

  // number of finite legal tokens
  uint32_t nfin = nlegal;
  if (mink == K::kNegInf) {
    uint32_t ninf = 0u;
    walk_row<DT, true>(sl, lane, [&](const uint32_t (&key)[8], const uint32_t (&)[8],
                                     uint32_t lm) {
#pragma unroll
      for (int j = 0; j < 8; ++j) ninf += (((lm >> j) & 1u) && key[j] == K::kNegInf) ? 1u : 0u;
    });
    ninf = wave_reduce<OpSum>(ninf);
    if (lane == 0) red.v[par][w][0] = ninf;
    __syncthreads();
    uint32_t t = 0u;
    for (int ww = 0; ww < kWaves; ++ww) t += red.v[par][ww][0];
    par ^= 1;
    nfin = uni(nlegal - t);
  }

  const double m = (double)K::value(maxk);
  const bool topk_on = !greedy && kk > 0 && (uint32_t)kk < nfin;

  // -- source selection (hit test) -------------------------------------------
  bool use_pool = !overflow && !(a.flags & QS_FLAG_FORCE_MISS) && !no_trunc;
  const uint32_t* pk = &pool_key[w][0];
  const uint32_t* pid = &pool_id[w][0];
  const int my_cnt = (int)min(my_wcnt, (uint32_t)kPoolPerWave);

  // walk the chosen source
  auto walk = [&](auto&& f) {
    if (use_pool) walk_pool(pk, pid, my_cnt, lane, f);
    else walk_row<DT, false>(sl, lane, f);
  };

  // block sum of an fp64 per-lane value computed by a walk
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

  // mass of tokens with key > lo_excl (fp64)
  auto mass_above = [&](uint32_t lo_excl) -> double {
    double s = 0.0;
    walk([&](const uint32_t (&key)[8], const uint32_t (&)[8], uint32_t vm) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (((vm >> j) & 1u) && key[j] > lo_excl) s += weight<DT>(key[j], m, invT);
    });
    return block_sum_f64(s);
  };

  double w_f = -1.0;  // mass of every finite legal token, when known
  if (use_pool) {
    if (topk_on) {
      use_pool = ccount >= (uint32_t)kk;
    } else if (greedy) {
      use_pool = true;  // t <= sample max <= row max: the maximum is in the pool
    } else if (topp_on) {
      if (need_bg) {
        double wc = mass_above(0u);
        w_f = wc + bg * exp((m_ref - m) * invT);
        use_pool = wc >= p * w_f * (1.0 + 1e-9);
      } else {
        use_pool = false;
      }
    } else {
      use_pool = ccount == nfin;  // everything is kept: the pool must hold all of F
    }
  }
  const uint32_t src_lo = use_pool ? tkey : K::kNegInf + 1u;  // every source key >= src_lo
  int rounds = 0;
  bool failed = false;

  // -- quaternary three-pivot search on counts (top-k) ---------------------------
  uint32_t kap = 0u, n_keep_k = 0u;
  if (topk_on) {
    uint32_t lo = src_lo - 1u, hi = maxk;
    bool found = false;
    while (!found) {
      if (rounds >= 48) { failed = true; break; }
      uint32_t d = hi - lo, tau[3];
#pragma unroll
      for (int n = 0; n < 3; ++n)
        tau[n] = d >= 4u ? lo + (uint32_t)(((uint64_t)d * (uint64_t)(n + 1)) >> 2)
                         : min(lo + (uint32_t)n, hi - 1u);
      uint32_t N[3] = {0u, 0u, 0u};
      MinCnt mc[3] = {{0xFFFFFFFFu, 0u}, {0xFFFFFFFFu, 0u}, {0xFFFFFFFFu, 0u}};
      walk([&](const uint32_t (&key)[8], const uint32_t (&)[8], uint32_t vm) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if ((vm >> j) & 1u) {
            uint32_t x = key[j];
#pragma unroll
            for (int n = 0; n < 3; ++n) {
              if (x > tau[n]) {
                ++N[n];
                if (x < mc[n].key) { mc[n].key = x; mc[n].cnt = 1u; }
                else if (x == mc[n].key) { ++mc[n].cnt; }
              }
            }
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

  // -- final boundary (pstar, n_keep): keep key > pstar, and the first n_keep
  //    ids of key == pstar --------------------------------------------------
  uint32_t pstar = K::kNegInf;  // keep-all: every source key is above it
  uint32_t n_keep = 0u;
  double w_p = 0.0, w_star = 0.0;
  if (greedy) {
    pstar = maxk;
    n_keep = 1u;
    w_star = 1.0;
    w_p = 1.0;
  } else if (!failed) {
    double w_k;
    double w_kap = topk_on ? weight<DT>(kap, m, invT) : 0.0;
    if (topk_on) {
      w_k = mass_above(kap) + (double)n_keep_k * w_kap;
    } else {
      w_k = (w_f >= 0.0) ? w_f : mass_above(0u);
    }
    if (topp_on) {
      // quaternary three-pivot search on fp64 mass inside K
      const double target = p * w_k;
      uint32_t lo = (topk_on ? kap : src_lo) - 1u, hi = maxk;
      const uint32_t excl = topk_on ? kap : 0u;  // per-token terms only for key > excl
      bool found = false;
      while (!found) {
        if (rounds >= 96) { failed = true; break; }
        uint32_t d = hi - lo, tau[3];
#pragma unroll
        for (int n = 0; n < 3; ++n)
          tau[n] = d >= 4u ? lo + (uint32_t)(((uint64_t)d * (uint64_t)(n + 1)) >> 2)
                           : min(lo + (uint32_t)n, hi - 1u);
        double M[3] = {0.0, 0.0, 0.0};
        MinCnt mc[3] = {{0xFFFFFFFFu, 0u}, {0xFFFFFFFFu, 0u}, {0xFFFFFFFFu, 0u}};
        walk([&](const uint32_t (&key)[8], const uint32_t (&)[8], uint32_t vm) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            uint32_t x = key[j];
            if (((vm >> j) & 1u) && x > excl && x > tau[0]) {
              double wt = weight<DT>(x, m, invT);
#pragma unroll
              for (int n = 0; n < 3; ++n) {
                if (x > tau[n]) {
                  M[n] += wt;
                  if (x < mc[n].key) { mc[n].key = x; mc[n].cnt = 1u; }
                  else if (x == mc[n].key) { ++mc[n].cnt; }
                }
              }
            }
          }
        });
#pragma unroll
        for (int n = 0; n < 3; ++n) {
          M[n] = wave_sum_f64(M[n]);
          mc[n] = wave_reduce_mc(mc[n]);
        }
        if (lane == 0) {
#pragma unroll
          for (int n = 0; n < 3; ++n) {
            uint64_t b = __double_as_longlong(M[n]);
            red.v[par][w][4 * n] = (uint32_t)b;
            red.v[par][w][4 * n + 1] = (uint32_t)(b >> 32);
            red.v[par][w][4 * n + 2] = mc[n].key;
            red.v[par][w][4 * n + 3] = mc[n].cnt;
          }
        }
        __syncthreads();
#pragma unroll
        for (int n = 0; n < 3; ++n) {
          M[n] = 0.0;
          mc[n] = MinCnt{0xFFFFFFFFu, 0u};
          for (int ww = 0; ww < kWaves; ++ww) {
            M[n] += __longlong_as_double(((uint64_t)red.v[par][ww][4 * n + 1] << 32) |
                                         red.v[par][ww][4 * n]);
            mc[n] = mc_merge(mc[n], MinCnt{red.v[par][ww][4 * n + 2], red.v[par][ww][4 * n + 3]});
          }
          // the boundary bucket of the top-k set holds only n_keep_k tokens
          if (topk_on && kap > tau[n]) {
            M[n] += (double)n_keep_k * w_kap;
            if (kap < mc[n].key) mc[n] = MinCnt{kap, n_keep_k};
          }
          M[n] = uni(M[n]);
          mc[n].key = uni(mc[n].key);
          mc[n].cnt = uni(mc[n].cnt);
        }
        par ^= 1;
        ++rounds;
#pragma unroll
        for (int n = 0; n < 3; ++n) {
          if (!found && M[n] >= target) {
            double wz = weight<DT>(mc[n].key, m, invT);
            double below = M[n] - (double)mc[n].cnt * wz;
            if (below < target) {
              found = true;
              pstar = mc[n].key;
              w_star = wz;
              // smallest count of boundary tokens that reaches the target
              double need = (target - below) / wz;
              uint32_t c = mc[n].cnt;
              uint32_t nk = need <= 1.0 ? 1u : (need >= (double)c ? c : (uint32_t)ceil(need));
              while (nk > 1u && below + (double)(nk - 1u) * wz >= target) --nk;
              while (nk < c && below + (double)nk * wz < target) ++nk;
              n_keep = nk;
              w_p = below + (double)nk * wz;
            }
          }
        }
        if (!found) {
#pragma unroll
          for (int n = 0; n < 3; ++n) {
            if (M[n] >= target) lo = tau[n] > lo ? tau[n] : lo;
            else hi = tau[n] < hi ? tau[n] : hi;
          }
        }
      }
    } else if (topk_on) {
      pstar = kap;
      n_keep = n_keep_k;
      w_star = w_kap;
      w_p = w_k;
    } else {
      pstar = K::kNegInf;
      n_keep = 0u;
      w_p = w_k;
    }
  }
  if (failed) {
    finish_error(QS_ROW_INTERNAL);
    return;
  }

  // -- walk A: per-wave counts of key > pstar and key == pstar, and q mass ------
  const double inv_wp = 1.0 / w_p;
  uint32_t gt = 0u, ties = 0u;
  double qgt = 0.0;
  walk([&](const uint32_t (&key)[8], const uint32_t (&)[8], uint32_t vm) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if ((vm >> j) & 1u) {
        if (key[j] > pstar) {
          ++gt;
          qgt += weight<DT>(key[j], m, invT) / w_p;
        } else if (key[j] == pstar) {
          ++ties;
        }
      }
    }
  });
  gt = wave_reduce<OpSum>(gt);
  ties = wave_reduce<OpSum>(ties);
  qgt = wave_sum_f64(qgt);
  if (lane == 0) {
    info.gt[w] = gt;
    info.ties[w] = ties;
    info.q[w] = qgt;
  }
  __syncthreads();
  uint32_t total_ties = 0u;
  for (int ww = 0; ww < kWaves; ++ww) total_ties += info.ties[ww];
  total_ties = uni(total_ties);
  if (pstar == K::kNegInf) n_keep = 0u;

  // -- walk B: id of the n_keep-th boundary token (earliest ids are kept) -------
  uint32_t id_cut = 0xFFFFFFFFu;
  if (n_keep < total_ties) {
    uint32_t before = 0u;
    int tw = 0;
    for (int ww = 0; ww < kWaves; ++ww) {
      uint32_t t = info.ties[ww];
      if (before + t >= n_keep) { tw = ww; break; }
      before += t;
    }
    const uint32_t want = n_keep - before;  // 1-based rank inside wave tw
    if (w == tw) {
      uint32_t seen = 0u;
      bool done = false;
      walk([&](const uint32_t (&key)[8], const uint32_t (&id)[8], uint32_t vm) {
        if (done) return;
        uint32_t tb = 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          tb |= ((((vm >> j) & 1u) && key[j] == pstar) ? 1u : 0u) << j;
        uint32_t total;
        uint32_t excl = wave_excl_small((uint32_t)__popc(tb), total);
        if (seen + total >= want) {
          // the lane whose range covers rank `want`
          uint32_t lo_r = seen + excl, hi_r = seen + excl + (uint32_t)__popc(tb);
          if (lo_r < want && want <= hi_r) {
            uint32_t need = want - lo_r;  // 1-based inside this lane
            uint32_t c = 0u;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              if ((tb >> j) & 1u) {
                ++c;
                if (c == need) red.v[par][0][39] = id[j];
              }
            }
          }
          done = true;
        }
        seen += total;
      });
    }
    __syncthreads();
    id_cut = uni(red.v[par][0][39]);
    par ^= 1;
  }

  // sampling uniform
  double u = 0.0;
  const bool sampled = SAMPLE && !greedy;
  if (sampled) {
    if (a.uniforms) u = a.uniforms[r];
    else u = (double)philox_u24(a.seed[r], a.offset[r]) * (1.0 / 16777216.0);
  }
  u = uni(u);

  // per-wave kept counts -> list offsets, cumulative q, and the wave holding u
  const double q_star = w_star / w_p;
  uint32_t my_off = 0u, n_p = 0u;
  double my_cum = 0.0;
  int sw = -1;
  {
    uint32_t tb = 0u;
    double cum = 0.0;
    for (int ww = 0; ww < kWaves; ++ww) {
      uint32_t t = info.ties[ww];
      uint32_t avail = n_keep > tb ? n_keep - tb : 0u;
      uint32_t kt = t < avail ? t : avail;
      tb += t;
      uint32_t kept = info.gt[ww] + kt;
      double qw = info.q[ww] + (double)kt * q_star;
      if (ww == w) { my_off = n_p; my_cum = cum; }
      if (sampled && sw < 0 && kept > 0u && u < cum + qw) sw = ww;
      n_p += kept;
      cum += qw;
    }
  }
  my_off = uni(my_off);
  n_p = uni(n_p);
  my_cum = uni(my_cum);
  sw = uni(sw);

  // -- walk D: outputs ------------------------------------------------------------
  zero_outputs();
  int32_t* ids_row = a.cand_ids ? a.cand_ids + (size_t)r * a.cand_cap : nullptr;
  float* probs_row = a.cand_probs ? a.cand_probs + (size_t)r * a.cand_cap : nullptr;
  const uint32_t cap = (uint32_t)a.cand_cap;
  uint32_t pos_base = my_off;
  double cbase = my_cum;
  int my_token = -1;         // set in wave sw
  int last_pos_id = -1;      // last kept id with q > 0 in this wave
  walk([&](const uint32_t (&key)[8], const uint32_t (&id)[8], uint32_t vm) {
    uint32_t pb = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bool in = ((vm >> j) & 1u) &&
                (key[j] > pstar || (key[j] == pstar && n_keep > 0u && id[j] <= id_cut));
      pb |= (in ? 1u : 0u) << j;
    }
    uint32_t total;
    uint32_t pos = pos_base + wave_excl_small((uint32_t)__popc(pb), total);
    double qv[8];
    double lane_sum = 0.0;
    uint32_t mword = 0u;
    int mwi = -1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      qv[j] = 0.0;
      if ((pb >> j) & 1u) {
        double q = greedy ? 1.0 : weight<DT>(key[j], m, invT) / w_p;
        qv[j] = q;
        lane_sum += q;
        float qf = (float)q;
        if (ids_row && pos < cap) ids_row[pos] = (int32_t)id[j];
        if (probs_row && pos < cap) probs_row[pos] = qf;
        if (dense_row) dense_row[id[j]] = qf;
        if (q > 0.0) last_pos_id = (int)id[j];
        int wi = (int)(id[j] >> 5);
        if (wi != mwi) {
          if (mwi >= 0 && mask_row) atomicOr(mask_row + mwi, mword);
          mwi = wi;
          mword = 0u;
        }
        mword |= 1u << (id[j] & 31u);
        ++pos;
      }
    }
    if (mwi >= 0 && mask_row) atomicOr(mask_row + mwi, mword);
    pos_base += total;
    if (w == sw && my_token < 0) {
      double incl = wave_incl_scan_f64(lane_sum, lane);
      double wtotal = __shfl(incl, 63, 64);
      double c = cbase + (incl - lane_sum);
      int hit = -1;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        c += qv[j];
        if (hit < 0 && ((pb >> j) & 1u) && u < c) hit = (int)id[j];
      }
      uint64_t hb = ballot(hit >= 0);
      if (hb) {
        int fl = __ffsll((unsigned long long)hb) - 1;
        my_token = __shfl(hit, fl, 64);
      }
      cbase += wtotal;
    }
  });

  // token: from wave sw; if rounding left u at or above the total, the last
  // kept id with q > 0
  int lp = last_pos_id;
  {
    uint32_t lpu = wave_reduce<OpMax>((uint32_t)(lp + 1));
    if (lane == 0) {
      red.v[par][w][0] = lpu;
      red.v[par][w][1] = (uint32_t)(my_token + 1);
    }
  }
  __syncthreads();
  int token = -1;
  if (greedy) {
    token = -1;
    for (int ww = 0; ww < kWaves && token < 0; ++ww)
      if (red.v[par][ww][0] > 0u) token = (int)red.v[par][ww][0] - 1;
  } else if (sampled) {
    if (sw >= 0) {
      token = (int)red.v[par][sw][1] - 1;
      // u fell past wave sw's last cumulative sum only by rounding
      if (token < 0 && red.v[par][sw][0] > 0u) token = (int)red.v[par][sw][0] - 1;
    }
    if (token < 0) {
      for (int ww = kWaves - 1; ww >= 0 && token < 0; --ww)
        if (red.v[par][ww][0] > 0u) token = (int)red.v[par][ww][0] - 1;
    }
  }
  par ^= 1;

  if (tid == 0) {
    const bool over = a.cand_ids || a.cand_probs ? n_p > cap : false;
    a.status[r] = over ? QS_ROW_CAND_OVERFLOW : QS_ROW_OK;
    if (a.cand_count) a.cand_count[r] = (int32_t)n_p;
    if (SAMPLE) {
      a.tokens[r] = token;
      if (sampled && !a.uniforms) a.offset[r] = a.offset[r] + 1u;
    }
    if (a.dbg) {
      a.dbg[4 * r + 0] = use_pool ? 0 : 1;
      a.dbg[4 * r + 1] = rounds;
      a.dbg[4 * r + 2] = (int32_t)ccount;
      a.dbg[4 * r + 3] = (int32_t)n_p;
    }
  }
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
  sl.wb = min(a.V, w * a.seg);
  sl.we = min(a.V, (w + 1) * a.seg);
  uint32_t maxk = 0u, mink = 0xFFFFFFFFu, nlegal = 0u, best_id = 0xFFFFFFFFu;
  walk_row<DT, true>(sl, lane, [&](const uint32_t (&key)[8], const uint32_t (&id)[8],
                                   uint32_t lm) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bool legal = (lm >> j) & 1u;
      uint32_t kx = legal ? key[j] : 0u;
      uint32_t kn = legal ? key[j] : 0xFFFFFFFFu;
      if (kx > maxk) { maxk = kx; best_id = id[j]; }  // ids ascend along a lane
      mink = kn < mink ? kn : mink;
    }
    nlegal += (uint32_t)__popc(lm);
  });
  uint32_t wmax = wave_reduce<OpMax>(maxk);
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
      uint32_t x = red.v[0][ww][0], c = red.v[0][ww][1];
      if (x > mx || (x == mx && c < bid)) { mx = x; bid = c; }
      uint32_t y = red.v[0][ww][2];
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
// Launchers (host side of this translation unit).
int seg_for(int V) {
  int s = (V + kWaves - 1) / kWaves;
  return (s + 31) & ~31;
}

hipError_t launch_filter(const FilterArgs& a, int dtype, bool sample, int B, hipStream_t st) {
  dim3 grid((unsigned)B), block(kThreads);
  if (dtype == QS_F32) {
    if (sample) hipLaunchKernelGGL((filter_rows_kernel<0, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((filter_rows_kernel<0, false>), grid, block, 0, st, a);
  } else {
    if (sample) hipLaunchKernelGGL((filter_rows_kernel<1, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((filter_rows_kernel<1, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_argmax(const ArgmaxArgs& a, int dtype, int B, hipStream_t st) {
  dim3 grid((unsigned)B), block(kThreads);
  if (dtype == QS_F32) hipLaunchKernelGGL((argmax_rows_kernel<0>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((argmax_rows_kernel<1>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace qs
