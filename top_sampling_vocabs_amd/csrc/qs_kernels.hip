// Exact top-k / top-p filter-and-sample kernels for gfx950 (MI355X).
//
// One 1024-thread workgroup owns one row. Its 16 wave64s each own a
// contiguous slice of the vocabulary (a multiple of 32 tokens, so every
// packed-mask word belongs to one wave), which keeps every per-wave walk in
// token-id order and makes the outputs deterministic.
//
// Per row (page "Qrita", overall framework and key designs 1-3):
//  1. sigma-truncation (key design 1): the first 512-token step of each
//     slice is a sample (8192 tokens) for mean, sigma and the sample maximum;
//     the threshold t = t0 - 0.2|t0| uses the Gaussian quantile of k/V
//     (top-k) or of p under the mass-weighted Gaussian (top-p). One pipelined
//     pass over the row then compacts the legal tokens with z >= t into a
//     per-wave LDS pool, in id order, counts legal tokens, checks for NaN,
//     and for rows with top-k off accumulates the mass below t.
//  2. hit test: |Z_t| >= k (top-k), or mass(Z_t) >= p * W (top-p only);
//     otherwise every later step runs over the full row (the page's
//     fallback Z_s = Z).
//  3. quaternary three-pivot search (key design 2) for the k-th largest
//     value: pivots at 1/4, 1/2, 3/4 of the current key interval; one fused
//     pass counts N_tau, the minimum above tau and its multiplicity for all
//     three pivots; it stops when N_tau >= k and N_tau - N_zm < k. Pivots are
//     order-preserving integer keys, so a search ends within 8 (bf16) or 16
//     (fp32) rounds even when values repeat. For bf16 pools the pass runs over
//     a per-key histogram of the pool instead of its elements.
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
#include "qs_stream.hpp"
#include "../../include/qs.h"

namespace qs {

typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ s16x2 as_s2(uint32_t x) { return __builtin_bit_cast(s16x2, x); }
__device__ __forceinline__ u16x2 as_u2(uint32_t x) { return __builtin_bit_cast(u16x2, x); }
__device__ __forceinline__ uint32_t bits_of(s16x2 x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ uint32_t bits_of(u16x2 x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) {
  return (m & a) | (~m & b);
}

constexpr int kHistBins = 2048;   // bf16 pool histogram (keys tkey .. tkey+2047)

// Relative error bound of one hardware exp2 (v_exp_f32), taken as 4 ulp.
constexpr double kExp2Err = 2.384185791015625e-07;  // 2^-22

// fp64 weight of a key relative to the row maximum: exp((z - m) / T).
template <int DT>
__device__ __forceinline__ double weight(uint32_t key, double m, double invT) {
  return exp64(((double)Keys<DT>::value(key) - m) * invT);
}

// The sigma-truncation threshold as a value (page "Qrita", key design 1 and
// the lookup table of the training-strategy paragraph): delta = Phi^-1(1 -
// k/V) for top-k; for top-p the mass-weighted Gaussian N(mu + sigma^2/T,
// sigma^2), truncated at the sample maximum, gives the value above which a
// fraction p of the mass lies. t = t0 - 0.2|t0|, never above the sample max.
// Returns -inf when every finite legal token must be a candidate.
__device__ __forceinline__ double truncation_value(double n_s, double sum, double sumsq,
                                                   double ms, double frac_legal, int V,
                                                   bool greedy, bool topk_on, int k,
                                                   bool topp_on, double p, double invT) {
  const double ninf = -__builtin_inf();
  if (n_s < 1.0) return ninf;
  if (greedy) return ms;
  const double mu = sum / n_s;
  const double var = sumsq / n_s - mu * mu;
  const double sd = var > 0.0 ? sqrt(var) : 0.0;
  double t0;
  if (topk_on) {
    const double q = (double)k / (frac_legal * (double)V);
    if (!(q < 1.0)) return ninf;
    t0 = mu + sd * (1.4142135623730951 * erfcinv(2.0 * q));
  } else if (topp_on) {
    if (!(sd > 0.0)) return ninf;
    const double mp = mu + sd * sd * invT;
    const double a = (ms - mp) / sd;
    const double c = (1.0 - p) * 0.5 * erfc(-a * 0.7071067811865476);
    if (!(c > 0.0)) return ninf;
    t0 = mp - sd * (1.4142135623730951 * erfcinv(2.0 * c));
  } else {
    return ninf;
  }
  double t = t0 - 0.2 * fabs(t0);
  if (!(t < ms)) t = ms;
  if (!(t > -3.0e38)) return ninf;
  return t;
}

// The largest bf16 / fp32 value <= t (t finite), as raw bits.
template <int DT>
__device__ __forceinline__ uint32_t raw_floor(double t) {
  const uint32_t b = __float_as_uint(__double2float_rd(t));
  if constexpr (DT == 0) return b;
  uint32_t h = b >> 16;
  if ((b & 0x80000000u) && (b & 0xFFFFu)) h += 1u;  // negative: round away from 0
  return h;
}

// ---------------------------------------------------------------------------
template <int DT, bool SAMPLE>
__global__ void __launch_bounds__(kThreads) filter_rows_kernel(FilterArgs a) {
  using K = Keys<DT>;
  using PL = PoolLayout<DT>;
  using PKey = typename PL::KeyT;
  constexpr uint32_t kCap = (uint32_t)PL::kPerWave;
  __shared__ __align__(16) uint8_t pool_raw[kPoolBytes];
  __shared__ __align__(16) uint4 lut[DT == 1 ? 256 : 1];
  __shared__ uint32_t hist[DT == 1 ? kHistBins : 1];
  __shared__ RedScratch red;
  __shared__ struct {
    uint32_t cnt[kWaves];
    uint32_t gt[kWaves];
    uint32_t ties[kWaves];
    double q[kWaves];
  } info;

  PKey* const pool_key = reinterpret_cast<PKey*>(pool_raw);
  uint16_t* const pool_id = reinterpret_cast<uint16_t*>(pool_raw + sizeof(PKey) * kWaves * kCap);

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
  sl.wb = uni(min(V, w * a.seg));
  sl.we = uni(min(V, (w + 1) * a.seg));
  const int W = (V + 31) >> 5;

  uint32_t* mask_row = a.keep_mask ? a.keep_mask + (size_t)r * W : nullptr;
  float* dense_row = a.dense ? a.dense + (size_t)r * V : nullptr;

  // Zero this wave's share of the mask and dense outputs and wait until the
  // stores have completed, so that this wave's later scatter into the same
  // slice lands after them.
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
  if (!(isfinite(Tf) && Tf >= 0.0f) || kk < 0 || !(pf > 0.0f && pf <= 1.0f)) {
    finish_error(QS_ROW_BAD_PARAM);
    return;
  }
  const bool greedy = (Tf == 0.0f);
  const double invT = greedy ? 0.0 : 1.0 / (double)Tf;
  const double p = (double)pf;
  const bool topp_on = !greedy && pf < 1.0f;
  // top-k is requested for k in [1, V); whether k < |F| is known after the pass
  const bool topk_req = !greedy && kk > 0 && kk < V;
  const bool need_bg = topp_on && !topk_req;
  const bool no_trunc = (a.flags & QS_FLAG_NO_TRUNCATION) != 0u;

  if constexpr (DT == 1) {  // pair masks of every legal byte: 0xFFFF per legal token
    if (tid < 256) {
      uint32_t v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v[q] = ((((uint32_t)tid >> (2 * q)) & 1u) ? 0x0000FFFFu : 0u) |
               ((((uint32_t)tid >> (2 * q + 1)) & 1u) ? 0xFFFF0000u : 0u);
      lut[tid] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  }

  // -- one pass over the row, with the sample taken from its first step --------
  constexpr int D = DT == 1 ? 8 : 4;
  RowReader<DT, D> rd(sl, lane);
  const int nst = rd.n;
#pragma unroll
  for (int i = 0; i < D; ++i)
    if (i < nst) rd.issue(i, i);

  // sample statistics of step 0 (legal finite tokens)
  double s_n = 0.0, s_sum = 0.0, s_sq = 0.0, s_all = 0.0;
  uint32_t s_maxk = 0u;
  if (nst > 0) {
    Raw<DT> raw;
    uint32_t mb;
    rd.fetch(0, 0, raw, mb);
    const int e = rd.first(0);
    s_all = (double)max(0, min(8, min(sl.we, sl.wb + kStep) - e));
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
  {
    double st[4] = {s_n, s_sum, s_sq, s_all};
#pragma unroll
    for (int i = 0; i < 4; ++i) st[i] = wave_sum_f64(st[i]);
    const uint32_t mx = wave_reduce<OpMax>(s_maxk);
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint64_t b = __double_as_longlong(st[i]);
        red.v[par][w][2 * i] = (uint32_t)b;
        red.v[par][w][2 * i + 1] = (uint32_t)(b >> 32);
      }
      red.v[par][w][8] = mx;
    }
  }
  __syncthreads();  // also publishes the pair-mask table
  {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    uint32_t mx = 0u;
    for (int ww = 0; ww < kWaves; ++ww) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[i] += __longlong_as_double(((uint64_t)red.v[par][ww][2 * i + 1] << 32) |
                                       red.v[par][ww][2 * i]);
      const uint32_t m2 = red.v[par][ww][8];
      mx = m2 > mx ? m2 : mx;
    }
    s_n = uni(acc[0]); s_sum = uni(acc[1]); s_sq = uni(acc[2]); s_all = uni(acc[3]);
    s_maxk = uni(mx);
  }
  par ^= 1;

  const double ms = s_n >= 1.0 ? (double)K::value(s_maxk) : 0.0;
  const double tval = truncation_value(s_n, s_sum, s_sq, ms, s_all > 0.0 ? s_n / s_all : 0.0,
                                       V, greedy, topk_req, kk, topp_on, p, invT);
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
  uint32_t nlegal = 0u, pcnt = 0u;
  int32_t nmin = DT == 1 ? 0x7FFF : 0x7FFFFFFF;  // smallest legal signed value
  uint32_t nmin2 = 0x7FFF7FFFu;                  // bf16: packed per half
  uint32_t nmax2 = 0u, nmax1 = 0u;               // largest legal raw bits (POS pass)
  double bg_sum = 0.0;     // sum of exp2((z - bg_ref) c) over legal finite z < t
  float bg_wx = 0.0f;      // sum of w |x| (error bound)
  float bg_w32 = 0.0f;     // sum of w in fp32 (error bound)
  PKey* const my_pk = pool_key + w * kCap;
  uint16_t* const my_pid = pool_id + w * kCap;

  auto pass = [&](auto bg_on, auto pos_t) {
    constexpr bool BG = decltype(bg_on)::value;
    // POS: the threshold is a positive value, so a legal token is a candidate
    // iff its raw bits, read as a signed integer, are >= those of t (negative
    // values have the sign bit set); no magnitude transform is needed.
    constexpr bool POS = decltype(pos_t)::value;
    auto step = [&](const Raw<DT>& raw, uint32_t mb, int e) {
      nlegal += (uint32_t)__popc(mb);
      uint32_t cb;
      float sw = 0.0f, swx = 0.0f;
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
            rl = bfi(pm[q], d, 0x80008000u);  // illegal -> 0x8000 (lowest as signed)
            // a legal negative NaN has raw bits above 0xFF80
            nmax2 = bits_of(__builtin_elementwise_max(as_u2(nmax2), as_u2(rl)));
          } else {
            // signed value of each half: +magnitude or -magnitude
            const uint32_t mag = d & 0x7FFF7FFFu;
            const uint32_t sg = bits_of(as_s2(d) >> 15);
            const uint32_t sv = bits_of(as_s2(mag ^ sg) - as_s2(sg));
            rl = bfi(pm[q], sv, 0x80008000u);   // illegal -> lowest
            nmin2 = bits_of(__builtin_elementwise_min(as_s2(nmin2),
                                                      as_s2(bfi(pm[q], sv, 0x7FFF7FFFu))));
          }
          dl[q] = bits_of(__builtin_elementwise_sub_sat(as_s2(t2m1), as_s2(rl)));  // <0 iff cand
          if constexpr (BG) {
            const uint32_t cm = bits_of(as_s2(dl[q]) >> 15);        // 0xFFFF per candidate
            const uint32_t zb = bfi(pm[q] & ~cm, d, 0xFF80FF80u);   // others -> -inf
            const float zlo = __uint_as_float(zb << 16);
            const float zhi = __uint_as_float(zb & 0xFFFF0000u);
            const float xlo = fmaxf((zlo - bg_ref) * bg_c, -200.0f);
            const float xhi = fmaxf((zhi - bg_ref) * bg_c, -200.0f);
            const float wlo = __builtin_amdgcn_exp2f(xlo);
            const float whi = __builtin_amdgcn_exp2f(xhi);
            sw += wlo + whi;
            swx = fmaf(wlo, -xlo, fmaf(whi, -xhi, swx));
          }
        }
        const uint32_t cA = __builtin_amdgcn_perm(dl[1], dl[0], 0x0B0A0908u);
        const uint32_t cB = __builtin_amdgcn_perm(dl[3], dl[2], 0x0B0A0908u);
        cb = __builtin_amdgcn_sad_u8(cB & 0x80402010u, 0u,
                                     __builtin_amdgcn_sad_u8(cA & 0x08040201u, 0u, 0u));
      } else {
        cb = 0u;
#pragma unroll
        for (int j = 7; j >= 0; --j) {
          const uint32_t d = raw.r[j];
          const uint32_t mj = (uint32_t)__builtin_amdgcn_sbfe((int)mb, j, 1);
          int32_t rl;
          if constexpr (POS) {
            rl = (int32_t)bfi(mj, d, 0x80000000u);  // illegal -> INT_MIN
            nmax1 = max(nmax1, (uint32_t)rl);       // legal negative NaN > 0xFF800000
          } else {
            const uint32_t mag = d & 0x7FFFFFFFu;
            const uint32_t sv = (d & 0x80000000u) ? 0u - mag : mag;
            rl = (int32_t)bfi(mj, sv, 0x80000000u);
            nmin = min(nmin, (int32_t)bfi(mj, sv, 0x7FFFFFFFu));
          }
          const bool cand = rl >= tS;
          cb = cb * 2u + (cand ? 1u : 0u);
          if constexpr (BG) {
            const float z = (mj && !cand) ? __uint_as_float(d) : -__builtin_inff();
            const float x = fmaxf((z - bg_ref) * bg_c, -200.0f);
            const float wv = __builtin_amdgcn_exp2f(x);
            sw += wv;
            swx = fmaf(wv, -x, swx);
          }
        }
      }
      if constexpr (BG) {
        bg_sum += (double)sw;
        bg_w32 += sw;
        bg_wx += swx;
      }
      pcnt = append_candidates<DT>(cb, raw, (uint32_t)(e - sl.wb), pcnt, my_pk, my_pid);
    };
    for (int s0 = 0; s0 < nst; s0 += D) {
#pragma unroll
      for (int i = 0; i < D; ++i) {
        const int st = s0 + i;
        if (st < nst) {
          Raw<DT> raw;
          uint32_t mb;
          rd.fetch(st, i, raw, mb);
          step(raw, mb, rd.first(st));
          if (st + D < nst) rd.issue(st + D, i);
        }
      }
    }
  };
  const bool pos_t = tS > 0;
  if (need_bg) {
    if (pos_t) pass(std::true_type{}, std::true_type{});
    else pass(std::true_type{}, std::false_type{});
  } else {
    if (pos_t) pass(std::false_type{}, std::true_type{});
    else pass(std::false_type{}, std::false_type{});
  }
  // smallest legal signed value (a negative NaN lies below -inf)
  if constexpr (DT == 1) {
    const s16x2 v = as_s2(nmin2);
    nmin = min((int32_t)v.x, (int32_t)v.y);
    const uint32_t hmax = max(nmax2 & 0xFFFFu, nmax2 >> 16);
    if (hmax > 0xFF80u) nmin = -0x7FFF;  // raw bits of a negative NaN
  } else {
    if (nmax1 > 0xFF800000u) nmin = min(nmin, -0x7FFFFFFF);  // raw bits of a negative NaN
  }

  // -- reduce the pass -------------------------------------------------------------
  nlegal = wave_reduce<OpSum>(nlegal);
  const uint32_t nmin_u = wave_reduce<OpMin>((uint32_t)nmin ^ 0x80000000u);  // signed order
  bg_sum = wave_sum_f64(bg_sum);
  const double bg_wx64 = wave_sum_f64((double)bg_wx);
  const double bg_w64 = wave_sum_f64((double)bg_w32);
  if (lane == 0) {
    red.v[par][w][0] = nlegal;
    red.v[par][w][1] = nmin_u;
    info.cnt[w] = pcnt;
    const uint64_t b0 = __double_as_longlong(bg_sum), b1 = __double_as_longlong(bg_wx64);
    const uint64_t b2 = __double_as_longlong(bg_w64);
    red.v[par][w][2] = (uint32_t)b0; red.v[par][w][3] = (uint32_t)(b0 >> 32);
    red.v[par][w][4] = (uint32_t)b1; red.v[par][w][5] = (uint32_t)(b1 >> 32);
    red.v[par][w][6] = (uint32_t)b2; red.v[par][w][7] = (uint32_t)(b2 >> 32);
  }
  __syncthreads();
  uint32_t ccount = 0u, my_wcnt = 0u;
  bool overflow = false, neg_nan = false;
  double bg_err = 0.0;
  {
    uint32_t nl = 0u, mn = 0xFFFFFFFFu;
    double b0 = 0.0, b1 = 0.0, b2 = 0.0;
    for (int ww = 0; ww < kWaves; ++ww) {
      nl += red.v[par][ww][0];
      const uint32_t y = red.v[par][ww][1];
      mn = y < mn ? y : mn;
      const uint32_t c = info.cnt[ww];
      if (ww == w) my_wcnt = c;
      ccount += c;
      overflow = overflow || c > kCap;
      b0 += __longlong_as_double(((uint64_t)red.v[par][ww][3] << 32) | red.v[par][ww][2]);
      b1 += __longlong_as_double(((uint64_t)red.v[par][ww][5] << 32) | red.v[par][ww][4]);
      b2 += __longlong_as_double(((uint64_t)red.v[par][ww][7] << 32) | red.v[par][ww][6]);
    }
    nlegal = uni(nl);
    const int32_t lowest = (int32_t)(mn ^ 0x80000000u);
    const int32_t neg_inf_s = DT == 1 ? -0x7F80 : -0x7F800000;
    neg_nan = uni(lowest < neg_inf_s);
    bg_sum = uni(b0);
    // per term: exp2 error plus the argument's three roundings (ln2 * 3 * 2^-24 |x|),
    // plus the fp32 accumulation of 8 terms per step
    bg_err = uni(kExp2Err * b2 + 1.24e-7 * b1 + 4.2e-7 * b2 + 1e-30);
  }
  ccount = uni(ccount);
  my_wcnt = uni(my_wcnt);
  overflow = uni(overflow);
  par ^= 1;

  const PKey* pk = my_pk;
  const uint16_t* pid = my_pid;
  const int my_cnt = (int)min(my_wcnt, kCap);
  // pool usable: complete, 16-bit ids fit, not forced off
  const bool pool_ok = !overflow && ccount > 0u && !(a.flags & QS_FLAG_FORCE_MISS) &&
                       !no_trunc && a.seg <= 65536;

  // -- row statistics: max, argmax, non-finite, -inf count ----------------------
  // From the pool when it holds the maximum (t never exceeds the sample max),
  // otherwise from a walk over the row.
  uint32_t maxk = 0u, max_id = 0xFFFFFFFFu, nfin = nlegal;
  bool nonfinite = neg_nan;
  {
    uint32_t mk = 0u, mid = 0xFFFFFFFFu, mn = 0xFFFFFFFFu, ninf = 0u;
    auto track = [&](const uint32_t (&key)[8], const uint32_t (&id)[8], uint32_t lm) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if ((lm >> j) & 1u) {
          if (key[j] > mk) { mk = key[j]; mid = id[j]; }  // ids ascend along a lane
          mn = key[j] < mn ? key[j] : mn;
          ninf += key[j] == K::kNegInf ? 1u : 0u;
        }
      }
    };
    if (pool_ok) walk_pool<DT>(pk, pid, my_cnt, (uint32_t)sl.wb, lane, track);
    else walk_row<DT, true>(sl, lane, track);
    const uint32_t wmax = wave_reduce<OpMax>(mk);
    const uint32_t cid = wave_reduce<OpMin>(mk == wmax ? mid : 0xFFFFFFFFu);
    mn = wave_reduce<OpMin>(mn);
    ninf = wave_reduce<OpSum>(ninf);
    if (lane == 0) {
      red.v[par][w][0] = wmax; red.v[par][w][1] = cid;
      red.v[par][w][2] = mn; red.v[par][w][3] = ninf;
    }
    __syncthreads();
    uint32_t gm = 0u, gid = 0xFFFFFFFFu, gmn = 0xFFFFFFFFu, gninf = 0u;
    for (int ww = 0; ww < kWaves; ++ww) {
      const uint32_t x = red.v[par][ww][0], c = red.v[par][ww][1];
      if (x > gm || (x == gm && c < gid)) { gm = x; gid = c; }
      const uint32_t y = red.v[par][ww][2];
      gmn = y < gmn ? y : gmn;
      gninf += red.v[par][ww][3];
    }
    par ^= 1;
    maxk = uni(gm);
    max_id = uni(gid);
    if (!pool_ok) {
      nfin = uni(nlegal - gninf);
      nonfinite = nonfinite || uni(gmn < K::kNegInf);
    }
    nonfinite = nonfinite || maxk >= K::kPosInf;
  }

  // -- row status --------------------------------------------------------------
  if (nlegal == 0u) { finish_error(QS_ROW_EMPTY); return; }
  if (nonfinite) { finish_error(QS_ROW_NONFINITE); return; }
  if (maxk <= K::kNegInf) { finish_error(QS_ROW_ALL_NEG_INF); return; }

  const double m = (double)K::value(maxk);
  // with a usable pool, |F| >= |Z_t|, so k < |Z_t| already settles k < |F|;
  // otherwise the row walk above counted |F| exactly
  const bool topk_on = !greedy && kk > 0 &&
                       (pool_ok ? (uint32_t)kk < ccount : (uint32_t)kk < nfin);

  // -- source selection (hit test) -------------------------------------------
  bool use_pool = pool_ok;
  double w_f = -1.0, w_f_err = 0.0, w_pool = 0.0;
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
  if (use_pool) {
    if (greedy) {
      use_pool = true;
    } else if (topk_on) {
      use_pool = true;  // kk < |Z_t|
    } else if (topp_on && need_bg) {
      double s = 0.0;
      walk_pool<DT>(pk, pid, my_cnt, (uint32_t)sl.wb, lane,
                    [&](const uint32_t (&key)[8], const uint32_t (&)[8], uint32_t vm) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if ((vm >> j) & 1u) s += weight<DT>(key[j], m, invT);
      });
      w_pool = block_sum_f64(s);
      const double scale = exp64(((double)bg_ref - m) * invT);
      w_f = w_pool + bg_sum * scale;
      w_f_err = bg_err * scale;
      use_pool = w_pool >= p * (w_f + w_f_err) * (1.0 + 1e-9);
    } else if (topp_on) {
      use_pool = false;  // k >= |Z_t| but the mass below t is unknown
    } else {
      // everything is kept: the pool must hold all of F, and |F| is unknown
      use_pool = false;
    }
  }
  if (!use_pool) w_f_err = 0.0;
  uint32_t nf_exact = nfin;
  if (!use_pool && pool_ok) {
    // the row walk above ran on the pool: count |F| on the row now
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
    nf_exact = uni(nlegal - t);
  }
  const bool topk_eff = !greedy && kk > 0 && (uint32_t)kk < nf_exact;
  const uint32_t src_lo = use_pool ? tkey : K::kNegInf + 1u;  // every source key >= src_lo

  // -- per-key histogram of a bf16 pool ------------------------------------------
  const bool use_hist = DT == 1 && use_pool && !greedy && (maxk - src_lo) < (uint32_t)kHistBins;
  if constexpr (DT == 1) {
    if (use_hist) {
    for (int b = tid; b < kHistBins; b += kThreads) hist[b] = 0u;
    __syncthreads();
    walk_pool<DT>(pk, pid, my_cnt, (uint32_t)sl.wb, lane,
                  [&](const uint32_t (&key)[8], const uint32_t (&)[8], uint32_t vm) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if ((vm >> j) & 1u) atomicAdd(&hist[key[j] - src_lo], 1u);
    });
    __syncthreads();
    }
  }
  const uint32_t nbins = use_hist ? maxk - src_lo + 1u : 0u;

  // items of the searches: (key, multiplicity) from the histogram, else tokens
  auto for_items = [&](auto&& f) {
    if (DT == 1 && use_hist) {
      for (uint32_t b = (uint32_t)tid; b < nbins; b += kThreads) {
        const uint32_t c = hist[DT == 1 ? b : 0u];
        if (c) f(src_lo + b, c);
      }
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

  // mass of source items with key > lo_excl
  auto mass_above = [&](uint32_t lo_excl) -> double {
    double s = 0.0;
    for_items([&](uint32_t key, uint32_t c) {
      if (key > lo_excl) s += (double)c * weight<DT>(key, m, invT);
    });
    return block_sum_f64(s);
  };

  int rounds = 0;
  bool failed = false;

  // -- quaternary three-pivot search on counts (top-k) ---------------------------
  uint32_t kap = 0u, n_keep_k = 0u;
  if (topk_eff) {
    uint32_t lo = src_lo - 1u, hi = maxk;
    bool found = false;
    while (!found) {
      if (rounds >= 48) { failed = true; break; }
      const uint32_t d = hi - lo;
      uint32_t tau[3];
#pragma unroll
      for (int n = 0; n < 3; ++n)
        tau[n] = d >= 4u ? lo + (uint32_t)(((uint64_t)d * (uint64_t)(n + 1)) >> 2)
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
    const double w_kap = topk_eff ? weight<DT>(kap, m, invT) : 0.0;
    double w_k;
    if (topk_eff) w_k = mass_above(kap) + (double)n_keep_k * w_kap;
    else if (w_f >= 0.0 && use_pool) w_k = w_f;
    else w_k = mass_above(0u);
    if (topp_on) {
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
        while (!found) {
          if (rounds >= 96) { failed = true; break; }
          const uint32_t d = hi - lo;
          uint32_t tau[3];
#pragma unroll
          for (int n = 0; n < 3; ++n)
            tau[n] = d >= 4u ? lo + (uint32_t)(((uint64_t)d * (uint64_t)(n + 1)) >> 2)
                             : min(lo + (uint32_t)n, hi - 1u);
          double M[3] = {0.0, 0.0, 0.0};
          MinCnt mc[3] = {{0xFFFFFFFFu, 0u}, {0xFFFFFFFFu, 0u}, {0xFFFFFFFFu, 0u}};
          for_items([&](uint32_t x, uint32_t c) {
            if (x > excl && x > tau[0]) {
              const double wt = (double)c * weight<DT>(x, m, invT);
#pragma unroll
              for (int n = 0; n < 3; ++n) {
                if (x > tau[n]) {
                  M[n] += wt;
                  if (x < mc[n].key) { mc[n].key = x; mc[n].cnt = c; }
                  else if (x == mc[n].key) { mc[n].cnt += c; }
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
            if (topk_eff && kap > tau[n]) {
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
              const double wz = weight<DT>(mc[n].key, m, invT);
              const double below = M[n] - (double)mc[n].cnt * wz;
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
                w_p = below + (double)nk * wz;
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
              if (M[n] >= target) lo = tau[n] > lo ? tau[n] : lo;
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
        w_k = w_pool + block_sum_f64(s);
        err = 0.0;
      }
    } else if (topk_eff) {
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
  if (pstar == K::kNegInf) n_keep = 0u;

  // -- walk A: per-wave counts of key > pstar and key == pstar, and q mass ------
  const double inv_wp = 1.0 / w_p;
  {
    uint32_t gt = 0u, ties = 0u;
    double qgt = 0.0;
    walk([&](const uint32_t (&key)[8], const uint32_t (&)[8], uint32_t vm) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if ((vm >> j) & 1u) {
          if (key[j] > pstar) {
            ++gt;
            qgt += weight<DT>(key[j], m, invT) * inv_wp;
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
  }
  __syncthreads();
  uint32_t total_ties = 0u;
  for (int ww = 0; ww < kWaves; ++ww) total_ties += info.ties[ww];
  total_ties = uni(total_ties);

  // -- walk B: id of the n_keep-th boundary token (earliest ids are kept) -------
  uint32_t id_cut = 0xFFFFFFFFu;
  if (greedy) {
    id_cut = max_id;
  } else if (n_keep < total_ties) {
    uint32_t before = 0u;
    int tw = 0;
    for (int ww = 0; ww < kWaves; ++ww) {
      const uint32_t t = info.ties[ww];
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
        const uint32_t excl = wave_excl_small((uint32_t)__popc(tb), total);
        if (seen + total >= want) {
          const uint32_t lo_r = seen + excl, hi_r = seen + excl + (uint32_t)__popc(tb);
          if (lo_r < want && want <= hi_r) {
            const uint32_t need = want - lo_r;  // 1-based inside this lane
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
  const double q_star = w_star * inv_wp;
  uint32_t my_off = 0u, n_p = 0u;
  double my_cum = 0.0;
  int sw = -1;
  {
    uint32_t tb = 0u;
    double cum = 0.0;
    for (int ww = 0; ww < kWaves; ++ww) {
      const uint32_t t = info.ties[ww];
      const uint32_t avail = n_keep > tb ? n_keep - tb : 0u;
      const uint32_t kt = t < avail ? t : avail;
      tb += t;
      const uint32_t kept = info.gt[ww] + kt;
      const double qw = info.q[ww] + (double)kt * q_star;
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
      const bool in = ((vm >> j) & 1u) &&
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
        const double q = greedy ? 1.0 : weight<DT>(key[j], m, invT) * inv_wp;
        qv[j] = q;
        lane_sum += q;
        const float qf = (float)q;
        if (ids_row && pos < cap) ids_row[pos] = (int32_t)id[j];
        if (probs_row && pos < cap) probs_row[pos] = qf;
        if (dense_row) dense_row[id[j]] = qf;
        if (q > 0.0) last_pos_id = (int)id[j];
        const int wi = (int)(id[j] >> 5);
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
      const double incl = wave_incl_scan_f64(lane_sum, lane);
      const double wtotal = __shfl(incl, 63, 64);
      double c = cbase + (incl - lane_sum);
      int hit = -1;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        c += qv[j];
        if (hit < 0 && ((pb >> j) & 1u) && u < c) hit = (int)id[j];
      }
      const uint64_t hb = ballot(hit >= 0);
      if (hb) {
        const int fl = __ffsll((unsigned long long)hb) - 1;
        my_token = __shfl(hit, fl, 64);
      }
      cbase += wtotal;
    }
  });

  // token: from wave sw; if rounding left u at or above the total, the last
  // kept id with q > 0
  {
    const uint32_t lpu = wave_reduce<OpMax>((uint32_t)(last_pos_id + 1));
    if (lane == 0) {
      red.v[par][w][0] = lpu;
      red.v[par][w][1] = (uint32_t)(my_token + 1);
    }
  }
  __syncthreads();
  int token = -1;
  if (greedy) {
    token = (int)max_id;
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
    const bool over = (a.cand_ids || a.cand_probs) ? n_p > cap : false;
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
