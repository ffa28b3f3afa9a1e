// Device building blocks for the gfx950 filter/sample kernels: order-preserving
// keys, wave64 DPP reductions, ballot-based scans, block reductions through LDS,
// Philox4x32-10 and the row layout every kernel shares.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace qs {

constexpr int kThreads = 1024;            // one workgroup per row
constexpr int kWaves = kThreads / 64;     // 16 wave64s
constexpr int kChunk = 8;                 // elements a lane handles per step
constexpr int kStep = 64 * kChunk;        // 512 elements per wave step
constexpr int kPoolBytes = 98304;         // LDS candidate pool per workgroup
constexpr int kResidentMaxSteps = 20;     // longest slice held in registers (steps)

// Candidate pool entry layout per dtype: key plus the token id relative to the
// wave's slice start (16 bits, so slices of at most 65536 tokens).
template <int DT> struct PoolLayout;
template <> struct PoolLayout<0> {   // fp32: 4-byte key + 2-byte id
  using KeyT = uint32_t;
  static constexpr int kPerWave = 1024;
};
template <> struct PoolLayout<1> {   // bf16: 2-byte key + 2-byte id
  using KeyT = uint16_t;
  static constexpr int kPerWave = 1536;
};
static_assert(kWaves * PoolLayout<0>::kPerWave * 6 <= kPoolBytes, "fp32 pool size");
static_assert(kWaves * PoolLayout<1>::kPerWave * 4 <= kPoolBytes, "bf16 pool size");
static_assert((PoolLayout<0>::kPerWave * 2) % 16 == 0, "pool rows stay 16-byte aligned");

// ---------------------------------------------------------------------------
// Order-preserving unsigned keys: the sign-magnitude bit pattern mapped to
// offset binary. key(a) < key(b) iff a < b and key(a) == key(b) iff a == b for
// non-NaN values (-0 and +0 share one key, as IEEE compares them equal); -inf
// maps to kNegInf, +inf to kPosInf, positive NaNs above kPosInf and negative
// NaNs below kNegInf. bf16 keys use 16 bits.
template <int DT> struct Keys;

template <> struct Keys<0> {  // float32
  static constexpr uint32_t kNegInf = 0x00800000u;
  static constexpr uint32_t kPosInf = 0xFF800000u;
  static constexpr uint32_t kMax = 0xFFFFFFFFu;
  // sign-magnitude -> offset binary: 0x80000000 +/- magnitude (both zeros 0x80000000)
  __device__ __forceinline__ static uint32_t of(uint32_t bits) {
    const uint32_t mag = bits & 0x7FFFFFFFu;
    return (bits & 0x80000000u) ? 0x80000000u - mag : 0x80000000u + mag;
  }
  __device__ __forceinline__ static uint32_t raw(uint32_t key) {
    return key >= 0x80000000u ? key - 0x80000000u : 0x80000000u | (0x80000000u - key);
  }
  __device__ __forceinline__ static float value(uint32_t key) { return __uint_as_float(raw(key)); }
};

template <> struct Keys<1> {  // bfloat16
  static constexpr uint32_t kNegInf = 0x0080u;
  static constexpr uint32_t kPosInf = 0xFF80u;
  static constexpr uint32_t kMax = 0xFFFFu;
  __device__ __forceinline__ static uint32_t of(uint32_t bits16) {
    const uint32_t mag = bits16 & 0x7FFFu;
    return (bits16 & 0x8000u) ? 0x8000u - mag : 0x8000u + mag;
  }
  __device__ __forceinline__ static uint32_t raw(uint32_t key) {
    return key >= 0x8000u ? key - 0x8000u : 0x8000u | (0x8000u - key);
  }
  __device__ __forceinline__ static float value(uint32_t key) {
    return __uint_as_float(raw(key) << 16);
  }
};

// ---------------------------------------------------------------------------
// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1, so that
// register arrays are only ever indexed by constants.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// ---------------------------------------------------------------------------
// Lane helpers.
__device__ __forceinline__ int lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// number of set bits of `mask` in lanes strictly below this lane
__device__ __forceinline__ uint32_t count_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Wave-uniform values made explicit (scalar registers).
__device__ __forceinline__ uint32_t uni(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}
__device__ __forceinline__ int32_t uni(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ double uni(double v) {
  uint64_t b = __double_as_longlong(v);
  uint32_t lo = uni((uint32_t)b), hi = uni((uint32_t)(b >> 32));
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ bool uni(bool v) { return uni((uint32_t)v) != 0u; }

// ---------------------------------------------------------------------------
// Wave64 all-reductions. Inside each 16-lane row: DPP quad_perm xor-1,
// quad_perm xor-2, row_half_mirror, row_mirror (every lane of the row ends
// with the row total); across the four rows: readlane of lanes 0/16/32/48.
// The combination order is fixed, so fp64 sums are deterministic.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  uint64_t b = __double_as_longlong(v);
  uint32_t lo = dpp_u32<CTRL>((uint32_t)b);
  uint32_t hi = dpp_u32<CTRL>((uint32_t)(b >> 32));
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  uint64_t b = __double_as_longlong(v);
  uint32_t lo = readlane_u32((uint32_t)b, l), hi = readlane_u32((uint32_t)(b >> 32), l);
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}

struct OpSum { __device__ static uint32_t f(uint32_t a, uint32_t b) { return a + b; } };
struct OpMax { __device__ static uint32_t f(uint32_t a, uint32_t b) { return a > b ? a : b; } };
struct OpMin { __device__ static uint32_t f(uint32_t a, uint32_t b) { return a < b ? a : b; } };

template <class Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v) {
  v = Op::f(v, dpp_u32<kDppXor1>(v));
  v = Op::f(v, dpp_u32<kDppXor2>(v));
  v = Op::f(v, dpp_u32<kDppHalfMirror>(v));
  v = Op::f(v, dpp_u32<kDppMirror>(v));
  uint32_t a = readlane_u32(v, 0), b = readlane_u32(v, 16);
  uint32_t c = readlane_u32(v, 32), d = readlane_u32(v, 48);
  return Op::f(Op::f(a, b), Op::f(c, d));
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<kDppXor1>(v);
  v += dpp_f64<kDppXor2>(v);
  v += dpp_f64<kDppHalfMirror>(v);
  v += dpp_f64<kDppMirror>(v);
  double a = readlane_f64(v, 0), b = readlane_f64(v, 16);
  double c = readlane_f64(v, 32), d = readlane_f64(v, 48);
  return (a + b) + (c + d);
}

// Inclusive prefix sums over the 64 lanes with DPP: shifts by 1, 2, 4, 8
// within each row of 16 lanes (lanes shifted in from outside the row read 0),
// then row_bcast:15 adds the last lane of rows 0 and 2 to rows 1 and 3, and
// row_bcast:31 adds lane 31 to rows 2 and 3. incl_shift1 moves every lane's
// value to the next lane (0 into lane 0).
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppWfShr1 = 0x138;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_rm(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_rm_f64(double v) {
  const uint64_t b = __double_as_longlong(v);
  const uint32_t lo = dpp_rm<CTRL, ROW_MASK>((uint32_t)b);
  const uint32_t hi = dpp_rm<CTRL, ROW_MASK>((uint32_t)(b >> 32));
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint32_t scan_incl_u32(uint32_t x) {
  x += dpp_rm<kDppRowShr1, 0xF>(x);
  x += dpp_rm<kDppRowShr2, 0xF>(x);
  x += dpp_rm<kDppRowShr4, 0xF>(x);
  x += dpp_rm<kDppRowShr8, 0xF>(x);
  x += dpp_rm<kDppRowBcast15, 0xA>(x);
  x += dpp_rm<kDppRowBcast31, 0xC>(x);
  return x;
}
__device__ __forceinline__ double scan_incl_f64(double x) {
  x += dpp_rm_f64<kDppRowShr1, 0xF>(x);
  x += dpp_rm_f64<kDppRowShr2, 0xF>(x);
  x += dpp_rm_f64<kDppRowShr4, 0xF>(x);
  x += dpp_rm_f64<kDppRowShr8, 0xF>(x);
  x += dpp_rm_f64<kDppRowBcast15, 0xA>(x);
  x += dpp_rm_f64<kDppRowBcast31, 0xC>(x);
  return x;
}
__device__ __forceinline__ double incl_shift1_f64(double incl) {
  return dpp_rm_f64<kDppWfShr1, 0xF>(incl);
}

// (minimum key, number of occurrences of that minimum) pairs.
struct MinCnt {
  uint32_t key;
  uint32_t cnt;
};
__device__ __forceinline__ MinCnt mc_merge(MinCnt a, MinCnt b) {
  MinCnt r;
  r.key = a.key < b.key ? a.key : b.key;
  r.cnt = (a.key == r.key ? a.cnt : 0u) + (b.key == r.key ? b.cnt : 0u);
  return r;
}
template <int CTRL>
__device__ __forceinline__ MinCnt dpp_mc(MinCnt v) {
  return MinCnt{dpp_u32<CTRL>(v.key), dpp_u32<CTRL>(v.cnt)};
}
__device__ __forceinline__ MinCnt wave_reduce_mc(MinCnt v) {
  v = mc_merge(v, dpp_mc<kDppXor1>(v));
  v = mc_merge(v, dpp_mc<kDppXor2>(v));
  v = mc_merge(v, dpp_mc<kDppHalfMirror>(v));
  v = mc_merge(v, dpp_mc<kDppMirror>(v));
  MinCnt a{readlane_u32(v.key, 0), readlane_u32(v.cnt, 0)};
  MinCnt b{readlane_u32(v.key, 16), readlane_u32(v.cnt, 16)};
  MinCnt c{readlane_u32(v.key, 32), readlane_u32(v.cnt, 32)};
  MinCnt d{readlane_u32(v.key, 48), readlane_u32(v.cnt, 48)};
  return mc_merge(mc_merge(a, b), mc_merge(c, d));
}

// ---------------------------------------------------------------------------
// Block reduction scratch: each wave deposits wave-uniform values in its slot,
// one barrier, then every thread combines the 16 slots in wave order. Two
// parities alternate so one barrier per reduction suffices.
constexpr int kSlots = 40;
struct RedScratch {
  uint32_t v[2][kWaves][kSlots];
};

// ---------------------------------------------------------------------------
// exp(x) in fp64 for the weights exp((z - m) / T), x <= ~0: x = n ln2 + r with
// n = rint(x / ln2) and a two-part ln2, |r| <= ln2/2, then the degree-11 Taylor
// polynomial of e^r (truncation < 7e-15 relative) and a power-of-two scale.
__device__ __forceinline__ double exp64(double x) {
  if (!(x > -745.0)) return 0.0;
  const double n = rint(x * 1.4426950408889634);
  const double r = fma(-n, 2.3190468138462996e-17, fma(-n, 0.6931471805599453, x));
  double q = 2.5052108385441720e-08;             // 1/11!
  q = fma(q, r, 2.7557319223985893e-07);         // 1/10!
  q = fma(q, r, 2.7557319223985888e-06);         // 1/9!
  q = fma(q, r, 2.4801587301587302e-05);         // 1/8!
  q = fma(q, r, 1.9841269841269841e-04);         // 1/7!
  q = fma(q, r, 1.3888888888888889e-03);         // 1/6!
  q = fma(q, r, 8.3333333333333333e-03);         // 1/5!
  q = fma(q, r, 4.1666666666666667e-02);         // 1/4!
  q = fma(q, r, 1.6666666666666667e-01);         // 1/3!
  q = fma(q, r, 0.5);
  q = fma(q, r, 1.0);
  q = fma(q, r, 1.0);
  return ldexp(q, (int)n);
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of the
// two-multiplier S-box on a 4x32 counter, key advanced by the Weyl constants
// between rounds.
__device__ __forceinline__ uint32_t philox_u24(uint64_t seed, uint64_t offset) {
  uint32_t c0 = (uint32_t)offset, c1 = (uint32_t)(offset >> 32), c2 = 0u, c3 = 0u;
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return c0 >> 8;
}

// ---------------------------------------------------------------------------
// Packed 16-bit views of a 32-bit register (two bf16 tokens per register).
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ s16x2 as_s2(uint32_t x) { return __builtin_bit_cast(s16x2, x); }
__device__ __forceinline__ u16x2 as_u2(uint32_t x) { return __builtin_bit_cast(u16x2, x); }
__device__ __forceinline__ uint32_t bits_of(s16x2 x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ uint32_t bits_of(u16x2 x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) {
  return (m & a) | (~m & b);
}

// The sigma-truncation threshold as a value (page "Qrita", key design 1 and
// the lookup table of the training-strategy paragraph): delta = Phi^-1(1 -
// k/V) for top-k; for top-p the mass-weighted Gaussian N(mu + sigma^2/T,
// sigma^2), truncated at the sample maximum, gives the value above which a
// fraction p of the mass lies. t = t0 - 0.2|t0|, never above the sample max.
// The quantiles are single precision: t only decides how many tokens are
// compacted, never which tokens are kept. Returns -inf when every finite
// legal token must be a candidate.
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
    t0 = mu + sd * (1.4142135623730951 * (double)erfcinvf((float)(2.0 * q)));
  } else if (topp_on) {
    if (!(sd > 0.0)) return ninf;
    const double mp = mu + sd * sd * invT;
    const double a = (ms - mp) / sd;
    const double c = (1.0 - p) * 0.5 * (double)erfcf((float)(-a * 0.7071067811865476));
    if (!(c > 0.0)) return ninf;
    t0 = mp - sd * (1.4142135623730951 * (double)erfcinvf((float)(2.0 * c)));
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

}  // namespace qs
