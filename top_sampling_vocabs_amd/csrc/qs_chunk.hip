// Chunked first pass of the filter for bf16 rows (layout and contract in
// qs_chunk.hpp).
//
// A persistent workgroup of 4 wave64s scans a run of consecutive chunks
// (16384 tokens: 4 segments of 4096, one per wave), as many workgroups as
// fit the GPU. Chunks are numbered chunk-major (chunk q is chunk q / B of row
// q mod B), so that a run mixes rows, and with them the heavier rows whose
// top-p cut needs the background histogram, evenly over the workgroups. Each wave streams its segments through a register ring of 8
// steps of 512 tokens (16 bytes per lane and step): the step just processed is
// refilled at once with the same step of the next chunk, so a wave always has
// 8 requests in flight, also while it finishes a chunk or computes a row's
// threshold. Per token: legality from the packed bitmask, the candidate test
// against the row's threshold (legality applied to the 8 result bits of a
// lane), a cheap test for infinities and NaN (an exact look at the step only
// when one is present), the count of legal tokens, and, for rows whose top-p
// cut needs the mass below the threshold, one LDS atomic into a histogram
// with one bin per bf16 value (the workgroup's one synchronisation, per such
// chunk). Candidates go to a per-wave LDS pool in id order, one round per
// candidate of the fullest lane, and are copied out per segment.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qs_chunk.hpp"
#include "qs_device.hpp"

namespace qs {
namespace chunk {
namespace {

// Order keys of two bf16 tokens as signed 16-bit values: +magnitude for a
// positive sign, -magnitude for a negative one, so that both zeros map to 0
// and the keys compare like the values (NaN lies beyond the infinities).
__device__ __forceinline__ uint32_t skey2(uint32_t d) {
  const uint32_t s = bits_of(as_s2(d) >> 15);  // 0xFFFF in each negative half
  return bits_of(as_u2((d & 0x7FFF7FFFu) ^ s) - as_u2(s));
}
__device__ __forceinline__ int32_t skey1(uint32_t raw16) {
  const int32_t mag = (int32_t)(raw16 & 0x7FFFu);
  return (raw16 & 0x8000u) ? -mag : mag;
}
// bf16 bits of the signed key (either zero -> +0)
__device__ __forceinline__ uint32_t raw_of_skey(int32_t s) {
  return s < 0 ? 0x8000u | (uint32_t)(-s) : (uint32_t)s;
}

constexpr int32_t kInfS = 0x7F80;   // key of +inf (-inf: -kInfS)

// Standard normal quantile for q in (0, 1): Abramowitz & Stegun 26.2.23 (a
// rational approximation in sqrt(-2 ln q), absolute error below 4.5e-4).
__device__ __forceinline__ float norm_quantile(float q) {
  const float qq = q < 0.5f ? q : 1.0f - q;
  const float t = __builtin_amdgcn_sqrtf(-2.0f * __logf(qq));
  const float x = t - __fdividef(2.515517f + t * (0.802853f + t * 0.010328f),
                                 1.0f + t * (1.432788f + t * (0.189269f + t * 0.001308f)));
  return q < 0.5f ? -x : x;
}
// Standard normal distribution function: Abramowitz & Stegun 26.2.17
// (absolute error below 7.5e-8).
__device__ __forceinline__ float norm_cdf(float x) {
  const float ax = fabsf(x);
  const float k = __builtin_amdgcn_rcpf(1.0f + 0.2316419f * ax);
  const float poly =
      k * (0.319381530f +
           k * (-0.356563782f + k * (1.781477937f + k * (-1.821255978f + k * 1.330274429f))));
  const float tail = 0.3989422804f * __expf(-0.5f * ax * ax) * poly;
  return x >= 0.0f ? 1.0f - tail : tail;
}

// The sigma-truncation threshold (page "Qrita", key design 1): t0 = mu +
// delta sigma with delta the Gaussian quantile of 1 - k / V_legal (top-k),
// or for top-p the value above which a fraction p of the mass of the
// mass-weighted Gaussian N(mu + sigma^2 / T, sigma^2), truncated at the sample
// maximum, lies; then t = t0 - 0.2 |t0|, never above the sample maximum.
// Single precision, hardware reciprocal / square root / log and published
// approximations: t only decides how many tokens are compacted, never which
// are kept (every chunk of a row computes it from the same sample with the
// same instructions, so the row has one threshold). -inf: every legal finite
// token.
__device__ __forceinline__ float chunk_threshold(float n_s, float sum, float sumsq, float ms,
                                                 float frac_legal, int V, bool topk_on, int k,
                                                 bool topp_on, float p, float T) {
  const float ninf = -__builtin_inff();
  if (n_s < 32.0f) return ninf;   // too few legal finite sample tokens
  const float inv_n = __builtin_amdgcn_rcpf(n_s);
  const float mu = sum * inv_n;
  const float var = sumsq * inv_n - mu * mu;
  const float sd = var > 0.0f ? __builtin_amdgcn_sqrtf(var) : 0.0f;
  float t0;
  if (topk_on) {
    const float q = __fdividef((float)k, frac_legal * (float)V);
    if (!(q < 1.0f)) return ninf;
    t0 = mu + sd * norm_quantile(1.0f - q);
  } else if (topp_on) {
    if (!(sd > 0.0f)) return ninf;
    const float mp = mu + sd * sd / T;
    const float c = (1.0f - p) * norm_cdf(__fdividef(ms - mp, sd));
    if (!(c > 0.0f)) return ninf;
    t0 = mp + sd * norm_quantile(c);
  } else {
    return ninf;
  }
  float t = t0 - 0.2f * fabsf(t0);
  if (!(t < ms)) t = ms;
  if (!(t > -3.0e38f)) return ninf;
  return t;
}

// The largest bf16 value <= t (finite), as raw bits.
__device__ __forceinline__ uint32_t bf16_floor(float t) {
  const uint32_t b = __float_as_uint(t);
  uint32_t h = b >> 16;
  if ((b & 0x80000000u) && (b & 0xFFFFu)) h += 1u;  // negative: round away from 0
  return h;
}

// exp(x) in double precision for the background mass: range reduction by ln 2
// (a two-part constant) and the degree-11 Taylor polynomial of exp on
// |r| <= ln 2 / 2 (truncation below 2^-56 relative), as in the filter's other
// kernels. Every coefficient is set where it is used (an empty asm makes it
// opaque), so that the compiler does not hold the eleven double constants in
// registers across the whole scan loop for this rarely taken path.
__device__ __forceinline__ double kconst(double c) {
  asm volatile("" : "+s"(c));
  return c;
}
__device__ __forceinline__ double exp64_k(double x) {
  if (!(x > -745.0)) return 0.0;
  const double n = rint(x * kconst(1.4426950408889634));
  const double r =
      fma(-n, kconst(2.3190468138462996e-17), fma(-n, kconst(0.6931471805599453), x));
  double q = kconst(2.5052108385441720e-08);       // 1/11!
  q = fma(q, r, kconst(2.7557319223985893e-07));   // 1/10!
  q = fma(q, r, kconst(2.7557319223985888e-06));   // 1/9!
  q = fma(q, r, kconst(2.4801587301587302e-05));   // 1/8!
  q = fma(q, r, kconst(1.9841269841269841e-04));   // 1/7!
  q = fma(q, r, kconst(1.3888888888888889e-03));   // 1/6!
  q = fma(q, r, kconst(8.3333333333333333e-03));   // 1/5!
  q = fma(q, r, kconst(4.1666666666666667e-02));   // 1/4!
  q = fma(q, r, kconst(1.6666666666666667e-01));   // 1/3!
  q = fma(q, r, 0.5);
  q = fma(q, r, 1.0);
  q = fma(q, r, 1.0);
  return ldexp(q, (int)n);
}

// Wave64 sum of floats in a fixed combination order.
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += __uint_as_float(dpp_u32<kDppXor1>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kDppXor2>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kDppHalfMirror>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kDppMirror>(__float_as_uint(v)));
  const float a = __uint_as_float(readlane_u32(__float_as_uint(v), 0));
  const float b = __uint_as_float(readlane_u32(__float_as_uint(v), 16));
  const float c = __uint_as_float(readlane_u32(__float_as_uint(v), 32));
  const float d = __uint_as_float(readlane_u32(__float_as_uint(v), 48));
  return (a + b) + (c + d);
}

// A row's state as wave 0 computed it for its workgroup.
struct RowState {
  float T;
  uint32_t thr;     // bf16 bits of the threshold value, kThrNone or kThrAll
  int32_t tS;       // its order key
  uint32_t mode;    // 1: greedy row; 2: top-p cut without top-k (background mass needed)
};

__global__ void __launch_bounds__(kThreads, 4) scan_bf16_kernel(Args a) {
  __shared__ __align__(16) uint32_t hist[kBgBins + 64];   // + one dump bin per lane
  __shared__ __align__(16) uint32_t pool[kWaves][kSegCap];
  __shared__ __align__(16) uint4 lut[256];
  __shared__ double red_d[kWaves], red_e[kWaves];
  __shared__ RowState rst[2];   // a row's state from wave 0, by parity of the row change
  __shared__ double rh_tab[kBgExact / 128u];   // per exact binade: exp(-spacing / T)

  // this workgroup's run: chunks [b C / G, (b + 1) C / G) of the G workgroups
  const int64_t C = (int64_t)a.B * a.S;
  const int q0 = (int)((int64_t)blockIdx.x * C / gridDim.x);
  const int q1 = (int)((int64_t)(blockIdx.x + 1) * C / gridDim.x);
  if (q0 >= q1) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = uni(tid >> 6);
  const int V = a.V, S = a.S, B = a.B;
  const int W = (V + 31) >> 5;
  const int range = (int)(((uint32_t)V * 2u + 15u) & ~15u);  // bytes of a row's buffer

  // -- the requests of chunk qq: the row's sample and this wave's mask words,
  // then the segment's steps (they return in this order) ------------------------------------
  // sample: run lane / 4 of 32 tokens, 8 of them per lane
  const int run = lane >> 2, part = lane & 3;
  const int s0 = run * a.stride;
  const int se = s0 + part * 8;
  auto rsrc_of = [&](int rr) {
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.logits + (size_t)rr * a.row_bytes), (short)0, range, 0x00020000);
  };
  auto bm_of = [&](int rr) -> const uint32_t* {
    return a.bitmask ? a.bitmask + (size_t)rr * a.bm_stride : nullptr;
  };
  // (the row's T, k and p too: vector loads, in order with the rest, so that
  // no wait for them stalls the ring)
  auto issue_meta = [&](int qq, uint4& sx, uint32_t& sm, uint32_t (&mw)[2], uint32_t (&pr)[3]) {
    const int cc = qq / B, rr = qq - cc * B;
    const __amdgpu_buffer_rsrc_t rs = rsrc_of(rr);
    const uint32_t* const bm = bm_of(rr);
    sx = make_uint4(0u, 0u, 0u, 0u);
    sm = 0u;
    if (w == 0) {   // (wave 0 computes the row's threshold for the workgroup)
      pr[0] = __float_as_uint(a.T[rr]);
      pr[1] = (uint32_t)a.k[rr];
      pr[2] = __float_as_uint(a.p[rr]);
    }
    if (w == 0 && s0 < V) {
      sx = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, se * 2, 0, 0));
      sm = bm ? bm[s0 >> 5] : 0xFFFFFFFFu;
    }
    const int lo = cc * kTokens + w * kSegTokens;
    const int w0 = lo >> 5;
    const int wlim = bm ? min(W, (min(V, lo + kSegTokens) + 31) >> 5) : 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int wi = w0 + lane + 64 * i;
      mw[i] = wi < wlim ? bm[wi] : 0u;
    }
  };
  uint4 xs[kSteps];
  // where the steps of chunk qq come from: the row's buffer and this lane's
  // byte offset (the whole offset in the address register: it is the part the
  // range check covers; requests past the row read zeros)
  auto step_src = [&](int qq, __amdgpu_buffer_rsrc_t& rs, int& voff) {
    const int cc = qq / B, rr = qq - cc * B;
    rs = rsrc_of(rr);
    voff = (cc * kTokens + w * kSegTokens + lane * 8) * 2;
  };
  auto issue_step = [&](const __amdgpu_buffer_rsrc_t& rs, int voff, auto stc) {
    constexpr int st = decltype(stc)::value;
    xs[st] = __builtin_bit_cast(uint4,
                                __builtin_amdgcn_raw_buffer_load_b128(rs, voff + st * 1024, 0, 0));
  };

  uint4 sx;
  uint32_t sm, mw[2], pr[3];
  issue_meta(q0, sx, sm, mw, pr);
  {
    __amdgpu_buffer_rsrc_t rs;
    int voff;
    step_src(q0, rs, voff);
    static_for<0, kSteps>([&](auto stc) { issue_step(rs, voff, stc); });
  }

  // -- tables: pair masks of a legal byte, the cleared histogram ----------------------------
  {
    const uint32_t e = (uint32_t)tid;  // 256 entries, one per thread
    uint32_t v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[q] = (((e >> (2 * q)) & 1u) ? 0x0000FFFFu : 0u) |
             (((e >> (2 * q + 1)) & 1u) ? 0xFFFF0000u : 0u);
    lut[e] = make_uint4(v[0], v[1], v[2], v[3]);
    uint4* const h4 = reinterpret_cast<uint4*>(hist);
    for (int i = tid; i < (kBgBins + 64) / 4; i += kThreads) h4[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();

  // legal bits of step st: byte (lane & 3) of segment word 16 st + lane / 4,
  // held by lane (st & 3) * 16 + lane / 4 in mw[st / 4]
  const int bp_addr = (lane >> 2) * 4;
  const uint32_t bsh = (uint32_t)(lane & 3) * 8u;
  const uint32_t dump2 = (uint32_t)(kBgBins + lane) * 0x10001u;
  // the lumps of the background histogram: 16 bins each, spread by lane
  const uint32_t lump_lo2 = (uint32_t)(lane & 15) * 0x10001u;
  const uint32_t lump_hi2 = (kBgTop + (uint32_t)(lane & 15)) * 0x10001u;
  uint32_t* const my_pool = pool[w];

  int cur_r = -1, rpar = 0;
  float Tf = 1.0f;
  bool greedy = false, need_bg = false, any_cand = false, tpos = true;
  int32_t tS = 0;
  uint32_t thr = kThrNone;
  for (int q = q0; q < q1; ++q) {
    const int c = q / B, r = q - c * B;
    const int seg_lo = c * kTokens + w * kSegTokens;   // this wave's segment (may lie past V)
    const bool has_next = q + 1 < q1;
    // -- the row's parameters and threshold (once per row, by wave 0) ---------------------
    if (r != cur_r) {
      cur_r = r;
      if (w == 0) {
      const float T0 = __uint_as_float(uni(pr[0]));
      const int kk = (int)uni(pr[1]);
      const float pf = __uint_as_float(uni(pr[2]));
      const bool bad = !(isfinite(T0) && T0 >= 0.0f) || kk < 0 || !(pf > 0.0f && pf <= 1.0f);
      const bool gr = !bad && T0 == 0.0f;
      const bool topk_on = !bad && !gr && kk > 0 && kk < V;
      const bool topp_on = !bad && !gr && pf < 1.0f;
      thr = kThrNone;
      tS = 0;
      if (topk_on || topp_on) {
        float n = 0.0f, sum = 0.0f, sq = 0.0f;
        int32_t mx = -32768;
        uint32_t ntok = 0u;
        const uint32_t d4[4] = {sx.x, sx.y, sx.z, sx.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t raw = (d4[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
          const bool in = s0 < V && se + j < V;
          ntok += in ? 1u : 0u;
          const bool legal = in && ((sm >> (part * 8 + j)) & 1u);
          const int32_t s = skey1(raw);
          if (legal && s > -kInfS && s < kInfS) {
            const float v = __uint_as_float(raw << 16);
            n += 1.0f;
            sum += v;
            sq = fmaf(v, v, sq);
            mx = s > mx ? s : mx;
          }
        }
        n = wave_sum_f32(n);
        sum = wave_sum_f32(sum);
        sq = wave_sum_f32(sq);
        const uint32_t tn = wave_reduce<OpSum>(ntok);
        const int32_t smx = (int32_t)wave_reduce<OpMax>((uint32_t)(mx + 32768)) - 32768;
        const float ms = n >= 1.0f ? __uint_as_float(raw_of_skey(smx) << 16) : 0.0f;
        const float tval = chunk_threshold(n, sum, sq, ms,
                                           tn > 0u ? __fdividef(n, (float)tn) : 0.0f, V,
                                           topk_on, kk, topp_on, pf, T0);
        if (tval > -__builtin_inff()) {
          tS = skey1(bf16_floor(tval));
          if (tS <= -kInfS) tS = -kInfS + 1;
          thr = raw_of_skey(tS);
        } else {
          tS = -kInfS + 1;
          thr = kThrAll;
        }
      }
      if (lane == 0) {
        RowState st;
        st.T = T0;
        st.thr = thr;
        st.tS = tS;
        st.mode = (gr ? 1u : 0u) | (topp_on && !topk_on ? 2u : 0u);
        rst[rpar] = st;
      }
      }
      __syncthreads();   // the row's state
      const RowState st = rst[rpar];
      rpar ^= 1;
      Tf = uni(st.T);
      thr = uni(st.thr);
      tS = uni(st.tS);
      greedy = (uni(st.mode) & 1u) != 0u;
      need_bg = (uni(st.mode) & 2u) != 0u;
      any_cand = thr != kThrNone;
      tpos = tS > 0;
    }
    // -- the next chunk's sample and mask words, ahead of its steps -------------------------
    uint4 sx_n = make_uint4(0u, 0u, 0u, 0u);
    uint32_t sm_n = 0u, mw_n[2] = {0u, 0u}, pr_n[3] = {0u, 0u, 0u};
    // (without a next chunk the refills read past the buffer's range: zeros,
    // no memory traffic, and no register copies for a conditional load)
    __amdgpu_buffer_rsrc_t rs_n = rsrc_of(r);
    int voff_n = 0x40000000;
    if (has_next) {
      issue_meta(q + 1, sx_n, sm_n, mw_n, pr_n);
      step_src(q + 1, rs_n, voff_n);
    }

    // -- the pass over this wave's segment ----------------------------------------------------
    // The candidate test, as one signed 16-bit comparison of the raw bits:
    // for tS > 0, key >= tS iff the bits read as int16 are >= tS (negative
    // values read as negative numbers); for tS <= 0, key >= tS iff the bits
    // read as uint16 are <= 0x8000 + |tS|, i.e. (bits ^ 0x8000) as int16 <=
    // |tS|. The sign of a saturating difference gives either result.
    // (one code path for both: a uniform xor mask and result inversion; two
    // instantiations of the pass would each hold the ring in other registers)
    const uint32_t tcmp = tpos ? ((uint32_t)(tS - 1) & 0xFFFFu) * 0x10001u
                               : ((uint32_t)(-tS) & 0xFFFFu) * 0x10001u;
    const uint32_t txor = tpos ? 0u : 0x80008000u;
    const uint32_t tinv = tpos ? 0u : 0xFFu;
    const bool bmr = a.bitmask != nullptr;
    uint32_t pcnt = 0u, n_legal = 0u, nmax = 0u;
    int32_t gkey = -32768;
    uint32_t gid = 0xFFFFFFFFu;
    static_for<0, kSteps>([&](auto stc) {
        constexpr int st = decltype(stc)::value;
        uint32_t m8 = 0xFFu;
        if (bmr)
          m8 = __builtin_amdgcn_ubfe(
              (uint32_t)__builtin_amdgcn_ds_bpermute(bp_addr + (st & 3) * 64, (int)mw[st >> 2]),
              bsh, 8u);
        const int e0 = seg_lo + st * 512 + lane * 8;   // this lane's first token
        const uint32_t d4[4] = {xs[st].x, xs[st].y, xs[st].z, xs[st].w};
        if (seg_lo + (st + 1) * 512 > V) {             // a step that ends past the row
          const int rem = V - e0;
          m8 &= rem >= 8 ? 0xFFu : (rem > 0 ? (1u << rem) - 1u : 0u);
        }
        n_legal += (uint32_t)__popc(m8);
        // a negative NaN anywhere (the largest bits as uint16 exceed -inf's;
        // the up to 7 tokens past the row's end in its last 16 bytes count
        // too: a flag only sends the row to the exact paths)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          nmax = bits_of(__builtin_elementwise_max(as_u2(nmax), as_u2(d4[j])));
        // (an empty asm that reads both running values keeps their updates in
        // this step: sunk to the segment's end, they would keep every step's
        // tokens alive and the refills would need other registers and copies)
        asm volatile("" ::"v"(nmax), "v"(n_legal));
        if (greedy) {  // ids ascend along the lane: a strictly larger key moves the best
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int32_t kj = skey1((d4[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu);
            if (((m8 >> j) & 1u) && kj > gkey) {
              gkey = kj;
              gid = (uint32_t)(e0 + j);
            }
          }
        }
        if (need_bg) {
          // bin of each legal token: 16 + magnitude - 2^-12's bits, lumps
          // below and above, + kBgSide for a negative sign; illegal tokens go
          // to this lane's dump bin
          const uint4 nb4 = lut[m8];
          const uint32_t nb[4] = {nb4.x, nb4.y, nb4.z, nb4.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t bi = bits_of(__builtin_elementwise_sub_sat(
                as_u2(d4[j] & 0x7FFF7FFFu), as_u2((kBgMagLo - 16u) * 0x10001u)));
            bi = bits_of(__builtin_elementwise_max(as_u2(bi), as_u2(lump_lo2)));
            bi = bits_of(__builtin_elementwise_min(as_u2(bi), as_u2(lump_hi2)));
            const u16x2 sg = as_u2(d4[j]) >> (unsigned short)15;
            bi = bits_of(sg * as_u2(kBgSide * 0x10001u) + as_u2(bi));
            bi = bfi(nb[j], bi, dump2);
            __hip_atomic_fetch_add(hist + (bi & 0xFFFFu), 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
            __hip_atomic_fetch_add(hist + (bi >> 16), 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
          }
        }
        if (any_cand) {
          uint32_t dl[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            dl[j] = bits_of(__builtin_elementwise_sub_sat(as_s2(tcmp), as_s2(d4[j] ^ txor)));
          // sign bits of the 8 differences -> bits 0..7 (perm selectors 8..11
          // replicate the sign of a 16-bit half into a byte)
          const uint32_t cA = __builtin_amdgcn_perm(dl[1], dl[0], 0x0B0A0908u);
          const uint32_t cB = __builtin_amdgcn_perm(dl[3], dl[2], 0x0B0A0908u);
          const uint32_t sb =
              __builtin_amdgcn_sad_u8((cA & 0x08040201u) | (cB & 0x80402010u), 0u, 0u);
          const uint32_t c8 = (sb ^ tinv) & m8;
          const uint64_t anyb = ballot(c8 != 0u);
          if (anyb) {
            const uint32_t off0 = (uint32_t)(st * 512 + lane * 8);
            // the bits of token j (0..7) of this lane in the high half, low half zero
            auto entry = [&](uint32_t j) {
              const uint32_t sel =
                  (__umul24(j & 3u, 0x0202u) << 16) + 0x01000C0Cu;
              const uint32_t lo = __builtin_amdgcn_perm(d4[1], d4[0], sel);
              const uint32_t hi = __builtin_amdgcn_perm(d4[3], d4[2], sel);
              return (j < 4u ? lo : hi) + off0 + j;
            };
            if (ballot((c8 & (c8 - 1u)) != 0u) == 0u) {
              // at most one candidate a lane: its place is the count of lanes below
              const uint32_t tot = (uint32_t)__popcll(anyb);
              if (pcnt + tot <= (uint32_t)kSegCap && c8 != 0u)
                my_pool[pcnt + count_below(anyb)] = entry((uint32_t)__builtin_ctz(c8));
              pcnt += tot;
            } else {
              const uint32_t cnt = (uint32_t)__popc(c8);
              const uint32_t incl = scan_incl_u32(cnt);
              const uint32_t tot = uni(readlane_u32(incl, 63));
              if (pcnt + tot <= (uint32_t)kSegCap) {
                // one candidate of every lane per round, lowest ids first
                uint32_t* dst = my_pool + pcnt + (incl - cnt);
                uint32_t cb = c8;
                while (ballot(cb != 0u)) {
                  if (cb) {
                    const uint32_t j = (uint32_t)__builtin_ctz(cb);
                    cb &= cb - 1u;
                    *dst++ = entry(j);
                  }
                }
              }
              pcnt += tot;
            }
          }
        }
        issue_step(rs_n, voff_n, stc);                  // refill the ring
    });

    // -- this segment's summary and candidates -------------------------------------------------
    {
      const uint32_t nl = wave_reduce<OpSum>(n_legal);
      const uint32_t nmx = max(nmax & 0xFFFFu, nmax >> 16);
      const bool neg_nan = ballot(nmx > 0xFF80u) != 0u;
      int32_t gm = -32768;
      uint32_t gi = 0xFFFFFFFFu;
      if (greedy) {
        gm = (int32_t)wave_reduce<OpMax>((uint32_t)(gkey + 32768)) - 32768;
        gi = wave_reduce<OpMin>(gkey == gm ? gid : 0xFFFFFFFFu);
      }
      const bool over = pcnt > (uint32_t)kSegCap;
      const size_t seg = (size_t)(r * S + c) * kWaves + w;
      if (lane == 0) {
        SegSummary s;
        s.cand = over ? 0u : pcnt;
        s.n_legal = nl;
        s.flags = (over ? kOverflow : 0u) | (neg_nan ? kNegNaN : 0u);
        s.pad0 = 0u;
        s.gmax = gm;
        s.gid = gi;
        s.thr = thr;
        s.n_cand = pcnt;
        a.segs[seg] = s;
      }
      if (!over) {
        uint32_t* const dst = a.cands + seg * kSegCap;
        for (uint32_t i = lane; i < pcnt; i += 64) dst[i] = my_pool[i];
      }
    }

    // -- rows whose top-p cut needs it: the mass below the threshold ---------------------------
    // The histogram gathers a row's consecutive chunks of this workgroup; the
    // last of them carries their mass, the others zero.
    if (need_bg) {
      const uint32_t tmag = thr & 0x7FFFu;
      const bool tneg = (thr & 0x8000u) != 0u;
      const bool exact_t = thr != kThrAll && tmag >= kBgMagLo && tmag < kBgMagLo + kBgExact;
      ChunkMass m;
      m.m_bg = 0.0;
      m.err = 0.0;
      m.flags = exact_t ? 0u : kBgInexact;
      m.pad[0] = m.pad[1] = m.pad[2] = 0u;
      if (!(has_next && (q + 1) - (q + 1) / B * B == r)) {
        const double invT = 1.0 / (double)Tf;
        const double vt = exact_t ? (double)__uint_as_float(thr << 16) : 0.0;
        constexpr int kRuns = (int)(kBgExact / 16u);      // exact runs per side
        constexpr uint32_t kE0 = kBgMagLo >> 7;           // the first exact binade's exponent
        // the ratio exp(-d / T) of each exact binade (d its spacing, 2^(e - 134))
        if (w == 0 && lane < (int)(kBgExact / 128u))
          rh_tab[lane] = exp64_k(-ldexp(1.0, (int)(kE0 + (uint32_t)lane) - 134) * invT);
        __syncthreads();  // every wave's histogram counts; the ratios
        // runs of 16 bins, 64-byte aligned, one binade's equally spaced values
        // apiece: exact run u of a side holds magnitudes kBgMagLo + 16 u + i.
        // Threads 0 .. 255 take runs t and t + 256 of the 2 kRuns; the four
        // lumps go to the last four threads, which have one run only. Every
        // bin is read and cleared by its thread.
        double part_sum = 0.0, part_err = 0.0;
        for (int t = tid; t < 2 * kRuns; t += kThreads) {
          const bool neg = t >= kRuns;
          const int u = neg ? t - kRuns : t;
          uint4* const hv =
              reinterpret_cast<uint4*>(hist + (neg ? kBgSide : 0u) + 16u + 16u * (uint32_t)u);
          const uint32_t mg0 = kBgMagLo + 16u * (uint32_t)u;
          // background entries: values below v_t (positive values grow with
          // the magnitude, negative ones fall with it)
          int lo, hi;  // background magnitudes mg0 + lo .. mg0 + hi - 1
          if (!neg) {
            lo = 0;
            hi = tneg ? 0 : (int)min(16u, tmag > mg0 ? tmag - mg0 : 0u);
          } else {
            lo = tneg ? (int)min(16u, tmag >= mg0 ? tmag - mg0 + 1u : 0u) : 0;
            hi = 16;
          }
          // weights exp((v - v_t) / T) are geometric along the run: Horner
          // from the largest background value down (four bins a read)
          const double rh = rh_tab[(mg0 >> 7) - kE0];
          double h = 0.0;
          double vtop;
          if (!neg) {  // the largest background value is magnitude hi - 1
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const uint4 v4 = hv[i4];
              hv[i4] = make_uint4(0u, 0u, 0u, 0u);
              const uint32_t cq[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
              for (int i1 = 0; i1 < 4; ++i1)
                if (4 * i4 + i1 < hi) h = fma(h, rh, (double)cq[i1]);
            }
            vtop = (double)__uint_as_float((mg0 + (uint32_t)max(hi, 1) - 1u) << 16);
          } else {     // the largest background value is magnitude lo
#pragma unroll
            for (int i4 = 3; i4 >= 0; --i4) {
              const uint4 v4 = hv[i4];
              hv[i4] = make_uint4(0u, 0u, 0u, 0u);
              const uint32_t cq[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
              for (int i1 = 3; i1 >= 0; --i1)
                if (4 * i4 + i1 >= lo) h = fma(h, rh, (double)cq[i1]);
            }
            vtop = -(double)__uint_as_float((mg0 + (uint32_t)min(lo, 15)) << 16);
          }
          if (exact_t && h != 0.0) part_sum += exp64_k((vtop - vt) * invT) * h;
        }
        if (tid >= kThreads - 4) {
          // the lumps: magnitudes below 2^-12 (zeros among them) lie below a
          // positive v_t, weights within those of +-2^-12 (above a negative
          // v_t they are candidates, not background); magnitudes >= 512 on
          // the negative side (-inf among them) weigh at most
          // exp((-512 - v_t) / T), on the positive side they are candidates
          const int li = tid - (kThreads - 4);
          const bool neg = (li & 1) != 0, top = li >= 2;
          uint4* const hv = reinterpret_cast<uint4*>(hist + (neg ? kBgSide : 0u) +
                                                     (top ? kBgTop : 0u));
          uint32_t n = 0u;
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const uint4 v4 = hv[i4];
            n += (v4.x + v4.y) + (v4.z + v4.w);
            hv[i4] = make_uint4(0u, 0u, 0u, 0u);
          }
          if (exact_t && n != 0u) {
            if (!top && !tneg) {
              const double e = 2.44140625e-04;  // 2^-12
              part_sum += (double)n * exp64_k(-vt * invT);
              part_err += (double)n * (exp64_k((e - vt) * invT) - exp64_k((-e - vt) * invT));
            } else if (top && neg) {
              part_err += (double)n * exp64_k((-512.0 - vt) * invT);
            }
          }
        }
        const double ws = wave_sum_f64(part_sum);
        const double we = wave_sum_f64(part_err);
        if (lane == 0) {
          red_d[w] = ws;
          red_e[w] = we;
        }
        __syncthreads();  // partial sums; the cleared histogram
        if (tid == 0) {
          double tot = 0.0, err = 0.0;
          for (int i = 0; i < kWaves; ++i) {
            tot += red_d[i];
            err += red_e[i];
          }
          m.m_bg = tot;
          m.err = err;
        }
      }
      if (tid == 0) a.mass[(size_t)r * S + c] = m;
    }
    sx = sx_n;
    sm = sm_n;
    pr[0] = pr_n[0];
    pr[1] = pr_n[1];
    pr[2] = pr_n[2];
    mw[0] = mw_n[0];
    mw[1] = mw_n[1];
  }
}

int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace

hipError_t launch_scan_bf16(Args a, hipStream_t st) {
  // four resident workgroups per compute unit (every slot taken, so that each
  // unit gets the same number of chunks within one), each scanning a run of
  // consecutive chunks whose lengths differ by at most one
  const int64_t C = (int64_t)a.B * a.S;
  const int64_t slots = 4 * (int64_t)cu_count();
  const unsigned nblk = (unsigned)(C < slots ? C : slots);
  hipLaunchKernelGGL(scan_bf16_kernel, dim3(nblk), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace chunk
}  // namespace qs
