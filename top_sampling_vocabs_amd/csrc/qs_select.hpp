// Value-histogram path of the filter/sample kernel for bf16 rows held in
// registers.
//
// The kept set is the one a full stable sort by (-z, id) gives (page "Qrita",
// key design 3). Here it is found without a sort, a truncation threshold or a
// pivot search:
//  1. the slice is held in VGPRs as it arrives; every legal token is counted
//     in an LDS histogram with one bin per bf16 value of magnitude in
//     [2^-24, 512) and sign (smaller and larger magnitudes in lumps);
//  2. block-wide prefix sums over the bins, in descending value order, of the
//     counts and of the fp64 masses exp((v - m) / T) give the k-th largest
//     value with its tie quota (the page's stop test, evaluated at every value
//     at once) and then the value at which the descending mass of the top-k
//     set reaches p W_K, with the count of its ties that is needed;
//  3. one walk over the registers appends the tokens at or above that value to
//     the wave's id-ordered pool; the tie walk, the 16-wave prefix and the
//     output walk then write the mask, the id-ordered lists and the token.
// A row this path cannot settle exactly returns false and takes the general
// path: greedy rows, invalid parameters, empty rows, legal magnitudes >= 512,
// infinities or NaN, a maximum that is not a positive value of the bins, a
// boundary at or below zero or past the weight table, a top-p cut that the
// bound on the lumped small values leaves open, every token kept, and a pool
// that would overflow.
// Included by the kernels' translation unit inside namespace qs, after its
// packed 16-bit helpers.
#pragma once

#include "qs_proc.hpp"

// Per-row scalars shared through LDS by the general and the histogram paths.
struct RowInfo {
  uint32_t cnt[kWaves];
  uint32_t gt[kWaves];
  uint32_t ties[kWaves];
  double mass[kWaves];
  int32_t bsel;
  uint32_t sel_u[2];
  double sel_d[2];
  uint32_t sc_u[8];   // single-wave scan results
  double sc_d[2];
  uint64_t claim;      // (rank << 32 | ties needed) of the top-p boundary, min wins
};


template <bool SAMPLE, int NL, int P>
__device__ __forceinline__ bool select_row(const FilterArgs& a, const Slice& sl, int r, int w,
                                           int lane, int tid, int W, const uint32_t* bmrow,
                                           uint32_t* mask_row, float* dense_row,
                                           uint8_t* pool_raw, uint32_t (*stage)[kStageWords],
                                           uint4* lut, double* wtab, RedScratch& red,
                                           RowInfo& info, uint32_t* s_proc) {
  using K = Keys<1>;
  constexpr uint32_t kCap = (uint32_t)PoolLayout<1>::kPerWave;
  // entries per wave; 64 dump slots and two steps of the slice (64 lanes x 32 B) follow
  constexpr uint32_t kPool = kCap - 64u - 512u;
  constexpr int kMW = NL * (kStep / 32);
  constexpr int kML = (kMW + 63) / 64;
  int par = 0;
  // the draw's random input (the given uniform, or seed and offset of the
  // Philox draw), read now by scalar loads so that their latency hides
  // behind the pass
  uint64_t u_bits = 0u, seed_in = 0u;
  if (SAMPLE) {
    if (a.uniforms) u_bits = (uint64_t)__double_as_longlong(a.uniforms[r]);
    else { seed_in = a.seed[r]; u_bits = a.offset[r]; }
  }

  // -- requests: the slice's mask words, then every step of the slice ----------------
  const int lane_e = sl.wb + lane * kChunk;
  uint32_t mw[kML];
  {
    const uint32_t* const mwsrc = bmrow ? bmrow : reinterpret_cast<const uint32_t*>(sl.row);
    const int w0 = sl.wb >> 5;
    const int wlim = bmrow ? min(W, (sl.we + 31) >> 5) : 0;
#pragma unroll
    for (int i = 0; i < kML; ++i) {
      const int wi = w0 + lane + 64 * i;
      const bool in = lane + 64 * i < kMW && wi < wlim;
      const uint32_t v = mwsrc[in ? wi : 0];
      mw[i] = in ? v : 0u;
    }
  }
  // every step of the slice gets its own registers. The first kEarly steps are
  // requested now, the rest of the first kLook after the table barrier, and
  // step st + kLook once step st has been counted, so that the requests never
  // stall the wave for long
  constexpr int kLook = NL < 10 ? NL : 10;
  constexpr int kEarly = kLook < 4 ? kLook : 4;
  uint4 xs[NL];
  // the row through a buffer resource whose range ends at the row's last
  // 16-byte chunk: requests past it read zeros (masked as padding below), so
  // the address of a step is the lane's constant offset plus a scalar one
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(sl.row), (short)0, (int)(((uint32_t)sl.V * 2u + 15u) & ~15u),
      0x00020000);
  const int voff = lane_e * 2;
  auto issue = [&](auto stc) {
    constexpr int st = decltype(stc)::value;
    if constexpr (st < NL)
      xs[st] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rsrc, voff, st * kStep * 2, 0));
  };
  static_for<0, kEarly>(issue);
  proc::HistIds hids{};
  if constexpr (P) hids = proc::prefetch_ids(a, r, tid);

  // -- tables: legal pair masks, the cleared histogram, this slice's mask words ------
  uint32_t* const hist = reinterpret_cast<uint32_t*>(pool_raw);  // kBins + 64 dump bins
  // the pair-mask table right after the histogram, at a small LDS offset that
  // fits a load's immediate field (the pools overwrite both after the pass)
  lut = reinterpret_cast<uint4*>(pool_raw + (sel::kBins + 64) * 4);
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
  {
    uint4* const h4 = reinterpret_cast<uint4*>(hist);
    for (int i = tid; i < sel::kBins / 4; i += kThreads) h4[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  if (tid == 0) {
    info.claim = ~0ull;
    // no run holds rank k when k lies past the exact values (tiny values,
    // zeros among them, are not ranked): the k search then finds nothing and
    // the row declines
    info.sel_u[0] = sel::kNone;
  }
  // logit processors: the row's table (after the histogram and the pair-mask
  // table in the pools' LDS, its side part in the stage), built while the
  // first steps are in flight; the pass edits the tokens it flags
  proc::RowParams prm{};
  proc::Table pt{};
  if constexpr (P) {
    prm = proc::row_params<P>(a, r);
    pt = proc::table_at(pool_raw + (sel::kBins + 64) * 4 + 4096,
                        reinterpret_cast<uint8_t*>(&stage[0][0]));
    static_assert((sel::kBins + 64) * 4 + 4096 + proc::kMainBytes <= kPoolBytes,
                  "processor table");
    static_assert(proc::kSideBytes <= kWaves * kStageWords * 4, "processor side table");
    proc::build_clear(a, pt, tid, s_proc + 16);
  }
  __syncthreads();  // cleared histogram
  static_for<kEarly, kLook>(issue);
  if constexpr (P) {
    proc::build_mark(a, r, prm, pt, tid, s_proc + 16, hids);
    __syncthreads();  // marked
    if (!prm.ok || s_proc[16] != 0u) {
      if (mask_row && sl.we > sl.wb)
        for (int i = (sl.wb >> 5) + lane; i < ((sl.we + 31) >> 5); i += 64) mask_row[i] = 0u;
      if (dense_row)
        for (int i = sl.wb + lane; i < sl.we; i += 64) dense_row[i] = 0.0f;
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
      return true;
    }
    if (prm.need_cnt || prm.has_b) proc::build_ranks(a, r, prm, pt, tid, s_proc);
  }
  const bool p_any = P && (prm.has_h || prm.has_b);

  // -- the pass: count every legal token in its value bin ------------------------------
  // legal bits of step st: byte (lane & 3) of slice word 16 st + lane / 4, held
  // by lane (st & 3) * 16 + lane / 4 in mw[st / 4]
  const int bp_addr = (lane >> 2) * 4;               // byte address of lane lane / 4
  const uint32_t bsh = (uint32_t)(lane & 3) * 8u;     // this lane's byte of that word
  auto legal_word = [&](int st) -> uint32_t {
    return bmrow ? (uint32_t)__builtin_amdgcn_ds_bpermute(bp_addr + (st & 3) * 64,
                                                         (int)mw[st >> 2])
                 : 0xFFFFFFFFu;
  };
  auto legal_bits = [&](int st, uint32_t wd) -> uint32_t {
    uint32_t m8 = __builtin_amdgcn_ubfe(wd, bsh, 8u);
    if (sl.wb + (st + 1) * kStep > sl.we) {  // a step that ends past the slice
      const int rem = sl.we - (lane_e + st * kStep);
      m8 &= rem >= 8 ? 0xFFu : (rem > 0 ? (1u << rem) - 1u : 0u);
    }
    return m8;
  };
  // the legal words run two steps ahead and the pair masks one step ahead of
  // the counting, so no wait for them also waits for the step's LDS atomics
  // (LDS requests complete in order)
  uint32_t wdv[NL];
  uint32_t mbv[NL];
  uint4 nbv[NL];
  wdv[0] = legal_word(0);
  if constexpr (NL > 1) wdv[1] = legal_word(1);
  mbv[0] = legal_bits(0, wdv[0]);
  nbv[0] = lut[mbv[0]];
  // logit processors: this lane's history bits (low byte) and bias bits (next
  // byte) of a step, read one step ahead like the legal bits (bits past the
  // slice are masked by the legal bits)
  uint32_t pwv[NL];
  auto proc_bits = [&](int st) -> uint32_t {
    const int e0 = lane_e + st * kStep;  // below 16 slices of NL steps: inside the bitmaps
    const uint32_t sh = (uint32_t)e0 & 31u;
    const uint32_t hw = prm.has_h ? (pt.hbits[e0 >> 5] >> sh) & 0xFFu : 0u;
    const uint32_t bw = prm.has_b ? (pt.bbits[e0 >> 5] >> sh) & 0xFFu : 0u;
    return hw | (bw << 8);
  };
  if constexpr (P) {
    static_assert(16 * NL * kStep <= proc::kMaxV, "slices inside the processor bitmaps");
    pwv[0] = p_any ? proc_bits(0) : 0u;
  }
  uint32_t n_legal = 0u;
  // the largest legal raw bits read as signed 16-bit: positive values order
  // like their bits, negative ones lie below every positive one
  uint32_t vmax2 = 0x80008000u;
  const uint32_t dump2 = (uint32_t)(sel::kBins + lane) * 0x10001u;
  static_for<0, NL>([&](auto stc) {
    constexpr int st = decltype(stc)::value;
    if constexpr (st + 2 < NL) wdv[st + 2] = legal_word(st + 2);
    if constexpr (st + 1 < NL) {
      mbv[st + 1] = legal_bits(st + 1, wdv[st + 1]);
      nbv[st + 1] = lut[mbv[st + 1]];
      if constexpr (P) pwv[st + 1] = p_any ? proc_bits(st + 1) : 0u;
    }
    n_legal += (uint32_t)__popc(mbv[st]);
    issue(std::integral_constant<int, st + kLook>{});
    const uint4 nb4 = nbv[st];
    const uint32_t nb[4] = {nb4.x, nb4.y, nb4.z, nb4.w};
    if constexpr (P) {
      // the legal tokens the processors edit, rewritten before they are counted
      const uint32_t pw = pwv[st];
      uint32_t m = (pw | (pw >> 8)) & mbv[st];
      if (ballot(m != 0u)) {
        const uint32_t e0 = (uint32_t)(lane_e + st * kStep);
        uint32_t r4[4] = {xs[st].x, xs[st].y, xs[st].z, xs[st].w};
        while (m) {
          const uint32_t j = (uint32_t)__builtin_ctz(m);
          m &= m - 1u;
          const uint32_t sh = 16u * (j & 1u);
          uint32_t raw = 0u;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if ((uint32_t)q == (j >> 1)) raw = (r4[q] >> sh) & 0xFFFFu;
          const uint32_t nv = proc::edit_token<1>(pt, prm, e0 + j, raw, (pw >> j) & 1u,
                                                  (pw >> (8u + j)) & 1u) & 0xFFFFu;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if ((uint32_t)q == (j >> 1)) r4[q] = (r4[q] & ~(0xFFFFu << sh)) | (nv << sh);
        }
        xs[st] = make_uint4(r4[0], r4[1], r4[2], r4[3]);
      }
    }
    const uint32_t d4[4] = {xs[st].x, xs[st].y, xs[st].z, xs[st].w};
    uint32_t dm[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // illegal tokens (and the slice's padding) now read as -0: below every
      // positive boundary, so the later walks need no mask
      const uint32_t d = bfi(nb[q], d4[q], 0x80008000u);
      dm[q] = d;
      vmax2 = bits_of(__builtin_elementwise_max(as_s2(vmax2), as_s2(d)));
      __asm__ volatile("" : "+v"(vmax2));  // fold now: the operands are not held to the end
      uint32_t bi = bits_of(__builtin_elementwise_sub_sat(
          as_u2(d & 0x7FFF7FFFu), as_u2((sel::kMagLo - 16u) * 0x10001u)));
      bi = bits_of(__builtin_elementwise_min(as_u2(bi), as_u2(sel::kTop * 0x10001u)));
      {  // the sign's side: bin + sign * kSide, one packed multiply-add
        const uint32_t sg = bits_of(as_u2(d) >> 15);
        __asm__("v_pk_mad_u16 %0, %1, %2, %3" : "=v"(bi) : "v"(sg), "s"(sel::kSide * 0x10001u), "v"(bi));
      }
      bi = bfi(nb[q], bi, dump2);
      __asm__ volatile("" : "+v"(bi));  // two plain 16-bit extracts for the addresses
      __hip_atomic_fetch_add(hist + (bi & 0xFFFFu), 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_WORKGROUP);
      __hip_atomic_fetch_add(hist + (bi >> 16), 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    xs[st] = make_uint4(dm[0], dm[1], dm[2], dm[3]);
  });

  // -- parameters (only the scans below need them) -------------------------------------
  const float Tf = a.T[r];
  const int kk = a.k[r];
  const float pf = a.p[r];
  n_legal = wave_reduce<OpSum>(n_legal);
  {
    const s16x2 v = as_s2(vmax2);
    const uint32_t vm = wave_reduce<OpMax>((uint32_t)(max((int32_t)v.x, (int32_t)v.y) + 0x8000));
    if (lane == 0) { red.v[par][w][0] = n_legal; red.v[par][w][1] = vm; }
  }
  __syncthreads();  // the histogram is complete
  // invalid parameters and greedy rows: the general path (which reports them)
  if (!(isfinite(Tf) && Tf > 0.0f) || kk < 0 || !(pf > 0.0f && pf <= 1.0f)) return false;
  const double invT = 1.0 / (double)Tf;
  const double p = (double)pf;
  const bool topp_on = pf < 1.0f;
  const bool act16 = lane < kWaves;
  n_legal = uni(wave_reduce<OpSum>(act16 ? red.v[par][lane][0] : 0u));
  // the largest legal value, as raw bits (below 0x8000: positive)
  const int32_t raw_max =
      (int32_t)uni(wave_reduce<OpMax>(act16 ? red.v[par][lane][1] : 0u)) - 0x8000;
  par ^= 1;
  // a row error reported here: zero outputs, no token, no draw
  auto row_error = [&](int code) {
    if (mask_row && sl.we > sl.wb)
      for (int i = (sl.wb >> 5) + lane; i < ((sl.we + 31) >> 5); i += 64) mask_row[i] = 0u;
    if (dense_row)
      for (int i = sl.wb + lane; i < sl.we; i += 64) dense_row[i] = 0.0f;
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
  // an empty row, or a legal +inf or positive NaN (the largest legal bits)
  // (the empty check comes first)
  if (n_legal == 0u || raw_max >= 0x7F80) {
    row_error(n_legal == 0u ? QS_ROW_EMPTY : QS_ROW_NONFINITE);
    return true;
  }
  if (SAMPLE && !a.uniforms) u_bits = philox_u24(seed_in, u_bits);

  // -- runs of 16 values ----------------------------------------------------------------
  // Thread t < kRuns owns ranks 16 t .. 16 t + 15. Its counts are read from LDS
  // again in every phase (the row is still held in VGPRs).
  const bool run_t = tid < sel::kRuns;
  // counts of ranks 16 tid + 4 qd .. + 3, in rank order (one LDS read)
  auto run_quad = [&](int qd, uint32_t (&c4)[4]) {
    const uint32_t b0 = sel::run_bin0(tid);
    const bool pos = tid < (int)(sel::kExact / 16);
    const uint4 v = *reinterpret_cast<const uint4*>(hist + (pos ? b0 + 12u - 4u * (uint32_t)qd
                                                                : b0 + 4u * (uint32_t)qd));
    c4[0] = pos ? v.w : v.x; c4[1] = pos ? v.z : v.y;
    c4[2] = pos ? v.y : v.z; c4[3] = pos ? v.x : v.w;
  };
  // the maximum must be a positive exact value (below it: no positive token,
  // or only values below 2^-24; at or above 512: large values, +inf, NaN)
  if (raw_max < (int32_t)sel::kMagLo || raw_max >= (int32_t)(sel::kMagLo + sel::kExact))
    return false;
  const uint32_t rho_top = sel::kMagLo + sel::kExact - 1u - (uint32_t)raw_max;
  uint32_t ct = 0u;
  // the lumps: magnitudes below 2^-24 (zeros among them), and >= 512 with the
  // infinities and NaN (bins 0..15 and the top bin of each side)
  uint32_t tiny = 0u, huge = 0u;
  if (tid >= sel::kRuns && tid < sel::kRuns + 34) {
    const int q = tid - sel::kRuns;
    const uint32_t side = q >= 17 ? sel::kSide : 0u;
    const int j = q % 17;
    const uint32_t v = hist[side + (j < 16 ? (uint32_t)j : sel::kTop)];
    if (j < 16) tiny = v; else huge = v;
  }

  // -- fp64 masses relative to the maximum, block prefix sums in rank order -------------
  const double m = sel::rho_value(rho_top);
  // this run's 16 values are one spacing d apart, descending: their weights
  // are w0, w0 rh, ..., w0 rh^15 with w0 = exp((v0 - m) / T), rh = exp(-d / T).
  // Ranks above the maximum hold no token; the run holding the maximum starts
  // its weights there (w = 1), so no weight above 1 is ever formed (it could
  // overflow at a small T)
  auto run_w0 = [&]() {
    const uint32_t b = max(16u * (uint32_t)tid, rho_top);
    return exp64((sel::rho_value(b) - m) * invT);
  };
  auto run_rh = [&]() {
    const uint32_t mag0 = sel::rho_mag(16u * (uint32_t)tid);
    return exp64(-ldexp(1.0, (int)(mag0 >> 7) - 134) * invT);
  };
  double mt = 0.0;
  // the run's first weight and ratio, kept for the boundary searches
  double w0 = 0.0, rh = 0.0;
  if (run_t) {
    const uint32_t rho0 = 16u * (uint32_t)tid;
    w0 = run_w0();
    rh = run_rh();
    // the run's counts (four quads, read at once) and their Horner sum from
    // the last rank down
    uint32_t c4[4][4];
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) run_quad(qd, c4[qd]);
    double h = 0.0;
#pragma unroll
    for (int qd = 3; qd >= 0; --qd) {
      ct += (c4[qd][0] + c4[qd][1]) + (c4[qd][2] + c4[qd][3]);
#pragma unroll
      for (int k = 3; k >= 0; --k)
        if (rho0 + (uint32_t)(4 * qd + k) >= rho_top) h = fma(h, rh, (double)c4[qd][k]);
    }
    mt = w0 * h;
    // the weight table: every rank from the maximum down, as far as it reaches
    if (rho0 + 16u > rho_top && rho0 < rho_top + (uint32_t)sel::kTab) {
      double wi = w0;
#pragma unroll 1
      for (int i = 0; i < 16; ++i) {
        const uint32_t rho = rho0 + (uint32_t)i;
        if (rho >= rho_top) {
          if (rho < rho_top + (uint32_t)sel::kTab) wtab[rho - rho_top] = wi;
          wi *= rh;
        }
      }
    }
  }
  uint32_t c_excl, n_ex, n_tiny, n_huge;
  double m_excl, w_f;
  {
    const uint32_t ci = scan_incl_u32(ct);
    const double mi = scan_incl_f64(mt);
    const uint32_t ts = wave_reduce<OpSum>(tiny);
    const uint32_t hm = wave_reduce<OpSum>(huge);
    if (lane == 63) {
      red.v[par][w][0] = ci;
      const uint64_t b = __double_as_longlong(mi);
      red.v[par][w][1] = (uint32_t)b; red.v[par][w][2] = (uint32_t)(b >> 32);
      red.v[par][w][3] = ts; red.v[par][w][4] = hm;
    }
    __syncthreads();  // wave totals, the weight table
    // lane i holds wave i's totals: exclusive prefix over the waves
    const uint32_t tc = act16 ? red.v[par][lane][0] : 0u;
    const double tm = act16 ? __longlong_as_double(((uint64_t)red.v[par][lane][2] << 32) |
                                                   red.v[par][lane][1])
                            : 0.0;
    const uint32_t tci = scan_incl_u32(tc);
    const double tmi = scan_incl_f64(tm);
    const double tme = incl_shift1_f64(tmi);
    const int wu = uni(w);
    c_excl = readlane_u32(tci - tc, wu) + ci - ct;
    m_excl = readlane_f64(tme, wu) + (mi - mt);
    w_f = uni(readlane_f64(tmi, kWaves - 1));
    n_ex = uni(readlane_u32(tci, kWaves - 1));
    n_tiny = uni(wave_reduce<OpSum>(act16 ? red.v[par][lane][3] : 0u));
    n_huge = uni(wave_reduce<OpSum>(act16 ? red.v[par][lane][4] : 0u));
    par ^= 1;
  }
  // Legal values of magnitude >= 512 can only be negative here (the maximum is
  // below 512): -inf, finite values <= -512 and negative NaN. A negative NaN
  // is a row error; the others weigh at most exp((-512 - m) / T) each, and
  // when all of them together stay below 2^-60 of the mass they are left out
  // of every sum (as in the oracle's fp64 sums, where they change nothing
  // beyond the last place) and never kept. Otherwise the general path.
  if (n_huge) {
    uint32_t nan2 = 0u;  // largest raw bits as unsigned: negative NaNs above -inf
    static_for<0, NL>([&](auto stc) {
      constexpr int st = decltype(stc)::value;
      const uint32_t r4[4] = {xs[st].x, xs[st].y, xs[st].z, xs[st].w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        nan2 = bits_of(__builtin_elementwise_max(as_u2(nan2), as_u2(r4[q])));
    });
    const uint32_t nmax = max(nan2 & 0xFFFFu, nan2 >> 16);
    if (lane == 0) red.v[par][w][0] = 0u;
    const uint64_t bad = ballot(nmax > 0xFF80u);
    if (lane == 0 && bad) red.v[par][w][0] = 1u;
    __syncthreads();
    const bool neg_nan = uni(wave_reduce<OpMax>(act16 ? red.v[par][lane][0] : 0u)) != 0u;
    par ^= 1;
    if (neg_nan) {
      row_error(QS_ROW_NONFINITE);
      return true;
    }
    if (!((double)n_huge * exp64((-512.0 - m) * invT) <= 0x1p-60)) return false;
  }
  // the tiny values lie below every positive exact value: with a positive
  // maximum they only enter the total mass, within a bound
  if (n_ex + n_tiny + n_huge != n_legal) return false;
  const uint32_t n_fin = n_legal;
  // the tiny values' mass: n_tiny w(0), within n_tiny (w(2^-24) - w(-2^-24))
  double w_f_err = 0.0;
  if (n_tiny) {
    const double e = 5.9604644775390625e-08;  // 2^-24
    w_f += (double)n_tiny * exp64(-m * invT);
    w_f_err = (double)n_tiny * (exp64((e - m) * invT) - exp64((-e - m) * invT));
  }

  // -- top-k: the rank of the k-th largest value and its tie quota ----------------------
  const bool topk_on = kk > 0 && (uint32_t)kk < n_fin;
  uint32_t rho_k = sel::kNone, nk_k = 0u;
  double w_kap = 0.0, w_k = w_f;
  if (topk_on) {
    const uint32_t kq = (uint32_t)kk;
    if (run_t && c_excl < kq && kq <= c_excl + ct) {
      uint32_t cum = c_excl;
      double mb = m_excl, wi = w0;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        uint32_t c4[4];
        run_quad(qd, c4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t ci = c4[k];
          if (cum < kq && kq <= cum + ci) {
            info.sel_u[0] = (uint32_t)(16 * tid + 4 * qd + k);
            info.sel_u[1] = kq - cum;
            info.sel_d[0] = mb + (double)(kq - cum) * wi;
            info.sel_d[1] = wi;
          }
          if ((uint32_t)(16 * tid + 4 * qd + k) >= rho_top) {  // (no token above)
            cum += ci;
            mb += (double)ci * wi;
            wi *= rh;
          }
        }
      }
    }
    __syncthreads();
    rho_k = uni(info.sel_u[0]);
    nk_k = uni(info.sel_u[1]);
    w_k = uni(info.sel_d[0]);
    w_kap = uni(info.sel_d[1]);
    // a k-th value that is not positive needs the rank order to be the value
    // order: no tiny values between the signs
    if (rho_k >= sel::kExact && n_tiny != 0u) return false;
    w_f_err = 0.0;                           // the top-k set is exact
  }

  // -- top-p on the top-k set: the rank where the descending mass reaches p W_K ---------
  uint32_t rho_s, n_keep;
  double w_star;
  if (topp_on) {
    // the first value whose inclusive descending mass reaches the target; the
    // claim goes through an atomic minimum so that adjacent runs, whose sums
    // round differently, cannot both set it
    // with the tiny values' mass only bounded, the cut must be the same for
    // every reference mass in [w_k - err, w_k + err]
    const double target = p * (w_k + w_f_err), target_lo = p * (w_k - w_f_err);
    // runs whose sum reaches the target, with room for rounding: the running
    // sums below and the prefix sums differ by a few units in the last place
    // of the target's magnitude, far below the 1e-13 margin
    if (run_t && ct && m_excl < target && m_excl + mt >= target * (1.0 - 1e-13)) {
      double mb = m_excl, wi = w0;
      // the crossing value of this run (at most one: the sum only grows)
      uint32_t hit_rho = sel::kNone, hit_c = 0u;
      double hit_mb = 0.0, hit_w = 0.0;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        uint32_t c4[4];
        run_quad(qd, c4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t rho = (uint32_t)(16 * tid + 4 * qd + k);
          // tokens of this value inside the top-k set
          const uint32_t ci = !topk_on || rho < rho_k ? c4[k] : (rho == rho_k ? nk_k : 0u);
          if (rho >= rho_top) {  // (no token above)
            const double nb = mb + (double)ci * wi;
            if (ci && mb < target && nb >= target) {
              hit_rho = rho; hit_c = ci; hit_mb = mb; hit_w = wi;
            }
            mb = nb;
            wi *= rh;
          }
        }
      }
      if (hit_rho != sel::kNone) {
        const double need = (target - hit_mb) / hit_w;
        uint32_t nk = need <= 1.0 ? 1u : (need >= (double)hit_c ? hit_c : (uint32_t)ceil(need));
        while (nk > 1u && hit_mb + (double)(nk - 1u) * hit_w >= target) --nk;
        while (nk < hit_c && hit_mb + (double)nk * hit_w < target) ++nk;
        // the lower reference must give the same value and count; otherwise
        // claim 0 (a count of 0 never occurs in a real claim, and it wins)
        const bool same = hit_mb < target_lo && hit_mb + (double)nk * hit_w >= target_lo &&
                          (nk == 1u || hit_mb + (double)(nk - 1u) * hit_w < target_lo);
        __hip_atomic_fetch_min(&info.claim, same ? ((uint64_t)hit_rho << 32) | nk : 0ull,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
    __syncthreads();
    const uint64_t cl = info.claim;
    rho_s = uni((uint32_t)(cl >> 32));
    n_keep = uni((uint32_t)cl);
    // rounding left the target above every prefix, or the bound on the tiny
    // values' mass leaves the cut open: the general path
    if (rho_s == sel::kNone || n_keep == 0u || rho_s < rho_top) return false;
    w_star = 0.0;  // from the weight table below
  } else if (topk_on) {
    rho_s = rho_k;
    n_keep = nk_k;
    w_star = w_kap;
  } else {
    return false;  // everything kept: the general path
  }
  // A boundary that is not positive, or that lies past the weight table (2,048
  // values below the maximum): the extended mode. The weights of every rank
  // from the maximum to the boundary go to a table in the pools' LDS, every
  // wave reads its slice again for its counts and outputs (no pools), and
  // entries carry 0xFFFF - rank instead of the raw bits (ranks order like
  // the values, descending, when no tiny value lies between the signs).
  const bool ext = rho_s >= sel::kExact || rho_s >= rho_top + (uint32_t)sel::kTab;
  if (ext && n_tiny != 0u) return false;
  const uint32_t raw_star = sel::rho_mag(rho_s);        // bf16 bits of the boundary value
  uint32_t tab_base = sel::kMagLo + sel::kExact - 1u - rho_top;  // tabw[tab_base - raw]
  const double* tabw = wtab;
  if (ext) {
    double* const xt = reinterpret_cast<double*>(pool_raw);
    static_assert(sel::kRho * 8 <= kPoolBytes, "the extended weight table fits the pools");
    if (run_t) {
      const uint32_t rho0 = 16u * (uint32_t)tid;
      if (rho0 + 16u > rho_top && rho0 <= rho_s) {
        double wi = w0;
#pragma unroll 1
        for (int i = 0; i < 16; ++i) {
          const uint32_t rho = rho0 + (uint32_t)i;
          if (rho >= rho_top) {
            if (rho <= rho_s) xt[rho - rho_top] = wi;
            wi *= rh;
          }
        }
      }
    }
    __syncthreads();  // the table
    tabw = xt;
    tab_base = 0xFFFFu - rho_top;
  }
  if (topp_on) w_star = tabw[ext ? rho_s - rho_top : tab_base - raw_star];

  // -- compaction: tokens at or above the boundary, in id order, to the wave's pool ------
  // pool entry: raw bits << 16 | token offset in the slice (id order = entry order)
  uint32_t* const my_pool = reinterpret_cast<uint32_t*>(pool_raw) + w * kCap;
  // this slice's keep bits, one byte per lane and step: the layout of the mask
  // words (byte lane & 3 of slice word 16 st + lane / 4)
  uint8_t* const keep_bytes = reinterpret_cast<uint8_t*>(stage[w]) + lane;
  // (the pools overwrite the histogram: its last reads, in the searches above,
  // all precede the search barriers)
  uint32_t pcnt = 0u;
  const uint32_t t2m1 = ((raw_star - 1u) & 0xFFFFu) * 0x10001u;
  uint32_t* const dump = my_pool + kPool + lane;
  // this lane's chunks of the current two steps, staged in LDS so that a
  // round reads its token's bits by index (0..15 over both chunks)
  uint4* const my_chunks = reinterpret_cast<uint4*>(my_pool + kPool + 64u) + 2 * lane;
  const uint16_t* const chunk_bits = reinterpret_cast<const uint16_t*>(my_chunks);
  auto keep_bits = [&](const uint4& x) -> uint32_t {
    const uint32_t r4[4] = {x.x, x.y, x.z, x.w};
    uint32_t dl[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // positive raw bits order like their values, negative ones (illegal
      // tokens among them) lie below every positive one
      dl[q] = bits_of(__builtin_elementwise_sub_sat(as_s2(t2m1), as_s2(r4[q])));  // <0 iff kept
    }
    const uint32_t cA = __builtin_amdgcn_perm(dl[1], dl[0], 0x0B0A0908u);
    const uint32_t cB = __builtin_amdgcn_perm(dl[3], dl[2], 0x0B0A0908u);
    return __builtin_amdgcn_sad_u8(cB & 0x80402010u, 0u,
                                   __builtin_amdgcn_sad_u8(cA & 0x08040201u, 0u, 0u));
  };
  // two steps per group: one prefix sum and one set of rounds for both, so
  // the rounds follow the fuller lane of the pair rather than of each step
  if (!ext) static_for<0, (NL + 1) / 2>([&](auto gc) {
    constexpr int s0 = 2 * decltype(gc)::value;
    constexpr bool two = s0 + 1 < NL;
    const uint32_t cb0 = keep_bits(xs[s0]);
    keep_bytes[s0 * 64] = (uint8_t)cb0;
    uint32_t cb1 = 0u;
    if constexpr (two) {
      cb1 = keep_bits(xs[s0 + 1]);
      keep_bytes[(s0 + 1) * 64] = (uint8_t)cb1;
    }
    const uint32_t c0 = (uint32_t)__popc(cb0), c1 = (uint32_t)__popc(cb1);
    if (ballot((cb0 | cb1) != 0u)) {
      // both counts in one prefix sum (16-bit fields: each total is at most 512)
      const uint32_t cc = c0 | (c1 << 16);
      const uint32_t incl = scan_incl_u32(cc);
      const uint32_t excl = incl - cc;
      const uint32_t tot = readlane_u32(incl, 63);
      const uint32_t t0 = tot & 0xFFFFu, t1 = tot >> 16;
      // a pool that would overflow is not written (the row then declines)
      if (pcnt + t0 + t1 <= kPool) {
        if (c0) my_chunks[0] = xs[s0];
        if constexpr (two) {
          if (c1) my_chunks[1] = xs[s0 + 1];
        }
        // round r writes the lane's r-th token: of step s0 at base0 + r while
        // r < c0, of step s0 + 1 at base1 + (r - c0) after
        uint32_t* slot = my_pool + pcnt + (excl & 0xFFFFu);
        const int32_t jump = (int32_t)(t0 + (excl >> 16)) - (int32_t)((excl & 0xFFFFu) + c0);
        const uint32_t e0 = (uint32_t)(lane_e + s0 * kStep - sl.wb);
        uint32_t cb = cb0 | (cb1 << 8);
        // every lane writes each round, lanes without a token left to a slot
        // of their own past the pool, so the rounds need no branches (a lane
        // stays idle once it has run out, so its own slot may move on)
        for (;;) {
          const bool on = cb != 0u;
          if (!ballot(on)) break;
          // lowest set bit (all ones for an idle lane: its reads land in the
          // LDS next to its chunks and its entry goes to its dump slot)
          uint32_t j;
          __asm__("v_ffbl_b32 %0, %1" : "=v"(j) : "v"(cb));
          cb &= cb - 1u;
          const uint32_t key = chunk_bits[j];
          // all ones for a token of the second step, else zero
          const int32_t hm = __builtin_amdgcn_sbfe((int32_t)j, 3, 1);
          const uint32_t off = e0 + j + ((uint32_t)hm & (uint32_t)(kStep - 8));
          *(on ? slot + (hm & jump) : dump) = (key << 16) | off;
          ++slot;
        }
      }
      pcnt = uni(pcnt + t0 + t1);
    }
  });
  // per wave: tokens above the boundary and their mass, ties at it (every
  // entry is at or above the boundary value, which is positive)
  const int my_cnt = (int)min(pcnt, kPool);
  // entries above the boundary compare greater
  const uint32_t e_gt = ext ? ((0xFFFFu - rho_s) << 16) | 0xFFFFu : (raw_star << 16) | 0xFFFFu;
  uint32_t gt = 0u, ties = 0u;
  double mgt = 0.0;
  // KP consecutive entries per lane and round: one for short pools, four for
  // long ones (reads past my_cnt stay in this wave's pool region and are not
  // counted)
  auto load_entries = [&](auto kpc, int ib, uint32_t (&e)[4]) {
    constexpr int KP = decltype(kpc)::value;
    if constexpr (KP == 4) {
      const uint4 e4 = *reinterpret_cast<const uint4*>(my_pool + ib);
      e[0] = e4.x; e[1] = e4.y; e[2] = e4.z; e[3] = e4.w;
    } else {
      e[0] = my_pool[ib];
    }
  };
  const bool long_pool = uni(my_cnt) > 192;
  // A wave whose tokens at or above the boundary overflow its pool reads its
  // slice again instead (all steps requested at once, the legal bits from the
  // bitmask) and walks it: f(e, bits) per step with this lane's 8 tokens as
  // pool entries and the bits of those at or above the boundary
  const bool direct = ext || uni(pcnt) > kPool;
  // With logit processors the caller's row holds the unedited values: such a
  // wave first stores its edited registers (its own slice only; slices start
  // at multiples of a step) to the row's workspace copy and reads that instead
  const uint8_t* dsrc = sl.row;
  if (P && direct) {
    uint8_t* const cp = a.p_copy + (size_t)r * a.p_copy_bytes;
    static_for<0, NL>([&](auto stc) {
      constexpr int st = decltype(stc)::value;
      const int c = lane_e + st * kStep;
      if (c < sl.we) *reinterpret_cast<uint4*>(cp + 2 * (size_t)c) = xs[st];
    });
    dsrc = cp;
  }
  const __amdgpu_buffer_rsrc_t rsrc_d = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(dsrc), (short)0, (int)(((uint32_t)sl.V * 2u + 15u) & ~15u),
      0x00020000);
  // (write_keep: also store each step's keep byte in the mask staging, which
  // the compaction did not fill in the extended mode)
  uint32_t ext_cnt = 0u;
  auto direct_walk = [&](auto&& f, bool write_keep) __attribute__((always_inline)) {
    // steps in groups of 4: the group's requests go out together
    constexpr int kG = 4;
    static_for<0, (NL + kG - 1) / kG>([&](auto gc) {
      constexpr int g0 = decltype(gc)::value * kG;
      uint4 x[kG];
      uint32_t lbs[kG];
#pragma unroll
      for (int i = 0; i < kG; ++i) {
        const int st = g0 + i;
        const int e0 = lane_e + st * kStep;
        if (st < NL) {
          x[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                               rsrc_d, voff, st * kStep * 2, 0));
          uint32_t lb = 0u;
          if (e0 < sl.we) {
            lb = bmrow ? (bmrow[e0 >> 5] >> (e0 & 31)) & 0xFFu : 0xFFu;
            if (e0 + kChunk > sl.we) lb &= (1u << (sl.we - e0)) - 1u;
          }
          lbs[i] = lb;
        }
      }
#pragma unroll
      for (int i = 0; i < kG; ++i) {
        const int st = g0 + i;
        if (st < NL) {
          const uint32_t lb = lbs[i];
          uint32_t r4[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
          const uint32_t o0 = (uint32_t)(lane_e + st * kStep - sl.wb);
          uint32_t e[8];
          uint32_t cb = 0u;
          if (ext) {
            // rank of every exact value (tiny ones are absent, huge ones were
            // declined); legal tokens ranked at or above the boundary are kept
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
              const uint32_t raw = (r4[jj >> 1] >> (16 * (jj & 1))) & 0xFFFFu;
              const uint32_t mag = raw & 0x7FFFu;
              const uint32_t rk = (raw >> 15) ? sel::kExact + (mag - sel::kMagLo)
                                              : sel::kMagLo + sel::kExact - 1u - mag;
              const bool ok = ((lb >> jj) & 1u) && mag >= sel::kMagLo &&
                              mag < sel::kMagLo + sel::kExact && rk <= rho_s;
              cb |= (ok ? 1u : 0u) << jj;
              e[jj] = ((0xFFFFu - (rk & 0xFFFFu)) << 16) | (o0 + (uint32_t)jj);
            }
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t pm = (((lb >> (2 * q)) & 1u) ? 0x0000FFFFu : 0u) |
                                  (((lb >> (2 * q + 1)) & 1u) ? 0xFFFF0000u : 0u);
              r4[q] = bfi(pm, r4[q], 0x80008000u);  // illegal -> -0, below the boundary
            }
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
              e[jj] = (((r4[jj >> 1] >> (16 * (jj & 1))) & 0xFFFFu) << 16) | (o0 + (uint32_t)jj);
            cb = keep_bits(make_uint4(r4[0], r4[1], r4[2], r4[3]));
          }
          if (write_keep) {
            keep_bytes[st * 64] = (uint8_t)cb;
            ext_cnt += (uint32_t)__popc(cb);
          }
          if (ballot(cb != 0u)) f(e, cb);
        }
      }
    });
  };
  auto classify = [&](uint32_t e) __attribute__((always_inline)) {
    if (e > e_gt) {
      ++gt;
      mgt += tabw[tab_base - (e >> 16)];
    } else {
      ++ties;
    }
  };
  auto walk_a = [&](auto kpc) {
    constexpr int KP = decltype(kpc)::value;
    for (int i0 = 0; i0 < my_cnt; i0 += 64 * KP) {
      const int ib = i0 + KP * lane;
      uint32_t e[4];
      load_entries(kpc, ib, e);
#pragma unroll
      for (int k = 0; k < KP; ++k)
        if (ib + k < my_cnt) classify(e[k]);
    }
  };
  if (direct) {
    direct_walk([&](const uint32_t (&e)[8], uint32_t cb) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if ((cb >> k) & 1u) classify(e[k]);
    }, true);
    if (ext) pcnt = uni(wave_reduce<OpSum>(ext_cnt));
  } else if (long_pool) {
    walk_a(std::integral_constant<int, 4>{});
  } else {
    walk_a(std::integral_constant<int, 1>{});
  }
  gt = wave_reduce<OpSum>(gt);
  ties = wave_reduce<OpSum>(ties);
  mgt = wave_sum_f64(mgt);
  if (lane == 0) {
    info.cnt[w] = pcnt;
    info.gt[w] = gt;
    info.ties[w] = ties;
    info.mass[w] = mgt;
  }
  __syncthreads();

  // -- tie quota per wave, list offsets, masses, the sampled wave -----------------------
  double u = 0.0;
  if (SAMPLE) {
    if (a.uniforms) u = __longlong_as_double((long long)u_bits);
    else u = (double)(uint32_t)u_bits * (1.0 / 16777216.0);
  }
  u = uni(u);
  uint32_t my_off, n_p, my_kt, n_z = 0u;
  double w_p, my_cumw;
  int sw, last_w;
  {
    const uint32_t t = act16 ? info.ties[lane] : 0u;
    const uint32_t g = act16 ? info.gt[lane] : 0u;
    const double mg = act16 ? info.mass[lane] : 0.0;
    n_z = uni(wave_reduce<OpSum>(act16 ? info.cnt[lane] : 0u));
    const uint32_t tb = scan_incl_u32(t) - t;
    const uint32_t avail = n_keep > tb ? n_keep - tb : 0u;
    const uint32_t kt = t < avail ? t : avail;
    const uint32_t kept = g + kt;
    const double mw = mg + (double)kt * w_star;
    const uint32_t kincl = scan_incl_u32(kept);
    const double mincl = scan_incl_f64(mw);
    const double mex = incl_shift1_f64(mincl);
    const int wu = uni(w);
    my_off = readlane_u32(kincl - kept, wu);
    my_kt = readlane_u32(kt, wu);
    my_cumw = readlane_f64(mex, wu);
    n_p = readlane_u32(kincl, kWaves - 1);
    w_p = readlane_f64(mincl, kWaves - 1);
    const uint64_t pos = ballot(act16 && kept > 0u && mw > 0.0);
    last_w = pos ? 63 - __clzll((long long)pos) : -1;
    sw = -1;
    if (SAMPLE) {
      const uint64_t hit = ballot(act16 && kept > 0u && u < mincl * (1.0 / w_p));
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
  const double inv_wp = 1.0 / w_p;

  // -- outputs --------------------------------------------------------------------------
  // the output rows and the list capacity are held in VGPRs for the walk
  // below (scalar registers are scarce there)
  auto to_vgpr = [](uint32_t x) {
    uint32_t v;
    __asm__("v_mov_b32 %0, %1" : "=v"(v) : "s"(x));
    return v;
  };
  auto ptr_vgpr = [&](auto* ptr) {
    const uint64_t b = (uint64_t)(uintptr_t)ptr;
    return reinterpret_cast<decltype(ptr)>(
        (uintptr_t)(((uint64_t)to_vgpr((uint32_t)(b >> 32)) << 32) | to_vgpr((uint32_t)b)));
  };
  // (global address space: the stores stay global, not flat, instructions)
  using gi32 = __attribute__((address_space(1))) int32_t;
  using gf32 = __attribute__((address_space(1))) float;
  gi32* const ids_row =
      a.cand_ids ? (gi32*)ptr_vgpr(a.cand_ids + (size_t)r * a.cand_cap) : nullptr;
  gf32* const probs_row =
      a.cand_probs ? (gf32*)ptr_vgpr(a.cand_probs + (size_t)r * a.cand_cap) : nullptr;
  const uint32_t cap = to_vgpr((uint32_t)a.cand_cap);
  // this slice's mask words, gathered in LDS (a resident slice always fits)
  const int sw0 = sl.wb >> 5, sw1 = sl.we > sl.wb ? (sl.we + 31) >> 5 : sw0;
  uint32_t* const my_stage = stage[w];  // the keep bits, written by the compaction
  if (dense_row) {  // zero in memory first (the scatter below lands after these stores)
    for (int i = sl.wb + lane; i < sl.we; i += 64) dense_row[i] = 0.0f;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
  }
  // walk D: 64 KP consecutive entries per round, KP per lane, so that the
  // kept ones of a lane take consecutive list positions and the prefix sums
  // of a round serve KP entries
  uint32_t pos_base = my_off;
  uint32_t ties_seen = 0u;
  double cbase = my_cumw * inv_wp;
  int my_token = -1;
  double my_q = 0.0;
  // this lane's last kept entry with q > 0; entries never equal ~0u (their
  // offset field stays below the slice length)
  uint32_t last_e = ~0u;
  // KP entries per lane (consecutive ids), vbits marking the valid ones
  auto emit = [&](auto kpc, const auto& e, uint32_t vbits) __attribute__((always_inline)) {
    constexpr int KP = decltype(kpc)::value;
    uint32_t kb = 0u, tb = 0u;  // kept (above the boundary) and tie bits of the KP
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const bool valid = (vbits >> k) & 1u;
      kb |= (valid && e[k] > e_gt ? 1u : 0u) << k;
      tb |= (valid && e[k] <= e_gt ? 1u : 0u) << k;
    }
    const uint32_t tc = (uint32_t)__popc(tb);
    if (ballot(tc != 0u)) {
      // ties in id order: the first my_kt of this wave are kept; the bits of
      // the others are cleared from the keep mask
      const uint32_t tincl = KP == 1 ? count_below(ballot(tc != 0u)) + tc : scan_incl_u32(tc);
      uint32_t trank = ties_seen + tincl - tc;
#pragma unroll
      for (int k = 0; k < KP; ++k) {
        if ((tb >> k) & 1u) {
          if (trank < my_kt) kb |= 1u << k;
          else if (mask_row)
            __hip_atomic_fetch_and(my_stage + ((e[k] & 0xFFFFu) >> 5), ~(1u << (e[k] & 31u)),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          ++trank;
        }
      }
      ties_seen += KP == 1 ? (uint32_t)__popcll(ballot(tc != 0u)) : readlane_u32(tincl, 63);
    }
    const uint32_t kc = (uint32_t)__popc(kb);
    const uint32_t kincl = KP == 1 ? count_below(ballot(kc != 0u)) + kc : scan_incl_u32(kc);
    uint32_t pos = pos_base + kincl - kc;
    double qv[KP];
    double lane_sum = 0.0;
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      qv[k] = 0.0;
      if ((kb >> k) & 1u) {
        const int id = (int)(sl.wb + (e[k] & 0xFFFFu));
        const double q = tabw[tab_base - (e[k] >> 16)] * inv_wp;
        qv[k] = q;
        lane_sum += q;
        const float qf = (float)q;
        // (streaming stores: the outputs go straight on to memory instead of
        // waiting in L2 for the end of the kernel)
        if (pos < cap) {
          if (ids_row) __builtin_nontemporal_store(id, ids_row + pos);
          if (probs_row) __builtin_nontemporal_store(qf, probs_row + pos);
        }
        if (dense_row) dense_row[id] = qf;
        if (q > 0.0) last_e = e[k];
        ++pos;
      }
    }
    pos_base += KP == 1 ? (uint32_t)__popcll(ballot(kc != 0u)) : readlane_u32(kincl, 63);
    if (SAMPLE && w == sw && my_token < 0) {
      const double incl = scan_incl_f64(lane_sum);
      double cu = cbase + (incl - lane_sum);
      int hit = -1;
      double hq = 0.0;
#pragma unroll
      for (int k = 0; k < KP; ++k) {
        cu += qv[k];
        if (hit < 0 && ((kb >> k) & 1u) && u < cu) {
          hit = (int)(sl.wb + (e[k] & 0xFFFFu));
          hq = qv[k];
        }
      }
      const uint64_t hbits = ballot(hit >= 0);
      if (hbits) {
        const int fl = __ffsll((unsigned long long)hbits) - 1;
        my_token = __shfl(hit, fl, 64);
        my_q = readlane_f64(hq, fl);
      }
      cbase += readlane_f64(incl, 63);
    }
  };
  auto walk_d = [&](auto kpc) {
    constexpr int KP = decltype(kpc)::value;
    for (int i0 = 0; i0 < my_cnt; i0 += 64 * KP) {
      const int ib = i0 + KP * lane;
      uint32_t e[4];
      load_entries(kpc, ib, e);
      uint32_t vb = 0u;
#pragma unroll
      for (int k = 0; k < KP; ++k) vb |= (ib + k < my_cnt ? 1u : 0u) << k;
      emit(kpc, e, vb);
    }
  };
  if (direct) {
    direct_walk([&](const uint32_t (&e)[8], uint32_t cb) {
      emit(std::integral_constant<int, 8>{}, e, cb);
    }, false);
  } else if (long_pool) {
    walk_d(std::integral_constant<int, 4>{});
  } else {
    walk_d(std::integral_constant<int, 1>{});
  }
  if (mask_row) {
    for (int i = lane; i < sw1 - sw0; i += 64)
      __builtin_nontemporal_store(my_stage[i], mask_row + sw0 + i);
  }
  // the token: from wave sw; if rounding left u at or above wave sw's last
  // cumulative sum, that wave's last kept id with q > 0; if u lies past every
  // wave, the last kept id with q > 0 of the row
  const int last_pos_id = last_e == ~0u ? -1 : (int)(sl.wb + (last_e & 0xFFFFu));
  const int last_id = (int)wave_reduce<OpMax>((uint32_t)(last_pos_id + 1)) - 1;
  if (SAMPLE) {
    double last_q = 0.0;
    if (a.logprobs) {
      const double last_pos_q = last_e == ~0u ? 0.0 : tabw[tab_base - (last_e >> 16)] * inv_wp;
      last_q = last_token_q(last_pos_id, last_pos_q, last_id);
    }
    if (lane == 0) {
      if (w == sw) {
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
    if (SAMPLE && !a.uniforms) a.offset[r] = a.offset[r] + 1u;
    if (a.dbg) {
      a.dbg[4 * r + 0] = 0;
      a.dbg[4 * r + 1] = 0;
      a.dbg[4 * r + 2] = (int32_t)n_z;
      a.dbg[4 * r + 3] = (int32_t)n_p;
    }
  }
  return true;
}
