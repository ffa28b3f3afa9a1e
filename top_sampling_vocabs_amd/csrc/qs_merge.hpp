// Per-row merge of the chunked first pass (bf16 rows): the second half of
// the filter for rows whose chunks were scanned by the chunk kernel.
//
// The chunk workgroups of a row left, in the caller's workspace, a summary per
// chunk and the chunk's candidates (legal tokens at or above the row's
// sigma-truncation threshold t, in id order). One workgroup per row then:
//  1. combines the summaries: legal count, extreme keys (row statuses), the
//     greedy token, and the exact mass of the legal tokens below t;
//  2. loads the candidates into LDS in id order (a wave per segment, the
//     segment's place in the list from a scan of the counts) and counts them
//     in a histogram with one bin per bf16 value above t;
//  3. block prefix sums of counts and fp64 masses exp((v - m) / T) over the
//     bins in descending value give the k-th largest value with its tie
//     quota (the page's stop test, evaluated at every value at once) and the
//     value at which the descending mass of the top-k set reaches p W_K, with
//     the count of its ties that is needed (page "Qrita", key designs 2-3);
//  4. per-wave counts over the id-ordered candidates, a 16-wave prefix of the
//     tie quota (earliest ids first), list offsets and masses, and the output
//     walk: packed mask, id-ordered lists, dense probabilities, and the draw
//     by inverse CDF in id order.
// A row this path cannot settle returns false and takes the kernel's other
// paths, which read the row itself: a threshold above the k-th value or the
// top-p cut (a truncation miss, page "Qrita" key design 1: Z_s = Z), more
// candidates than the LDS holds, values spanning more than the histogram,
// a background mass that is not exact, and rows that keep every token.
// Included by the kernels' translation unit inside namespace qs, after the
// value-histogram path.
#pragma once

namespace mrg {
constexpr int kWin = kHistBins;                     // value bins above the threshold
constexpr uint32_t kPoolMax = kPoolBytes / 4;       // candidates held in LDS
constexpr int kIdBits = 20;                         // pool entry: bin << 20 | token id
constexpr uint32_t kIdMask = (1u << kIdBits) - 1u;
constexpr int kMaskWords = kWaves * kStageWords;    // keep-mask words staged in LDS
constexpr int32_t kInfS = 0x7F80;                   // order key of +inf

__device__ __forceinline__ int32_t skey1(uint32_t raw16) {
  const int32_t mag = (int32_t)(raw16 & 0x7FFFu);
  return (raw16 & 0x8000u) ? -mag : mag;
}
__device__ __forceinline__ double skey_value(int32_t s) {
  const uint32_t raw = s < 0 ? 0x8000u | (uint32_t)(-s) : (uint32_t)s;
  return (double)__uint_as_float(raw << 16);
}
}  // namespace mrg

template <bool SAMPLE>
__device__ __forceinline__ bool merge_row(const FilterArgs& a, int r, int tid, int w, int lane,
                                          uint8_t* pool_raw, uint32_t* mstage, uint32_t* hist,
                                          double* binw, RedScratch& red, RowInfo& info) {
  using chunk::SegSummary;
  const int S = a.S;                     // chunks of the row
  const int NS = S * chunk::kWaves;      // segments of the row
  const int V = a.V;
  const int W = (V + 31) >> 5;
  const bool act16 = lane < kWaves;

  // -- 1. one round trip: wave 0 reads the segments' summaries, the row's
  // parameters and its chunks' background masses; every wave reads the first
  // 64 candidates of up to kSpec of its segments (checked against the counts
  // after the barrier). The histogram and the staged mask words are cleared
  // meanwhile.
  // red.v[0][0][*]: row scalars; red.v[1]: the segments' candidate list bases
  uint32_t* const row_u = red.v[0][0];
  uint32_t* const base_s = &red.v[1][0][0];   // [NS + 1] list bases of the segments
  uint32_t* const pool = reinterpret_cast<uint32_t*>(pool_raw);
  const uint32_t* const crow = a.ws_cands + (size_t)r * NS * chunk::kSegCap;
  constexpr int kSpec = 4;
  uint32_t spec[kSpec];
#pragma unroll
  for (int i = 0; i < kSpec; ++i) {
    const int sg = w + kWaves * i;
    spec[i] = sg < NS ? crow[(size_t)sg * chunk::kSegCap + lane] : 0u;
  }
  if (w == 0) {
    // (buffer loads: issued here with the summaries, not deferred to the use)
    auto ld32 = [&](const void* base, int idx) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<void*>(base), (short)0, 0x7FFFFFF0, 0x00020000);
      return __builtin_amdgcn_raw_buffer_load_b32(rs, idx * 4, 0, 0);
    };
    const uint32_t pT = ld32(a.T, r), pk = ld32(a.k, r), pp = ld32(a.p, r);
    uint32_t pu0 = 0u, pu1 = 0u, ps0 = 0u, ps1 = 0u;
    if (SAMPLE) {
      if (a.uniforms) {
        pu0 = ld32(a.uniforms, 2 * r);
        pu1 = ld32(a.uniforms, 2 * r + 1);
      } else {
        pu0 = ld32(a.offset, 2 * r);
        pu1 = ld32(a.offset, 2 * r + 1);
        ps0 = ld32(a.seed, 2 * r);
        ps1 = ld32(a.seed, 2 * r + 1);
      }
    }
    double mb = 0.0, me = 0.0;
    uint32_t bad_m = 0u;
    if (lane < S) {
      const chunk::ChunkMass cm = a.ws_mass[(size_t)r * S + lane];
      mb = cm.m_bg;
      me = cm.err;
      bad_m = cm.flags;
    }
    uint32_t n_legal = 0u, fl = 0u, thr_hi = 0u, thr_lo = 0xFFFFFFFFu;
    uint32_t gmax = 0u, gid = 0xFFFFFFFFu;
    uint32_t cc[4];
    // consecutive segments per lane (id order), all eight loads in flight at
    // once (range-checked: past the row's summaries they read zeros, unused)
    uint4 sv[4][2];
    {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<SegSummary*>(a.ws_segs + (size_t)r * NS), (short)0,
          NS * (int)sizeof(SegSummary), 0x00020000);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          sv[i][h] = __builtin_bit_cast(
              uint4, __builtin_amdgcn_raw_buffer_load_b128(
                         rs, (lane * 4 + i) * (int)sizeof(SegSummary) + 16 * h, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sg = lane * 4 + i;
      cc[i] = 0u;
      if (sg < NS) {
        SegSummary s;
        s.cand = sv[i][0].x;
        s.n_legal = sv[i][0].y;
        s.flags = sv[i][0].z;
        s.gmax = (int32_t)sv[i][1].x;
        s.gid = sv[i][1].y;
        s.thr = sv[i][1].z;
        cc[i] = s.cand;
        n_legal += s.n_legal;
        fl |= s.flags;
        thr_hi = max(thr_hi, s.thr);
        thr_lo = min(thr_lo, s.thr);
        const uint32_t gk = (uint32_t)(s.gmax + 32768);
        if (gk > gmax) { gmax = gk; gid = s.gid; }   // the first segment holding the maximum
      }
    }
    const uint32_t c4 = cc[0] + cc[1] + cc[2] + cc[3];
    const uint32_t incl = scan_incl_u32(c4);
    uint32_t b = incl - c4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (lane * 4 + i < NS) base_s[lane * 4 + i] = b;
      b += cc[i];
    }
    const uint32_t tot = readlane_u32(incl, 63);
    const uint32_t gm = wave_reduce<OpMax>(gmax);
    const uint32_t gi = wave_reduce<OpMin>(gmax == gm ? gid : 0xFFFFFFFFu);
    n_legal = wave_reduce<OpSum>(n_legal);
    fl = wave_reduce<OpMax>(fl & chunk::kOverflow) | wave_reduce<OpMax>(fl & chunk::kNegNaN);
    thr_hi = wave_reduce<OpMax>(thr_hi);
    thr_lo = wave_reduce<OpMin>(thr_lo);
    mb = wave_sum_f64(mb);
    me = wave_sum_f64(me);
    bad_m = wave_reduce<OpMax>(bad_m);
    if (lane == 0) {
      base_s[NS] = tot;
      row_u[0] = n_legal;
      row_u[1] = gm;
      row_u[2] = fl | (thr_hi != thr_lo ? chunk::kOverflow : 0u);  // (never: one threshold a row)
      row_u[3] = gi;
      row_u[4] = thr_hi;
      row_u[5] = tot;
      row_u[6] = pT;
      row_u[7] = pk;
      row_u[8] = pp;
      row_u[9] = pu0;
      row_u[10] = pu1;
      row_u[11] = ps0;
      row_u[12] = ps1;
      info.sc_d[0] = mb;
      info.sc_d[1] = me;
      info.sc_u[0] = bad_m;
      info.sc_u[1] = 0u;   // the largest candidate bin (+1)
    }
  }
  for (int i = tid; i < mrg::kWin; i += kThreads) hist[i] = 0u;
  if (a.keep_mask && W <= mrg::kMaskWords)
    for (int i = tid; i < W; i += kThreads) mstage[i] = 0u;
  __syncthreads();
  const float Tf = __uint_as_float(uni(row_u[6]));
  const int kk = (int)uni(row_u[7]);
  const float pf = __uint_as_float(uni(row_u[8]));
  uint64_t u_bits = 0u, seed_in = 0u;
  if (SAMPLE) {
    u_bits = ((uint64_t)uni(row_u[10]) << 32) | uni(row_u[9]);
    seed_in = ((uint64_t)uni(row_u[12]) << 32) | uni(row_u[11]);
  }
  const uint32_t n_legal = uni(row_u[0]);
  const int32_t gmax = (int32_t)uni(row_u[1]) - 32768;   // greedy rows: the largest key
  const uint32_t flags = uni(row_u[2]);
  const uint32_t argmax = uni(row_u[3]);
  const uint32_t thr = uni(row_u[4]);
  const uint32_t N = uni(row_u[5]);

  uint32_t* const mask_row = a.keep_mask ? a.keep_mask + (size_t)r * W : nullptr;
  float* const dense_row = a.dense ? a.dense + (size_t)r * V : nullptr;
  int32_t* const ids_out = a.cand_ids ? a.cand_ids + (size_t)r * a.cand_cap : nullptr;
  float* const probs_out = a.cand_probs ? a.cand_probs + (size_t)r * a.cand_cap : nullptr;

  // -- 2. row statuses and greedy rows (settled from the summaries alone) -----------------
  // A negative NaN (flagged by the chunks, legal or not) leaves the row to the
  // other paths. Otherwise a legal +inf or positive NaN is a candidate of any
  // threshold (checked in step 3) or the greedy maximum, and the legal tokens
  // are all -inf when no finite one passes the keep-all threshold.
  const bool bad = !(isfinite(Tf) && Tf >= 0.0f) || kk < 0 || !(pf > 0.0f && pf <= 1.0f);
  const bool greedy_row = !bad && Tf == 0.0f;
  if (!bad && n_legal != 0u && (flags & chunk::kNegNaN)) return false;
  int code = QS_ROW_OK;
  if (bad) code = QS_ROW_BAD_PARAM;
  else if (n_legal == 0u) code = QS_ROW_EMPTY;
  else if (greedy_row && gmax >= mrg::kInfS) code = QS_ROW_NONFINITE;
  else if (greedy_row && gmax == -mrg::kInfS) code = QS_ROW_ALL_NEG_INF;
  else if (!greedy_row && thr == chunk::kThrAll && N == 0u && !(flags & chunk::kOverflow))
    code = QS_ROW_ALL_NEG_INF;
  const bool greedy = code == QS_ROW_OK && greedy_row;
  // one point mass at the greedy token, or all zeros for an error row
  auto settle_point = [&](int code_, bool greedy_) {
    const uint32_t am = greedy_ ? argmax : 0xFFFFFFFFu;
    if (mask_row)
      for (int i = tid; i < W; i += kThreads)
        mask_row[i] = greedy_ && (uint32_t)i == (am >> 5) ? 1u << (am & 31u) : 0u;
    if (dense_row)
      for (int i = tid; i < V; i += kThreads) dense_row[i] = (uint32_t)i == am ? 1.0f : 0.0f;
    if (tid == 0) {
      a.status[r] = code_;
      if (SAMPLE) {
        a.tokens[r] = greedy_ ? (int32_t)am : -1;
        if (a.logprobs) a.logprobs[r] = greedy_ ? 0.0f : __builtin_nanf("");
      }
      if (greedy_) {
        if (ids_out) ids_out[0] = (int32_t)am;
        if (probs_out) probs_out[0] = 1.0f;
      }
      if (a.cand_count) a.cand_count[r] = greedy_ ? 1 : 0;
      if (a.dbg) {
        a.dbg[4 * r + 0] = 2;
        a.dbg[4 * r + 1] = 0;
        a.dbg[4 * r + 2] = greedy_ ? 1 : 0;
        a.dbg[4 * r + 3] = greedy_ ? 1 : 0;
      }
    }
  };
  if (code != QS_ROW_OK || greedy) {
    settle_point(code, greedy);
    return true;
  }

  // -- which rows the candidates settle -----------------------------------------------------
  const bool topk_on = kk > 0 && kk < V;
  const bool topp_on = pf < 1.0f;
  const bool need_bg = topp_on && !topk_on;
  if (thr >= chunk::kThrNone || (flags & chunk::kOverflow) || N > mrg::kPoolMax || N == 0u)
    return false;
  if (!topk_on && !topp_on) return false;              // every token kept
  if (topk_on && N < (uint32_t)kk) return false;       // the k-th value lies below t
  // masks wider than the LDS stage: cleared in memory here, bits set there
  const bool mask_direct = mask_row && W > mrg::kMaskWords;
  if (V > (int)mrg::kIdMask) return false;
  const int32_t tS = mrg::skey1(thr);
  double m_bg = 0.0, m_bg_err = 0.0;
  // -- 3. candidates into LDS (id order), histogram of their values ------------------------
  if (need_bg) {
    m_bg = uni(info.sc_d[0]);
    m_bg_err = uni(info.sc_d[1]);
    if (uni(info.sc_u[0]) != 0u) return false;        // a background mass that is not exact
  }
  if (dense_row || mask_direct) {
    // zero in memory first (the scatter below lands after these stores)
    if (dense_row)
      for (int i = tid; i < V; i += kThreads) dense_row[i] = 0.0f;
    if (mask_direct)
      for (int i = tid; i < W; i += kThreads) mask_row[i] = 0u;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  // Candidates: entry i of segment sg goes to pool[base_s[sg] + i] (id
  // order). Wave w takes segments w, w + 16, ...; the first 64 entries of its
  // first kSpec segments arrived with step 1, the rest are read now, two
  // segments at a time, eight loads a lane each (past a segment's count the
  // range-checked buffer loads read zeros).
  {
    uint32_t top = 0u;
    bool nonfin = false;
    auto put = [&](uint32_t e, int sg, uint32_t j) {
      nonfin |= (e >> 16) - 0x7F80u < 0x80u;   // +inf or a positive NaN
      const uint32_t bin = (uint32_t)(mrg::skey1(e >> 16) - tS);
      const uint32_t binc = bin < (uint32_t)mrg::kWin ? bin : (uint32_t)mrg::kWin - 1u;
      top = max(top, bin + 1u);
      pool[j] = (binc << mrg::kIdBits) | ((uint32_t)sg * (uint32_t)chunk::kSegTokens + (e & 0xFFFFu));
      __hip_atomic_fetch_add(hist + binc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
#pragma unroll
    for (int i = 0; i < kSpec; ++i) {
      const int sg = w + kWaves * i;
      if (sg < NS) {
        const uint32_t b0 = uni(base_s[sg]), n = uni(base_s[sg + 1]) - b0;
        if ((uint32_t)lane < n) put(spec[i], sg, b0 + (uint32_t)lane);
      }
    }
    for (int sg0 = w; sg0 < NS; sg0 += 2 * kWaves) {
      const int sgs[2] = {sg0, sg0 + kWaves};
      uint32_t b[2], n[2], st[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        b[h] = sgs[h] < NS ? uni(base_s[sgs[h]]) : 0u;
        n[h] = sgs[h] < NS ? uni(base_s[sgs[h] + 1]) - b[h] : 0u;
        st[h] = sgs[h] < w + kWaves * kSpec ? 64u : 0u;    // entries already taken
      }
      const uint32_t rest = max(n[0] > st[0] ? n[0] - st[0] : 0u, n[1] > st[1] ? n[1] - st[1] : 0u);
      for (uint32_t i0 = 0u; i0 < rest; i0 += 512u) {
        uint32_t ev[2][8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
              const_cast<uint32_t*>(crow + (size_t)(sgs[h] < NS ? sgs[h] : 0) * chunk::kSegCap),
              (short)0, (int)(n[h] * 4u), 0x00020000);
#pragma unroll
          for (int k = 0; k < 8; ++k)
            ev[h][k] = __builtin_amdgcn_raw_buffer_load_b32(
                rs, (int)((st[h] + i0 + (uint32_t)(lane + 64 * k)) * 4u), 0, 0);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const uint32_t ii = st[h] + i0 + (uint32_t)(lane + 64 * k);
            if (ii < n[h]) put(ev[h][k], sgs[h], b[h] + ii);
          }
        }
      }
    }
    top = wave_reduce<OpMax>(top);
    if (ballot(nonfin)) top |= 0x80000000u;
    if (lane == 0)
      __hip_atomic_fetch_max(&info.sc_u[1], top, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  if (SAMPLE && !a.uniforms) u_bits = philox_u24(seed_in, u_bits);
  __syncthreads();  // pool, histogram, the largest bin
  const uint32_t top_bin = uni(info.sc_u[1]);
  if (top_bin & 0x80000000u) {   // a legal +inf or positive NaN among the candidates
    __syncthreads();             // (the staged mask words are not read again)
    settle_point(QS_ROW_NONFINITE, false);
    return true;
  }
  // candidates beyond the bins (a value span wider than the histogram)
  if (top_bin > (uint32_t)mrg::kWin) return false;
  const int32_t max_s = tS + (int32_t)top_bin - 1;    // the row's largest legal value

  // -- 4. bins in descending value: weights, prefix sums, the boundaries ------------------
  const double invT = 1.0 / (double)Tf;
  const double p = (double)pf;
  const double m = mrg::skey_value(max_s);
  const int bme = mrg::kWin - 1 - tid;  // this thread's bin: descending value as tid grows
  const int32_t sk_me = tS + bme;
  const uint32_t c_me = hist[bme];
  const double w_me = sk_me <= max_s ? exp64((mrg::skey_value(sk_me) - m) * invT) : 0.0;
  binw[bme] = w_me;
  const double mt = (double)c_me * w_me;
  uint32_t c_excl;
  double m_excl, m_tot;
  int par = 0;
  {
    const uint32_t ci = scan_incl_u32(c_me);
    const double mi = scan_incl_f64(mt);
    if (lane == 63) {
      red.v[par][w][0] = ci;
      const uint64_t b = __double_as_longlong(mi);
      red.v[par][w][1] = (uint32_t)b;
      red.v[par][w][2] = (uint32_t)(b >> 32);
    }
    if (tid == 0) {
      info.claim = ~0ull;
      info.sel_u[0] = sel::kNone;
    }
    __syncthreads();  // wave totals, bin weights
    const uint32_t tc = act16 ? red.v[par][lane][0] : 0u;
    const double tm = act16 ? __longlong_as_double(((uint64_t)red.v[par][lane][2] << 32) |
                                                   red.v[par][lane][1])
                            : 0.0;
    const uint32_t tci = scan_incl_u32(tc);
    const double tmi = scan_incl_f64(tm);
    const double tme = incl_shift1_f64(tmi);
    const int wu = uni(w);
    c_excl = readlane_u32(tci - tc, wu) + ci - c_me;
    m_excl = readlane_f64(tme, wu) + (mi - mt);
    m_tot = uni(readlane_f64(tmi, kWaves - 1));
    par ^= 1;
  }

  // top-k: the bin of the k-th largest value and its tie quota
  uint32_t bk = 0xFFFFFFFFu, nk = 0u;
  double w_k = 0.0, w_kap = 0.0;
  if (topk_on) {
    const uint32_t kq = (uint32_t)kk;
    if (c_excl < kq && kq <= c_excl + c_me) {
      info.sel_u[0] = (uint32_t)bme;
      info.sel_u[1] = kq - c_excl;
      info.sel_d[0] = m_excl + (double)(kq - c_excl) * w_me;
      info.sel_d[1] = w_me;
    }
    __syncthreads();
    bk = uni(info.sel_u[0]);
    nk = uni(info.sel_u[1]);
    w_k = uni(info.sel_d[0]);
    w_kap = uni(info.sel_d[1]);
    if (bk == sel::kNone) return false;  // (never: N >= k candidates)
  }
  // the reference mass of top-p: the top-k set, or every legal token (the
  // candidates plus the background mass, known within a bound)
  double w_ref = w_k, w_err = 0.0;
  if (!topk_on) {
    const double sc = exp64((mrg::skey_value(tS) - m) * invT);
    w_ref = m_tot + m_bg * sc;
    w_err = m_bg_err * sc;
  }

  // top-p on the top-k set: the first value whose descending mass reaches p W
  uint32_t b_star, n_keep;
  double w_star;
  if (topp_on) {
    const double target = p * (w_ref + w_err), target_lo = p * (w_ref - w_err);
    // tokens of this bin inside the top-k set
    const uint32_t cK = !topk_on || (uint32_t)bme > bk ? c_me : ((uint32_t)bme == bk ? nk : 0u);
    if (cK && m_excl < target && m_excl + (double)cK * w_me >= target * (1.0 - 1e-13)) {
      const double need = (target - m_excl) / w_me;
      uint32_t nn = need <= 1.0 ? 1u : (need >= (double)cK ? cK : (uint32_t)ceil(need));
      while (nn > 1u && m_excl + (double)(nn - 1u) * w_me >= target) --nn;
      while (nn < cK && m_excl + (double)nn * w_me < target) ++nn;
      if (m_excl + (double)nn * w_me >= target) {
        // the lower reference must give the same value and count; otherwise
        // claim 0 (never a real claim), and the row takes the other paths
        const bool same = m_excl < target_lo && m_excl + (double)nn * w_me >= target_lo &&
                          (nn == 1u || m_excl + (double)(nn - 1u) * w_me < target_lo);
        __hip_atomic_fetch_min(&info.claim, same ? ((uint64_t)tid << 32) | nn : 0ull,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
    __syncthreads();
    const uint64_t cl = info.claim;
    const uint32_t rank = uni((uint32_t)(cl >> 32));
    n_keep = uni((uint32_t)cl);
    // no claim: the target lies past the candidates' mass (a truncation miss
    // of a row with top-k off) or the bound leaves the cut open
    if (rank >= (uint32_t)mrg::kWin || n_keep == 0u) return false;
    b_star = (uint32_t)(mrg::kWin - 1) - rank;
    w_star = binw[b_star];
  } else {
    b_star = bk;
    n_keep = nk;
    w_star = w_kap;
  }

  // -- 5. per-wave counts over the id-ordered candidates ------------------------------------
  const uint32_t per = ((N + kWaves - 1) / kWaves + 3u) & ~3u;
  const uint32_t lo_w = min(N, (uint32_t)w * per), hi_w = min(N, lo_w + per);
  const uint32_t e_gt = ((b_star + 1u) << mrg::kIdBits) - 1u;  // entries above compare greater
  {
    uint32_t gt = 0u, ties = 0u;
    double mgt = 0.0;
    for (uint32_t i0 = lo_w; i0 < hi_w; i0 += 256u) {
      const uint32_t ib = i0 + 4u * (uint32_t)lane;
      if (ib < hi_w) {
        const uint4 e4 = *reinterpret_cast<const uint4*>(pool + ib);
        const uint32_t e[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (ib + (uint32_t)q < hi_w) {
            if (e[q] > e_gt) {
              ++gt;
              mgt += binw[e[q] >> mrg::kIdBits];
            } else if ((e[q] >> mrg::kIdBits) == b_star) {
              ++ties;
            }
          }
        }
      }
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

  // tie quota per wave (earliest ids first), list offsets, masses, the sampled wave
  double u = 0.0;
  if (SAMPLE) {
    if (a.uniforms) u = __longlong_as_double((long long)u_bits);
    else u = (double)(uint32_t)u_bits * (1.0 / 16777216.0);
  }
  u = uni(u);
  uint32_t my_off, n_p, my_kt;
  double w_p, my_cumw;
  int sw, last_w;
  {
    const uint32_t t = act16 ? info.ties[lane] : 0u;
    const uint32_t g = act16 ? info.gt[lane] : 0u;
    const double mg = act16 ? info.mass[lane] : 0.0;
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

  // -- 6. outputs: 256 consecutive entries a round, four per lane ----------------------------
  using gi32 = __attribute__((address_space(1))) int32_t;
  using gf32 = __attribute__((address_space(1))) float;
  gi32* const ids_row = (gi32*)ids_out;
  gf32* const probs_row = (gf32*)probs_out;
  const uint32_t cap = (uint32_t)a.cand_cap;
  uint32_t pos_base = my_off;
  uint32_t ties_seen = 0u;
  double cbase = my_cumw * inv_wp;
  int my_token = -1;
  double my_q = 0.0;
  uint32_t last_e = ~0u;   // this lane's last kept entry with q > 0 (entries never equal ~0u)
  for (uint32_t i0 = lo_w; i0 < hi_w; i0 += 256u) {
    const uint32_t ib = i0 + 4u * (uint32_t)lane;
    uint32_t e[4] = {0u, 0u, 0u, 0u};
    if (ib < hi_w) {
      const uint4 e4 = *reinterpret_cast<const uint4*>(pool + ib);
      e[0] = e4.x; e[1] = e4.y; e[2] = e4.z; e[3] = e4.w;
    }
    uint32_t kb = 0u, tb = 0u;  // entries above the boundary, and ties at it
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool valid = ib + (uint32_t)q < hi_w;
      kb |= (valid && e[q] > e_gt ? 1u : 0u) << q;
      tb |= (valid && (e[q] >> mrg::kIdBits) == b_star ? 1u : 0u) << q;
    }
    const uint32_t tc = (uint32_t)__popc(tb);
    if (ballot(tc != 0u)) {
      const uint32_t tincl = scan_incl_u32(tc);
      uint32_t trank = ties_seen + tincl - tc;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if ((tb >> q) & 1u) {
          if (trank < my_kt) kb |= 1u << q;
          ++trank;
        }
      }
      ties_seen += readlane_u32(tincl, 63);
    }
    const uint32_t kc = (uint32_t)__popc(kb);
    const uint32_t kincl = scan_incl_u32(kc);
    uint32_t pos = pos_base + kincl - kc;
    double qv[4];
    double lane_sum = 0.0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      qv[q] = 0.0;
      if ((kb >> q) & 1u) {
        const uint32_t id = e[q] & mrg::kIdMask;
        const double qq = binw[e[q] >> mrg::kIdBits] * inv_wp;
        qv[q] = qq;
        lane_sum += qq;
        const float qf = (float)qq;
        if (pos < cap) {
          if (ids_row) __builtin_nontemporal_store((int32_t)id, ids_row + pos);
          if (probs_row) __builtin_nontemporal_store(qf, probs_row + pos);
        }
        if (dense_row) dense_row[id] = qf;
        if (mask_direct)
          __hip_atomic_fetch_or(mask_row + (id >> 5), 1u << (id & 31u), __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
        else if (mask_row)
          __hip_atomic_fetch_or(mstage + (id >> 5), 1u << (id & 31u), __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_WORKGROUP);
        if (qq > 0.0) last_e = e[q];
        ++pos;
      }
    }
    pos_base += readlane_u32(kincl, 63);
    if (SAMPLE && w == sw && my_token < 0) {
      const double incl = scan_incl_f64(lane_sum);
      double cu = cbase + (incl - lane_sum);
      int hit = -1;
      double hq = 0.0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        cu += qv[q];
        if (hit < 0 && ((kb >> q) & 1u) && u < cu) {
          hit = (int)(e[q] & mrg::kIdMask);
          hq = qv[q];
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
  }
  __syncthreads();  // the staged mask words
  if (mask_row && !mask_direct)
    for (int i = tid; i < W; i += kThreads) __builtin_nontemporal_store(mstage[i], mask_row + i);
  // the token: from wave sw; if rounding left u at or above wave sw's last
  // cumulative sum, that wave's last kept id with q > 0; if u lies past every
  // wave, the last kept id with q > 0 of the row
  const int last_pos_id = last_e == ~0u ? -1 : (int)(last_e & mrg::kIdMask);
  const int last_id = (int)wave_reduce<OpMax>((uint32_t)(last_pos_id + 1)) - 1;
  if (SAMPLE) {
    double last_q = 0.0;
    if (a.logprobs) {
      const double last_pos_q =
          last_e == ~0u ? 0.0 : binw[last_e >> mrg::kIdBits] * inv_wp;
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
      a.dbg[4 * r + 0] = 2;
      a.dbg[4 * r + 1] = 0;
      a.dbg[4 * r + 2] = (int32_t)N;
      a.dbg[4 * r + 3] = (int32_t)n_p;
    }
  }
  return true;
}
