"""Shared helpers: move seeded workloads to the GPU, run the C-ABI through the
binding, and compare every output with the CPU oracle row by row."""

import numpy as np

import oracle

PROB_RTOL = 1e-6          # relative tolerance on probabilities (fp32 outputs)
PROB_FLOOR = 2.0 ** -126  # absolute floor for underflowing tails
CDF_BAND = 1e-6           # tokens are compared exactly unless u is this close to a CDF step


def to_device(w, device="cuda"):
    import torch
    d = {}
    if w.dtype == "bf16":
        d["logits"] = torch.from_numpy(w.logits.view(np.int16)).to(device).view(torch.bfloat16)
    else:
        d["logits"] = torch.from_numpy(w.logits).to(device)
    d["T"] = torch.from_numpy(w.T).to(device)
    d["k"] = torch.from_numpy(w.k).to(device)
    d["p"] = torch.from_numpy(w.p).to(device)
    d["bitmask"] = None if w.bitmask is None else \
        torch.from_numpy(w.bitmask.view(np.int32)).to(device)
    d["seed"] = torch.from_numpy(w.seeds.view(np.int64)).to(device)
    d["offset"] = torch.from_numpy(w.offsets.view(np.int64).copy()).to(device)
    return d


def words_u32(t):
    return t.cpu().numpy().view(np.uint32)


def prob_close(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    return np.all(np.abs(got - want) <= PROB_RTOL * np.abs(want) + PROB_FLOOR)


class Report:
    def __init__(self):
        self.rows = 0
        self.band_rows = 0
        self.cdf_band = 0
        self.failures = []

    def fail(self, msg):
        if len(self.failures) < 20:
            self.failures.append(msg)

    def check(self):
        assert not self.failures, "\n".join(self.failures)
        # a token may differ from the oracle's only where u lies within CDF_BAND
        # of a step, and then only by summation order (fp64 on both sides):
        # at most one such row per thousand
        assert self.cdf_band <= max(1, self.rows // 1000), \
            f"{self.cdf_band} tokens differ within the CDF band over {self.rows} rows"


def compare_filter(w, res, out, rows, rep, cand_cap=None, check_dense=True):
    """Compare filter outputs for `rows` with oracle results `res` ({row: RowResult})."""
    V = w.V
    status = out["status"].cpu().numpy()
    mask = words_u32(out["keep_mask"]) if "keep_mask" in out else None
    cids = out["cand_ids"].cpu().numpy() if "cand_ids" in out else None
    cpr = out["cand_probs"].cpu().numpy() if "cand_probs" in out else None
    ccnt = out["cand_count"].cpu().numpy() if "cand_count" in out else None
    dense = out["dense"].cpu().numpy() if ("dense" in out and check_dense) else None
    for r in rows:
        rr = res[r]
        rep.rows += 1
        want_status = rr.status
        n_p = len(rr.kept) if rr.status == oracle.ROW_OK else 0
        if rr.status == oracle.ROW_OK and cids is not None and n_p > cids.shape[1]:
            want_status = oracle.ROW_CAND_OVERFLOW
        if status[r] != want_status:
            # an in-band row may overflow the list in one variant and not the other
            rep.fail(f"row {r}: status {status[r]} != {want_status}")
            continue
        if rr.status != oracle.ROW_OK:
            if mask is not None and mask[r].any():
                rep.fail(f"row {r}: error row with a non-zero mask")
            if ccnt is not None and ccnt[r] != 0:
                rep.fail(f"row {r}: error row with cand_count {ccnt[r]}")
            if dense is not None and dense[r].any():
                rep.fail(f"row {r}: error row with non-zero dense probs")
            continue
        options = [(rr.kept, rr.q)] + list(rr.alternatives)
        if rr.alternatives:
            rep.band_rows += 1
        # which option does the GPU mask match?
        got_kept = None
        if mask is not None:
            gm = mask[r]
            for kept, q in options:
                if np.array_equal(gm, oracle.keep_mask_words(kept, V)):
                    got_kept = (kept, q)
                    break
            if got_kept is None:
                gk = np.nonzero(oracle.legal_from_bitmask(gm, V))[0]
                rep.fail(f"row {r}: mask mismatch |gpu|={len(gk)} |orc|={len(rr.kept)} "
                         f"first diff ids {np.setxor1d(gk, rr.kept)[:8]} margin {rr.margin:.3g}")
                continue
        else:
            got_kept = options[0]
        kept, q = got_kept
        if ccnt is not None:
            if ccnt[r] != len(kept):
                rep.fail(f"row {r}: cand_count {ccnt[r]} != {len(kept)}")
                continue
            n = min(len(kept), cids.shape[1])
            if not np.array_equal(cids[r, :n], kept[:n]):
                rep.fail(f"row {r}: candidate ids differ")
                continue
            if not prob_close(cpr[r, :n], q[:n].astype(np.float32)):
                bad = np.argmax(np.abs(cpr[r, :n] - q[:n]) / (q[:n] + 1e-300))
                rep.fail(f"row {r}: cand prob {cpr[r, bad]} vs {q[bad]}")
                continue
        if dense is not None:
            want = np.zeros(V, np.float64)
            want[kept] = q
            if not prob_close(dense[r], want.astype(np.float32)):
                rep.fail(f"row {r}: dense probs differ")
                continue


def compare_tokens(res, tokens, rows, rep, uniforms=None, offsets_in=None,
                   offsets_out=None, seeds=None):
    """Tokens against the oracle's CDF walk with the same u (fixed uniforms, or
    the oracle's own Philox from seeds and the incoming offsets)."""
    tokens = tokens.cpu().numpy()
    for r in rows:
        rr = res[r]
        if rr.status != oracle.ROW_OK:
            if tokens[r] != -1:
                rep.fail(f"row {r}: error row token {tokens[r]}")
            if offsets_out is not None and offsets_out[r] != offsets_in[r]:
                rep.fail(f"row {r}: error row advanced its offset")
            continue
        if rr.greedy:
            if tokens[r] != rr.kept[0]:
                rep.fail(f"row {r}: greedy token {tokens[r]} != {rr.kept[0]}")
            if offsets_out is not None and offsets_out[r] != offsets_in[r]:
                rep.fail(f"row {r}: greedy row advanced its offset")
            continue
        if uniforms is not None:
            u = float(uniforms[r])
        else:
            u = oracle.uniform(int(seeds[r]), int(offsets_in[r]))
            if offsets_out[r] != offsets_in[r] + 1:
                rep.fail(f"row {r}: offset {offsets_out[r]} != {offsets_in[r] + 1}")
        ok = False
        dmin = np.inf
        for kept, q in [(rr.kept, rr.q)] + list(rr.alternatives):
            tok, dist = oracle.sample_from(kept, q, u)
            dmin = min(dmin, dist)
            ok = ok or tok == tokens[r]
        if not ok:
            if dmin < CDF_BAND:
                rep.cdf_band += 1
            else:
                rep.fail(f"row {r}: token {tokens[r]} != oracle (u={u}, dist={dmin:.3g})")


LOGPROB_ATOL = 1e-6  # the probabilities' 1e-6 relative tolerance, on the log scale


def compare_logprobs(res, tokens, logprobs, cand_count, rows, rep):
    """The drawn token's log-probability against the oracle's, for the token the
    GPU drew: NaN on error rows, 0 on greedy rows, else log q of that token
    within LOGPROB_ATOL plus the float32 rounding of the result. Rows that kept
    an adjacent top-p prefix (a different set, so different q) are skipped."""
    tokens = tokens.cpu().numpy()
    lp = logprobs.cpu().numpy().astype(np.float64)
    cc = cand_count.cpu().numpy()
    for r in rows:
        rr = res[r]
        want = oracle.token_logprob(rr, int(tokens[r]))
        if rr.status != oracle.ROW_OK:
            if not np.isnan(lp[r]):
                rep.fail(f"row {r}: error row logprob {lp[r]}")
            continue
        if not rr.greedy and cc[r] != len(rr.kept):
            continue
        if not abs(lp[r] - want) <= LOGPROB_ATOL + 1.2e-7 * abs(want):
            rep.fail(f"row {r}: logprob {lp[r]} != {want}")
