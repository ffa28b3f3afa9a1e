"""Exact speculative-decoding verification over candidate lists (CPU oracle).

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module.

Rule (page "第 9 讲 · 生成与推测解码", section 5.2, the exact rule of Leviathan et
al. and Chen et al.): a draft token x drawn from the draft distribution q is
accepted with probability min(1, p(x)/q(x)), p being the target distribution;
on rejection one token is drawn from max(0, p - q) renormalised. The page shows
that the output is then distributed exactly as p.

Both distributions arrive as id-ascending candidate lists (ids, float32 probs)
as the filter writes them; a token outside a list has probability 0 there.
Decisions, in float64 on the float32 list values widened exactly:
  accept    iff u_accept * q(x) < p(x)            (u_accept in [0, 1))
  residual  r(y) = max(0, p(y) - q(y)) for y in the target list, R = sum r
  resample  the first y in id order with u_resample * R < cumsum(r)(y); if
            rounding leaves none, the last y with r(y) > 0
  R == 0    (rounding only: p <= q everywhere although p(x) < q(x)) draw from
            p itself the same way
Row errors: BAD_PARAM for a negative count; EMPTY when either list is empty
(or the target list holds no positive probability); CAND_OVERFLOW when either count
exceeds its list's capacity (the list is truncated, so p or q is unknown),
BAD_PARAM when x is not in the draft list or a uniform lies outside [0, 1).
"""

import numpy as np

from .sampling import ROW_BAD_PARAM, ROW_CAND_OVERFLOW, ROW_EMPTY, ROW_OK


def _prob(ids, probs, tok):
    i = int(np.searchsorted(ids, tok))
    if i < len(ids) and int(ids[i]) == tok:
        return float(probs[i]), True
    return 0.0, False


def _inverse_cdf(ids, w, target):
    """First id whose running sum of w (id order) exceeds target; else the last
    id with w > 0. Returns (token, distance of target to the nearest step)."""
    cum = 0.0
    dist = abs(target)
    last = -1
    for i in range(len(ids)):
        if w[i] > 0.0:
            last = i
        cum += float(w[i])
        dist = min(dist, abs(target - cum))
        if target < cum:
            return int(ids[i]), dist
    return (int(ids[last]) if last >= 0 else -1), dist


def spec_verify_row(t_ids, t_probs, t_count, t_cap, d_ids, d_probs, d_count, d_cap,
                    x, u_accept, u_resample):
    """Returns (status, token, accepted, distance); distance is how close the
    resampling target came to a CDF step (inf when nothing was resampled)."""
    if t_count < 0 or d_count < 0:
        return ROW_BAD_PARAM, -1, 0, np.inf
    if t_count == 0 or d_count == 0:
        return ROW_EMPTY, -1, 0, np.inf
    if t_count > t_cap or d_count > d_cap:
        return ROW_CAND_OVERFLOW, -1, 0, np.inf
    t_ids = np.asarray(t_ids[:t_count], np.int64)
    t_p = np.asarray(t_probs[:t_count], np.float32).astype(np.float64)
    d_ids = np.asarray(d_ids[:d_count], np.int64)
    d_p = np.asarray(d_probs[:d_count], np.float32).astype(np.float64)
    qx, in_draft = _prob(d_ids, d_p, x)
    if not in_draft or not (0.0 <= u_accept < 1.0) or not (0.0 <= u_resample < 1.0):
        return ROW_BAD_PARAM, -1, 0, np.inf
    px, _ = _prob(t_ids, t_p, x)
    if u_accept * qx < px:
        return ROW_OK, int(x), 1, np.inf
    q_at = np.array([_prob(d_ids, d_p, int(y))[0] for y in t_ids])
    r = np.maximum(0.0, t_p - q_at)
    R = 0.0
    for v in r:  # id order
        R += float(v)
    if R > 0.0:
        tok, dist = _inverse_cdf(t_ids, r, u_resample * R)
    else:
        P = 0.0
        for v in t_p:
            P += float(v)
        if not P > 0.0:  # every listed target probability underflowed
            return ROW_EMPTY, -1, 0, np.inf
        tok, dist = _inverse_cdf(t_ids, t_p, u_resample * P)
    return ROW_OK, tok, 0, dist


def spec_verify_batch(t_ids, t_probs, t_count, d_ids, d_probs, d_count, x, u_accept,
                      u_resample, rows=None):
    """Row loop over [B, cap] lists: {row: (status, token, accepted, distance)}."""
    B = len(x)
    rows = range(B) if rows is None else rows
    tc, dc = t_ids.shape[1], d_ids.shape[1]
    return {r: spec_verify_row(t_ids[r], t_probs[r], int(t_count[r]), tc, d_ids[r],
                               d_probs[r], int(d_count[r]), dc, int(x[r]),
                               float(u_accept[r]), float(u_resample[r]))
            for r in rows}
