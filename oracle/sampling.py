"""Plain CPU definition of batched top-k / top-p filtering and sampling (fp64).

TEST INFRASTRUCTURE: this is the oracle the HIP path is checked against. Only
tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import it.
It shares no code with the product package and imports nothing from it.

What it computes, per row, and where each step comes from:

* Contract order (page "Attention算完，还没有选出下一个token", section 02, the
  reference convention): temperature and score rules first, then the legal-token
  mask, then top-k with renormalisation, then top-p as the shortest prefix of the
  descending-probability order whose cumulative mass reaches p, then
  renormalisation and sampling.
* Greedy is a separate argmax path when the temperature is 0 (same page,
  section 02 note; page "Sampling 系统设计", the temperature section): no softmax
  and no random number. Ties go to the lowest token id (page "第 9 讲 · 生成与推测解码",
  exercise 1 answer: the tie is broken by vocabulary order).
* Illegal tokens become -inf before top-k (first page, section 05 step list).
* An empty candidate set is an explicit error, never a substituted token (first
  page, section 03); NaN and all -inf rows are handled explicitly (section 07).
* Ties at the top-k / top-p boundary keep the earliest token ids (page "Qrita",
  key design 3: the prefix-sum quota keeps the earliest N_keep duplicates).
* Temperature divides the logits, equivalently p^(1/T) renormalised (lecture
  page, section 3.3).
* Sampling walks the kept candidates in token-id order and returns the first id
  whose cumulative probability exceeds u (first page, the widget in section 02:
  "CDF by token id"; lecture page section 3.1: one O(k) scan).

The method on the Qrita page reaches exactly the full-vocabulary sort result
("identical to full-vocabulary sorting", key design 3), so this oracle is that
definition written out: a stable sort by (-logit, token id) of each full row,
then prefix slices and fp64 cumulative sums. There is no truncation, pivoting,
blocking or fusion here.

Readings where the pages are silent:
* top-p boundary is ">= p" (cumulative mass *reaching* p; worked answer to
  exercise 7 on the lecture page keeps 3 tokens when the sum hits 0.9 exactly);
* ranking uses the exact logit z, not a rounded z/T;
* the top-p reference mass is the mass of the top-k set (top-k renormalises
  first), or of all finite legal tokens when top-k is off;
* k = 0 means top-k off, k >= |F| keeps every finite legal token, p = 1 means
  top-p off; T < 0, T not finite, k < 0, p <= 0, p > 1 or p NaN is BAD_PARAM;
* status precedence: EMPTY (no legal token), then NONFINITE (NaN or +inf at a
  legal position), then ALL_NEG_INF (every legal logit is -inf);
* bitmask bit order: token i is bit (i & 31) of 32-bit word (i >> 5);
* legal -inf tokens are never kept; finite kept tokens stay kept even if their
  probability underflows;
* the CDF interval is right-open: token j is chosen iff cum_{j-1} <= u < cum_j;
  if rounding leaves u at or above the final sum, the last kept id with q > 0.
"""

from dataclasses import dataclass, field

import numpy as np

# Row status codes of the contract.
ROW_OK = 0
ROW_EMPTY = 1
ROW_ALL_NEG_INF = 2
ROW_NONFINITE = 3
ROW_BAD_PARAM = 4
ROW_CAND_OVERFLOW = 5

# Width of the band around the top-p boundary inside which two correct fp64
# implementations that sum in different orders may keep adjacent prefixes.
TOP_P_BAND = 1e-9


@dataclass
class RowResult:
    status: int
    kept: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    q: np.ndarray = field(default_factory=lambda: np.zeros(0, np.float64))
    greedy: bool = False
    n_finite: int = 0
    k_size: int = 0          # |K|, the top-k set size (|F| when top-k is off)
    w_k: float = 0.0         # mass of K (weights relative to the row maximum)
    margin: float = np.inf   # top-p boundary margin / W_K (inf when top-p off)
    alternatives: list = field(default_factory=list)  # adjacent prefixes in the band


def bf16_bits_to_float64(bits):
    """Widen bfloat16 bit patterns (uint16) exactly to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def legal_from_bitmask(words, V):
    """Token i is legal iff bit (i & 31) of word (i >> 5) is set; bits >= V ignored."""
    words = np.asarray(words, dtype=np.uint32)
    ids = np.arange(V, dtype=np.int64)
    return ((words[ids >> 5] >> (ids & 31).astype(np.uint32)) & 1).astype(bool)


def params_valid(T, k, p):
    T = float(T)
    p = float(p)
    if not np.isfinite(T) or T < 0.0:
        return False
    if int(k) < 0:
        return False
    if not np.isfinite(p) or p <= 0.0 or p > 1.0:
        return False
    return True


def filter_row(z, T, k, p, legal=None, band=TOP_P_BAND):
    """Filter one row of logits.

    z: float64 array of logits (already widened exactly from fp32 / bf16).
    T: temperature as the float32 value the caller passes, widened to float64.
    k: top-k (0 = off). p: top-p (1 = off). legal: bool array or None (all legal).
    Returns a RowResult with the kept ids in ascending order and their
    renormalised probabilities (float64).
    """
    z = np.asarray(z, dtype=np.float64)
    V = z.shape[0]
    T = float(np.float32(T))
    p = float(np.float32(p))
    k = int(k)

    # 0. parameters
    if not params_valid(T, k, p):
        return RowResult(ROW_BAD_PARAM)

    # 1. legal set
    if legal is None:
        legal = np.ones(V, dtype=bool)
    legal_ids = np.nonzero(legal)[0]
    if legal_ids.size == 0:
        return RowResult(ROW_EMPTY)

    # 2. NaN or +inf at a legal position (illegal positions were overwritten by -inf)
    zl = z[legal_ids]
    if np.any(np.isnan(zl)) or np.any(zl == np.inf):
        return RowResult(ROW_NONFINITE)

    # 3. finite legal set F
    fin = legal_ids[zl > -np.inf]
    if fin.size == 0:
        return RowResult(ROW_ALL_NEG_INF)
    zf = z[fin]

    # 4. greedy
    if T == 0.0:
        top = zf.max()
        tok = int(fin[np.nonzero(zf == top)[0][0]])
        return RowResult(ROW_OK, kept=np.array([tok], np.int64),
                         q=np.array([1.0]), greedy=True, n_finite=int(fin.size),
                         k_size=1, w_k=1.0)

    # 5. descending order by (-z, id): stable sort on -z keeps ascending ids in ties
    order = np.argsort(-zf, kind="stable")
    pi = fin[order]
    zpi = zf[order]

    # 6. top-k
    n = pi.size
    kk = n if (k == 0 or k >= n) else k
    K = pi[:kk]
    zK = zpi[:kk]

    # 7. weights relative to the row maximum, fp64, summed in pi order
    w = np.exp((zK - zpi[0]) / T)
    cum = np.cumsum(w)
    w_k = float(cum[-1])

    # 8. top-p: shortest prefix whose cumulative mass reaches p * W_K
    margin = np.inf
    alternatives = []
    if p < 1.0:
        target = p * w_k
        j = int(np.searchsorted(cum, target, side="left"))  # first cum_j >= target
        j = min(j, kk - 1)
        below = cum[j - 1] if j > 0 else 0.0
        m_lo = (target - below) / w_k
        m_hi = (cum[j] - target) / w_k
        margin = min(m_lo, m_hi)
        if m_lo < band and j >= 1:
            alternatives.append(j)        # one fewer kept token
        if m_hi < band and j + 1 < kk:
            alternatives.append(j + 2)    # one more kept token
        npk = j + 1
    else:
        npk = kk

    # 9. renormalise over P (W_P is the pi-order prefix sum at the cut)
    w_p = float(cum[npk - 1])
    P = K[:npk]
    q = w[:npk] / w_p

    # 10. outputs in ascending token id
    asc = np.argsort(P, kind="stable")
    alts = []
    for m in alternatives:
        Pa = K[:m]
        wa = w[:m] / float(cum[m - 1])
        aa = np.argsort(Pa, kind="stable")
        alts.append((Pa[aa], wa[aa]))
    return RowResult(ROW_OK, kept=P[asc], q=q[asc], n_finite=int(n), k_size=kk,
                     w_k=w_k, margin=margin, alternatives=alts)


def sample_from(kept, q, u):
    """Inverse CDF in ascending token-id order with a right-open interval.

    Returns (token, distance) where distance is the smallest |u - cum_j| seen
    over the walk (how close u is to a CDF boundary).
    """
    cum = 0.0
    dist = abs(u)
    last_pos = -1
    for i in range(len(kept)):
        if q[i] > 0.0:
            last_pos = i
        cum += float(q[i])
        dist = min(dist, abs(u - cum))
        if u < cum:
            return int(kept[i]), dist
    if last_pos < 0:
        return -1, dist
    return int(kept[last_pos]), dist


def token_logprob(res, token):
    """Log-probability of the drawn token under the distribution it was drawn
    from: after temperature, mask, top-k, top-p and renormalisation (page
    "Sampling 系统设计：从 logits 到可控生成", section on logprobs: a sampler may
    return the chosen token's log-probability and must say which distribution
    it refers to; this is that reading). Greedy rows draw from a point mass,
    so 0; error rows have no token, so NaN.
    """
    if res.status != ROW_OK or token < 0:
        return float("nan")
    if res.greedy:
        return 0.0
    i = int(np.searchsorted(res.kept, token))
    assert i < len(res.kept) and int(res.kept[i]) == token, "token outside P"
    return float(np.log(res.q[i]))


def keep_mask_words(kept, V):
    """Packed keep mask for one row: uint32[ceil(V/32)], LSB-first."""
    W = (V + 31) // 32
    words = np.zeros(W, dtype=np.uint32)
    for i in np.asarray(kept, dtype=np.int64):
        words[i >> 5] |= np.uint32(1) << np.uint32(i & 31)
    return words


def argmax_row(z, legal=None):
    """Greedy selection without softmax or RNG: (status, token)."""
    z = np.asarray(z, dtype=np.float64)
    V = z.shape[0]
    if legal is None:
        legal = np.ones(V, dtype=bool)
    legal_ids = np.nonzero(legal)[0]
    if legal_ids.size == 0:
        return ROW_EMPTY, -1
    zl = z[legal_ids]
    if np.any(np.isnan(zl)) or np.any(zl == np.inf):
        return ROW_NONFINITE, -1
    fin = legal_ids[zl > -np.inf]
    if fin.size == 0:
        return ROW_ALL_NEG_INF, -1
    zf = z[fin]
    return ROW_OK, int(fin[np.nonzero(zf == zf.max())[0][0]])


def top_logprobs_row(ids, probs, count, cap, n):
    """The n most probable tokens of a candidate list and their log-probabilities
    under the final distribution (page "Sampling 系统设计：从 logits 到可控生成",
    logprobs section: besides the chosen token's log-probability a sampler may
    return the top tokens with theirs). Order: probability descending (the
    list's float32 values compared exactly), ties by ascending id. Returns
    (status, ids[n], logprobs[n]); slots past the list's length hold id -1 and
    -inf. A negative count is BAD_PARAM; a count above cap is a list the filter
    truncated, CAND_OVERFLOW (all slots -1 / -inf either way)."""
    out_i = np.full(n, -1, np.int64)
    out_l = np.full(n, -np.inf)
    if count < 0:
        return ROW_BAD_PARAM, out_i, out_l
    if count > cap:
        return ROW_CAND_OVERFLOW, out_i, out_l
    q = np.asarray(probs[:count], np.float32)
    t = np.asarray(ids[:count], np.int64)
    order = sorted(range(count), key=lambda i: (-float(q[i]), int(t[i])))[:n]
    for j, i in enumerate(order):
        out_i[j] = t[i]
        out_l[j] = np.log(np.float64(q[i])) if q[i] > 0 else -np.inf
    return ROW_OK, out_i, out_l
