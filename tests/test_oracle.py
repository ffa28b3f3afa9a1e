"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here calls the HIP path. Each test targets a mistake the oracle could
plausibly contain (wrong sort direction, wrong tie order, '>' instead of '>=',
top-p mass measured before top-k renormalisation, mask applied after top-k,
temperature as p^T instead of p^(1/T), dropped renormalisation, off-by-one in
the cut, NaN at an illegal position treated as an error, legal -inf kept).
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy import special, stats

import oracle
from oracle import exact_filter, brute_force_filter, filter_row, sample_from

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _examples():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


EXAMPLES = _examples()


# --- pages' worked examples, exact mode --------------------------------------

@pytest.mark.parametrize("ex", EXAMPLES, ids=[e["name"] for e in EXAMPLES])
def test_worked_example_exact(ex):
    probs = [Fraction(x) for x in ex["probs"]]
    kept, q = exact_filter(probs, k=ex["k"], p=Fraction(ex["p"]),
                           inv_t=ex["inv_t"], legal=ex["legal"])
    assert kept == ex["kept"]
    assert q == [Fraction(x) for x in ex["q"]]
    if "printed_q" in ex:  # the page prints 3 decimals
        assert np.allclose([float(x) for x in q], ex["printed_q"], atol=5e-4)
    if "not_kept" in ex:
        assert kept != ex["not_kept"]


@pytest.mark.parametrize("ex", EXAMPLES, ids=[e["name"] for e in EXAMPLES])
def test_worked_example_brute_force(ex):
    """The subset enumerator (no sort) agrees with the pages too."""
    w = [Fraction(x) ** ex["inv_t"] for x in ex["probs"]]
    kept, q = brute_force_filter(w, k=ex["k"], p=Fraction(ex["p"]), legal=ex["legal"])
    assert kept == ex["kept"]
    assert q == [Fraction(x) for x in ex["q"]]


def test_other_order_would_keep_two():
    """Top-p first on the full distribution keeps A/B (the page's counter-example),
    which our order must not produce."""
    probs = [Fraction(2, 5), Fraction(3, 10), Fraction(1, 5), Fraction(1, 10)]
    kept_p_first, _ = exact_filter(probs, k=0, p=Fraction(1, 2))
    assert kept_p_first == [0, 1]
    kept, q = exact_filter(probs, k=2, p=Fraction(1, 2))
    assert kept == [0] and q == [1]


@pytest.mark.parametrize("ex", EXAMPLES, ids=[e["name"] for e in EXAMPLES])
def test_worked_example_logits_fp64(ex):
    """The fp64 oracle on logits log(p) reproduces the printed probabilities.

    Exercise 7 lands exactly on the boundary (0.5+0.3+0.1 = 0.9). The contract
    passes p as float32, and float32(0.9) = 0.89999998 sits 2.4e-8 below it, so
    the logits path keeps the printed 3 tokens with a margin of that size; the
    3-token answer may also appear as an in-band alternative."""
    probs = np.array([float(Fraction(x)) for x in ex["probs"]])
    z = np.log(probs)
    T = 1.0 / ex["inv_t"]
    legal = None if ex["legal"] is None else np.array(ex["legal"])
    res = filter_row(z, T, ex["k"], float(Fraction(ex["p"])), legal)
    assert res.status == oracle.ROW_OK
    want_ids = ex["kept"]
    want_q = [float(Fraction(x)) for x in ex["q"]]
    options = [(list(res.kept), list(res.q))] + [(list(a), list(b)) for a, b in res.alternatives]
    ok = any(ids == want_ids and np.allclose(qq, want_q, rtol=1e-12, atol=0)
             for ids, qq in options)
    assert ok, (options, want_ids, want_q)
    if ex["name"] == "exercise7":
        assert res.margin < 1e-7


# --- empty set composition ----------------------------------------------------

def test_empty_set_composition():
    """Page 1 section 03: top-k=2 first, then a C/D-only constraint leaves no
    candidate. Composing the keep-mask of the first call with the constraint
    as a bitmask gives EMPTY; writing -inf outside the kept set and then
    applying the constraint gives ALL_NEG_INF. Both are explicit errors."""
    z = np.log(np.array([0.4, 0.3, 0.2, 0.1]))
    first = filter_row(z, 1.0, 2, 1.0)
    assert list(first.kept) == [0, 1]
    keep = oracle.keep_mask_words(first.kept, 4)
    constraint = oracle.keep_mask_words([2, 3], 4)
    both = oracle.legal_from_bitmask(keep & constraint, 4)
    assert filter_row(z, 1.0, 0, 1.0, both).status == oracle.ROW_EMPTY
    z2 = z.copy()
    z2[[2, 3]] = -np.inf
    assert filter_row(z2, 1.0, 0, 1.0, np.array([False, False, True, True])).status \
        == oracle.ROW_ALL_NEG_INF
    # and the correct order (mask first) is not empty
    res = filter_row(z, 1.0, 2, 1.0, np.array([False, False, True, True]))
    assert list(res.kept) == [2, 3]
    assert np.allclose(res.q, [2 / 3, 1 / 3], rtol=1e-12)


# --- statuses -------------------------------------------------------------------

def test_status_precedence_and_illegal_nan():
    z = np.array([0.0, np.nan, 1.0, -np.inf])
    # NaN at an illegal position is overwritten by -inf: OK
    r = filter_row(z, 1.0, 0, 1.0, np.array([True, False, True, True]))
    assert r.status == oracle.ROW_OK and list(r.kept) == [0, 2]
    # NaN at a legal position
    assert filter_row(z, 1.0, 0, 1.0).status == oracle.ROW_NONFINITE
    # +inf at a legal position
    z2 = np.array([0.0, np.inf, 1.0])
    assert filter_row(z2, 1.0, 0, 1.0).status == oracle.ROW_NONFINITE
    # nothing legal beats NaN: EMPTY first
    assert filter_row(z, 1.0, 0, 1.0, np.zeros(4, bool)).status == oracle.ROW_EMPTY
    # all legal logits -inf
    z3 = np.array([-np.inf, 5.0, -np.inf])
    assert filter_row(z3, 1.0, 0, 1.0, np.array([True, False, True])).status \
        == oracle.ROW_ALL_NEG_INF
    # the greedy path reports the same statuses
    assert oracle.argmax_row(z)[0] == oracle.ROW_NONFINITE
    assert oracle.argmax_row(z3, np.array([True, False, True]))[0] == oracle.ROW_ALL_NEG_INF


@pytest.mark.parametrize("T,k,p", [(-1.0, 0, 1.0), (np.nan, 0, 1.0), (np.inf, 0, 1.0),
                                   (1.0, -1, 1.0), (1.0, 0, 0.0), (1.0, 0, -0.5),
                                   (1.0, 0, 1.5), (1.0, 0, np.nan), (0.0, -3, 0.5)])
def test_bad_params(T, k, p):
    assert filter_row(np.zeros(5), T, k, p).status == oracle.ROW_BAD_PARAM


def test_legal_neg_inf_never_kept():
    z = np.array([1.0, -np.inf, 0.5, -np.inf])
    r = filter_row(z, 1.0, 10, 1.0)
    assert list(r.kept) == [0, 2]
    assert r.n_finite == 2


def test_bitmask_bit_order():
    """Token i is bit (i & 31) of word (i >> 5): ids 0, 31, 32 and 40."""
    words = np.array([0x80000001, 0x00000101], dtype=np.uint32)
    legal = oracle.legal_from_bitmask(words, 41)
    assert list(np.nonzero(legal)[0]) == [0, 31, 32, 40]
    assert (oracle.keep_mask_words([0, 31, 32, 40], 41) == words).all()


# --- greedy ----------------------------------------------------------------------

def test_greedy_is_first_argmax():
    rng = np.random.default_rng(1)
    for _ in range(50):
        z = rng.integers(-3, 3, size=17).astype(np.float64)
        legal = rng.random(17) < 0.7
        if not legal.any():
            continue
        ids = np.nonzero(legal)[0]
        want = int(ids[np.argmax(z[ids])])  # numpy returns the first maximum
        assert oracle.argmax_row(z, legal) == (oracle.ROW_OK, want)
        r = filter_row(z, 0.0, 5, 0.3, legal)
        assert r.greedy and list(r.kept) == [want] and list(r.q) == [1.0]


def test_small_temperature_limit_is_argmax():
    """T -> 0 concentrates the filtered distribution on the argmax (lecture page
    section 3.3)."""
    z = np.array([0.1, 2.0, 1.9, 2.0, -1.0])
    r = filter_row(z, 1e-4, 0, 1.0)
    top = r.q[list(r.kept).index(1)]
    assert top > 0.49 and r.q[list(r.kept).index(3)] > 0.49  # tie shares the mass
    r2 = filter_row(np.array([0.1, 2.0, 1.9, 1.0]), 1e-4, 0, 1.0)
    assert r2.q[1] == pytest.approx(1.0)


# --- special cases that reduce to library routines ------------------------------------

def test_no_truncation_is_softmax():
    rng = np.random.default_rng(2)
    for T in (0.5, 1.0, 1.7):
        z = rng.normal(size=300) * 2
        legal = rng.random(300) < 0.6
        r = filter_row(z, T, 0, 1.0, legal)
        ids = np.nonzero(legal)[0]
        want = special.softmax(z[ids] / np.float32(T).astype(np.float64))
        assert list(r.kept) == list(ids)
        assert np.allclose(r.q, want, rtol=1e-12, atol=0)


def test_topk_distinct_matches_argpartition():
    rng = np.random.default_rng(3)
    for _ in range(20):
        z = rng.normal(size=1000)
        k = int(rng.integers(1, 200))
        r = filter_row(z, 1.0, k, 1.0)
        want = np.sort(np.argpartition(-z, k - 1)[:k])
        assert list(r.kept) == list(want)
        assert np.allclose(r.q, special.softmax(z[want]), rtol=1e-12)


def test_topp_invariants():
    """Shortest prefix reaching p: the kept mass reaches p*W_K and dropping the
    least-ranked kept token falls below it; every kept token outranks every
    dropped one in (z desc, id asc); q sums to 1."""
    rng = np.random.default_rng(4)
    for _ in range(40):
        V = 500
        z = np.round(rng.normal(size=V) * 2, 1)  # many exact ties
        k = int(rng.integers(0, 300))
        p = float(np.float32(rng.uniform(0.05, 0.99)))
        r = filter_row(z, 1.0, k, p)
        if r.margin < 1e-9:
            continue
        kept = list(r.kept)
        rank = {i: j for j, i in enumerate(sorted(range(V), key=lambda i: (-z[i], i)))}
        Kset = sorted(range(V), key=lambda i: rank[i])[:r.k_size]
        dropped = [i for i in range(V) if i not in set(kept)]
        worst_kept = max(rank[i] for i in kept)
        assert all(rank[i] > worst_kept for i in dropped)
        wK = np.exp(z[Kset] - z.max())
        w = {i: math.exp(z[i] - z.max()) for i in range(V)}
        mass = sum(w[i] for i in kept)
        target = p * wK.sum()
        assert mass >= target * (1 - 1e-12)
        last = max(kept, key=lambda i: rank[i])
        assert mass - w[last] < target * (1 + 1e-12)
        assert abs(sum(r.q) - 1.0) < 1e-12
        assert len(kept) <= (k if k else V)


# --- brute force on tiny vocabularies -----------------------------------------------

def _exact_weights(z, T):
    m = max(x for x in z if x != -np.inf)
    return [Fraction(float(np.exp((x - m) / T))) if x != -np.inf else Fraction(0)
            for x in z]


def test_brute_force_tiny_rows():
    """Random V <= 8 rows with forced ties, -inf and masks: the sort-based fp64
    oracle and the sort-free subset enumerator agree on the kept set (rows whose
    top-p boundary lies within 1e-12 of the threshold are skipped: there the two
    only differ by fp64 summation order)."""
    rng = np.random.default_rng(5)
    checked = 0
    for _ in range(600):
        V = int(rng.integers(1, 9))
        z = rng.integers(-2, 3, size=V).astype(np.float64)
        z[rng.random(V) < 0.15] = -np.inf
        legal = rng.random(V) < 0.8
        k = int(rng.integers(0, V + 2))
        p = float(np.float32(rng.choice([1.0, rng.uniform(0.05, 1.0)])))
        T = float(np.float32(rng.choice([1.0, 0.5, 2.0])))
        r = filter_row(z, T, k, p, legal)
        zz = np.where(legal, z, -np.inf)
        if not legal.any():
            assert r.status == oracle.ROW_EMPTY
            continue
        if not np.isfinite(zz).any():
            assert r.status == oracle.ROW_ALL_NEG_INF
            continue
        assert r.status == oracle.ROW_OK
        if r.margin < 1e-12:
            continue
        w = _exact_weights(zz, np.float64(np.float32(T)))
        kept, q = brute_force_filter(w, k=k, p=Fraction(p))
        assert list(r.kept) == kept, (z, legal, k, p, T)
        assert np.allclose(r.q, [float(x) for x in q], rtol=1e-12)
        checked += 1
    assert checked > 300


def test_tie_keeps_earliest_ids():
    """Qrita key design 3: boundary duplicates keep the earliest token ids."""
    z = np.array([1.0, 3.0, 2.0, 2.0, 2.0, 2.0, 0.0])
    r = filter_row(z, 1.0, 3, 1.0)
    assert list(r.kept) == [1, 2, 3]
    r = filter_row(z, 1.0, 0, 0.6)
    # weights e^0, e^-1 x4 ...: mass order 1, then 2,3,4,5
    w = np.exp(z - 3.0)
    cum = np.cumsum(np.concatenate([[w[1]], w[2:6]]))
    n = int(np.searchsorted(cum, 0.6 * w.sum()) + 1)
    assert list(r.kept) == sorted([1, 2, 3, 4, 5][:n])


# --- sampling ----------------------------------------------------------------------

def test_cdf_walk_intervals_exact():
    """Right-open CDF in token-id order: for q = [4/9,3/9,2/9] on ids 0,1,2, u in
    [0,4/9) -> 0, [4/9,7/9) -> 1, [7/9,1) -> 2."""
    kept = np.array([0, 1, 2])
    q = np.array([4 / 9, 3 / 9, 2 / 9])
    assert sample_from(kept, q, 0.0)[0] == 0
    assert sample_from(kept, q, 0.4444)[0] == 0
    assert sample_from(kept, q, 0.4445)[0] == 1
    assert sample_from(kept, q, 0.7777)[0] == 1
    assert sample_from(kept, q, 0.7778)[0] == 2
    assert sample_from(kept, q, 0.999999)[0] == 2
    # u at or beyond a rounded total falls back to the last id with q > 0
    assert sample_from(np.array([3, 7, 9]), np.array([0.5, 0.5, 0.0]), 1.0)[0] == 7


def test_sampling_frequencies_match_q():
    """Over a uniform grid of u the CDF walk hits each kept id with frequency q
    (closed form P(token = i) = q_i)."""
    rng = np.random.default_rng(6)
    z = rng.normal(size=64) * 1.5
    r = filter_row(z, 0.8, 20, 0.9)
    n = 200000
    u = (np.arange(n) + 0.5) / n
    toks = [sample_from(r.kept, r.q, x)[0] for x in u]
    counts = np.array([toks.count(i) for i in r.kept]) / n
    assert np.allclose(counts, r.q, atol=2.0 / n + 1e-12)


def test_philox_uniform_statistics():
    """Statistical properties (the known-answer pin is in
    test_philox_rocrand.py): the generator's uniforms pass chi-square and independence checks, differ across seeds, and
    distinct counters give distinct outputs (Philox is a bijection)."""
    us = np.array([oracle.uniform(12345, off) for off in range(20000)])
    hist, _ = np.histogram(us, bins=40, range=(0, 1))
    assert stats.chisquare(hist).pvalue > 1e-4
    assert abs(np.corrcoef(us[:-1], us[1:])[0, 1]) < 0.03
    vs = np.array([oracle.uniform(seed, 0) for seed in range(20000)])
    hist, _ = np.histogram(vs, bins=40, range=(0, 1))
    assert stats.chisquare(hist).pvalue > 1e-4
    outs = {oracle.philox4x32((c, 0, 0, 0), (7, 9)) for c in range(4096)}
    assert len(outs) == 4096
    assert all(0.0 <= x < 1.0 for x in us)
    assert oracle.uniform(1, 2) != oracle.uniform(1, 3)
    assert oracle.uniform(1, 2) != oracle.uniform(2, 2)


def test_philox_round_is_invertible():
    """Each Philox round is a bijection of the 4-word block for a fixed round key
    (the multipliers are odd): undo one round by hand and recover the input."""
    rng = np.random.default_rng(7)
    M0, M1 = oracle.philox.PHILOX_M0, oracle.philox.PHILOX_M1
    inv0 = pow(M0, -1, 1 << 32)
    inv1 = pow(M1, -1, 1 << 32)
    for _ in range(200):
        c = [int(x) for x in rng.integers(0, 1 << 32, size=4, dtype=np.uint64)]
        key = [int(x) for x in rng.integers(0, 1 << 32, size=2, dtype=np.uint64)]
        o0, o1, o2, o3 = oracle.philox4x32(c, key, rounds=1)
        c0 = (o3 * inv0) & 0xFFFFFFFF
        c2 = (o1 * inv1) & 0xFFFFFFFF
        hi0 = (M0 * c0) >> 32
        hi1 = (M1 * c2) >> 32
        c1 = o0 ^ hi1 ^ key[0]
        c3 = o2 ^ hi0 ^ key[1]
        assert [c0, c1, c2, c3] == c


# --- batch layer -------------------------------------------------------------------

def test_batch_decodes_bf16_and_bitmask():
    import workloads
    w = workloads.make(3, B=6, V=1000)
    res = oracle.filter_batch(w.logits, "bf16", w.T, w.k, w.p, w.bitmask)
    for r in range(6):
        z = oracle.bf16_bits_to_float64(w.logits[r])
        legal = oracle.legal_from_bitmask(w.bitmask[r], 1000)
        assert np.array_equal(res[r].kept, filter_row(z, w.T[r], w.k[r], w.p[r], legal).kept)
        assert legal[res[r].kept].all()
    # bf16 decode is exact widening: 0x3F80 -> 1.0, 0xC040 -> -3.0, 0xFF80 -> -inf
    assert list(oracle.bf16_bits_to_float64(np.array([0x3F80, 0xC040, 0xFF80], np.uint16))) \
        == [1.0, -3.0, -np.inf]
    out = oracle.sample_batch(res, w.seeds, w.offsets)
    for r in range(6):
        tok, off, u, _ = out[r]
        if res[r].status == oracle.ROW_OK:
            assert tok in set(res[r].kept)
            assert off == 1


def test_topp_cut_reaching_p_exactly_fp64():
    """When the cumulative mass equals p * W_K exactly in fp64 the cut keeps that
    prefix ('reaching' p, lecture page exercise 7 answer). Equal logits give
    weights of exactly 1, and p = 0.25, 0.5, 0.75 are exact in float32."""
    z = np.zeros(4)
    for p, n in ((0.25, 1), (0.5, 2), (0.75, 3)):
        r = filter_row(z, 1.0, 0, p)
        assert list(r.kept) == list(range(n))
        assert np.allclose(r.q, [1.0 / n] * n)
    # same with a top-k cut first: k=3 of 6 equal tokens, p=2/3 is not exact in
    # float32, so use W_K = 4 (k=4) and p = 0.5 -> 2 tokens
    r = filter_row(np.zeros(6), 1.0, 4, 0.5)
    assert list(r.kept) == [0, 1]


def test_cdf_walk_right_open_on_exact_boundary():
    """u equal to a cumulative sum moves to the next token (right-open interval)."""
    kept = np.array([2, 5, 9])
    q = np.array([0.5, 0.25, 0.25])
    assert sample_from(kept, q, 0.5)[0] == 5
    assert sample_from(kept, q, 0.75)[0] == 9
    assert sample_from(kept, q, 0.0)[0] == 2


def test_signed_zeros_tie():
    """-0.0 and +0.0 compare equal, so they are a tie broken by token id."""
    z = np.array([-1.0, -0.0, 0.0, -0.0, -2.0])
    assert list(filter_row(z, 1.0, 1, 1.0).kept) == [1]
    assert list(filter_row(z, 1.0, 2, 1.0).kept) == [1, 2]
    assert oracle.argmax_row(z) == (oracle.ROW_OK, 1)


# --- the drawn token's log-probability ---------------------------------------

@pytest.mark.parametrize("ex", EXAMPLES, ids=[e["name"] for e in EXAMPLES])
def test_token_logprob_worked_examples(ex):
    """For every kept token of the pages' worked examples the log-probability
    is the log of the page's exact renormalised fraction."""
    probs = np.array([float(Fraction(x)) for x in ex["probs"]])
    legal = None if ex["legal"] is None else np.array(ex["legal"])
    res = filter_row(np.log(probs), 1.0 / ex["inv_t"], ex["k"], float(Fraction(ex["p"])), legal)
    for tok, qf in zip(ex["kept"], ex["q"]):
        want = np.log(float(Fraction(qf)))
        assert abs(oracle.token_logprob(res, tok) - want) < 1e-6


def test_token_logprob_log_softmax_without_truncation():
    """With top-k and top-p off the final distribution is the softmax of z/T
    over the legal tokens, so the log-probability is scipy's log-softmax."""
    from scipy.special import log_softmax
    rng = np.random.default_rng(11)
    z = rng.normal(0, 3, 300)
    legal = rng.random(300) < 0.6
    T = float(np.float32(0.7))  # the contract passes T as float32
    res = filter_row(z, T, 0, 1.0, legal)
    ls = log_softmax(z[legal] / T)
    ids = np.flatnonzero(legal)
    for j in (0, 17, 101, len(ids) - 1):
        assert abs(oracle.token_logprob(res, int(ids[j])) - ls[j]) < 1e-12


def test_token_logprob_uniform_and_degenerate():
    # k equal logits kept by top-k: each has probability 1/k
    res = filter_row(np.zeros(40), 1.0, 8, 1.0)
    assert abs(oracle.token_logprob(res, 3) + np.log(8)) < 1e-15
    # a single kept token: probability 1
    z = np.arange(20, dtype=np.float64)
    res = filter_row(z, 1.0, 1, 1.0)
    assert oracle.token_logprob(res, 19) == 0.0
    # greedy: a point mass
    res = filter_row(z, 0.0, 0, 1.0)
    assert res.greedy and oracle.token_logprob(res, 19) == 0.0
    # error rows: no token
    res = filter_row(np.full(20, np.nan), 1.0, 0, 1.0)
    assert np.isnan(oracle.token_logprob(res, -1))
    # the kept probabilities exponentiate back to one
    res = filter_row(np.random.default_rng(3).normal(0, 2, 500), 1.3, 60, 0.8)
    tot = sum(np.exp(oracle.token_logprob(res, int(t))) for t in res.kept)
    assert abs(tot - 1.0) < 1e-12


# --- exact speculative verification ------------------------------------------

def _dyadic_dist(rng, n, den=64):
    """n probabilities that are multiples of 1/den, summing to exactly 1, some 0."""
    cuts = np.sort(rng.choice(np.arange(1, den), n - 1, replace=True))
    w = np.diff(np.concatenate([[0], cuts, [den]])).astype(np.float64)
    return (w / den).astype(np.float32)


def _out_distribution(t_ids, t_p, d_ids, d_p, n_grid=512):
    """Output distribution of the verifier when x ~ q, u_accept and u_resample
    uniform: every x in the draft list weighted by q(x), both uniforms on a
    midpoint grid. Also returns the acceptance rate."""
    grid = (np.arange(n_grid) + 0.5) / n_grid
    out = {}
    acc_rate = 0.0
    for x, qx in zip(d_ids, d_p):
        if qx == 0.0:
            continue
        acc = 0
        for u1 in grid:
            st, tok, a, _ = oracle.spec_verify_row(t_ids, t_p, len(t_ids), len(t_ids), d_ids, d_p,
                                                   len(d_ids), len(d_ids), int(x), u1, 0.5)
            acc += a
        pa = acc / n_grid
        acc_rate += float(qx) * pa
        out[int(x)] = out.get(int(x), 0.0) + float(qx) * pa
        if pa < 1.0:
            for u2 in grid:
                st, tok, a, _ = oracle.spec_verify_row(t_ids, t_p, len(t_ids), len(t_ids), d_ids,
                                                       d_p, len(d_ids), len(d_ids), int(x), 0.999999,
                                                       u2)
                if a == 0:
                    out[tok] = out.get(tok, 0.0) + float(qx) * (1.0 - pa) / n_grid
    return out, acc_rate


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_spec_verify_output_is_target(seed):
    """The page's claim: accept-or-resample outputs exactly the target p, and the
    acceptance rate is sum(min(p, q)) = 1 - TV(p, q) (grid resolution 1/512)."""
    rng = np.random.default_rng(seed)
    V = 9
    ids = np.arange(V)
    p = _dyadic_dist(rng, V)
    q = _dyadic_dist(rng, V)
    t_keep = p > 0
    d_keep = q > 0
    out, acc = _out_distribution(ids[t_keep], p[t_keep], ids[d_keep], q[d_keep])
    for y in range(V):
        assert abs(out.get(y, 0.0) - float(p[y])) < 4.0 / 512, (y, out.get(y), p[y])
    assert abs(acc - float(np.minimum(p, q).sum())) < 2.0 / 512
    assert abs(acc - (1.0 - 0.5 * float(np.abs(p - q).sum()))) < 2.0 / 512


def test_spec_verify_lecture_exercise_3():
    """Lecture exercise 3 and its answer (page "第 9 讲 · 生成与推测解码",
    exercises): p = (0.5, 0.3, 0.2), q = (0.2, 0.5, 0.3) give the acceptance
    rate 0.7, a residual that renormalises to (1, 0, 0) (every rejection
    resamples token 0), and P(output 0) = 0.2 + 0.3 = 0.5 (grid 1/1000)."""
    ids = np.arange(3)
    p = np.array([0.5, 0.3, 0.2], np.float32)
    q = np.array([0.2, 0.5, 0.3], np.float32)
    out, acc = _out_distribution(ids, p, ids, q, n_grid=1000)
    assert abs(acc - 0.7) < 2e-3, acc
    for x in ids:
        for u2 in (0.0, 0.3, 0.77, 0.999):
            st, tok, a, _ = oracle.spec_verify_row(ids, p, 3, 3, ids, q, 3, 3, int(x), 0.999999,
                                                   u2)
            assert st == oracle.ROW_OK
            assert a == 1 or tok == 0, (x, u2, tok)   # residual (1, 0, 0)
    assert abs(out.get(0, 0.0) - 0.5) < 2e-3, out
    assert abs(out.get(1, 0.0) - 0.3) < 2e-3 and abs(out.get(2, 0.0) - 0.2) < 2e-3, out


def test_spec_verify_special_cases():
    ids = np.array([3, 7, 11, 20])
    p = np.array([0.5, 0.25, 0.125, 0.125], np.float32)
    # identical distributions: every draft token is accepted
    for x in ids:
        for u1 in (0.0, 0.5, 0.999):
            st, tok, a, _ = oracle.spec_verify_row(ids, p, 4, 4, ids, p, 4, 4, int(x), u1, 0.3)
            assert st == oracle.ROW_OK and a == 1 and tok == x
    # a draft token the target excludes is always rejected; the residual is
    # p - q where positive: here only id 3 (p 0.5 > q 0.25) and id 11
    q = np.array([0.25, 0.25, 0.0, 0.5], np.float32)   # id 11 has q 0 but is listed
    d_ids = ids
    t_ids = np.array([3, 7, 11])
    tp = np.array([0.5, 0.25, 0.25], np.float32)
    for u2, want in ((0.0, 3), (0.49, 3), (0.51, 11), (0.99, 11)):
        st, tok, a, _ = oracle.spec_verify_row(t_ids, tp, 3, 3, d_ids, q, 4, 4, 20, 0.0, u2)
        assert st == oracle.ROW_OK and a == 0 and tok == want, (u2, tok)
    # accept iff u * q(x) < p(x): x = 7, p = q = 0.25 always; x = 3 (p > q) always
    assert oracle.spec_verify_row(t_ids, tp, 3, 3, d_ids, q, 4, 4, 3, 0.999, 0.5)[2] == 1
    # errors
    assert oracle.spec_verify_row(t_ids, tp, 0, 3, d_ids, q, 4, 4, 3, 0.1, 0.1)[0] == oracle.ROW_EMPTY
    assert oracle.spec_verify_row(t_ids, tp, 3, 2, d_ids, q, 4, 4, 3, 0.1, 0.1)[0] == \
        oracle.ROW_CAND_OVERFLOW
    assert oracle.spec_verify_row(t_ids, tp, 3, 3, d_ids, q, 4, 4, 5, 0.1, 0.1)[0] == \
        oracle.ROW_BAD_PARAM
    assert oracle.spec_verify_row(t_ids, tp, 3, 3, d_ids, q, 4, 4, 3, 1.0, 0.1)[0] == \
        oracle.ROW_BAD_PARAM


# --- repetition / presence penalties ------------------------------------------

def test_penalties_hand_example():
    """Positive logits divide, negative multiply, then the presence penalty is
    subtracted; a repeated history token is penalised once; ids outside [0, V)
    are ignored; untouched tokens keep their bits."""
    z = np.array([2.0, -2.0, 1.0, 0.5, -0.0], np.float32)
    st, out = oracle.apply_penalties_row(z, "f32", np.array([0, 1, 0, 7, -1]), 5, 5, 2.0, 0.5)
    assert st == oracle.ROW_OK
    assert out.tolist() == [0.5, -4.5, 1.0, 0.5, -0.0]
    # the identity parameters change nothing
    st, out = oracle.apply_penalties_row(z, "f32", np.array([0, 1, 2, 3, 4]), 5, 5, 1.0, 0.0)
    assert np.array_equal(out.view(np.uint32), z.view(np.uint32))
    # count 0: nothing; bad parameters: unchanged and flagged
    assert np.array_equal(oracle.apply_penalties_row(z, "f32", np.array([0]), 0, 1, 2.0, 1.0)[1], z)
    for rep, pres, cnt in ((0.0, 0.0, 1), (-1.0, 0.0, 1), (np.nan, 0.0, 1), (1.0, np.inf, 1),
                           (1.0, 0.0, 2), (1.0, 0.0, -1)):
        st, out = oracle.apply_penalties_row(z, "f32", np.array([0]), cnt, 1, rep, pres)
        assert st == oracle.ROW_BAD_PARAM and np.array_equal(out, z)


def test_penalties_bf16_rounding():
    """bf16 rows: the float32 result is rounded to nearest even. 1.0 / 3 =
    0.33333334 lies between bf16 0.33203125 and 0.333984375, nearer the
    latter; -1.0 * 1.5 - 0.0 = -1.5 is exact."""
    z = np.array([0x3F80, 0xBF80], np.uint16)  # 1.0, -1.0
    st, out = oracle.apply_penalties_row(z, "bf16", np.array([0]), 1, 1, 3.0, 0.0)
    assert out[0] == 0x3EAB and out[1] == 0xBF80  # 0.333984375
    st, out = oracle.apply_penalties_row(z, "bf16", np.array([1]), 1, 1, 1.5, 0.0)
    assert out[1] == 0xBFC0  # -1.5
    # ties round to even: 1 + 2^-8 (bits 0x3F808000) -> 1.0, 1 + 3*2^-8 -> 1 + 2^-6
    assert oracle.penalties._to_bf16_bits(np.array([1 + 2**-8], np.float32))[0] == 0x3F80
    assert oracle.penalties._to_bf16_bits(np.array([1 + 3 * 2**-8], np.float32))[0] == 0x3F82


def test_logit_bias_hand_example():
    z = np.array([1.0, -2.0, 0.5, 3.0], np.float32)
    st, out = oracle.apply_logit_bias_row(z, "f32", np.array([2, 0, 9, -1]),
                                          np.array([-0.25, 4.0, 7.0, 1.0], np.float32), 4, 4)
    assert st == oracle.ROW_OK and out.tolist() == [5.0, -2.0, 0.25, 3.0]
    # only the first `count` entries apply
    st, out = oracle.apply_logit_bias_row(z, "f32", np.array([3, 1]), np.array([1.0, 1.0],
                                          np.float32), 1, 2)
    assert out.tolist() == [1.0, -2.0, 0.5, 4.0]
    # a token listed twice, a non-finite value, a bad count: unchanged and flagged
    for ids, vals, cnt in (([1, 1], [1.0, 2.0], 2), ([1, 2], [np.inf, 0.0], 2),
                           ([1, 2], [1.0, 1.0], 3), ([1, 2], [1.0, 1.0], -1)):
        st, out = oracle.apply_logit_bias_row(z, "f32", np.array(ids), np.array(vals, np.float32),
                                              cnt, 2)
        assert st == oracle.ROW_BAD_PARAM and np.array_equal(out, z)
    # bf16: 1.0 + 2^-9 rounds back to 1.0 (below half an ulp), 1.0 + 2^-7 is exact
    zb = np.array([0x3F80, 0x3F80], np.uint16)
    st, out = oracle.apply_logit_bias_row(zb, "bf16", np.array([0, 1]),
                                          np.array([2**-9, 2**-7], np.float32), 2, 2)
    assert out.tolist() == [0x3F80, 0x3F81]


def test_frequency_penalty_hand_example():
    """f times the number of occurrences, after the repetition and presence
    terms: id 0 occurs 3 times, id 1 once."""
    z = np.array([2.0, -2.0, 1.0], np.float32)
    st, out = oracle.apply_penalties_row(z, "f32", np.array([0, 1, 0, 0]), 4, 4, 2.0, 0.5, 0.25)
    assert st == oracle.ROW_OK
    assert out.tolist() == [2.0 / 2 - 0.5 - 0.75, -2.0 * 2 - 0.5 - 0.25, 1.0]
    # f = 0 is the plain repetition / presence result
    st, out0 = oracle.apply_penalties_row(z, "f32", np.array([0, 1, 0, 0]), 4, 4, 2.0, 0.5, 0.0)
    assert out0.tolist() == [0.5, -4.5, 1.0]
    # a non-finite f, or a history longer than the limit with f != 0, flags the row
    assert oracle.apply_penalties_row(z, "f32", np.array([0]), 1, 1, 1.0, 0.0, np.nan)[0] == \
        oracle.ROW_BAD_PARAM
    long_h = np.zeros(5000, np.int64)
    assert oracle.apply_penalties_row(z, "f32", long_h, 5000, 5000, 1.0, 0.0, 0.1)[0] == \
        oracle.ROW_BAD_PARAM
    assert oracle.apply_penalties_row(z, "f32", long_h, 5000, 5000, 1.0, 0.0, 0.0)[0] == \
        oracle.ROW_OK


def test_top_logprobs_worked_example():
    """The page's top-p example keeps A/B/C at 4/9, 3/9, 2/9: the top two are A
    and B with log(4/9) and log(1/3). Ties go to the lower id; slots past the
    list are (-1, -inf)."""
    probs = np.array([4 / 9, 3 / 9, 2 / 9], np.float32)
    st, ti, tl = oracle.top_logprobs_row(np.array([0, 1, 2]), probs, 3, 3, 2)
    assert st == oracle.ROW_OK and ti.tolist() == [0, 1]
    assert np.allclose(tl, np.log(probs[:2].astype(np.float64)))
    st, ti, tl = oracle.top_logprobs_row(np.array([3, 5, 9]), np.array([0.25, 0.5, 0.25],
                                         np.float32), 3, 3, 5)
    assert ti.tolist() == [5, 3, 9, -1, -1] and np.isneginf(tl[3:]).all()
    # a count above the capacity is a truncated list (the filter's overflow
    # status); a negative count is bad input
    assert oracle.top_logprobs_row(np.array([1]), np.array([1.0], np.float32), 2, 1, 1)[0] == \
        oracle.ROW_CAND_OVERFLOW
    assert oracle.top_logprobs_row(np.array([1]), np.array([1.0], np.float32), -1, 1, 1)[0] == \
        oracle.ROW_BAD_PARAM
    # against a brute-force ordering of a random list with many ties
    rng = np.random.default_rng(5)
    ids = np.sort(rng.choice(1000, 200, replace=False))
    pr = rng.choice([0.5, 0.25, 0.125, 0.0], 200).astype(np.float32)
    st, ti, tl = oracle.top_logprobs_row(ids, pr, 200, 200, 30)
    best = sorted(zip(-pr.astype(np.float64), ids))[:30]
    assert ti.tolist() == [int(b[1]) for b in best]
