"""Exact-arithmetic modes of the oracle: rational weights and brute force.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module.

* ``exact_filter`` runs the contract on probabilities given as fractions, the
  way the pages print their worked examples (page "Attention算完，还没有选出下一个token",
  sections 02 and 03; lecture page "第 9 讲 · 生成与推测解码", exercises 7 and 8).
  Temperature T = 1/n (n a positive integer) is applied as p_i ** n and then
  renormalised (lecture page, section 3.3: temperature is p^(1/T) renormalised),
  so every number stays rational and a cut that lands exactly on p is decided
  exactly.
* ``brute_force_filter`` finds the same sets without any sorting, by enumerating
  subsets of a tiny vocabulary: top-k is the unique subset of size min(k, |F|)
  that beats every outsider in (weight, then lower id); top-p is, among subsets
  of K whose mass reaches p * W_K, one of minimum size, then maximum mass, then
  lexicographically smallest ids. It pins the sort-based definition from
  outside.
"""

from fractions import Fraction
from itertools import combinations


def _weights(probs, inv_t):
    return [Fraction(x) ** inv_t for x in probs]


def exact_filter(probs, k=0, p=Fraction(1), inv_t=1, legal=None):
    """Contract on rational probabilities. Returns (kept ids ascending, q list)
    or (None, None) for an empty legal set.

    probs: sequence of Fractions (original probabilities, temperature 1).
    inv_t: 1/T as a positive integer (T = 1, 1/2, 1/3, ...).
    """
    n = len(probs)
    legal = [True] * n if legal is None else list(legal)
    w = _weights(probs, inv_t)
    F = [i for i in range(n) if legal[i] and w[i] > 0]
    if not F:
        return None, None
    # descending weight, ascending id among equals
    pi = sorted(F, key=lambda i: (-w[i], i))
    kk = len(pi) if (k == 0 or k >= len(pi)) else k
    K = pi[:kk]
    wk = sum(w[i] for i in K)
    p = Fraction(p)
    if p < 1:
        target = p * wk
        acc = Fraction(0)
        P = []
        for i in K:
            P.append(i)
            acc += w[i]
            if acc >= target:
                break
    else:
        P = K
    wp = sum(w[i] for i in P)
    kept = sorted(P)
    return kept, [w[i] / wp for i in kept]


def _beats(w, i, j):
    return w[i] > w[j] or (w[i] == w[j] and i < j)


def brute_force_filter(w, k=0, p=Fraction(1), legal=None):
    """Enumerate subsets of a tiny vocabulary (len(w) <= 12) with exact weights.

    w: list of non-negative exact weights (Fraction or int); weight 0 means -inf.
    Returns (kept ids ascending, q list) or (None, None) for an empty F.
    """
    n = len(w)
    legal = [True] * n if legal is None else list(legal)
    F = [i for i in range(n) if legal[i] and w[i] > 0]
    if not F:
        return None, None
    kk = len(F) if (k == 0 or k >= len(F)) else k
    K = None
    for S in combinations(F, kk):
        rest = [j for j in F if j not in S]
        if all(_beats(w, i, j) for i in S for j in rest):
            if K is not None:
                raise AssertionError("top-k set is not unique")
            K = list(S)
    wk = sum((Fraction(w[i]) for i in K), Fraction(0))
    p = Fraction(p)
    if p < 1:
        target = p * wk
        best = None
        for size in range(1, kk + 1):
            cands = []
            for S in combinations(sorted(K), size):
                m = sum((Fraction(w[i]) for i in S), Fraction(0))
                if m >= target:
                    cands.append((m, S))
            if cands:
                top = max(m for m, _ in cands)
                best = min(S for m, S in cands if m == top)
                break
        P = list(best)
    else:
        P = K
    wp = sum((Fraction(w[i]) for i in P), Fraction(0))
    kept = sorted(P)
    return kept, [Fraction(w[i]) / wp for i in kept]
