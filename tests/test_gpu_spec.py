"""Parity of the speculative verifier (qs_spec_verify, through the C ABI) with
the oracle's exact rule. Target and draft candidate lists are made on the host
by the oracle's filter from seeded logits (the draft's logits are the target's
plus noise), so no input comes from the HIP path. Accept flags and statuses
are compared exactly; tokens exactly unless the resampling target lies within
1e-9 of a step of the cumulative residual (summation order)."""

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

STEP_BAND = 1e-9


def _lists(z, T, k, p, cap):
    """Oracle filter of each row -> (ids [B, cap] int32, probs float32, count)."""
    B = z.shape[0]
    ids = np.zeros((B, cap), np.int32)
    pr = np.zeros((B, cap), np.float32)
    cnt = np.zeros(B, np.int32)
    for r in range(B):
        res = oracle.filter_row(z[r].astype(np.float64), T[r], k[r], p[r])
        n = len(res.kept)
        assert n <= cap
        ids[r, :n] = res.kept
        pr[r, :n] = res.q.astype(np.float32)
        cnt[r] = n
    return ids, pr, cnt


def _case(rng, B, V, sigma, noise, ks, ps):
    z_t = rng.normal(0, sigma, (B, V)).astype(np.float32)
    z_d = (z_t + rng.normal(0, noise, (B, V))).astype(np.float32)
    T = rng.choice([0.7, 1.0, 1.3], B).astype(np.float32)
    k = rng.choice(ks, B).astype(np.int32)
    p = rng.choice(ps, B).astype(np.float32)
    ti, tp, tc = _lists(z_t, T, k, p, V)
    di, dp, dc = _lists(z_d, T, k, p, V)
    # draft tokens drawn from the draft lists
    x = np.array([oracle.sample_from(di[r, :dc[r]], dp[r, :dc[r]].astype(np.float64),
                                     rng.random())[0] for r in range(B)], np.int32)
    u1 = rng.random(B)
    u1[::3] = 0.999999  # force rejections where p(x) < q(x)
    u2 = rng.random(B)
    return dict(ti=ti, tp=tp, tc=tc, di=di, dp=dp, dc=dc, x=x, u1=u1, u2=u2)


def _run_and_compare(qs, c):
    import torch
    dev = "cuda"
    g = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in c.items()}
    out = qs.spec_verify(g["ti"], g["tp"], g["tc"], g["di"], g["dp"], g["dc"], g["x"],
                         g["u1"], g["u2"])
    torch.cuda.synchronize()
    tok = out["tokens"].cpu().numpy()
    acc = out["accepted"].cpu().numpy()
    st = out["status"].cpu().numpy()
    want = oracle.spec_verify_batch(c["ti"], c["tp"], c["tc"], c["di"], c["dp"], c["dc"],
                                    c["x"], c["u1"], c["u2"])
    n_rej = band = 0
    for r, (ws, wt, wa, dist) in want.items():
        assert st[r] == ws, (r, st[r], ws)
        assert acc[r] == wa, (r, acc[r], wa)
        n_rej += ws == oracle.ROW_OK and wa == 0
        if tok[r] != wt:
            assert dist < STEP_BAND, (r, tok[r], wt, dist)
            band += 1
    return n_rej, band


@pytest.fixture(scope="module")
def qs():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import top_sampling_vocabs_amd as qs
    qs.load()
    return qs


def test_spec_verify_parity(qs):
    rng = np.random.default_rng(21)
    c = _case(rng, B=48, V=6000, sigma=3.0, noise=1.0, ks=[0, 20, 200], ps=[1.0, 0.9, 0.6])
    print("spec verify B=48 V=6000", flush=True)
    n_rej, band = _run_and_compare(qs, c)
    assert n_rej >= 8, n_rej  # the residual draw is exercised
    assert band <= 1


def test_spec_verify_long_draft_list(qs):
    """Draft lists longer than the LDS stage (16384 entries): q is looked up in
    memory instead."""
    rng = np.random.default_rng(22)
    c = _case(rng, B=6, V=40000, sigma=0.2, noise=0.2, ks=[0], ps=[0.99])
    assert (c["dc"] > 16384).all()
    c["u1"][:] = 0.999999
    print("spec verify long lists B=6 V=40000", flush=True)
    n_rej, band = _run_and_compare(qs, c)
    assert n_rej >= 3 and band <= 1


def test_spec_verify_row_errors(qs):
    rng = np.random.default_rng(23)
    c = _case(rng, B=8, V=3000, sigma=2.0, noise=0.5, ks=[50], ps=[1.0])
    c["dc"][0] = 0                       # empty draft list
    c["tc"][1] = 0                       # empty target list
    c["tc"][2] = c["ti"].shape[1] + 1    # count beyond capacity
    c["u1"][3] = 1.0                     # uniform outside [0, 1)
    c["dc"][4] = -2                      # negative count
    absent = np.setdiff1d(np.arange(3000), c["di"][5, :c["dc"][5]])[0]
    c["x"][5] = absent                   # x is not in the draft list
    # identical lists: always accepted
    c["di"][6], c["dp"][6], c["dc"][6] = c["ti"][6], c["tp"][6], c["tc"][6]
    c["x"][6] = c["ti"][6, 0]
    c["u1"][6] = 0.999999
    _run_and_compare(qs, c)
