"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Masks and candidate ids are compared bit-exactly; probabilities within 1e-6
relative (floor 2^-126); tokens exactly for the same u unless u lies within
1e-6 of a CDF step; statuses and RNG offsets exactly. Rows whose top-p cut sits
within 1e-9 * W_K of the threshold may keep the adjacent prefix (counted).
"""

import numpy as np
import pytest

import oracle
import workloads
from _harness import (Report, compare_filter, compare_logprobs, compare_tokens, to_device,
                      words_u32)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qs():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import top_sampling_vocabs_amd as qs
    qs.load()
    return qs


def run_all(qs, d, uniforms=None, flags=0, cand_cap=None, V=None):
    import torch
    cap = cand_cap if cand_cap is not None else V
    out = qs.sample(d["logits"], d["T"], d["k"], d["p"], d["bitmask"],
                    seed=d["seed"], offset=d["offset"], uniforms=uniforms,
                    keep_mask=True, cand_cap=cap, dense=True, debug=True, logprobs=True,
                    flags=flags)
    torch.cuda.synchronize()
    return out


def check_workload(qs, w, rows=None, seed=0, flags=0, cand_cap=None, dense=True):
    import torch
    rows = list(range(w.B)) if rows is None else rows
    d = to_device(w)
    uni = np.random.default_rng(seed).random(w.B)
    uni_t = torch.from_numpy(uni).cuda()
    out = run_all(qs, d, uniforms=uni_t, flags=flags, cand_cap=cand_cap, V=w.V)
    res = oracle.filter_batch(w.logits, w.dtype, w.T, w.k, w.p, w.bitmask, rows=rows)
    rep = Report()
    compare_filter(w, res, out, rows, rep, check_dense=dense)
    compare_tokens(res, out["tokens"], rows, rep, uniforms=uni)
    compare_logprobs(res, out["tokens"], out["logprobs"], out["cand_count"], rows, rep)
    # filter_mask gives the same mask and lists
    fm = qs.filter_mask(d["logits"], d["T"], d["k"], d["p"], d["bitmask"],
                        cand_cap=cand_cap or w.V, flags=flags)
    torch.cuda.synchronize()
    assert np.array_equal(words_u32(fm["keep_mask"]), words_u32(out["keep_mask"]))
    assert np.array_equal(fm["cand_count"].cpu().numpy(), out["cand_count"].cpu().numpy())
    rep.check()
    return rep, out


SMALL = {1: dict(B=4, V=32000), 2: dict(B=24, V=20000), 3: dict(B=48, V=9000),
         4: dict(B=24, V=16384), 5: dict(B=100, V=9000)}


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_parity_small(qs, cfg):
    w = workloads.make(cfg, **SMALL[cfg])
    print(f"workload {cfg} B={w.B} V={w.V}", flush=True)
    rep, out = check_workload(qs, w, seed=cfg)
    assert rep.band_rows <= max(1, w.B // 50)


@pytest.mark.parametrize("stream", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 2, 5, 31, 33, 100, 511, 513, 1000, 5003, 8193, 40000])
def test_parity_ragged(qs, dtype, V, stream):
    """Odd vocabulary sizes (ragged final step, partial mask word, V < one wave
    step), many exact ties (rounded logits), -inf, and every parameter mode;
    rows held in registers and rows streamed through the prefetch ring."""
    import torch
    rng = np.random.default_rng(V * 7 + (dtype == "bf16"))
    B = 36
    z = np.round(rng.normal(size=(B, V)) * 2, 1).astype(np.float32)
    z[rng.random((B, V)) < 0.02] = -np.inf
    bits = rng.random((B, V)) < rng.uniform(0.2, 1.0, size=(B, 1))
    bits[np.arange(B), rng.integers(0, V, size=B)] = True
    k = rng.integers(0, max(2, V + 3), size=B).astype(np.int32)
    k[::4] = 0
    p = rng.uniform(0.05, 1.0, size=B).astype(np.float32)
    p[1::5] = 1.0
    T = rng.uniform(0.3, 2.0, size=B).astype(np.float32)
    T[2::9] = 0.0
    es = 2 if dtype == "bf16" else 4
    stride = -(-V // (16 // es)) * (16 // es)
    if dtype == "bf16":
        logits = np.zeros((B, stride), np.uint16)
        logits[:, :V] = workloads.f32_to_bf16_bits(z)
    else:
        logits = np.zeros((B, stride), np.float32)
        logits[:, :V] = z
    w = workloads.Workload(cfg=0, dtype=dtype, logits=logits, T=T, k=k, p=p,
                           bitmask=workloads.pack_bits(bits),
                           seeds=np.arange(B, dtype=np.uint64),
                           offsets=np.zeros(B, np.uint64))
    d = to_device(w)
    d["logits"] = d["logits"][:, :V]  # row stride stays padded
    w.logits = logits[:, :V]
    uni = rng.random(B)
    out = run_all(qs, d, uniforms=torch.from_numpy(uni).cuda(), V=V,
                  flags=qs.FLAG_STREAM if stream else 0)
    res = oracle.filter_batch(w.logits, dtype, T, k, p, w.bitmask)
    rep = Report()
    compare_filter(w, res, out, range(B), rep)
    compare_tokens(res, out["tokens"], range(B), rep, uniforms=uni)
    compare_logprobs(res, out["tokens"], out["logprobs"], out["cand_count"], range(B), rep)
    rep.check()


def test_path_invariance(qs):
    """Forced fallback and no truncation run every search over the full row; the
    pivot-search switch replaces the histogram scan by the quaternary search;
    the stream switch reads the row through the prefetch ring instead of the
    register-resident pass; the binary-pivot switch searches with one pivot per
    round. Every variant gives bitwise identical outputs (page "Qrita" ablation
    runs D to G compute the same result as run A)."""
    import torch
    variants = (qs.FLAG_FORCE_MISS, qs.FLAG_NO_TRUNCATION, qs.FLAG_PIVOT_SEARCH,
                qs.FLAG_STREAM, qs.FLAG_STREAM | qs.FLAG_PIVOT_SEARCH,
                qs.FLAG_BINARY_PIVOT | qs.FLAG_PIVOT_SEARCH,
                qs.FLAG_BINARY_PIVOT | qs.FLAG_FORCE_MISS)
    for cfg in (1, 2, 3, 5):
        w = workloads.make(cfg, **SMALL[cfg])
        d = to_device(w)
        uni = torch.from_numpy(np.random.default_rng(9).random(w.B)).cuda()
        base = run_all(qs, d, uniforms=uni, V=w.V)
        for flags in variants:
            print(f"workload {cfg} flags {flags}", flush=True)
            alt = run_all(qs, d, uniforms=uni, flags=flags, V=w.V)
            for key in ("keep_mask", "cand_count", "dense", "tokens", "status"):
                assert torch.equal(base[key], alt[key]), (cfg, flags, key)
            assert lists_equal(base, alt), (cfg, flags)
            # log q in fp64 from either path's weights, rounded to float32
            assert np.allclose(base["logprobs"].cpu().numpy(), alt["logprobs"].cpu().numpy(),
                               rtol=2.4e-7, atol=1e-9, equal_nan=True), (cfg, flags)
            dbg = alt["debug"].cpu().numpy()
            ok = base["status"].cpu().numpy() == 0
            if flags in (qs.FLAG_FORCE_MISS, qs.FLAG_NO_TRUNCATION,
                         qs.FLAG_BINARY_PIVOT | qs.FLAG_FORCE_MISS):
                assert (dbg[ok, 0] == 1).all()  # every OK row took the full-row path
            if flags == qs.FLAG_BINARY_PIVOT | qs.FLAG_FORCE_MISS:
                # one pivot per round never needs fewer rounds than three
                quad = run_all(qs, d, uniforms=uni, flags=qs.FLAG_FORCE_MISS, V=w.V)
                qr = quad["debug"].cpu().numpy()[ok, 1]
                assert (dbg[ok, 1] >= qr).all(), (cfg, dbg[ok, 1], qr)


SWITCHES = ("FLAG_FORCE_MISS", "FLAG_NO_TRUNCATION", "FLAG_PIVOT_SEARCH", "FLAG_STREAM",
            "FLAG_BINARY_PIVOT", "FLAG_SORT_SUBSET")


@pytest.mark.parametrize("switch", SWITCHES)
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_switches_match_oracle(qs, cfg, switch):
    """Every ablation switch (page "Qrita", ablation table: runs B, D, E, F, G,
    I and the page's own design, Q) against the oracle directly, on every
    workload at reduced size: masks, lists, probabilities, tokens and
    statuses, to the same tolerances as the normal path."""
    w = workloads.make(cfg, **SMALL[cfg])
    flags = getattr(qs, switch)
    if switch == "FLAG_BINARY_PIVOT":
        flags |= qs.FLAG_PIVOT_SEARCH
    print(f"workload {cfg} switch {switch}", flush=True)
    rep, out = check_workload(qs, w, seed=31 + cfg, flags=flags)
    dbg = out["debug"].cpu().numpy()
    ok = out["status"].cpu().numpy() == 0
    if switch in ("FLAG_FORCE_MISS", "FLAG_NO_TRUNCATION"):
        assert (dbg[ok, 0] == 1).all(), np.bincount(dbg[ok, 0])  # searched the full row


def lists_equal(a, b):
    """Candidate lists agree on their first cand_count entries (the rest of each
    row is not written)."""
    cnt = a["cand_count"].cpu().numpy()
    cap = a["cand_ids"].shape[1]
    ia, ib = a["cand_ids"].cpu().numpy(), b["cand_ids"].cpu().numpy()
    pa = a["cand_probs"].cpu().numpy().view(np.uint32)
    pb = b["cand_probs"].cpu().numpy().view(np.uint32)
    for r in range(len(cnt)):
        n = min(int(cnt[r]), cap)
        if not (np.array_equal(ia[r, :n], ib[r, :n]) and np.array_equal(pa[r, :n], pb[r, :n])):
            return False
    return True


def test_determinism(qs):
    import torch
    w = workloads.make(5, **SMALL[5])
    d = to_device(w)
    a = qs.sample(d["logits"], d["T"], d["k"], d["p"], d["bitmask"], seed=d["seed"],
                  offset=d["offset"].clone(), keep_mask=True, cand_cap=4096, dense=True)
    b = qs.sample(d["logits"], d["T"], d["k"], d["p"], d["bitmask"], seed=d["seed"],
                  offset=d["offset"].clone(), keep_mask=True, cand_cap=4096, dense=True)
    torch.cuda.synchronize()
    for key in ("tokens", "status", "keep_mask", "cand_count", "dense"):
        assert torch.equal(a[key], b[key]), key
    assert lists_equal(a, b)


def test_philox_stream_and_offsets(qs):
    """Tokens drawn from the library's own Philox match the oracle's Philox walk;
    sampled rows advance their offset by exactly one, greedy and error rows not
    at all; a second call continues the stream from the advanced offsets."""
    import torch
    w = workloads.make(5, **SMALL[5])
    w.T[3] = 0.0
    w.offsets[:] = np.random.default_rng(3).integers(0, 1 << 40, size=w.B).astype(np.uint64)
    d = to_device(w)
    res = oracle.filter_batch(w.logits, w.dtype, w.T, w.k, w.p, w.bitmask)
    off0 = w.offsets.copy()
    for call in range(2):
        before = d["offset"].cpu().numpy().view(np.uint64).copy()
        out = qs.sample(d["logits"], d["T"], d["k"], d["p"], d["bitmask"],
                        seed=d["seed"], offset=d["offset"])
        torch.cuda.synchronize()
        after = d["offset"].cpu().numpy().view(np.uint64).copy()
        rep = Report()
        compare_tokens(res, out["tokens"], range(w.B), rep, offsets_in=before,
                       offsets_out=after, seeds=w.seeds)
        rep.check()
    sampled = np.array([res[r].status == 0 and not res[r].greedy for r in range(w.B)])
    assert np.array_equal(after - off0, np.where(sampled, 2, 0).astype(np.uint64))


def test_sampling_statistics(qs):
    """One filtered row replicated with distinct seeds: token frequencies match
    the oracle's q (chi-square with bins pooled to expectation >= 5, and total
    variation within the finite-sample scale)."""
    import torch
    from scipy import stats
    rng = np.random.default_rng(11)
    V = 3000
    z = (rng.normal(size=V) * 1.5).astype(np.float32)
    n = 20000
    logits = torch.from_numpy(np.tile(z, (n, 1))).cuda()
    T = torch.full((n,), 0.8, dtype=torch.float32, device="cuda")
    k = torch.full((n,), 200, dtype=torch.int32, device="cuda")
    p = torch.full((n,), 0.9, dtype=torch.float32, device="cuda")
    seed = torch.arange(n, dtype=torch.int64, device="cuda") * 7919 + 5
    offset = torch.zeros(n, dtype=torch.int64, device="cuda")
    out = qs.sample(logits, T, k, p, seed=seed, offset=offset)
    torch.cuda.synchronize()
    toks = out["tokens"].cpu().numpy()
    rr = oracle.filter_row(z.astype(np.float64), 0.8, 200, 0.9)
    assert set(np.unique(toks)) <= set(rr.kept.tolist())
    counts = np.array([(toks == i).sum() for i in rr.kept], dtype=np.float64)
    expect = rr.q * n
    order = np.argsort(expect)
    obs_b, exp_b, acc_o, acc_e = [], [], 0.0, 0.0
    for i in order:
        acc_o += counts[i]
        acc_e += expect[i]
        if acc_e >= 5:
            obs_b.append(acc_o)
            exp_b.append(acc_e)
            acc_o = acc_e = 0.0
    if acc_e > 0:
        obs_b[-1] += acc_o
        exp_b[-1] += acc_e
    pval = stats.chisquare(obs_b, exp_b).pvalue
    assert pval > 1e-4, pval
    tv = 0.5 * np.abs(counts / n - rr.q).sum()
    # finite-sample TV scale ~ sum_i sqrt(q_i (1-q_i) / n) * sqrt(2/pi) / 2
    scale = 0.5 * np.sqrt(2 / np.pi) * np.sqrt(rr.q * (1 - rr.q) / n).sum()
    assert tv < 1.5 * scale + 0.005, (tv, scale)


def test_argmax_parity(qs):
    import torch
    for cfg in (1, 2, 3, 5):
        w = workloads.make(cfg, **SMALL[cfg])
        d = to_device(w)
        tok, st = qs.argmax(d["logits"], d["bitmask"])
        torch.cuda.synchronize()
        want = oracle.argmax_batch(w.logits, w.dtype, w.bitmask)
        for r in range(w.B):
            assert (st[r].item(), tok[r].item()) == want[r], (cfg, r)


def test_argmax_ties_and_specials(qs):
    import torch
    z = np.array([[1.0, 3.0, 3.0, 2.0],
                  [np.nan, 0.0, 1.0, 1.0],
                  [-np.inf, -np.inf, -np.inf, -np.inf],
                  [0.0, np.inf, 1.0, 2.0],
                  [5.0, 5.0, 5.0, 5.0],
                  [-1.0, -1.0, -3.0, -0.5]], np.float32)
    zz = np.zeros((6, 8), np.float32)
    zz[:, :4] = z
    bits = np.ones((6, 4), bool)
    bits[1, 0] = False      # NaN at an illegal position is fine
    bits[3, 1] = False      # so is +inf
    bits[5, 3] = False
    t = torch.from_numpy(zz).cuda()[:, :4]
    bm = torch.from_numpy(workloads.pack_bits(bits).view(np.int32)).cuda()
    tok, st = qs.argmax(t, bm)
    torch.cuda.synchronize()
    assert st.cpu().tolist() == [0, 0, 2, 0, 0, 0]
    assert tok.cpu().tolist() == [1, 2, -1, 3, 0, 0]


def test_error_rows_and_bad_params(qs):
    import torch
    V = 700
    B = 10
    rng = np.random.default_rng(5)
    z = rng.normal(size=(B, V)).astype(np.float32)
    bits = np.ones((B, V), bool)
    bits[0] = False                    # EMPTY
    z[1, 17] = np.nan                  # NONFINITE
    z[2] = -np.inf                     # ALL_NEG_INF
    z[3, 5] = np.inf                   # NONFINITE (+inf)
    z[4, 9] = np.nan
    bits[4, 9] = False                 # NaN at an illegal position: OK
    T = np.ones(B, np.float32)
    k = np.full(B, 20, np.int32)
    p = np.full(B, 0.9, np.float32)
    T[5] = -1.0                        # BAD_PARAM
    k[6] = -2                          # BAD_PARAM
    p[7] = 1.5                         # BAD_PARAM
    p[8] = 0.0                         # BAD_PARAM
    T[9] = np.nan                      # BAD_PARAM
    w = workloads.Workload(cfg=0, dtype="f32", logits=z, T=T, k=k, p=p,
                           bitmask=workloads.pack_bits(bits),
                           seeds=np.arange(B, dtype=np.uint64), offsets=np.zeros(B, np.uint64))
    d = to_device(w)
    out = run_all(qs, d, V=V)
    st = out["status"].cpu().tolist()
    assert st == [1, 3, 2, 3, 0, 4, 4, 4, 4, 4]
    off = d["offset"].cpu().numpy()
    assert off.tolist() == [0, 0, 0, 0, 1, 0, 0, 0, 0, 0]
    tok = out["tokens"].cpu().numpy()
    assert (tok[[0, 1, 2, 3, 5, 6, 7, 8, 9]] == -1).all()
    res = oracle.filter_batch(z, "f32", T, k, p, w.bitmask)
    rep = Report()
    compare_filter(w, res, out, range(B), rep)
    rep.check()


def test_candidate_overflow(qs):
    import torch
    w = workloads.make(3, B=12, V=9000)
    d = to_device(w)
    out = qs.sample(d["logits"], d["T"], d["k"], d["p"], d["bitmask"],
                    uniforms=torch.full((w.B,), 0.5, dtype=torch.float64, device="cuda"),
                    keep_mask=True, cand_cap=8)
    torch.cuda.synchronize()
    res = oracle.filter_batch(w.logits, w.dtype, w.T, w.k, w.p, w.bitmask)
    rep = Report()
    compare_filter(w, res, out, range(w.B), rep)
    rep.check()
    st = out["status"].cpu().numpy()
    assert (st == 5).sum() == sum(len(res[r].kept) > 8 for r in range(w.B))


@pytest.mark.slow
@pytest.mark.parametrize("cfg,rows", [(1, None), (2, None), (3, 24), (4, 12), (5, 24)])
def test_parity_full_size(qs, cfg, rows):
    """Full-size workloads in the launch configuration the bench times; the
    oracle checks a seeded sample of rows (all rows for the small workloads)."""
    w = workloads.make(cfg)
    print(f"full workload {cfg} B={w.B} V={w.V}", flush=True)
    if rows is None:
        pick = list(range(w.B))
    else:
        pick = sorted(np.random.default_rng(cfg).choice(w.B, size=rows, replace=False).tolist())
        if cfg == 4:  # every row kind
            pick = sorted(set(pick) | {0, 1, 2})
        if cfg == 5:  # include every degenerate row
            empty = np.nonzero(~w.bitmask.any(axis=1))[0]
            ninf = np.nonzero((w.logits == 0xFF80).all(axis=1))[0]
            nan = np.nonzero(((w.logits & 0x7FFF) > 0x7F80).any(axis=1))[0]
            pick = sorted(set(pick) | set(empty[:4].tolist()) | set(ninf.tolist())
                          | set(nan.tolist()))
    rep, out = check_workload(qs, w, rows=pick, seed=100 + cfg, cand_cap=8192, dense=False)
    dbg = out["debug"].cpu().numpy()
    if w.dtype == "bf16":
        # 151936-token bf16 rows are held in registers by the per-row kernel:
        # nearly all are settled by the value histogram (no search rounds)
        assert (dbg[:, 0] != 2).all(), np.bincount(dbg[:, 0])
        assert (dbg[:, 1] == 0).mean() > 0.95, np.bincount(dbg[:, 1])
    if cfg == 4:
        # near-flat rows hit the truncated pool; bimodal and heavy-tail rows fall back
        kinds = np.arange(w.B) % 3
        assert (dbg[kinds == 0, 0] == 0).mean() > 0.9
        # radix select: at most four 8-bit levels per search
        assert dbg[:, 1].max() <= 8, np.bincount(dbg[:, 1])
        # rows that miss search the full row for top-k, then go on with the top-k set
        assert (dbg[kinds != 0, 0] == 3).mean() > 0.9, np.bincount(dbg[kinds != 0, 0])


@pytest.mark.parametrize("B,V", [(32, 262144), (12, 200000)])
def test_parity_long_bf16_rows(qs, B, V):
    """bf16 rows longer than the per-row kernel's register tiers take the
    chunked first pass (workspace) and the per-row merge; the rows it declines
    take the per-row kernel's streamed paths. Both must match the oracle on a
    sample of rows (every row kind of the headline mix)."""
    w = workloads.make(3, B=B, V=V)
    print(f"long bf16 rows B={w.B} V={w.V}", flush=True)
    pick = sorted(np.random.default_rng(V).choice(w.B, size=min(w.B, 9), replace=False).tolist())
    pick = sorted(set(pick) | {0, 1, 2})
    rep, out = check_workload(qs, w, rows=pick, seed=7, cand_cap=16384, dense=False)
    dbg = out["debug"].cpu().numpy()
    assert (dbg[:, 0] == 2).mean() > 0.3, np.bincount(dbg[:, 0])   # the chunked path ran


@pytest.mark.parametrize("cfg", [3, 2])
def test_parity_rows_past_16bit_slices(qs, cfg):
    """Rows of more than 2^20 tokens (the longest the tests take): each wave's
    slice then holds more than 65536 tokens, so the candidate pools (16-bit
    offsets) are not used and every search runs over the whole row; bf16 rows
    of this length also skip the chunked pass. Masks, lists, dense
    probabilities and tokens must match the oracle (bf16: top-k, top-p and both;
    fp32: top-k with top-p and a greedy row)."""
    # (a row length whose rows start on 16-byte boundaries; not a multiple of
    # a wave step)
    w = workloads.make(cfg, B=4, V=(1 << 20) + 4136)
    print(f"rows past 16-bit slices cfg={cfg} B={w.B} V={w.V} {w.dtype}", flush=True)
    check_workload(qs, w, seed=11, cand_cap=w.V, dense=True)


@pytest.mark.parametrize("cfg", [5, 2])
def test_parity_many_rows(qs, cfg):
    """A batch of 66,000 short rows: a launch grid past 65,535 workgroups (one
    per row) and per-row offsets past 2^22 elements. Rows sampled across the
    batch, the first and last among them, must match the oracle (bf16: the
    mixed batch with error rows; fp32: top-k / top-p rows and greedy rows)."""
    w = workloads.make(cfg, B=66000, V=72)
    print(f"many rows cfg={cfg} B={w.B} V={w.V} {w.dtype}", flush=True)
    rng = np.random.default_rng(cfg)
    pick = sorted(set(rng.choice(w.B, size=240, replace=False).tolist()) | {0, 1, w.B - 2, w.B - 1})
    check_workload(qs, w, rows=pick, seed=13, dense=True)


def test_topp_background_extremes(qs):
    """Rows with top-k off whose background (legal tokens below the truncation
    threshold) lies outside the exact bf16 value bins: values of magnitude
    >= 512 or below 2^-12, exact zeros, legal -inf, +inf, and very large or
    very small temperatures. Their mass test and top-p cut go through the error
    bound and, where it is too wide, the exact fp64 walk or the full row; every
    output must still match the oracle."""
    rng = np.random.default_rng(77)
    B, V = 14, 9000
    z = (3.0 * rng.standard_normal((B, V))).astype(np.float32)
    T = np.ones(B, np.float32)
    p = np.full(B, 0.9, np.float32)
    z[0] += 1000.0                      # background >= 512 above zero
    z[1] -= 1000.0                      # background <= -512
    z[2] *= 1e-4                        # most values below 2^-12
    z[3, rng.random(V) < 0.5] = 0.0     # exact zeros
    z[4, rng.random(V) < 0.2] = -np.inf # legal -inf
    z[5, 17] = np.inf                   # +inf at a legal position
    T[6] = 50.0                         # nearly flat weights
    T[7] = 0.05                         # sharply peaked weights
    p[8], p[9], p[10] = 0.999, 0.01, 0.5
    z[11, :40] = 600.0                  # ties far above the rest
    z[12] = np.where(rng.random(V) < 0.5, 600.0, -600.0)
    T[13], z[13] = 0.5, z[13] * 1e-3    # tiny values, small temperature
    bits = workloads._random_bitmask(rng, B, V, 0.3)
    bits[5, 17] = True
    w = workloads.Workload(cfg=3, dtype="bf16", logits=workloads.f32_to_bf16_bits(z),
                           T=T, k=np.zeros(B, np.int32), p=p,
                           bitmask=workloads.pack_bits(bits),
                           seeds=np.arange(B, dtype=np.uint64),
                           offsets=np.zeros(B, np.uint64))
    rep, out = check_workload(qs, w, seed=5)
    st = out["status"].cpu().numpy()
    assert st[5] == oracle.ROW_NONFINITE
    dbg = out["debug"].cpu().numpy()
    # candidate keys spanning more than the 1024-key histogram: some rows are
    # settled by the radix select on the pool (two 8-bit levels of the bf16
    # key per search), and the pivot rounds the ablation switches keep
    # settle the same rows identically
    assert (dbg[:, 1] >= 2).any(), dbg.tolist()
    d = to_device(w)
    pv = qs.filter_mask(d["logits"], d["T"], d["k"], d["p"], d["bitmask"], cand_cap=w.V,
                        debug=True, flags=qs.FLAG_PIVOT_SEARCH)
    fm = qs.filter_mask(d["logits"], d["T"], d["k"], d["p"], d["bitmask"], cand_cap=w.V,
                        debug=True)
    import torch
    torch.cuda.synchronize()
    assert np.array_equal(words_u32(pv["keep_mask"]), words_u32(fm["keep_mask"]))
    assert (pv["debug"].cpu().numpy()[:, 1] >= 3).any()


@pytest.mark.gpu
def test_small_temperature_large_logits(qs):
    """bf16 rows with logits in the upper exact binades (spacing 1 and 2) and
    temperatures down to 0.001: the weights (v - m) / T of values above the
    maximum would overflow, so the value-histogram path must start the run
    that holds the maximum at the maximum. Every row is settled by that path
    (no search rounds) and must match the oracle."""
    rng = np.random.default_rng(91)
    B, V = 12, 9000
    z = (300.0 + 20.0 * rng.standard_normal((B, V))).astype(np.float32)
    z[6:] = (450.0 + 15.0 * rng.standard_normal((6, V))).astype(np.float32)
    z = np.minimum(z, 510.0)
    T = np.array([0.001, 0.005, 0.02, 0.1, 0.001, 0.02] * 2, np.float32)
    k = np.array([0, 5, 50, 0, 3, 0, 0, 7, 0, 100, 1, 0], np.int32)
    p = np.array([0.9, 1.0, 0.5, 0.99, 0.7, 0.3, 0.95, 1.0, 0.6, 0.8, 1.0, 0.999],
                 np.float32)
    bits = workloads._random_bitmask(rng, B, V, 0.5)
    w = workloads.Workload(cfg=3, dtype="bf16", logits=workloads.f32_to_bf16_bits(z),
                           T=T, k=k, p=p, bitmask=workloads.pack_bits(bits),
                           seeds=np.arange(B, dtype=np.uint64),
                           offsets=np.zeros(B, np.uint64))
    rep, out = check_workload(qs, w, seed=6)
    assert (out["status"].cpu().numpy() == 0).all()
    dbg = out["debug"].cpu().numpy()
    assert (dbg[:, 1] == 0).all(), dbg.tolist()


@pytest.mark.gpu
def test_histogram_pool_overflow_direct(qs):
    """bf16 rows whose kept set is larger than the value-histogram path's
    pools (every token legal, a large temperature and p close to 1, a
    positive boundary value): the waves whose pools overflow emit their
    outputs from a second read of their slice, so these rows stay on the
    histogram path (no search rounds) like the rows with a small kept set,
    and so does a flat row whose boundary is negative. All must match the
    oracle: lists, masks, dense probabilities and tokens."""
    rng = np.random.default_rng(123)
    B, V = 6, 40000
    z = (3.0 * rng.standard_normal((B, V))).astype(np.float32)
    z[:2] += 20.0
    z[2] = (0.05 * rng.standard_normal(V)).astype(np.float32)
    T = np.array([3.0, 3.0, 1.0, 1.0, 1.0, 1.0], np.float32)
    k = np.zeros(B, np.int32)
    p = np.array([0.99, 0.95, 0.999, 0.5, 0.9, 0.7], np.float32)
    bits = np.ones((B, V), bool)
    w = workloads.Workload(cfg=3, dtype="bf16", logits=workloads.f32_to_bf16_bits(z),
                           T=T, k=k, p=p, bitmask=workloads.pack_bits(bits),
                           seeds=np.arange(B, dtype=np.uint64),
                           offsets=np.zeros(B, np.uint64))
    rep, out = check_workload(qs, w, seed=8, cand_cap=65536)
    dbg = out["debug"].cpu().numpy()
    assert (dbg[:, 0] == 0).all() and (dbg[:, 1] == 0).all(), dbg.tolist()
    assert (dbg[:3, 3] > 16 * 960).all(), dbg.tolist()   # kept sets larger than the pools


@pytest.mark.gpu
def test_topk_rank_among_zero_logits(qs):
    """bf16 rows holding a few positive logits and thousands of exact zeros,
    with k between the count of non-zero logits and the count of legal tokens:
    the k-th largest value is 0, which the value histogram does not rank, so
    those rows must leave that path and still match the oracle (top-k alone
    and top-k followed by top-p). Ordinary top-k rows run first in the same
    launch (more rows than compute units), so a workgroup that ran one of them
    left its selection in LDS before a zero row reuses the unit."""
    rng = np.random.default_rng(4242)
    B, V = 600, 9000
    z = (3.0 * rng.standard_normal((B, V))).astype(np.float32)
    k = rng.integers(20, 200, size=B).astype(np.int32)
    p = np.ones(B, np.float32)
    zero_rows = np.arange(320, B)
    for r in zero_rows:
        z[r] = 0.0
        pos = rng.choice(V, size=10, replace=False)
        z[r, pos] = rng.uniform(0.5, 4.0, size=10)
        neg = rng.choice(V, size=50, replace=False)
        z[r, neg] = -rng.uniform(0.5, 4.0, size=50)
        k[r] = rng.integers(11, 2000)
        p[r] = 1.0 if r % 2 else rng.uniform(0.3, 0.99)
    bits = workloads._random_bitmask(rng, B, V, 0.6)
    w = workloads.Workload(cfg=3, dtype="bf16", logits=workloads.f32_to_bf16_bits(z),
                           T=np.ones(B, np.float32), k=k, p=p,
                           bitmask=workloads.pack_bits(bits),
                           seeds=np.arange(B, dtype=np.uint64),
                           offsets=np.zeros(B, np.uint64))
    rows = list(range(0, 320, 16)) + zero_rows.tolist()
    rep, out = check_workload(qs, w, rows=rows, seed=12, cand_cap=V, dense=False)
    assert (out["status"].cpu().numpy()[zero_rows] == 0).all()


def test_histogram_far_and_negative_boundaries(qs):
    """bf16 rows whose top-k or top-p boundary value is negative (a large
    temperature with p close to 1, or k above half the legal tokens), or lies
    more than 2,048 values below the maximum (log-uniform magnitudes): the
    value-histogram path builds the weights of every rank down to the
    boundary and reads the row again for its outputs, so these rows stay on
    that path (no search rounds). A row with exact zeros between the signs
    leaves it for the truncation path. All must match the oracle."""
    rng = np.random.default_rng(2024)
    B, V = 8, 40000
    z = (3.0 * rng.standard_normal((B, V))).astype(np.float32)
    z[3] = np.exp2(rng.uniform(-12, 8, V)).astype(np.float32)
    z[4, rng.random(V) < 0.2] = 0.0
    T = np.array([1.5, 1.0, 1.0, 1000.0, 1.5, 1.44, 1.0, 1.0], np.float32)
    k = np.array([0, 30000, 25000, 0, 0, 0, 50, 0], np.int32)
    p = np.array([0.99, 1.0, 0.95, 0.9, 0.99, 0.989, 1.0, 0.9], np.float32)
    bits = np.ones((B, V), bool)
    bits[5] = rng.random(V) < 0.3
    bits[5, 0] = True
    w = workloads.Workload(cfg=3, dtype="bf16", logits=workloads.f32_to_bf16_bits(z),
                           T=T, k=k, p=p, bitmask=workloads.pack_bits(bits),
                           seeds=np.arange(B, dtype=np.uint64),
                           offsets=np.zeros(B, np.uint64))
    rep, out = check_workload(qs, w, seed=12, cand_cap=V)
    dbg = out["debug"].cpu().numpy()
    on_path = [0, 1, 2, 3, 5, 6, 7]
    assert (dbg[on_path, 0] == 0).all() and (dbg[on_path, 1] == 0).all(), dbg.tolist()
    assert dbg[4, 1] >= 1 or dbg[4, 0] != 0, dbg.tolist()   # zeros between the signs


def test_histogram_huge_negative_logits(qs):
    """bf16 rows holding a few huge negative logits among ordinary ones (a
    logit bias of -1000, legal -inf tokens, values below -512): their weights
    are below 2^-60 of the row's mass, so the value-histogram path leaves them
    out of its sums and keeps these rows (no search rounds), top-k and top-p
    alike; a large temperature, which gives them weight, sends the row to the
    truncation path; a legal negative NaN is a row error. All must match the
    oracle."""
    rng = np.random.default_rng(99)
    B, V = 10, 30000
    z = (3.0 * rng.standard_normal((B, V))).astype(np.float32)
    for r in range(B):
        ids = rng.choice(V, size=12, replace=False)
        z[r, ids[:6]] = -1000.0
        z[r, ids[6:9]] = -np.inf
        z[r, ids[9:]] = -600.0
    T = np.array([1.0, 1.0, 0.7, 1.3, 1.0, 1.0, 1.0, 400.0, 1.0, 1.0], np.float32)
    k = np.array([50, 0, 200, 0, 20, 0, 1000, 0, 0, 0], np.int32)
    p = np.array([1.0, 0.9, 0.95, 0.99, 0.8, 0.5, 0.9, 0.9, 0.97, 0.9], np.float32)
    bits = rng.random((B, V)) < 0.3
    for r in range(B):
        bits[r, np.nonzero(z[r] < -500)[0]] = True   # the outliers are legal
    w = workloads.Workload(cfg=3, dtype="bf16", logits=workloads.f32_to_bf16_bits(z),
                           T=T, k=k, p=p, bitmask=workloads.pack_bits(bits),
                           seeds=np.arange(B, dtype=np.uint64),
                           offsets=np.zeros(B, np.uint64))
    w.logits[9, int(np.nonzero(bits[9])[0][5])] = 0xFFC1   # a legal negative NaN
    rep, out = check_workload(qs, w, seed=4, cand_cap=V)
    dbg = out["debug"].cpu().numpy()
    st = out["status"].cpu().numpy()
    assert st[9] == oracle.ROW_NONFINITE
    on_path = [0, 1, 2, 3, 4, 5, 6, 8]
    assert (dbg[on_path, 0] == 0).all() and (dbg[on_path, 1] == 0).all(), dbg.tolist()


@pytest.mark.gpu
def test_histogram_error_rows(qs):
    """bf16 error rows: no legal token (EMPTY) and a legal +inf (NONFINITE),
    which the value-histogram path reports itself, and rows whose every legal
    value is -inf (ALL_NEG_INF, also with NaN at illegal positions), which
    the truncation path reports. Rows mixing -inf with finite negative values
    or -0 are not errors. Statuses, zeroed outputs and tokens must match the
    oracle."""
    rng = np.random.default_rng(2024)
    B, V = 8, 30000
    z = (3.0 * rng.standard_normal((B, V))).astype(np.float32)
    bits = rng.random((B, V)) < 0.3
    bits[0] = False                                   # EMPTY
    z[1, np.nonzero(bits[1])[0][3]] = np.inf          # NONFINITE
    z[2] = -np.inf                                    # ALL_NEG_INF
    z[3, bits[3]] = -np.inf                           # ALL_NEG_INF (legal ones only)
    z[3, np.nonzero(~bits[3])[0][:5]] = np.nan
    z[4] = -np.inf
    z[4, np.nonzero(bits[4])[0][7]] = -3.0            # one finite legal value: not an error
    z[5] = -np.inf
    z[5, np.nonzero(bits[5])[0][2]] = -0.0            # -0 among -inf: not an error
    z[6] = -np.abs(z[6]) - 1.0                        # all negative: not an error
    T = np.ones(B, np.float32)
    k = np.full(B, 40, np.int32)
    p = np.full(B, 0.9, np.float32)
    w = workloads.Workload(cfg=3, dtype="bf16", logits=workloads.f32_to_bf16_bits(z),
                           T=T, k=k, p=p, bitmask=workloads.pack_bits(bits),
                           seeds=np.arange(B, dtype=np.uint64),
                           offsets=np.zeros(B, np.uint64))
    rep, out = check_workload(qs, w, seed=6, cand_cap=V)
    st = out["status"].cpu().numpy()
    assert st[:4].tolist() == [oracle.ROW_EMPTY, oracle.ROW_NONFINITE, oracle.ROW_ALL_NEG_INF,
                               oracle.ROW_ALL_NEG_INF], st.tolist()
    assert (st[4:] == oracle.ROW_OK).all(), st.tolist()
    dbg = out["debug"].cpu().numpy()
    assert (dbg[:2] == 0).all(), dbg.tolist()        # reported by the histogram path
