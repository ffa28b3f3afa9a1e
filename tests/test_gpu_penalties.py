"""Parity of the in-place repetition / presence penalties (qs_apply_penalties,
through the C ABI) with the oracle: every logit of every row bit for bit, for
float32 and bfloat16 rows, histories with repeated and out-of-range ids, and
rows with invalid parameters; then the sampling path on the penalised rows
against the oracle's filter of the oracle's penalised rows."""

import numpy as np
import pytest

import oracle
import workloads
from _harness import Report, compare_filter, compare_tokens, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qs():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import top_sampling_vocabs_amd as qs
    qs.load()
    return qs


def _history(rng, B, V, cap):
    hist = rng.integers(0, V, (B, cap)).astype(np.int32)
    hist[:, 1::7] = hist[:, 0::7][:, :hist[:, 1::7].shape[1]]  # repeats
    hist[:, 5::11] = rng.choice([-3, V, V + 9], hist[:, 5::11].shape)  # out of range
    cnt = rng.integers(0, cap + 1, B).astype(np.int32)
    return hist, cnt


@pytest.mark.parametrize("freq_on", [False, True])
@pytest.mark.parametrize("cap", [600, 9000])  # one round held in registers; several rounds
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_penalties_bitwise(qs, dtype, cap, freq_on):
    import torch
    rng = np.random.default_rng(31 + (dtype == "bf16") + cap)
    B, V = 40, 20011
    z = rng.normal(0, 3, (B, V)).astype(np.float32)
    z[0, :50] = 0.0
    z[1, :50] = -0.0
    z[2, 10] = np.nan
    z[3, :20] = -np.inf
    if dtype == "bf16":
        host = (z.view(np.uint32) >> 16).astype(np.uint16)
        dev = torch.from_numpy(host.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        host = z
        dev = torch.from_numpy(z).cuda()
    hist, cnt = _history(rng, B, V, cap)
    hist[0, :40] = np.arange(40)
    hist[1, :40] = np.arange(40)
    hist[2, 0], hist[3, 0] = 10, 5
    cnt[:4] = 40
    rep = rng.choice([1.0, 1.2, 0.8, 2.5], B).astype(np.float32)
    pres = rng.choice([0.0, 0.5, -0.3], B).astype(np.float32)
    rep[5], pres[6], cnt[7] = 0.0, np.inf, cap + 1  # invalid rows
    rep[8] = np.nan
    # frequency penalties (sorted-history counts); with cap 9000 the rows over
    # 4096 entries and f != 0 are flagged
    freq = rng.choice([0.0, 0.1, -0.2, 0.05], B).astype(np.float32) if freq_on else None
    if freq_on:
        freq[9] = np.inf
    if cap > 4096:
        cnt[8:] = rng.integers(4097, cap + 1, B - 8)
    print(f"penalties {dtype} B={B} V={V} cap={cap} freq={freq_on}", flush=True)
    st = qs.apply_penalties(dev, torch.from_numpy(hist).cuda(), torch.from_numpy(cnt).cuda(),
                            torch.from_numpy(rep).cuda(), torch.from_numpy(pres).cuda(),
                            None if freq is None else torch.from_numpy(freq).cuda())
    torch.cuda.synchronize()
    want_st, want = oracle.apply_penalties_batch(host, dtype, hist, cnt, rep, pres, freq)
    assert np.array_equal(st.cpu().numpy(), want_st)
    got = dev.view(torch.int16).cpu().numpy().view(np.uint16) if dtype == "bf16" else \
        dev.cpu().numpy()
    bits = (lambda a: a.view(np.uint16)) if dtype == "bf16" else (lambda a: a.view(np.uint32))
    diff = np.argwhere(bits(got) != bits(want))
    assert len(diff) == 0, diff[:10]
    assert (want_st[[5, 6, 7, 8]] == oracle.ROW_BAD_PARAM).all()


def test_penalties_then_sample(qs):
    """The sampling path reads the penalised bf16 rows like any other: the kept
    sets and tokens match the oracle's filter of the oracle's penalised rows."""
    import torch
    w = workloads.make(3, B=24, V=9000)
    rng = np.random.default_rng(33)
    hist, cnt = _history(rng, w.B, w.V, 300)
    rep = np.full(w.B, 1.3, np.float32)
    pres = np.full(w.B, 0.4, np.float32)
    d = to_device(w)
    st = qs.apply_penalties(d["logits"], torch.from_numpy(hist).cuda(),
                            torch.from_numpy(cnt).cuda(), torch.from_numpy(rep).cuda(),
                            torch.from_numpy(pres).cuda())
    _, pen = oracle.apply_penalties_batch(w.logits, w.dtype, hist, cnt, rep, pres)
    w.logits = pen
    uni = rng.random(w.B)
    out = qs.sample(d["logits"], d["T"], d["k"], d["p"], d["bitmask"],
                    uniforms=torch.from_numpy(uni).cuda(), keep_mask=True, cand_cap=w.V,
                    dense=True)
    torch.cuda.synchronize()
    assert (st.cpu().numpy() == 0).all()
    res = oracle.filter_batch(w.logits, w.dtype, w.T, w.k, w.p, w.bitmask)
    rep_ = Report()
    compare_filter(w, res, out, range(w.B), rep_)
    compare_tokens(res, out["tokens"], range(w.B), rep_, uniforms=uni)
    rep_.check()


@pytest.mark.parametrize("cap", [700, 6000])  # one round held in registers; several rounds
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_logit_bias_bitwise(qs, dtype, cap):
    """Additive bias lists: every logit bit for bit against the oracle, with ids
    outside [0, V), rows listing a token twice, a non-finite value or a bad
    count (left unchanged and flagged)."""
    import torch
    rng = np.random.default_rng(41 + (dtype == "bf16") + cap)
    B, V = 24, 30011
    z = rng.normal(0, 3, (B, V)).astype(np.float32)
    if dtype == "bf16":
        host = (z.view(np.uint32) >> 16).astype(np.uint16)
        dev = torch.from_numpy(host.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        host = z
        dev = torch.from_numpy(z).cuda()
    ids = np.stack([rng.permutation(V + 50)[:cap] - 25 for _ in range(B)]).astype(np.int32)
    vals = rng.normal(0, 5, (B, cap)).astype(np.float32)
    cnt = rng.integers(0, cap + 1, B).astype(np.int32)
    cnt[:4] = cap
    ids[0, 7] = ids[0, 3] = 11          # a token listed twice
    vals[1, 5] = np.nan                 # a non-finite value
    cnt[2] = cap + 1                    # count beyond capacity
    ids[3, 9] = ids[3, 2] = V + 3       # a repeated id outside [0, V) is ignored
    print(f"logit bias {dtype} B={B} V={V}", flush=True)
    st = qs.apply_logit_bias(dev, torch.from_numpy(ids).cuda(), torch.from_numpy(vals).cuda(),
                             torch.from_numpy(cnt).cuda())
    torch.cuda.synchronize()
    want_st, want = oracle.apply_logit_bias_batch(host, dtype, ids, vals, cnt)
    assert np.array_equal(st.cpu().numpy(), want_st)
    assert (want_st[:3] == oracle.ROW_BAD_PARAM).all() and want_st[3] == oracle.ROW_OK
    got = dev.view(torch.int16).cpu().numpy().view(np.uint16) if dtype == "bf16" else \
        dev.cpu().numpy().view(np.uint32)
    ref = want.view(np.uint16) if dtype == "bf16" else want.view(np.uint32)
    diff = np.argwhere(got != ref)
    assert len(diff) == 0, diff[:10]


def _edited_workload(w, hist, hcnt, rep, pres, freq, bids, bvals, bcnt):
    """The oracle's composition: penalties, then the bias, on the host rows;
    a row either processor flags is BAD_PARAM for the fused call."""
    import dataclasses
    st_p, z1 = oracle.apply_penalties_batch(w.logits, w.dtype, hist, hcnt, rep, pres, freq)
    st_b, z2 = oracle.apply_logit_bias_batch(z1, w.dtype, bids, bvals, bcnt)
    bad = (st_p != oracle.ROW_OK) | (st_b != oracle.ROW_OK)
    return dataclasses.replace(w, logits=z2), bad


@pytest.mark.parametrize("case", ["bf16_resident", "bf16_switch", "f32", "bf16_greedy",
                                  "bf16_direct", "bf16_penalties_only", "bf16_direct_penalties"])
def test_processed_matches_oracle(qs, case):
    """qs_sample_processed / qs_filter_mask_processed: penalties and bias
    applied inside the call (the caller's logits untouched) give the outputs
    of the oracle's filter and draw on the oracle's edited rows (penalties,
    then bias), bit for bit for masks and lists; rows with invalid processor
    arguments (either processor's, or too many edited ids) are BAD_PARAM.
    bf16 rows held in registers patch the edited tokens in place; fp32 rows,
    switched runs and greedy rows are selected from an edited copy in the
    workspace. bf16_direct: every token legal and kept sets larger than the
    histogram path's per-wave pools (and flat rows with a negative boundary),
    so waves read their slices again: from the edited copy, not the caller's
    row."""
    import torch
    rng = np.random.default_rng({"bf16_resident": 1, "bf16_switch": 2, "f32": 3,
                                 "bf16_greedy": 4, "bf16_direct": 5, "bf16_penalties_only": 6,
                                 "bf16_direct_penalties": 7}[case])
    # (the *_penalties cases pass repetition and presence penalties alone: no
    # frequency penalty, no bias list)
    pen_only = case in ("bf16_penalties_only", "bf16_direct_penalties")
    dtype = "f32" if case == "f32" else "bf16"
    B, V = 24, (20000 if dtype == "f32" else 40000)
    w = workloads.make(3 if dtype == "bf16" else 2, B=B, V=V, seed=int(rng.integers(1 << 30)))
    if case == "bf16_greedy":
        w.T[::2] = 0.0
    if case in ("bf16_direct", "bf16_direct_penalties"):
        w.bitmask = None
        w.k[:] = 0
        w.T[:] = np.where(np.arange(B) % 2 == 0, 3.0, 1.0).astype(np.float32)
        w.p[:] = rng.choice([0.95, 0.99, 0.999], B).astype(np.float32)
        flat = (0.05 * rng.standard_normal((4, V))).astype(np.float32)
        w.logits[B - 4:] = workloads.f32_to_bf16_bits(flat)
    hist, hcnt = _history(rng, B, V, 700)
    rep = rng.choice([1.0, 1.3, 0.7, 2.0], B).astype(np.float32)
    pres = rng.choice([0.0, 0.4, -0.2], B).astype(np.float32)
    freq = rng.choice([0.0, 0.1, 0.5], B).astype(np.float32)
    bcap = 300
    bids = np.stack([rng.choice(V, bcap, replace=False) for _ in range(B)]).astype(np.int32)
    bids[:, ::17] = -5                              # out of range: ignored
    bvals = rng.normal(0, 2, (B, bcap)).astype(np.float32)
    if case != "bf16_direct":
        bvals[:, ::5] = 40.0                        # pushed to the top
    bcnt = rng.integers(0, bcap + 1, B).astype(np.int32)
    if pen_only:
        freq = np.zeros(B, np.float32)
        bcnt = np.zeros(B, np.int32)
    # invalid rows: a bad repetition penalty, a repeated bias id, a non-finite
    # bias (a bad presence penalty and a history count past the capacity for
    # the penalties alone)
    rep[3] = 0.0
    if pen_only:
        pres[4] = np.nan
        hcnt[5] = 701
    else:
        bids[4, 1] = bids[4, 0] if bids[4, 0] >= 0 else 7
        bids[4, 0] = bids[4, 1]
        bcnt[4] = max(bcnt[4], 2)
        bvals[5, 0] = np.inf
        bcnt[5] = max(bcnt[5], 1)
    ew, bad = _edited_workload(w, hist, hcnt, rep, pres, freq, bids, bvals, bcnt)
    d = to_device(w)
    before = d["logits"].clone()
    groups = (("history", hist), ("history_count", hcnt), ("repetition", rep),
              ("presence", pres))
    if not pen_only:
        groups += (("frequency", freq), ("bias_ids", bids), ("bias_values", bvals),
                   ("bias_count", bcnt))
    P = {k: torch.from_numpy(v).cuda() for k, v in groups}
    uni = np.random.default_rng(8).random(B)
    flags = qs.FLAG_STREAM if case == "bf16_switch" else 0
    out = qs.sample(d["logits"], d["T"], d["k"], d["p"], d["bitmask"],
                    uniforms=torch.from_numpy(uni).cuda(), keep_mask=True, cand_cap=V,
                    dense=True, debug=True, logprobs=True, flags=flags, processors=P)
    fm = qs.filter_mask(d["logits"], d["T"], d["k"], d["p"], d["bitmask"], cand_cap=V,
                        flags=flags, processors=P)
    torch.cuda.synchronize()
    assert torch.equal(before, d["logits"])        # the caller's logits are only read
    st = out["status"].cpu().numpy()
    assert (st[bad] == oracle.ROW_BAD_PARAM).all(), (np.nonzero(bad)[0], st[bad])
    assert bad[[3, 4, 5]].all()
    good = [r for r in range(B) if not bad[r]]
    res = oracle.filter_batch(ew.logits, ew.dtype, ew.T, ew.k, ew.p, ew.bitmask, rows=good)
    rep_ = Report()
    compare_filter(ew, res, out, good, rep_)
    compare_tokens(res, out["tokens"], good, rep_, uniforms=uni)
    rep_.check()
    assert np.array_equal(fm["keep_mask"].cpu().numpy(), out["keep_mask"].cpu().numpy())
    dbg = out["debug"].cpu().numpy()
    if case == "bf16_resident":
        assert (dbg[good, 0] == 0).all() and (dbg[good, 1] == 0).all(), dbg[good].tolist()
    if case in ("bf16_direct", "bf16_direct_penalties"):  # kept sets past the pools
        hist_path = (dbg[good, 0] == 0) & (dbg[good, 1] == 0)
        assert (hist_path & (dbg[good, 3] > 16 * 960)).sum() >= 4, dbg[good].tolist()


def test_processed_limits(qs):
    """The fused call's limits: a row with more than 4096 bias entries, or
    with more than 4096 history entries and a frequency penalty, is
    BAD_PARAM; a longer history without a frequency penalty is applied like
    any other (5,000 entries here) and matches the oracle."""
    import torch
    rng = np.random.default_rng(77)
    B, V = 4, 30000
    w = workloads.make(3, B=B, V=V)
    hist = np.stack([rng.permutation(V)[:5000] for _ in range(B)]).astype(np.int32)
    hcnt = np.array([5000, 5000, 100, 0], np.int32)
    rep = np.full(B, 1.5, np.float32)
    pres = np.full(B, 0.2, np.float32)
    freq = np.array([0.0, 0.1, 0.1, 0.0], np.float32)
    bids = np.stack([rng.permutation(V)[:5000] for _ in range(B)]).astype(np.int32)
    bvals = rng.normal(0, 1, bids.shape).astype(np.float32)
    bcnt = np.array([10, 0, 4096, 4097], np.int32)
    ew, bad = _edited_workload(w, hist, hcnt, rep, pres, freq, bids, bvals, bcnt)
    bad = bad | (bcnt > 4096)
    assert bad.tolist() == [False, True, False, True]
    d = to_device(w)
    P = {k: torch.from_numpy(v).cuda() for k, v in (
        ("history", hist), ("history_count", hcnt), ("repetition", rep), ("presence", pres),
        ("frequency", freq), ("bias_ids", bids), ("bias_values", bvals), ("bias_count", bcnt))}
    uni = np.random.default_rng(9).random(B)
    out = qs.sample(d["logits"], d["T"], d["k"], d["p"], d["bitmask"],
                    uniforms=torch.from_numpy(uni).cuda(), keep_mask=True, cand_cap=V,
                    dense=True, logprobs=True, processors=P)
    torch.cuda.synchronize()
    st = out["status"].cpu().numpy()
    assert (st[bad] == oracle.ROW_BAD_PARAM).all() and (st[~bad] != oracle.ROW_BAD_PARAM).all(), st
    good = [0, 2]
    res = oracle.filter_batch(ew.logits, ew.dtype, ew.T, ew.k, ew.p, ew.bitmask, rows=good)
    rep_ = Report()
    compare_filter(ew, res, out, good, rep_)
    compare_tokens(res, out["tokens"], good, rep_, uniforms=uni)
    rep_.check()
