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
