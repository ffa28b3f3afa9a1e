"""Parity of qs_top_logprobs (through the C ABI) with the oracle: the n most
probable tokens of candidate lists made by the oracle's filter on the host (no
input from the HIP path). Ids exactly (float32 probabilities compared exactly,
ties by id); log-probabilities within 1e-6 + 1.2e-7 |logprob|."""

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qs():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import top_sampling_vocabs_amd as qs
    qs.load()
    return qs


# (n, cap): n <= 64 with cap <= 16384 takes the register path (per-wave top n,
# then one wave merges them; lanes sort their keys first from n = 16 on); the
# others the block-wide rounds
@pytest.mark.parametrize("n,cap", [(1, 9000), (15, 9000), (16, 9000), (20, 9000), (64, 9000),
                                   (65, 9000),
                                   (20, 17000), (700, 9000)])
def test_top_logprobs_parity(qs, n, cap):
    import torch
    w = workloads.make(3, B=24, V=9000)
    res = oracle.filter_batch(w.logits, w.dtype, w.T, w.k, w.p, w.bitmask)
    ids = np.zeros((w.B, cap), np.int32)
    pr = np.zeros((w.B, cap), np.float32)
    cnt = np.zeros(w.B, np.int32)
    for r, rr in res.items():
        m = len(rr.kept)
        ids[r, :m] = rr.kept
        pr[r, :m] = rr.q.astype(np.float32)
        cnt[r] = m
    pr[3, :cnt[3]] = np.float32(1.0 / max(cnt[3], 1))  # one row of exact ties
    cnt[5] = cap + 1                                     # a truncated list
    cnt[6] = -1                                          # a bad count
    print(f"top logprobs n={n} cap={cap}", flush=True)
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    ti, tl, st = qs.top_logprobs(g(ids), g(pr), g(cnt), n)
    torch.cuda.synchronize()
    ti, tl, st = ti.cpu().numpy(), tl.cpu().numpy().astype(np.float64), st.cpu().numpy()
    for r in range(w.B):
        ws, wi, wl = oracle.top_logprobs_row(ids[r], pr[r], int(cnt[r]), cap, n)
        assert st[r] == ws, r
        assert np.array_equal(ti[r], wi), (r, ti[r][:8], wi[:8])
        fin = np.isfinite(wl)
        assert np.array_equal(np.isfinite(tl[r]), fin), r
        assert (np.abs(tl[r][fin] - wl[fin]) <= 1e-6 + 1.2e-7 * np.abs(wl[fin])).all(), r
