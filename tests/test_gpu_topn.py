"""The top tokens written by the sampling launch itself (qs_sample_top_logprobs)
against the oracle's top_logprobs_row on the oracle's kept lists, and against
qs_top_logprobs run on the lists the same call wrote: ids bit for bit, log-
probabilities within 2e-6 absolute (the hardware log2), empty slots past the
list and for rows that are errors or whose list overflowed."""

import numpy as np
import pytest

import oracle
import workloads
from _harness import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qs():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import top_sampling_vocabs_amd as qs
    qs.load()
    return qs


@pytest.mark.parametrize("case", ["bf16_resident", "f32", "bf16_errors", "bf16_chunked",
                                  "bf16_switch", "small_lists", "overflow"])
@pytest.mark.parametrize("n", [1, 20, 64])
def test_top_n_in_launch(qs, case, n):
    import torch
    cfg, B, V = {"bf16_resident": (3, 24, 40000), "f32": (2, 16, 20000),
                 "bf16_errors": (5, 40, 9000), "bf16_chunked": (3, 6, 200000),
                 "bf16_switch": (3, 16, 30000), "small_lists": (1, 8, 6000),
                 "overflow": (3, 12, 30000)}[case]
    w = workloads.make(cfg, B=B, V=V, seed=1000 + n)
    if case == "small_lists":
        w.k[:] = np.arange(B) % 5 + 1          # lists of 1..5 entries (n exceeds some)
        w.p[:] = 1.0
    d = to_device(w)
    cap = 64 if case == "overflow" else V
    flags = qs.FLAG_STREAM if case == "bf16_switch" else 0
    uni = torch.from_numpy(np.random.default_rng(n).random(B)).cuda()
    ws = qs.workspace_for(d["logits"], cap) if case == "bf16_chunked" else None
    print(f"top-n {case} n={n} B={B} V={V}", flush=True)
    out = qs.sample(d["logits"], d["T"], d["k"], d["p"], d["bitmask"], uniforms=uni,
                    cand_cap=cap, flags=flags, top_n=n, workspace=ws)
    ref_i, ref_l, _ = qs.top_logprobs(out["cand_ids"], out["cand_probs"], out["cand_count"], n)
    torch.cuda.synchronize()
    st = out["status"].cpu().numpy()
    ti = out["top_ids"].cpu().numpy()
    tl = out["top_logprobs"].cpu().numpy()
    ri, rl = ref_i.cpu().numpy(), ref_l.cpu().numpy()
    cid = out["cand_ids"].cpu().numpy()
    cpr = out["cand_probs"].cpu().numpy()
    res = oracle.filter_batch(w.logits, w.dtype, w.T, w.k, w.p, w.bitmask)
    for r in range(B):
        if st[r] != oracle.ROW_OK:
            assert (ti[r] == -1).all() and np.isneginf(tl[r]).all(), (r, st[r], ti[r])
            continue
        # the same launch's lists, read by the separate kernel: identical slots
        assert np.array_equal(ti[r], ri[r]), (r, ti[r], ri[r])
        assert np.array_equal(tl[r].view(np.uint32), rl[r].view(np.uint32)), r
        # the oracle's kept set (the same ids as the list: the parity tests
        # check that) with the list's float32 probabilities, ordered by the
        # oracle's definition
        kept = res[r].kept
        assert np.array_equal(cid[r, :len(kept)], kept.astype(np.int32)), r
        q32 = cpr[r, :len(kept)]
        s_o, oi, ol = oracle.top_logprobs_row(kept, q32, len(kept), len(kept), n)
        assert s_o == oracle.ROW_OK
        assert np.array_equal(ti[r], oi.astype(np.int32)), (r, ti[r], oi)
        fin = np.isfinite(ol)
        assert np.array_equal(np.isfinite(tl[r]), fin)
        assert np.allclose(tl[r][fin], ol[fin], atol=2e-6, rtol=0), (r, tl[r], ol)
    if case == "overflow":
        assert (st == oracle.ROW_CAND_OVERFLOW).any()
    if case == "bf16_errors":
        assert (st != oracle.ROW_OK).any()


def test_top_n_arguments(qs):
    """top_n outside 1..64, or no candidate lists to read: refused before any
    launch."""
    import torch
    w = workloads.make(3, B=2, V=1000)
    d = to_device(w)
    uni = torch.zeros(2, dtype=torch.float64, device="cuda")
    for bad in (65, -1):
        with pytest.raises(RuntimeError):
            qs.sample(d["logits"], d["T"], d["k"], d["p"], d["bitmask"], uniforms=uni,
                      cand_cap=1000, top_n=bad)
    with pytest.raises(RuntimeError):   # the lists are the source: cand_cap required
        qs.sample(d["logits"], d["T"], d["k"], d["p"], d["bitmask"], uniforms=uni, top_n=5)
