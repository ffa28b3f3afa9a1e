"""qs_sample_noalloc (the library's fixed per-GPU scratch) against qs_sample
(a caller workspace): the same kernels, so every output must be identical,
on two calls in a row, the second one smaller than the first."""

import numpy as np
import pytest

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


def _same(a, b, name):
    a = a.cpu().numpy()
    b = b.cpu().numpy()
    assert a.dtype == b.dtype and a.shape == b.shape, name
    assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), name


def _both(qs, w, cand_cap):
    import torch
    d = to_device(w)
    off_ws = d["offset"].clone()
    off_na = d["offset"].clone()
    kw = dict(keep_mask=True, cand_cap=cand_cap, debug=True, logprobs=True)
    ref = qs.sample(d["logits"], d["T"], d["k"], d["p"], d["bitmask"], seed=d["seed"],
                    offset=off_ws, **kw)
    got = qs.sample_noalloc(d["logits"], d["T"], d["k"], d["p"], d["bitmask"],
                            seed=d["seed"], offset=off_na, **kw)
    torch.cuda.synchronize()
    for name in ("tokens", "status", "keep_mask", "cand_count", "logprobs", "debug"):
        _same(ref[name], got[name], name)
    # the lists up to each row's count (the rest of a row is not written)
    cnt = np.minimum(ref["cand_count"].cpu().numpy(), cand_cap)
    for name in ("cand_ids", "cand_probs"):
        a = ref[name].cpu().numpy()
        b = got[name].cpu().numpy()
        for r in range(w.B):
            assert np.array_equal(a[r, :cnt[r]].view(np.uint32), b[r, :cnt[r]].view(np.uint32)), \
                (name, r)
    _same(off_ws, off_na, "offset")
    return ref


def test_noalloc_matches_workspace_call_twice(qs):
    # 128 rows of 262144 bf16 tokens (the chunked pass, whose workspace the
    # scratch replaces; thirds top-k / top-p / both, 30 % legal bitmask), then
    # a smaller batch of the same kinds: the second call reuses the scratch
    # the first one left behind
    big = workloads.make(3, B=128, V=262144)
    print(f"noalloc call 1: B={big.B} V={big.V} {big.dtype}", flush=True)
    ref = _both(qs, big, 8192)
    assert (ref["debug"].cpu().numpy()[:, 0] == 2).mean() > 0.3   # the chunked path ran
    small = workloads.make(3, B=37, V=200000, seed=workloads.BASE_SEED + 77)
    print(f"noalloc call 2: B={small.B} V={small.V} {small.dtype}", flush=True)
    _both(qs, small, 4096)


def test_noalloc_fp32_rows(qs):
    # fp32 rows take no chunk workspace; the entry point still matches
    w = workloads.make(2, B=16, V=20000)
    print(f"noalloc fp32: B={w.B} V={w.V}", flush=True)
    _both(qs, w, 2048)
