"""Calls captured in a HIP graph (the library enqueues kernels only: no
allocation, copy or memset on the stream). Each replay advances the Philox
offsets like an eager call, so replay r must equal the r-th of the same calls
run eagerly; between replays the program runs eager work of its own and
synchronises."""
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


def _bits(t):
    import torch
    return t.view(torch.int32) if t.dtype == torch.float32 else t


@pytest.mark.parametrize("case", ["bf16_registers", "fp32", "bf16_chunked"])
def test_graph_replays_match_eager(qs, case):
    import torch
    w = {"bf16_registers": lambda: workloads.make(3, B=64),
         "fp32": lambda: workloads.make(2, B=16),
         "bf16_chunked": lambda: workloads.make(3, B=4, V=200000)}[case]()
    print(f"graph replays {case} B={w.B} V={w.V} {w.dtype}", flush=True)
    d = to_device(w)
    ws = qs.workspace_for(d["logits"], w.V)
    off0 = d["offset"].clone()
    R = 4

    def call():
        return qs.sample(d["logits"], d["T"], d["k"], d["p"], d["bitmask"], seed=d["seed"],
                         offset=d["offset"], keep_mask=True, cand_cap=w.V, logprobs=True,
                         workspace=ws)

    eager = []
    for _ in range(R):
        o = call()
        torch.cuda.synchronize()
        eager.append({k: v.clone() for k, v in o.items()} | {"offset": d["offset"].clone()})
    d["offset"].copy_(off0)
    torch.cuda.synchronize()
    # warm the allocator outside the capture, then capture one call on a side stream
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        call()
    torch.cuda.synchronize()
    d["offset"].copy_(off0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        out = call()
    torch.cuda.synchronize()
    d["offset"].copy_(off0)
    torch.cuda.synchronize()
    scratch = torch.zeros(1 << 20, device="cuda")
    for r in range(R):
        with torch.cuda.stream(cs):
            g.replay()
        torch.cuda.synchronize()
        got = {k: v.clone() for k, v in out.items()} | {"offset": d["offset"].clone()}
        want = eager[r]
        cnt = want["cand_count"]
        live = torch.arange(w.V, device=cnt.device)[None, :] < cnt.clamp(max=w.V)[:, None]
        for key in want:
            a, b = _bits(got[key]), _bits(want[key])
            if key in ("cand_ids", "cand_probs"):
                a, b = a[live], b[live]
            assert torch.equal(a, b), (case, r, key)
        scratch.add_(1.0)  # the program's own eager work between replays
        torch.cuda.synchronize()
