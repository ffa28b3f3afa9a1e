"""Calls on different streams at the same time (the header's concurrency
contract: the library keeps no state, each call has its own outputs and
workspace). Batches of every kernel path run concurrently on four streams and
must give, bit for bit, what the same calls give one after another."""
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


def _call(qs, d, uni, cap):
    return qs.sample(d["logits"], d["T"], d["k"], d["p"], d["bitmask"], uniforms=uni,
                     keep_mask=True, cand_cap=cap, dense=True, logprobs=True)


def test_concurrent_streams_match_serial(qs):
    import torch
    batches = [workloads.make(3, B=96),                    # bf16 rows in registers
               workloads.make(2, B=32),                    # fp32 truncation path
               workloads.make(3, B=8, V=200000),           # bf16 chunked pass (own workspace)
               workloads.make(5, B=96)]                    # error rows, per-row temperatures
    print("concurrent streams: " + ", ".join(f"B={w.B} V={w.V} {w.dtype}" for w in batches),
          flush=True)
    devs = [to_device(w) for w in batches]
    unis = [torch.from_numpy(np.random.default_rng(i).random(w.B)).cuda()
            for i, w in enumerate(batches)]
    caps = [w.V for w in batches]
    torch.cuda.synchronize()
    serial = []
    for d, u, c in zip(devs, unis, caps):
        serial.append(_call(qs, d, u, c))
        torch.cuda.synchronize()
    main = torch.cuda.current_stream()
    streams = [torch.cuda.Stream() for _ in batches]
    for rep in range(2):
        outs = []
        for s, d, u, c in zip(streams, devs, unis, caps):
            s.wait_stream(main)
            with torch.cuda.stream(s):
                outs.append(_call(qs, d, u, c))
        for s in streams:
            main.wait_stream(s)
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(outs, serial)):
            cnt = want["cand_count"]
            # list entries past a row's count are not written
            live = torch.arange(caps[i], device=cnt.device)[None, :] < cnt.clamp(max=caps[i])[:, None]
            for key in want:
                a, b = got[key], want[key]
                if a.dtype == torch.float32:  # bit patterns (error rows hold NaN)
                    a, b = a.view(torch.int32), b.view(torch.int32)
                if key in ("cand_ids", "cand_probs"):
                    a, b = a[live], b[live]
                assert torch.equal(a, b), (rep, i, key)


def _same(got, want, tag):
    import torch
    if isinstance(want, tuple):
        got, want = dict(enumerate(got)), dict(enumerate(want))
    cnt = want.get("cand_count")
    for key in want:
        a, b = got[key], want[key]
        if a.dtype == torch.float32:  # bit patterns (error rows hold NaN)
            a, b = a.view(torch.int32), b.view(torch.int32)
        if key in ("cand_ids", "cand_probs"):
            cap = a.shape[1]
            live = torch.arange(cap, device=a.device)[None, :] < cnt.clamp(max=cap)[:, None]
            a, b = a[live], b[live]
        assert torch.equal(a, b), (tag, key)


def test_concurrent_entry_points_match_serial(qs):
    """Different entry points at once: sampling with top-n outputs, sampling
    with fused penalties, greedy argmax and the sorted-subset filter."""
    import torch
    wb = workloads.make(3, B=64)
    wf = workloads.make(2, B=32)
    print(f"entry points on four streams: B={wb.B} V={wb.V} bf16, B={wf.B} V={wf.V} fp32",
          flush=True)
    db, df = to_device(wb), to_device(wf)
    rng = np.random.default_rng(5)
    ub = torch.from_numpy(rng.random(wb.B)).cuda()
    H = 512
    proc = {"history": torch.from_numpy(rng.integers(0, wb.V, size=(wb.B, H)).astype(np.int32)).cuda(),
            "history_count": torch.full((wb.B,), H, dtype=torch.int32, device="cuda"),
            "repetition": torch.full((wb.B,), 1.2, dtype=torch.float32, device="cuda"),
            "presence": torch.full((wb.B,), 0.3, dtype=torch.float32, device="cuda")}
    calls = [
        ("top_n", lambda: qs.sample(db["logits"], db["T"], db["k"], db["p"], db["bitmask"],
                                    uniforms=ub, keep_mask=True, cand_cap=wb.V, top_n=20)),
        ("processed", lambda: qs.sample(db["logits"], db["T"], db["k"], db["p"], db["bitmask"],
                                        uniforms=ub, keep_mask=True, cand_cap=wb.V,
                                        logprobs=True, processors=proc)),
        ("argmax", lambda: qs.argmax(df["logits"])),
        ("sorted_subset", lambda: qs.filter_mask(df["logits"], df["T"], df["k"], df["p"],
                                                 cand_cap=wf.V, dense=True,
                                                 flags=qs.FLAG_SORT_SUBSET)),
    ]
    torch.cuda.synchronize()
    serial = []
    for _, fn in calls:
        serial.append(fn())
        torch.cuda.synchronize()
    main = torch.cuda.current_stream()
    streams = [torch.cuda.Stream() for _ in calls]
    for rep in range(2):
        outs = []
        for s, (_, fn) in zip(streams, calls):
            s.wait_stream(main)
            with torch.cuda.stream(s):
                outs.append(fn())
        for s in streams:
            main.wait_stream(s)
        torch.cuda.synchronize()
        for (name, _), got, want in zip(calls, outs, serial):
            _same(got, want, (rep, name))
