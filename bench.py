"""Throughput of the fused filter+sample path on one MI355X.

One step = one qs_sample call over a whole batch: sigma-truncation pass,
pivot searches, tie quota, renormalisation, mask/candidate outputs and the
token draw, for every row. Inputs are resident in HBM before timing starts;
the calls rotate over several input sets whose total size exceeds the 256 MB
Infinity Cache, so the logits are read from HBM.

Prints one JSON line (rank 0, one GPU):
  value       rows per second over the whole timed region
  roofline    algorithmic bytes read per launch / mean launch duration (HIP
              events around every launch on the stream the kernel runs on),
              against the 8 TB/s HBM peak
  cpu_baseline  the CPU oracle on a bounded sample of the same rows
"""

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0
WORKLOAD_NAMES = {
    1: "B=4 V=32000 fp32 N(0,1)+6 on 16 ids, T=1 k=50 p=0.9",
    2: "B=64 V=128256 fp32 N(0,4)+20 ids N(8,2), per-row k/p/T, 10% greedy",
    3: "B=256 V=151936 bf16 N(0,9), thirds top-k/top-p/both, 30% legal bitmask",
    4: "B=1024 V=262144 fp32 near-flat/bimodal/heavy-tail, k=4096 p=0.99",
    5: "B=512 V=151936 bf16 as 3 + per-row T and degenerate rows, candidate lists",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--sets", type=int, default=4,
                    help="distinct input sets rotated through (default 4 > 256 MB MALL)")
    ap.add_argument("--cand-cap", type=int, default=0,
                    help="candidate-list capacity per row; 0 (the default): V, so every "
                         "kept token is written (the line counts rows whose kept set "
                         "overflowed a smaller capacity)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="the oracle baseline takes row chunks of the input sets, in "
                         "order and cyclically, until this much wall time has passed")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--flags", type=int, default=0)
    ap.add_argument("--eager", action="store_true",
                    help="time K eager launches instead of one replay of a HIP graph "
                         "holding the K launches")
    ap.add_argument("--spec", action="store_true",
                    help="instead of the headline line, time the speculative verifier "
                         "(qs_spec_verify) on candidate lists of the headline workload")
    ap.add_argument("--toplp", type=int, default=0, metavar="N",
                    help="instead of the headline line, time qs_top_logprobs (the N most "
                         "probable tokens) on candidate lists of the headline workload")
    ap.add_argument("--penalties", action="store_true",
                    help="instead of the headline line, time qs_apply_penalties (2048-token "
                         "histories) on the headline batch, alone and followed by qs_sample")
    ap.add_argument("--ablation", action="store_true",
                    help="instead of the headline line, print one line timing the path "
                         "switches (the Qrita page's ablation runs) on the headline "
                         "workload and at the page's ablation shape")
    ap.add_argument("--outliers", type=int, default=0, metavar="N",
                    help="set N random ids of every row to -1000 and make them legal (a "
                         "logit bias of -1000 on a few tokens), on top of the workload")
    ap.add_argument("--streams", type=int, default=1, metavar="N",
                    help="print one line for N independent batches in flight together: "
                         "the calls alternate over N streams captured in one graph, each "
                         "stream with input sets of its own (the default line is one "
                         "stream, one call after another)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, also run plain device copies of the "
                         "logits (known bytes) so counter runs can scale FETCH/WRITE sizes")
    return ap.parse_args()


class Prepared:
    """One input set on the device with preallocated outputs and the ctypes
    argument tuple for qs_sample (no Python-side allocation in the loop)."""

    def __init__(self, lib, w, cand_cap, flags, stream, workspace=None):
        import torch
        import top_sampling_vocabs_amd as qs
        dev = "cuda"
        self.w = w
        cand_cap = cand_cap if cand_cap > 0 else w.V  # 0: room for every kept token
        self.cand_cap = cand_cap
        if w.dtype == "bf16":
            self.logits = torch.from_numpy(w.logits.view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            self.logits = torch.from_numpy(w.logits).to(dev)
        self.T = torch.from_numpy(w.T).to(dev)
        self.k = torch.from_numpy(w.k).to(dev)
        self.p = torch.from_numpy(w.p).to(dev)
        self.bm = None if w.bitmask is None else \
            torch.from_numpy(w.bitmask.view(np.int32)).to(dev)
        self.seed = torch.from_numpy(w.seeds.view(np.int64)).to(dev)
        self.offset = torch.zeros(w.B, dtype=torch.int64, device=dev)
        W = (w.V + 31) // 32
        self.tokens = torch.empty(w.B, dtype=torch.int32, device=dev)
        self.status = torch.empty(w.B, dtype=torch.int32, device=dev)
        self.keep = torch.empty((w.B, W), dtype=torch.int32, device=dev)
        self.cids = torch.empty((w.B, cand_cap), dtype=torch.int32, device=dev)
        self.cprobs = torch.empty((w.B, cand_cap), dtype=torch.float32, device=dev)
        self.ccount = torch.empty(w.B, dtype=torch.int32, device=dev)
        # the caller-owned scratch (input sets of one shape may share one: the
        # calls run one after another on one stream)
        need = qs.workspace_bytes(w.B, w.V, 1 if w.dtype == "bf16" else 0, cand_cap)
        if workspace is None and need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        self.ws = workspace
        self.ws_bytes = need
        P = ctypes.c_void_p
        self.args = (
            P(self.logits.data_ptr()), 1 if w.dtype == "bf16" else 0, w.B, w.V, w.V,
            P(self.T.data_ptr()), P(self.k.data_ptr()), P(self.p.data_ptr()),
            None if self.bm is None else P(self.bm.data_ptr()),
            0 if self.bm is None else self.bm.stride(0),
            P(self.seed.data_ptr()), P(self.offset.data_ptr()), None,
            P(self.tokens.data_ptr()), None, P(self.keep.data_ptr()), P(self.cids.data_ptr()),
            P(self.cprobs.data_ptr()), P(self.ccount.data_ptr()), cand_cap, None,
            P(self.status.data_ptr()), None, flags,
            None if workspace is None else P(workspace.data_ptr()), need, stream)
        self.lib = lib

    # positions in the argument tuple, counted from its end
    _FLAGS, _DEBUG = -4, -5

    def call(self, stream=None, flags=None, debug=None):
        args = list(self.args)
        if flags is not None:
            args[self._FLAGS] = flags
        if debug is not None:
            args[self._DEBUG] = ctypes.c_void_p(debug.data_ptr())
        if stream is not None:
            args[-1] = stream
        rc = self.lib.qs_sample(*args)
        if rc != 0:
            raise RuntimeError(f"qs_sample returned {rc}")

    def outputs(self):
        return [t.clone() for t in (self.tokens, self.status, self.keep, self.cids,
                                    self.cprobs, self.ccount, self.offset)]


# the translation unit of the filter/sample kernel (the other entry points'
# kernels live in files of their own and do not change it)
FILTER_SOURCES = ("qs_device.hpp", "qs_filter.hpp", "qs_filter_bf16.hip", "qs_filter_f32.hip",
                  "qs_launch.hpp", "qs_select.hpp", "qs_stream.hpp", "qs_merge.hpp",
                  "qs_bins.hpp", "qs_chunk.hpp", "qs_chunk.hip", "qs_proc.hpp")


def source_digest():
    """sha256 over the sources the filter/sample kernel is built from: a stored
    counter reading applies only to the kernel it was taken on."""
    import hashlib
    csrc = os.path.join(ROOT, "top_sampling_vocabs_amd", "csrc")
    h = hashlib.sha256()
    for name in FILTER_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def stored_traffic(cfg):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE + WRITE_SIZE
    (scaled by a plain copy of known size), from profiles/, or None when the
    kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"filter_kernel_workload{cfg}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, _, v = line.partition(":")
                vals[key.strip()] = v.strip()
    if vals.get("source_digest") != source_digest():
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def copy_calibration(preps, reps=20):
    """Plain device-to-device copies of each input set's logits: a kernel of
    known bytes (read = write = logits size) for scaling counter readings."""
    import torch
    srcs = [p.logits for p in preps]
    dsts = [torch.empty_like(s) for s in srcs]
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        dsts[i % len(dsts)].copy_(srcs[i % len(srcs)])
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    nbytes = srcs[0].numel() * srcs[0].element_size()
    return {"bytes_read": nbytes, "bytes_written": nbytes, "ms": round(ms, 5),
            "gbs_rw": round(2 * nbytes / (ms / 1e3) / 1e9, 1)}


def time_graph(preps, K, flags=None):
    """Capture K launches (input sets in rotation) in one HIP graph on a side
    stream, replay it once untimed, then time one replay between two events on
    that stream. Returns (total ms, graph, capture stream)."""
    import torch
    cs = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(graph, stream=cs):
            sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for i in range(K):
                preps[i % len(preps)].call(sp, flags=flags)
    torch.cuda.synchronize()
    with torch.cuda.stream(cs):
        graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(cs):
        a.record(cs)
        graph.replay()
        b.record(cs)
    torch.cuda.synchronize()
    return a.elapsed_time(b), graph, cs


def streams_bench(args, lib):
    """Throughput with N independent batches in flight: call i runs on stream
    i % N with its own input set and outputs (2 sets a stream, so the sets do
    not fit the 256 MB MALL), all K calls captured in one graph whose streams
    fork from and join the capture stream. A kernel's slowest rows then share
    the GPU with the next kernel's first rows instead of leaving compute units
    idle. The outputs of a replay are checked against the same calls run
    eagerly on one stream (each set's calls keep their order)."""
    import torch
    N = args.streams
    cfg = args.workload
    sets = [workloads.make(cfg, seed=workloads.BASE_SEED + cfg + 1000 * i) for i in range(2 * N)]
    preps = [Prepared(lib, w, args.cand_cap, args.flags, None) for w in sets]
    K = args.steps - args.steps % (2 * N)
    for i in range(args.warmup):
        preps[i % len(preps)].call()
    torch.cuda.synchronize()
    for p_ in preps:
        p_.offset.zero_()
    torch.cuda.synchronize()
    for i in range(K):
        preps[i % len(preps)].call()
    torch.cuda.synchronize()
    eager_out = [p_.outputs() for p_ in preps]
    cs = torch.cuda.Stream()
    others = [torch.cuda.Stream() for _ in range(N - 1)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(graph, stream=cs):
            for o in others:
                o.wait_stream(cs)
            streams = [cs] + others
            for i in range(K):
                preps[i % len(preps)].call(ctypes.c_void_p(streams[i % N].cuda_stream))
            for o in others:
                cs.wait_stream(o)
    torch.cuda.synchronize()
    for p_ in preps:
        p_.offset.zero_()
    torch.cuda.synchronize()
    with torch.cuda.stream(cs):
        graph.replay()
    torch.cuda.synchronize()
    for p_, ref in zip(preps, eager_out):
        for a_, b_ in zip(p_.outputs(), ref):
            assert torch.equal(a_, b_), "multi-stream replay differs from eager launches"
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(cs):
        a.record(cs)
        graph.replay()
        b.record(cs)
    torch.cuda.synchronize()
    total_ms = a.elapsed_time(b)
    base = sets[0]
    bytes_read = workloads.bytes_read(base)
    gbs = bytes_read * K / (total_ms / 1e3) / 1e9
    print(json.dumps({
        "metric": "rows/sec and effective HBM GB/s (fraction of peak), B=256 V=151936",
        "value": round(base.B * K / (total_ms / 1e3), 1), "unit": "rows/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(total_ms / K, 5),
        "higher_is_better": True, "dtype": base.dtype, "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[cfg], "batch_rows": base.B, "vocab": base.V,
                   "input_sets": len(sets), "bytes_read_per_step": bytes_read,
                   "cand_cap": preps[0].cand_cap, "streams": N,
                   "launch": f"hip_graph over {N} streams (independent batches in flight)"},
        "aggregate": {"GBps": round(gbs, 1), "peak": HBM_PEAK_GBS,
                      "frac": round(gbs / HBM_PEAK_GBS, 4),
                      "basis": "algorithmic bytes of all calls / elapsed time; launches overlap"},
        "check": "every set's outputs equal to the same calls run eagerly on one stream",
    }), flush=True)


# Path switches of the library and the Qrita page's ablation runs they mirror
# (its runs C and J drop duplicate handling or sort the full row: not paths of
# this library).
ABLATION_RUNS = [
    ("A", "normal path: value histogram (bf16 in registers) / truncation hit + bucket select (fp32)", 0),
    ("B", "single streamed tier instead of the register tiers", 8),
    ("D", "forced fallback: quaternary searches over the full row", 1),
    ("E", "no truncation: quaternary searches over the full row", 2),
    ("F", "truncation hit, binary pivot (one pivot per round)", 16 | 4),
    ("G", "forced fallback, binary pivot", 16 | 1),
    ("Q", "truncation hit, quaternary search on bf16 pools (the page's design)", 4),
    ("I", "truncation hit, the candidate subset sorted in LDS (up to 8,192 candidates; "
          "larger subsets are searched)", 32),
]


class SpecPrepared:
    """Target and draft candidate lists of one input set, made on the device by
    the filter (draft logits = target logits + N(0, 0.5^2) noise, same T, k, p),
    draft tokens drawn from the draft lists, and the ctypes argument tuple of
    qs_spec_verify."""

    def __init__(self, lib, w, cap, stream, seed):
        import torch
        import top_sampling_vocabs_amd as qs
        dev = "cuda"
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        z = torch.from_numpy(w.logits.view(np.int16)).to(dev).view(torch.bfloat16)
        zd = (z.float() + 0.5 * torch.randn(z.shape, device=dev, generator=g)).to(torch.bfloat16)
        T = torch.from_numpy(w.T).to(dev)
        k = torch.from_numpy(w.k).to(dev)
        p = torch.from_numpy(w.p).to(dev)
        # sampled rows only (greedy rows have no draft distribution to verify)
        T = torch.where(T > 0, T, torch.ones_like(T))
        bm = None if w.bitmask is None else torch.from_numpy(w.bitmask.view(np.int32)).to(dev)
        self.t = qs.filter_mask(z, T, k, p, bm, cand_cap=cap)
        uni = torch.rand(w.B, dtype=torch.float64, device=dev, generator=g)
        self.d = qs.sample(zd, T, k, p, bm, uniforms=uni, cand_cap=cap)
        self.x = self.d["tokens"]
        self.u1 = torch.rand(w.B, dtype=torch.float64, device=dev, generator=g)
        self.u2 = torch.rand(w.B, dtype=torch.float64, device=dev, generator=g)
        self.out = {n: torch.empty(w.B, dtype=torch.int32, device=dev)
                    for n in ("tokens", "accepted", "status")}
        P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        self.args = (w.B, P(self.t["cand_ids"]), P(self.t["cand_probs"]), P(self.t["cand_count"]),
                     cap, P(self.d["cand_ids"]), P(self.d["cand_probs"]), P(self.d["cand_count"]),
                     cap, P(self.x), P(self.u1), P(self.u2), P(self.out["tokens"]),
                     P(self.out["accepted"]), P(self.out["status"]), stream)
        self.lib = lib

    def call(self, stream=None, flags=None):
        args = self.args if stream is None else self.args[:-1] + (stream,)
        rc = self.lib.qs_spec_verify(*args)
        if rc != 0:
            raise RuntimeError(f"qs_spec_verify returned {rc}")

    def bytes_read(self):
        """Algorithmic bytes: every row reads its counts, token and uniforms; a
        rejected row also reads the target list twice (mass, then draw) and the
        draft list once (8 bytes an entry)."""
        acc = self.out["accepted"].cpu().numpy()
        ok = self.out["status"].cpu().numpy() == 0
        tc = self.t["cand_count"].cpu().numpy().astype(np.int64)
        dc = self.d["cand_count"].cpu().numpy().astype(np.int64)
        rej = ok & (acc == 0)
        return int(len(acc) * 28 + (16 * tc[rej] + 8 * dc[rej]).sum()), float(acc[ok].mean()), \
            int(rej.sum()), int((~ok).sum())


def spec_bench(args, lib, stream):
    import torch
    cap = 16384
    preps = [SpecPrepared(lib, workloads.make(args.workload, seed=workloads.BASE_SEED +
                                              args.workload + 1000 * i), cap, stream, 77 + i)
             for i in range(args.sets)]
    for i in range(args.warmup):
        preps[i % len(preps)].call()
    torch.cuda.synchronize()
    ms, graph, cs = time_graph(preps, args.steps)
    per = ms / args.steps
    stats = [pr.bytes_read() for pr in preps]
    nbytes = sum(s[0] for s in stats) / len(stats)
    B = preps[0].args[0]
    line = {
        "metric": "speculative verification rows/sec over candidate lists, B=256 V=151936",
        "value": round(B / (per * 1e-3), 1), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(per, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": "candidate lists (cap 16384) of the B=256 V=151936 bf16 batch as "
                               "target, of the same logits + N(0, 0.5^2) as draft",
                   "accept_rate": round(float(np.mean([s[1] for s in stats])), 4),
                   "rejected_rows": [s[2] for s in stats], "error_rows": [s[3] for s in stats]},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (per * 1e-3) / 1e9, 1),
                     "peak": 8000.0, "unit": "GB/s",
                     "frac": round(nbytes / (per * 1e-3) / 8e12, 5), "traffic": None,
                     "bytes_per_launch": int(nbytes)},
    }
    print(json.dumps(line), flush=True)


class TopLPPrepared:
    """Candidate lists of one input set, made on the device by the filter, and
    the ctypes argument tuple of qs_top_logprobs for n slots a row."""

    def __init__(self, lib, w, cap, n, stream):
        import torch
        import top_sampling_vocabs_amd as qs
        dev = "cuda"
        z = torch.from_numpy(w.logits.view(np.int16)).to(dev).view(torch.bfloat16)
        T = torch.from_numpy(w.T).to(dev)
        T = torch.where(T > 0, T, torch.ones_like(T))
        k = torch.from_numpy(w.k).to(dev)
        p = torch.from_numpy(w.p).to(dev)
        bm = None if w.bitmask is None else torch.from_numpy(w.bitmask.view(np.int32)).to(dev)
        self.t = qs.filter_mask(z, T, k, p, bm, cand_cap=cap)
        self.ids = torch.empty(w.B, n, dtype=torch.int32, device=dev)
        self.lp = torch.empty(w.B, n, dtype=torch.float32, device=dev)
        self.status = torch.empty(w.B, dtype=torch.int32, device=dev)
        P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        self.args = (w.B, P(self.t["cand_ids"]), P(self.t["cand_probs"]), P(self.t["cand_count"]),
                     cap, n, P(self.ids), P(self.lp), P(self.status), stream)
        self.n = n
        self.lib = lib

    def call(self, stream=None, flags=None):
        args = self.args if stream is None else self.args[:-1] + (stream,)
        rc = self.lib.qs_top_logprobs(*args)
        if rc != 0:
            raise RuntimeError(f"qs_top_logprobs returned {rc}")

    def bytes_moved(self):
        """Algorithmic bytes: each row reads its count and its list once (8 bytes
        an entry) and writes n (id, logprob) slots."""
        tc = self.t["cand_count"].cpu().numpy().astype(np.int64)
        assert (self.status.cpu().numpy() == 0).all()
        return int(len(tc) * (4 + 8 * self.n) + 8 * tc.sum()), float(tc.mean())


def toplp_bench(args, lib, stream):
    import torch
    cap = 16384
    preps = [TopLPPrepared(lib, workloads.make(args.workload, seed=workloads.BASE_SEED +
                                               args.workload + 1000 * i), cap, args.toplp, stream)
             for i in range(args.sets)]
    for i in range(args.warmup):
        preps[i % len(preps)].call()
    torch.cuda.synchronize()
    ms, graph, cs = time_graph(preps, args.steps)
    per = ms / args.steps
    stats = [pr.bytes_moved() for pr in preps]
    nbytes = sum(s[0] for s in stats) / len(stats)
    B = preps[0].args[0]
    del graph

    # the sampling step alone, then with the separate call on its lists, then
    # with the top tokens written by the sampling launch itself
    # (qs_sample_top_logprobs); lists of capacity 16384 (every kept token of
    # this batch fits, and the separate call takes its register path)
    sets = [workloads.make(args.workload, seed=workloads.BASE_SEED + args.workload + 1000 * i)
            for i in range(args.sets)]
    samp = [Prepared(lib, w, cap, 0, stream) for w in sets]
    n = args.toplp

    class Then:
        def __init__(self, sp):
            import torch
            self.sp = sp
            P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
            self.ids = torch.empty(sp.w.B, n, dtype=torch.int32, device="cuda")
            self.lp = torch.empty(sp.w.B, n, dtype=torch.float32, device="cuda")
            self.st = torch.empty(sp.w.B, dtype=torch.int32, device="cuda")
            self.targs = (sp.w.B, P(sp.cids), P(sp.cprobs), P(sp.ccount), sp.cand_cap, n,
                          P(self.ids), P(self.lp), P(self.st))
            a_ = sp.args
            self.fargs = a_[:-3] + (n, P(self.ids), P(self.lp)) + a_[-3:]

        def call(self, stream=None, flags=None):
            self.sp.call(stream)
            rc = lib.qs_top_logprobs(*(self.targs + (stream,)))
            if rc != 0:
                raise RuntimeError(f"qs_top_logprobs returned {rc}")

    class Fused(Then):
        def call(self, stream=None, flags=None):
            rc = lib.qs_sample_top_logprobs(*(self.fargs[:-1] + (stream,)))
            if rc != 0:
                raise RuntimeError(f"qs_sample_top_logprobs returned {rc}")

    times = {}
    for name, calls in (("sample", samp), ("sample_then_top_logprobs", [Then(sp) for sp in samp]),
                        ("sample_with_top_logprobs", [Fused(sp) for sp in samp])):
        for i in range(args.warmup):
            calls[i % len(calls)].call()
        torch.cuda.synchronize()
        ms_, g_, cs_ = time_graph(calls, args.steps)
        del g_
        times[name] = round(ms_ / args.steps, 5)
        if name == "sample_with_top_logprobs":  # the same slots as the separate call
            ref = Then(calls[0].sp)
            ref.call()
            calls[0].call()
            torch.cuda.synchronize()
            assert torch.equal(calls[0].ids, ref.ids)
            assert torch.equal(calls[0].lp.view(torch.int32), ref.lp.view(torch.int32))
    line = {
        "metric": f"top-{args.toplp} logprobs rows/sec over candidate lists, B=256 V=151936",
        "value": round(B / (per * 1e-3), 1), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(per, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "candidate lists (cap 16384) of the B=256 V=151936 bf16 batch",
                   "n": args.toplp,
                   "mean_list_length": round(float(np.mean([s[1] for s in stats])), 1),
                   "sample_ms": times["sample"],
                   "sample_then_top_logprobs_ms": times["sample_then_top_logprobs"],
                   "sample_with_top_logprobs_in_launch_ms": times["sample_with_top_logprobs"]},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (per * 1e-3) / 1e9, 1),
                     "peak": 8000.0, "unit": "GB/s",
                     "frac": round(nbytes / (per * 1e-3) / 8e12, 5), "traffic": None,
                     "bytes_per_launch": int(nbytes)},
    }
    print(json.dumps(line), flush=True)


class PenaltyPrepared:
    """A 2048-token history per row (uniform ids, so about 2,030 distinct),
    repetition 1.2 and presence 0.3, and the ctypes tuple of qs_apply_penalties
    on the same device logits a Prepared set samples from."""

    H = 2048

    def __init__(self, lib, prep, seed):
        import torch
        w = prep.w
        rng = np.random.default_rng(seed)
        self.hist = torch.from_numpy(rng.integers(0, w.V, (w.B, self.H)).astype(np.int32)).cuda()
        self.cnt = torch.full((w.B,), self.H, dtype=torch.int32, device="cuda")
        self.rep = torch.full((w.B,), 1.2, dtype=torch.float32, device="cuda")
        self.pres = torch.full((w.B,), 0.3, dtype=torch.float32, device="cuda")
        self.status = torch.empty(w.B, dtype=torch.int32, device="cuda")
        P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        self.args = (P(prep.logits), 1 if w.dtype == "bf16" else 0, w.B, w.V, w.V, P(self.hist),
                     self.H, P(self.cnt), P(self.rep), P(self.pres), None, P(self.status), None)
        self.lib, self.prep, self.with_sample = lib, prep, False

    def call(self, stream=None, flags=None):
        rc = self.lib.qs_apply_penalties(*(self.args[:-1] + (stream,)))
        if rc != 0:
            raise RuntimeError(f"qs_apply_penalties returned {rc}")
        if self.with_sample:
            self.prep.call(stream)


def penalties_bench(args, lib, stream):
    """Penalties alone, then penalties + sample per step. Each set is
    penalised once for real (repetition 1.2, presence 0.3); the timed steps
    then apply repetition 1 and presence 0 to the same histories, which does
    the same loads, arithmetic and stores but leaves the rows as one real
    application made them (applying 1.2 over and over would drive the
    penalised logits to huge negative values no real row holds)."""
    import torch
    sets = [workloads.make(args.workload, seed=workloads.BASE_SEED + args.workload + 1000 * i)
            for i in range(args.sets)]
    preps = [Prepared(lib, w, args.cand_cap, args.flags, stream) for w in sets]
    pens = [PenaltyPrepared(lib, pr, 500 + i) for i, pr in enumerate(preps)]
    for pn in pens:
        pn.call(stream)
        pn.rep.fill_(1.0)
        pn.pres.fill_(0.0)
    torch.cuda.synchronize()
    out = {}
    for mode in ("penalties", "penalties+sample"):
        for pn in pens:
            pn.with_sample = mode != "penalties"
        for i in range(args.warmup):
            pens[i % len(pens)].call(stream)
        torch.cuda.synchronize()
        ms, graph, cs = time_graph(pens, args.steps)
        out[mode] = ms / args.steps
        del graph
    # the logit bias kernel on the same rows: 2048 distinct ids per row, bias 0
    # (the same work as any bias, rows unchanged)
    import top_sampling_vocabs_amd as qs

    class BiasCall:
        def __init__(self, pr, seed):
            g = torch.Generator()
            g.manual_seed(seed)
            w = pr.w
            self.ids = torch.stack([torch.randperm(w.V, generator=g)[:PenaltyPrepared.H]
                                    for _ in range(w.B)]).to(torch.int32).cuda()
            self.vals = torch.zeros(self.ids.shape, dtype=torch.float32, device="cuda")
            self.cnt = torch.full((w.B,), PenaltyPrepared.H, dtype=torch.int32, device="cuda")
            self.st = torch.empty(w.B, dtype=torch.int32, device="cuda")
            P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
            self.args = (P(pr.logits), 1 if w.dtype == "bf16" else 0, w.B, w.V, w.V, P(self.ids),
                         P(self.vals), PenaltyPrepared.H, P(self.cnt), P(self.st))

        def call(self, stream=None, flags=None):
            rc = lib.qs_apply_logit_bias(*(self.args + (stream,)))
            if rc != 0:
                raise RuntimeError(f"qs_apply_logit_bias returned {rc}")

    bias = [BiasCall(pr, 900 + i) for i, pr in enumerate(preps)]
    for i in range(args.warmup):
        bias[i % len(bias)].call(stream)
    torch.cuda.synchronize()
    ms, graph, cs = time_graph(bias, args.steps)
    out["logit_bias"] = ms / args.steps
    del graph

    class SeparateAll:
        """penalties, then the bias kernel, then sample: three launches"""

        def __init__(self, pn, bc):
            self.pn, self.bc = pn, bc

        def call(self, stream=None, flags=None):
            self.pn.with_sample = False
            self.pn.call(stream)
            self.bc.call(stream)
            self.pn.prep.call(stream)

    class FusedCall:
        """qs_sample_processed: the processors applied inside the sampling
        launch. The caller's rows are only read, so the real parameters
        (repetition 1.2, presence 0.3) are used on every step."""

        def __init__(self, pn, bc):
            pr, w = pn.prep, pn.prep.w
            dt = 1 if w.dtype == "bf16" else 0
            self.rep = torch.full((w.B,), 1.2, dtype=torch.float32, device="cuda")
            self.pres = torch.full((w.B,), 0.3, dtype=torch.float32, device="cuda")
            P = lambda t: t.data_ptr()  # noqa: E731
            self.proc = qsl.QsProcessors(
                P(pn.hist), PenaltyPrepared.H, P(pn.cnt), P(self.rep), P(self.pres), None,
                P(bc.ids) if bc else None, P(bc.vals) if bc else None,
                PenaltyPrepared.H if bc else 0, P(bc.cnt) if bc else None)
            nb = lib.qs_processors_workspace_bytes(w.B, w.V, dt)
            self.ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
            self.args = pr.args[:-4] + (pr.args[-4], ctypes.byref(self.proc),
                                        ctypes.c_void_p(self.ws.data_ptr()), nb, None)
            self.pr = pr

        def call(self, stream=None, flags=None):
            rc = lib.qs_sample_processed(*(self.args[:-1] + (stream,)))
            if rc != 0:
                raise RuntimeError(f"qs_sample_processed returned {rc}")

    from top_sampling_vocabs_amd import _lib as qsl
    modes = [("penalties+bias+sample", [SeparateAll(pn, bc) for pn, bc in zip(pens, bias)]),
             ("fused penalties+sample", [FusedCall(pn, None) for pn in pens]),
             ("fused penalties+bias+sample", [FusedCall(pn, bc) for pn, bc in zip(pens, bias)])]
    for mode, calls in modes:
        for i in range(args.warmup):
            calls[i % len(calls)].call(stream)
        torch.cuda.synchronize()
        ms, graph, cs = time_graph(calls, args.steps)
        out[mode] = ms / args.steps
        del graph
        if mode.startswith("fused"):
            # every row processed and sampled (none over the id limit; a kept
            # set larger than the candidate lists' capacity still samples)
            for c in calls:
                st = c.pr.status.cpu().numpy()
                bad = np.nonzero((st != qsl.ROW_OK) & (st != qsl.ROW_CAND_OVERFLOW))[0]
                if bad.size:
                    raise RuntimeError(f"{mode}: rows {bad.tolist()} not sampled, "
                                       f"statuses {st[bad].tolist()}")
    del qs
    B = preps[0].w.B
    H = PenaltyPrepared.H
    nbytes = B * (4 * H + 12 + 2 * 2 * H)  # ids, params, read + write of each penalised logit
    per = out["penalties"]
    line = {
        "metric": "rows/sec of penalties + sample, B=256 V=151936",
        "value": round(B / (out["fused penalties+sample"] * 1e-3), 1), "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(out["fused penalties+sample"], 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "B=256 V=151936 bf16 batch, 2048-token history per row, "
                               "repetition 1.2, presence 0.3, value = one fused launch",
                   "fused_penalties_sample_ms": round(out["fused penalties+sample"], 5),
                   "separate_penalties_then_sample_ms": round(out["penalties+sample"], 5),
                   "penalties_ms": round(per, 5),
                   "logit_bias_ms_2048_ids": round(out["logit_bias"], 5),
                   "separate_penalties_bias_sample_ms": round(out["penalties+bias+sample"], 5),
                   "fused_penalties_bias_sample_ms":
                       round(out["fused penalties+bias+sample"], 5)},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (per * 1e-3) / 1e9, 1),
                     "peak": 8000.0, "unit": "GB/s",
                     "frac": round(nbytes / (per * 1e-3) / 8e12, 5), "traffic": None,
                     "bytes_per_launch": nbytes},
    }
    print(json.dumps(line), flush=True)


def ablation(args, lib, stream):
    """Time every path switch on the headline workload and at the page's
    ablation shape; every switch gives identical outputs (the path-invariance
    test), so only time, search rounds and fallback rows differ."""
    import torch
    out = []
    for name in ("headline", "pages_ablation_shape"):
        if name == "headline":
            sets = [workloads.make(args.workload, seed=workloads.BASE_SEED + args.workload + 1000 * i)
                    for i in range(args.sets)]
        else:
            sets = [workloads.make_ablation(seed=workloads.BASE_SEED + 100 + 1000 * i)
                    for i in range(args.sets)]
        preps = [Prepared(lib, w, args.cand_cap, 0, stream) for w in sets]
        nbytes = workloads.bytes_read(sets[0])
        B = sets[0].B
        dbg = torch.zeros((B, 4), dtype=torch.int32, device="cuda")
        for run, what, flags in ABLATION_RUNS:
            for i in range(args.warmup):
                preps[i % len(preps)].call(flags=flags)
            preps[0].call(flags=flags, debug=dbg)
            torch.cuda.synchronize()
            d = dbg.cpu().numpy()
            st = preps[0].status.cpu().numpy()
            ok = st == 0
            total_ms, _, _ = time_graph(preps, args.steps, flags=flags)
            ms = total_ms / args.steps
            out.append({"workload": name, "run": run, "what": what, "flags": flags,
                        "ms_per_step": round(ms, 5),
                        "rows_per_s": round(B / (ms / 1e3), 1),
                        "gbs": round(nbytes / (ms / 1e3) / 1e9, 1),
                        "frac": round(nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                        "fallback_rows": int((d[ok, 0] == 1).sum()),
                        "rounds_mean": round(float(d[ok, 1].mean()), 3) if ok.any() else None,
                        "rounds_max": int(d[ok, 1].max()) if ok.any() else None})
            print(f"# {name} run {run}: {ms * 1e3:.1f} us/step", file=sys.stderr, flush=True)
        del preps
        torch.cuda.empty_cache()
    line = {"ablation": out, "steps": args.steps, "warmup": args.warmup,
            "input_sets": args.sets, "launch": "hip_graph",
            "shapes": {"headline": WORKLOAD_NAMES[args.workload],
                       "pages_ablation_shape": "B=1024 V=128256 fp32 N(0,2^2), k=50, p=0.9, T=1"}}
    print(json.dumps(line), flush=True)


def _oracle_chunk(task):
    """One oracle task in a worker process: filter + sample a few rows."""
    import oracle
    logits, dtype, T, k, p, bitmask, seeds, offsets = task
    res = oracle.filter_batch(logits, dtype, T, k, p, bitmask)
    oracle.sample_batch(res, seeds, offsets)
    return logits.shape[0]


def _oracle_warm(_):
    import oracle  # noqa: F401
    return os.getpid()


def cpu_cores():
    """Host threads the CPU baseline may use: the affinity set, capped at 16
    (the share of host cores that goes with one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.partition(":")[2].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(sets, seconds, chunk=None, procs=None):
    """Oracle throughput on a time-bounded sample, one oracle process per host
    core. Tasks are row chunks (16 rows, 4 for rows longer than 160000 so that
    the unfinished chunks at the deadline stay a small share) taken in order
    through the input sets
    (wrapping around); the clock starts once every worker has imported the
    oracle and stops after `seconds`, counting only finished chunks. Workers
    are fresh interpreters (spawn), so none inherits the parent's GPU state.
    Returns (rows/s, rows done, seconds, processes, chunk)."""
    import multiprocessing as mp
    procs = cpu_cores() if procs is None else procs
    B = sets[0].B
    if chunk is None:
        chunk = 16 if sets[0].V <= 160000 else 4

    def tasks():
        i = 0
        while True:
            w = sets[(i * chunk // B) % len(sets)]
            r0 = (i * chunk) % B
            r1 = min(r0 + chunk, B)
            yield (w.logits[r0:r1], w.dtype, w.T[r0:r1], w.k[r0:r1], w.p[r0:r1],
                   None if w.bitmask is None else w.bitmask[r0:r1],
                   w.seeds[r0:r1], w.offsets[r0:r1])
            i += 1

    ctx = mp.get_context("spawn")
    with ctx.Pool(procs) as pool:
        pool.map(_oracle_warm, range(procs), chunksize=1)
        done = 0
        t0 = time.perf_counter()
        for n in pool.imap_unordered(_oracle_chunk, tasks(), chunksize=1):
            done += n
            dt = time.perf_counter() - t0
            if dt >= seconds:
                break
        pool.terminate()
    return done / dt, done, dt, procs, chunk


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(rows are independent: a batch shards across GPUs with no communication)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import top_sampling_vocabs_amd as qs
    lib = qs.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.penalties:
        penalties_bench(args, lib, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        return
    if args.toplp:
        toplp_bench(args, lib, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        return
    if args.spec:
        spec_bench(args, lib, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        return
    if args.ablation:
        ablation(args, lib, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        return
    if args.streams > 1:
        streams_bench(args, lib)
        return
    cfg = args.workload
    base = workloads.make(cfg)
    sets = [base] + [workloads.make(cfg, seed=workloads.BASE_SEED + cfg + 1000 * i)
                     for i in range(1, args.sets)]
    if args.outliers:
        for i, w in enumerate(sets):
            workloads.add_outliers(w, args.outliers, -1000.0, seed=workloads.BASE_SEED + 77 + i)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    preps = [Prepared(lib, w, args.cand_cap, args.flags, stream) for w in sets[:1]]
    preps += [Prepared(lib, w, args.cand_cap, args.flags, stream, workspace=preps[0].ws)
              for w in sets[1:]]
    torch.cuda.synchronize()
    bytes_read = workloads.bytes_read(base)
    B = base.B

    for i in range(args.warmup):
        preps[i % len(preps)].call()
    torch.cuda.synchronize()

    K = args.steps
    n_sets = len(preps)
    if args.eager:
        # K eager launches, an event pair around each on the launch stream
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(K)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start_all = torch.cuda.Event(enable_timing=True)
        end_all = torch.cuda.Event(enable_timing=True)
        start_all.record()
        for i in range(K):
            ev[i][0].record()
            preps[i % n_sets].call()
            ev[i][1].record()
        end_all.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        total_ms = start_all.elapsed_time(end_all)
        per = np.array([a.elapsed_time(b) for a, b in ev])  # ms per launch
        launch_mode = "eager"
    else:
        # The K launches (input sets in rotation) captured in one HIP graph on
        # a side stream; one untimed replay, then the timed replay between two
        # events on that stream. A further replay from restarted Philox offsets
        # is checked against the same K launches run eagerly.
        for p_ in preps:
            p_.offset.zero_()
        torch.cuda.synchronize()
        for i in range(K):
            preps[i % n_sets].call()
        torch.cuda.synchronize()
        eager_out = [p_.outputs() for p_ in preps]
        for p_ in preps:
            p_.offset.zero_()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        total_ms, graph, cs = time_graph(preps, K)
        wall = time.perf_counter() - t0
        for p_ in preps:
            p_.offset.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(cs):
            graph.replay()
        torch.cuda.synchronize()
        for p_, ref in zip(preps, eager_out):
            for a_, b_ in zip(p_.outputs(), ref):
                assert torch.equal(a_, b_), "graph replay differs from eager launches"
        per = np.full(K, total_ms / K)
        launch_mode = "hip_graph"
    ms_step = total_ms / K
    rows_per_s = B * K / (total_ms / 1e3)
    mean_launch = float(per.mean())
    achieved = bytes_read / (mean_launch / 1e3) / 1e9

    # sanity: every row OK or an expected degenerate status
    st = preps[0].status.cpu().numpy()
    assert ((st == 0) | (st == 1) | (st == 2) | (st == 3) | (st == 5)).all(), np.unique(st)
    # rows of every input set whose kept set was longer than the lists (their
    # lists hold the first cand_cap entries only)
    overflow_rows = int(sum(int((p_.status == 5).sum()) for p_ in preps))

    copy = copy_calibration(preps) if args.copy_calibration else None

    cpu = None
    if not args.no_cpu:
        v, n, dt, procs, chunk = cpu_baseline(sets, args.cpu_seconds)
        cpu = {"value": round(v, 3), "unit": "rows/s", "cores": procs, "kind": "oracle",
               "sample": f"{n} rows of the same workload's {len(sets)} input sets in "
                         f"{chunk}-row chunks, filter + sample, {procs} oracle processes "
                         f"for {dt:.1f} s on {cpu_model()}"}

    line = {
        "metric": "rows/sec and effective HBM GB/s (fraction of peak), B=256 V=151936",
        "value": round(rows_per_s, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": base.dtype,
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[cfg] + (f", {args.outliers} ids/row at -1000"
                                                       if args.outliers else ""),
                   "batch_rows": B, "vocab": base.V,
                   "input_sets": len(sets), "bytes_read_per_step": bytes_read,
                   "cand_cap": preps[0].cand_cap,
                   "cand_overflow_rows": overflow_rows,
                   "launch": launch_mode, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic(cfg),
                     "kernel_ms_mean": round(mean_launch, 5),
                     "kernel_ms_p50": (round(float(np.median(per)), 5)
                                       if launch_mode == "eager" else None),
                     "kernel_ms_p99": (round(float(np.percentile(per, 99)), 5)
                                       if launch_mode == "eager" else None)},
        "cpu_baseline": cpu,
        "wall_s": round(wall, 3),
    }
    if copy is not None:
        line["copy_calibration"] = copy
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
