"""Known-answer pin of the oracle's Philox4x32-10 against an independent
implementation: rocRAND's Philox engine, built for the host from its header
source in the ROCm installation (no GPU). The pages fix only that the RNG state
is an explicit seed and offset advanced by what was consumed (page
"Attention算完，还没有选出下一个token", section 06); the generator is Salmon et
al.'s Philox4x32-10, and this test checks the oracle's rounds, multipliers, key
schedule and output word order against rocRAND's on counters with non-zero
high words, carries across 2^32, and the oracle's (seed, offset) layout: the
draw at offset n is rocRAND's first output after rocrand_init(seed, 0, 4 n)."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))
HEADER = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"
M32 = 0xFFFFFFFF


@pytest.fixture(scope="module")
def probe(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not (os.path.exists(HEADER) and os.path.exists(hipcc)):
        pytest.skip("rocRAND header or hipcc not available")
    exe = str(tmp_path_factory.mktemp("philox") / "probe")
    subprocess.run([hipcc, "-x", "hip", "--cuda-host-only", "-O1",
                    os.path.join(HERE, "philox_rocrand_probe.cpp"), "-o", exe],
                   check=True, capture_output=True, timeout=300)

    def run(lines):
        out = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True,
                             text=True, check=True, timeout=60).stdout.split("\n")
        return [tuple(int(x) for x in ln.split()) for ln in out if ln.strip()]
    return run


def _cases():
    rng = np.random.default_rng(20261202)
    cases = [
        ((0, 0, 0, 0), (0, 0)),
        ((0, 0, 0, 0), (5, 0)),
        ((1, 0, 0, 0), (0, 0)),
        ((M32, 0, 0, 0), (1, 2)),          # the next counter carries into word 1
        ((0, 1, 0, 0), (1, 2)),            # ... and lands here
        ((M32, M32, 0, 0), (M32, M32)),
        ((0, 0, 1, 0), (7, 9)),            # non-zero words 2 and 3
        ((0, 0, 0, 1), (7, 9)),
        ((0x12345678, 0x9ABCDEF0, 0x0FEDCBA9, 0x87654321), (0xDEADBEEF, 0xCAFEBABE)),
    ]
    for _ in range(32):
        c = tuple(int(x) for x in rng.integers(0, 1 << 32, size=4))
        k = tuple(int(x) for x in rng.integers(0, 1 << 32, size=2))
        cases.append((c, k))
    return cases


def test_blocks_match_rocrand(probe):
    cases = _cases()
    got = probe([f"w {c[0]} {c[1]} {c[2]} {c[3]} {k[0]} {k[1]}" for c, k in cases])
    assert len(got) == len(cases)
    for (c, k), want in zip(cases, got):
        assert philox.philox4x32(c, k) == want, (c, k)


def test_uniform_layout_matches_rocrand(probe):
    """The oracle's u at (seed, offset): counter (offset lo, offset hi, 0, 0),
    key (seed lo, seed hi), u = (x0 >> 8) 2^-24. Offsets cross 2^32 (the high
    counter word) and reach 2^61."""
    rng = np.random.default_rng(7)
    pairs = [(0, 0), (1, 1), (0xDEADBEEFDEADBEEF, 0), (3, (1 << 32) - 1), (3, 1 << 32),
             (3, (1 << 32) + 1), ((5 << 32) | 17, 123456789012), (42, (1 << 61) - 1)]
    pairs += [(int(s), int(o)) for s, o in zip(rng.integers(0, 1 << 63, size=24),
                                              rng.integers(0, 1 << 40, size=24))]
    got = probe([f"u {s} {o}" for s, o in pairs])
    for (s, o), (x0,) in zip(pairs, got):
        assert oracle.uniform(s, o) == (x0 >> 8) * 2.0 ** -24, (s, o)
