"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws inputs: logits, per-row parameters, legal-token
bitmasks, seeds and offsets. It holds none of the filtering or sampling
arithmetic, so both the CPU oracle and the HIP path can be fed from it.

The pages measure on real models and WikiText-2, which are not available here;
these seeded inputs stand in for them with the vocabulary sizes of the page's
models (128,256; 151,936; 262,144 ~ 262,208) and the logit shapes the
method's Gaussian prior assumes (page "Qrita", key design 1). Five workloads:

1. B=4, V=32000, fp32: N(0,1) plus +6 on 16 distinct random ids per row;
   T=1, k=50, p=0.9 for every row; no bitmask.
2. B=64, V=128256, fp32: N(0, 2^2) background, 20 distinct ids per row replaced
   by N(8, 2) (2 read as a variance: sigma = sqrt 2); per-row k ~ U{1..1024},
   p ~ U[0.5, 1.0), T ~ U[0.5, 1.5); 10% of rows (seeded) greedy, T = 0.
3. B=256, V=151936, bf16: N(0, 3^2) rounded to bf16 (many exact ties); row r
   in group r mod 3: 0 top-k only (k ~ U{20..200}, p = 1), 1 top-p only
   (p ~ U[0.8, 0.99), k = 0), 2 both; T = 1; packed bitmask with each bit set
   with probability 0.3 and at least one legal token per row.
4. B=1024, V=262144, fp32, rows by r mod 3: near-flat N(0, 0.01^2); bimodal
   (a random half of the ids at N(5, 0.1^2), the rest N(0, 0.1^2)); Gaussian
   N(0,1) with 1% of ids adding 3|Cauchy|; k = 4096, p = 0.99, T = 1.
5. B=512, V=151936, bf16: as 3 with per-row T ~ U[0.5, 1.5), plus degenerate
   rows chosen by a seeded permutation: 5% all-masked, 1% with one NaN at a
   legal position, 1% with every logit -inf.

Per-row Philox state: seed = (cfg << 32) | r, offset = 0.
"""

from dataclasses import dataclass

import numpy as np

BASE_SEED = 20260000

FULL_SHAPES = {1: (4, 32000), 2: (64, 128256), 3: (256, 151936),
               4: (1024, 262144), 5: (512, 151936)}
DTYPES = {1: "f32", 2: "f32", 3: "bf16", 4: "f32", 5: "bf16"}


@dataclass
class Workload:
    cfg: int
    dtype: str            # "f32" or "bf16"
    logits: np.ndarray    # float32 [B, V] or uint16 bf16 bits [B, V]
    T: np.ndarray         # float32 [B]
    k: np.ndarray         # int32 [B]
    p: np.ndarray         # float32 [B]
    bitmask: object       # uint32 [B, ceil(V/32)] or None
    seeds: np.ndarray     # uint64 [B]
    offsets: np.ndarray   # uint64 [B]

    @property
    def B(self):
        return self.logits.shape[0]

    @property
    def V(self):
        return self.logits.shape[1]

    @property
    def elem_bytes(self):
        return 2 if self.dtype == "bf16" else 4


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (round to nearest, ties to even)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def pack_bits(bits):
    """Pack a bool [B, V] array LSB-first into uint32 [B, ceil(V/32)] words."""
    B, V = bits.shape
    W = (V + 31) // 32
    padded = np.zeros((B, W * 32), dtype=np.uint8)
    padded[:, :V] = bits
    by = np.packbits(padded.reshape(B, W * 4, 8), axis=2, bitorder="little")
    return by.reshape(B, W * 4).view(np.uint32).copy()


def _random_bitmask(rng, B, V, density):
    bits = rng.random((B, V), dtype=np.float32) < density
    empty = np.nonzero(~bits.any(axis=1))[0]
    for r in empty:
        bits[r, rng.integers(0, V)] = True
    return bits


def _seeds(cfg, B):
    return (np.uint64(cfg) << np.uint64(32)) | np.arange(B, dtype=np.uint64)


def make(cfg, B=None, V=None, seed=None):
    """Build workload ``cfg`` (1..5). B and V default to the full sizes; smaller
    values keep every distribution and row mix, for tests the oracle finishes
    quickly. ``seed`` defaults to BASE_SEED + cfg."""
    fb, fv = FULL_SHAPES[cfg]
    B = fb if B is None else int(B)
    V = fv if V is None else int(V)
    rng = np.random.default_rng(BASE_SEED + cfg if seed is None else seed)
    T = np.ones(B, np.float32)
    k = np.zeros(B, np.int32)
    p = np.ones(B, np.float32)
    bitmask = None
    dtype = DTYPES[cfg]

    if cfg == 1:
        z = rng.standard_normal((B, V), dtype=np.float32)
        for r in range(B):
            z[r, rng.choice(V, size=min(16, V), replace=False)] += np.float32(6.0)
        k[:] = 50
        p[:] = 0.9
        logits = z
    elif cfg == 2:
        z = np.float32(2.0) * rng.standard_normal((B, V), dtype=np.float32)
        for r in range(B):
            ids = rng.choice(V, size=min(20, V), replace=False)
            z[r, ids] = np.float32(8.0) + np.float32(np.sqrt(2.0)) * \
                rng.standard_normal(ids.size, dtype=np.float32)
        k[:] = rng.integers(1, 1025, size=B)
        p[:] = rng.uniform(0.5, 1.0, size=B).astype(np.float32)
        T[:] = rng.uniform(0.5, 1.5, size=B).astype(np.float32)
        greedy = rng.permutation(B)[:max(1, int(round(0.1 * B)))]
        T[greedy] = 0.0
        logits = z
    elif cfg in (3, 5):
        z = np.float32(3.0) * rng.standard_normal((B, V), dtype=np.float32)
        logits = f32_to_bf16_bits(z)
        del z
        grp = np.arange(B) % 3
        kk = rng.integers(20, 201, size=B)
        pp = rng.uniform(0.8, 0.99, size=B).astype(np.float32)
        k[:] = np.where(grp == 1, 0, kk)
        p[:] = np.where(grp == 0, np.float32(1.0), pp)
        bits = _random_bitmask(rng, B, V, 0.3)
        if cfg == 5:
            T[:] = rng.uniform(0.5, 1.5, size=B).astype(np.float32)
            perm = rng.permutation(B)
            n_empty = max(1, int(round(0.05 * B)))
            n_nan = max(1, int(round(0.01 * B)))
            n_ninf = max(1, int(round(0.01 * B)))
            empty_rows = perm[:n_empty]
            nan_rows = perm[n_empty:n_empty + n_nan]
            ninf_rows = perm[n_empty + n_nan:n_empty + n_nan + n_ninf]
            bits[empty_rows] = False
            for r in nan_rows:
                legal_ids = np.nonzero(bits[r])[0]
                logits[r, legal_ids[rng.integers(0, legal_ids.size)]] = 0x7FC0
            logits[ninf_rows] = 0xFF80
        bitmask = pack_bits(bits)
        del bits
    elif cfg == 4:
        z = np.empty((B, V), np.float32)
        for r in range(B):
            kind = r % 3
            if kind == 0:
                z[r] = np.float32(0.01) * rng.standard_normal(V, dtype=np.float32)
            elif kind == 1:
                z[r] = np.float32(0.1) * rng.standard_normal(V, dtype=np.float32)
                hi = rng.permutation(V)[:V // 2]
                z[r, hi] += np.float32(5.0)
            else:
                z[r] = rng.standard_normal(V, dtype=np.float32)
                ids = rng.choice(V, size=max(1, V // 100), replace=False)
                z[r, ids] += np.float32(3.0) * np.abs(
                    rng.standard_cauchy(ids.size)).astype(np.float32)
        k[:] = 4096
        p[:] = 0.99
        logits = z
    else:
        raise ValueError(f"unknown workload {cfg}")

    return Workload(cfg=cfg, dtype=dtype, logits=np.ascontiguousarray(logits),
                    T=T, k=k, p=p, bitmask=bitmask, seeds=_seeds(cfg, B),
                    offsets=np.zeros(B, np.uint64))


# Shape of the ablation table on the Qrita page (B=1024, V=128256, k=50, p=0.9).
ABLATION_SHAPE = (1024, 128256)


def make_ablation(B=None, V=None, seed=None):
    """Inputs at the shape of the Qrita page's ablation table: B=1024,
    V=128256 (that page's first model's vocabulary), top-k 50, top-p 0.9,
    T = 1, no bitmask. The page does not describe its logits; fp32 N(0, 2^2)
    i.i.d. values stand in for them. Not one of the five parity workloads: it
    only feeds bench.py --ablation."""
    fb, fv = ABLATION_SHAPE
    B = fb if B is None else int(B)
    V = fv if V is None else int(V)
    rng = np.random.default_rng(BASE_SEED + 100 if seed is None else seed)
    logits = np.float32(2.0) * rng.standard_normal((B, V), dtype=np.float32)
    return Workload(cfg=0, dtype="f32", logits=np.ascontiguousarray(logits),
                    T=np.ones(B, np.float32), k=np.full(B, 50, np.int32),
                    p=np.full(B, 0.9, np.float32), bitmask=None, seeds=_seeds(0, B),
                    offsets=np.zeros(B, np.uint64))


def bytes_read(w):
    """Algorithmic bytes one filter+sample pass must read: the logits once, the
    bitmask once, and the per-row parameters (T, k, p: 4 B each; seed, offset:
    8 B each)."""
    total = w.B * w.V * w.elem_bytes + w.B * (4 + 4 + 4 + 8 + 8)
    if w.bitmask is not None:
        total += w.bitmask.size * 4
    return total


def add_outliers(w, n, value, seed):
    """Set n distinct random ids of every row to `value` (in the workload's
    dtype) and make them legal: the effect of a per-token logit bias that
    pushes a few tokens far down. Modifies w in place."""
    rng = np.random.default_rng(seed)
    B, V = w.logits.shape
    if w.dtype == "bf16":
        bits = np.frombuffer(np.float32(value).tobytes(), np.uint32)[0] >> 16
        v = np.uint16(bits)
    else:
        v = np.float32(value)
    for r in range(B):
        ids = rng.choice(V, size=n, replace=False)
        w.logits[r, ids] = v
        if w.bitmask is not None:
            for t in ids:
                w.bitmask[r, t >> 5] |= np.uint32(1) << np.uint32(t & 31)
