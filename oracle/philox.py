"""Philox4x32-10 counter-based generator, written from its published definition.

TEST INFRASTRUCTURE: part of the CPU oracle. Only tests/, __graft_entry__.smoke()
and bench.py's cpu_baseline leg may import it.

Source of the algorithm: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3", SC'11 — the Philox-4x32 bijection
with 10 rounds: each round multiplies counter words 0 and 2 by two fixed 32-bit
multipliers, takes the high/low halves of the 64-bit products, XORs the high
halves with the other two counter words and the two key words, and permutes;
between rounds the key is advanced by two Weyl increments.

Why it is here: the sampling contract needs an explicit per-row RNG state
(seed, offset) that the caller advances by what was actually consumed
(page "Attention算完，还没有选出下一个token", section 06; also page
"Sampling 系统设计", the seed/per-sequence generator discussion). The pages do
not name a generator; the plain reading used throughout is Philox4x32-10 with
counter = (offset_lo, offset_hi, 0, 0), key = (seed_lo, seed_hi) and a 24-bit
uniform u = (x0 >> 8) * 2**-24 in [0, 1).

Pinned by known answers from an independent implementation: rocRAND's
Philox4x32-10 engine, compiled for the host from its header source in the ROCm
installation (tests/test_philox_rocrand.py), on counters with non-zero high
words and carries across 2**32, and for the (seed, offset) layout above (the
draw at offset n is rocRAND's first output after rocrand_init(seed, 0, 4 n)).
The pages themselves print no Philox values.
"""

MASK32 = 0xFFFFFFFF

# Multipliers and Weyl key increments as published for Philox-4x32.
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9  # golden ratio
PHILOX_W1 = 0xBB67AE85  # sqrt(3) - 1

ROUNDS = 10


def _mul_hi_lo(a, b):
    prod = (a * b) & 0xFFFFFFFFFFFFFFFF
    return prod >> 32, prod & MASK32


def philox4x32(counter, key, rounds=ROUNDS):
    """Return the 4 output words for a 4-word counter and a 2-word key."""
    c0, c1, c2, c3 = (int(x) & MASK32 for x in counter)
    k0, k1 = (int(x) & MASK32 for x in key)
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + PHILOX_W0) & MASK32
            k1 = (k1 + PHILOX_W1) & MASK32
        hi0, lo0 = _mul_hi_lo(PHILOX_M0, c0)
        hi1, lo1 = _mul_hi_lo(PHILOX_M1, c2)
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0), lo1, (hi0 ^ c3 ^ k1), lo0
    return c0, c1, c2, c3


def uniform(seed, offset):
    """The single uniform a sampled row consumes at RNG position (seed, offset).

    counter = (offset low word, offset high word, 0, 0), key = (seed low word,
    seed high word); u = (x0 >> 8) / 2**24, so u is one of 2**24 equally
    spaced values in [0, 1).
    """
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    offset = int(offset) & 0xFFFFFFFFFFFFFFFF
    x0, _, _, _ = philox4x32(
        (offset & MASK32, offset >> 32, 0, 0), (seed & MASK32, seed >> 32))
    return (x0 >> 8) * (1.0 / 16777216.0)
