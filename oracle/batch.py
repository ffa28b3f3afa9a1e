"""Row loops over a [B, V] batch in the C-ABI's input layout.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module.

Inputs are host numpy arrays in exactly the layout the library reads: logits as
float32, or bfloat16 bit patterns stored as uint16; an optional packed uint32
legal-token bitmask of ceil(V/32) words per row; per-row float32 temperature and
top-p, int32 top-k, uint64 seed and offset. Each row is handed to
``sampling.filter_row`` on its own.
"""

import numpy as np

from .philox import uniform
from .sampling import (ROW_OK, argmax_row, bf16_bits_to_float64, filter_row,
                       legal_from_bitmask, sample_from)


def decode_logits(row, dtype):
    """One row of logits widened exactly to float64. dtype: 'f32' or 'bf16'."""
    if dtype == "bf16":
        return bf16_bits_to_float64(row)
    return np.asarray(row, dtype=np.float32).astype(np.float64)


def _legal(bitmask, r, V):
    if bitmask is None:
        return None
    return legal_from_bitmask(bitmask[r], V)


def filter_batch(logits, dtype, T, k, p, bitmask=None, rows=None):
    """Filter the listed rows (default: all). Returns {row: RowResult}."""
    B, V = logits.shape
    rows = range(B) if rows is None else rows
    out = {}
    for r in rows:
        out[r] = filter_row(decode_logits(logits[r], dtype), T[r], k[r], p[r],
                            _legal(bitmask, r, V))
    return out


def sample_batch(results, seeds, offsets, uniforms=None):
    """Sample every filtered row.

    Returns {row: (token, new_offset, u, distance_to_cdf_boundary)}. Rows that
    are not OK, and greedy rows, consume no random number: their offset is
    returned unchanged (and the token is -1 for error rows).
    """
    out = {}
    for r, res in results.items():
        off = int(offsets[r])
        if res.status != ROW_OK:
            out[r] = (-1, off, None, np.inf)
            continue
        if res.greedy:
            out[r] = (int(res.kept[0]), off, None, np.inf)
            continue
        if uniforms is not None:
            u = float(uniforms[r])
            new_off = off
        else:
            u = uniform(int(seeds[r]), off)
            new_off = off + 1
        tok, dist = sample_from(res.kept, res.q, u)
        out[r] = (tok, new_off, u, dist)
    return out


def argmax_batch(logits, dtype, bitmask=None, rows=None):
    """Greedy selection for the listed rows: {row: (status, token)}."""
    B, V = logits.shape
    rows = range(B) if rows is None else rows
    return {r: argmax_row(decode_logits(logits[r], dtype), _legal(bitmask, r, V))
            for r in rows}
