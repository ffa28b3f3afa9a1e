"""Exact top-k / top-p filtering and sampling for MI355X (gfx950).

The work runs in hand-written HIP kernels behind the C ABI declared in
include/qs.h (libqs.so, built in-tree). This package is the thin Python layer
over it: it turns torch tensors into device pointers and passes the current
stream. The library is loaded on first use; calls raise if it is missing.
"""

from ._lib import (  # noqa: F401
    filter_mask, sample, sample_noalloc, argmax, spec_verify, apply_penalties, apply_logit_bias, top_logprobs,
    processors_workspace_for,
    load, workspace_bytes, workspace_for,
    LIB_PATH,
    ROW_OK, ROW_EMPTY, ROW_ALL_NEG_INF, ROW_NONFINITE, ROW_BAD_PARAM,
    ROW_CAND_OVERFLOW, ROW_INTERNAL, FLAG_FORCE_MISS, FLAG_NO_TRUNCATION,
    FLAG_PIVOT_SEARCH, FLAG_STREAM, FLAG_BINARY_PIVOT, FLAG_SORT_SUBSET)

__version__ = "0.1.0"
