"""CPU oracle for exact top-k / top-p filtering and sampling.

TEST INFRASTRUCTURE. This package is the slow, obviously correct definition the
HIP path is compared with. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import, call or execute anything under oracle/. It shares
no code, header, table or constant generator with the product package
``top_sampling_vocabs_amd`` and imports nothing from it; the product package
never imports it.

Modules:
* ``sampling`` — fp64 definition: stable full-row sort, top-k, top-p, greedy,
  statuses, inverse-CDF walk in token-id order, the drawn token's
  log-probability, keep-mask packing.
* ``exact``    — rational-arithmetic mode for the pages' worked examples and a
  brute-force subset enumerator for tiny vocabularies.
* ``philox``   — Philox4x32-10 from its published definition, pinned by known
  answers from rocRAND's independent implementation (host build of its header).
* ``spec``     — exact speculative-decoding verification (accept with
  min(1, p/q), else resample from max(0, p - q)) over candidate lists.
* ``penalties`` — repetition and presence penalties over each row's history,
  and an additive logit bias list per row.
* ``batch``    — row loops over a whole [B, V] batch with the exact input layout
  the C-ABI uses (fp32 or bf16 bit patterns, packed uint32 bitmask).
"""

from .sampling import (  # noqa: F401
    ROW_OK, ROW_EMPTY, ROW_ALL_NEG_INF, ROW_NONFINITE, ROW_BAD_PARAM,
    ROW_CAND_OVERFLOW, TOP_P_BAND, RowResult, bf16_bits_to_float64,
    legal_from_bitmask, filter_row, sample_from, token_logprob, top_logprobs_row,
    keep_mask_words,
    argmax_row, params_valid)
from .exact import exact_filter, brute_force_filter  # noqa: F401
from .philox import philox4x32, uniform  # noqa: F401
from .batch import decode_logits, filter_batch, sample_batch, argmax_batch  # noqa: F401
from .spec import spec_verify_row, spec_verify_batch  # noqa: F401
from .penalties import (apply_penalties_row, apply_penalties_batch,  # noqa: F401
                        apply_logit_bias_row, apply_logit_bias_batch)
