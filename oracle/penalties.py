"""History-dependent logit processors applied before the sampling contract.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module.

Page "Sampling 系统设计：从 logits 到可控生成", repetition-penalty section: a
repetition penalty needs the sequence's earlier tokens and lowers the chance
that a token seen before is picked again; the page leaves the exact formula
open (frameworks differ in how they treat positive and negative logits) and
asks for a simple version in the right place, as a logits processor fed by
the sequence's history. The reading taken here, for each distinct token t in
the row's history with 0 <= t < V:
    z_t <- (z_t / r if z_t > 0 else z_t * r) - a
with r the repetition penalty (> 0; 1 disables it) and a the presence
penalty (0 disables it), each operation in float32 and rounded, the result
stored in the logits' dtype (bfloat16 round-to-nearest-even). A token repeated
in the history is penalised once. Other tokens are untouched. A row with r not
finite or <= 0, a not finite, or a history count outside [0, capacity] is
left unchanged and reported as BAD_PARAM. Applied to the raw logits, before
temperature and the rest of the contract. An optional frequency penalty f
then subtracts f times the token's count in the history (the counting variant
of the same idea: repeated use is penalised more), z_t <- z_t - f*n_t.
"""

import numpy as np

from .sampling import ROW_BAD_PARAM, ROW_OK


def _to_bf16_bits(x32):
    """float32 -> bfloat16 bits, round to nearest even (NaN kept quiet)."""
    b = np.asarray(x32, np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x32, np.float32))
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = ((b[nan] >> 16) | 0x40).astype(np.uint16)
    return r


FREQ_MAX_HISTORY = 4096  # the C ABI's limit on a history with a frequency penalty


def apply_penalties_row(z, dtype, history, count, cap, rep, pres, freq=0.0):
    """z: one row as stored (float32, or bfloat16 bits as uint16). Returns
    (status, new row as stored). A frequency penalty f (0 disables it) then
    subtracts f times the token's number of occurrences n in the history:
    z_t <- z_t - f*n, both operations in float32; with f != 0 the history may
    hold at most FREQ_MAX_HISTORY entries."""
    rep = np.float32(rep)
    pres = np.float32(pres)
    freq = np.float32(freq)
    if not (np.isfinite(rep) and rep > 0 and np.isfinite(pres) and np.isfinite(freq)) \
            or count < 0 or count > cap or (freq != 0 and count > FREQ_MAX_HISTORY):
        return ROW_BAD_PARAM, z.copy()
    counts = {}
    for t in history[:count]:
        counts[int(t)] = counts.get(int(t), 0) + 1
    out = z.copy()
    V = len(z)
    seen = set()
    for t in history[:count]:
        t = int(t)
        if t < 0 or t >= V or t in seen:
            continue
        seen.add(t)
        if dtype == "bf16":
            v = (np.uint32(z[t]) << np.uint32(16)).astype(np.uint32).view(np.float32)
        else:
            v = np.float32(z[t])
        v = np.float32(v / rep) if v > 0 else np.float32(v * rep)
        v = np.float32(v - pres)
        if freq != 0:
            v = np.float32(v - np.float32(freq * np.float32(counts[t])))
        out[t] = _to_bf16_bits(np.array([v]))[0] if dtype == "bf16" else v
    return ROW_OK, out


def apply_penalties_batch(logits, dtype, history, count, rep, pres, freq=None):
    """Row loop: (status [B] int32, new logits) in the input layout."""
    B = logits.shape[0]
    cap = history.shape[1]
    out = logits.copy()
    st = np.zeros(B, np.int32)
    for r in range(B):
        st[r], out[r] = apply_penalties_row(logits[r], dtype, history[r], int(count[r]), cap,
                                            rep[r], pres[r], 0.0 if freq is None else freq[r])
    return st, out


def apply_logit_bias_row(z, dtype, ids, vals, count, cap):
    """Additive logit bias (the processors list of page "Sampling 系统设计：从
    logits 到可控生成" ends with such per-token edits; a bias list is the plain
    reading): z_t <- z_t + b for each (t, b) of the row's first `count` entries
    with 0 <= t < V, in float32, stored in the logits' dtype. A row whose count
    lies outside [0, cap], whose values are not all finite, or that lists one
    token twice is left unchanged and reported as BAD_PARAM."""
    if count < 0 or count > cap:
        return ROW_BAD_PARAM, z.copy()
    V = len(z)
    vals = np.asarray(vals[:count], np.float32)
    if not np.isfinite(vals).all():
        return ROW_BAD_PARAM, z.copy()
    inside = [int(t) for t in ids[:count] if 0 <= int(t) < V]
    if len(set(inside)) != len(inside):
        return ROW_BAD_PARAM, z.copy()
    out = z.copy()
    for t, b in zip(ids[:count], vals):
        t = int(t)
        if t < 0 or t >= V:
            continue
        if dtype == "bf16":
            v = (np.uint32(z[t]) << np.uint32(16)).astype(np.uint32).view(np.float32)
        else:
            v = np.float32(z[t])
        v = np.float32(v + b)
        out[t] = _to_bf16_bits(np.array([v]))[0] if dtype == "bf16" else v
    return ROW_OK, out


def apply_logit_bias_batch(logits, dtype, ids, vals, count):
    """Row loop: (status [B] int32, new logits) in the input layout."""
    B = logits.shape[0]
    cap = ids.shape[1]
    out = logits.copy()
    st = np.zeros(B, np.int32)
    for r in range(B):
        st[r], out[r] = apply_logit_bias_row(logits[r], dtype, ids[r], vals[r], int(count[r]), cap)
    return st, out
