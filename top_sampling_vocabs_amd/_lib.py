"""ctypes binding of libqs.so (the C ABI in include/qs.h).

This layer only marshals arguments: tensors become device pointers, the
current torch stream becomes the hipStream_t. Every step of the filtering and
sampling runs in the HIP kernels; there is no CPU or torch fallback. If the
library is missing the first call raises.
"""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqs.so")

QS_OK = 0
QS_ERR_INVALID_ARG = 1
QS_ERR_WORKSPACE = 2
QS_ERR_HIP = 3

ROW_OK = 0
ROW_EMPTY = 1
ROW_ALL_NEG_INF = 2
ROW_NONFINITE = 3
ROW_BAD_PARAM = 4
ROW_CAND_OVERFLOW = 5
ROW_INTERNAL = 6

QS_F32 = 0
QS_BF16 = 1

FLAG_FORCE_MISS = 1
FLAG_NO_TRUNCATION = 2
FLAG_PIVOT_SEARCH = 4
FLAG_STREAM = 8
FLAG_BINARY_PIVOT = 16
FLAG_SORT_SUBSET = 32

# size of the fixed per-GPU scratch behind qs_sample_noalloc (QS_SCRATCH_BYTES)
SCRATCH_BYTES = 64 << 20

EXPORTS = ("qs_workspace_bytes", "qs_filter_mask", "qs_sample", "qs_sample_noalloc", "qs_argmax",
           "qs_processors_workspace_bytes", "qs_sample_processed", "qs_filter_mask_processed",
           "qs_sample_top_logprobs",
           "qs_spec_verify",
           "qs_apply_penalties", "qs_apply_logit_bias", "qs_top_logprobs", "qs_version")

_lib = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int
_u32 = ctypes.c_uint32
_sz = ctypes.c_size_t


class QsProcessors(ctypes.Structure):
    """The C struct QsProcessors: device pointers of the logit processors."""
    _fields_ = [("history", ctypes.c_void_p), ("history_cap", ctypes.c_int64),
                ("history_count", ctypes.c_void_p), ("repetition_penalty", ctypes.c_void_p),
                ("presence_penalty", ctypes.c_void_p), ("frequency_penalty", ctypes.c_void_p),
                ("bias_ids", ctypes.c_void_p), ("bias_values", ctypes.c_void_p),
                ("bias_cap", ctypes.c_int64), ("bias_count", ctypes.c_void_p)]


def load(path=LIB_PATH):
    """Load libqs.so and declare the C signatures. Raises if it is missing."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m top_sampling_vocabs_amd.build`")
    lib = ctypes.CDLL(path, mode=ctypes.RTLD_LOCAL)
    lib.qs_workspace_bytes.restype = _sz
    lib.qs_workspace_bytes.argtypes = [_i64, _i64, _i32, _i64]   # B, V, dtype, cand_cap
    lib.qs_filter_mask.restype = _i32
    lib.qs_filter_mask.argtypes = [
        _p, _i32, _i64, _i64, _i64,          # logits, dtype, B, V, row_stride
        _p, _p, _p,                          # temperature, top_k, top_p
        _p, _i64,                            # bitmask, bitmask_stride
        _p, _p, _p, _p, _i64,                # keep_mask, cand_ids, cand_probs, cand_count, cand_cap
        _p, _p, _p, _u32,                    # dense, row_status, debug, flags
        _p, _sz, _p]                         # workspace, workspace_bytes, stream
    lib.qs_sample.restype = _i32
    lib.qs_sample.argtypes = [
        _p, _i32, _i64, _i64, _i64,
        _p, _p, _p,
        _p, _i64,
        _p, _p, _p, _p, _p,                  # seed, offset, uniforms, tokens, logprobs
        _p, _p, _p, _p, _i64,
        _p, _p, _p, _u32,
        _p, _sz, _p]
    lib.qs_sample_noalloc.restype = _i32
    lib.qs_sample_noalloc.argtypes = lib.qs_sample.argtypes[:-3] + [_p]
    lib.qs_processors_workspace_bytes.restype = _sz
    lib.qs_processors_workspace_bytes.argtypes = [_i64, _i64, _i32]   # B, V, dtype
    lib.qs_sample_processed.restype = _i32
    lib.qs_sample_processed.argtypes = lib.qs_sample.argtypes[:-3] + [_p, _p, _sz, _p]
    lib.qs_sample_top_logprobs.restype = _i32
    lib.qs_sample_top_logprobs.argtypes = lib.qs_sample.argtypes[:-3] + [_i64, _p, _p, _p, _sz,
                                                                         _p]
    lib.qs_filter_mask_processed.restype = _i32
    lib.qs_filter_mask_processed.argtypes = lib.qs_filter_mask.argtypes[:-3] + [_p, _p, _sz, _p]
    lib.qs_argmax.restype = _i32
    lib.qs_argmax.argtypes = [_p, _i32, _i64, _i64, _i64, _p, _i64, _p, _p, _p]
    lib.qs_spec_verify.restype = _i32
    lib.qs_spec_verify.argtypes = [
        _i64, _p, _p, _p, _i64,              # B, target ids, probs, count, cap
        _p, _p, _p, _i64,                    # draft ids, probs, count, cap
        _p, _p, _p,                          # draft tokens, u_accept, u_resample
        _p, _p, _p, _p]                      # tokens, accepted, row_status, stream
    lib.qs_apply_penalties.restype = _i32
    lib.qs_apply_penalties.argtypes = [
        _p, _i32, _i64, _i64, _i64,          # logits, dtype, B, V, row_stride
        _p, _i64, _p,                        # history, history_cap, history_count
        _p, _p, _p, _p, _p]                  # repetition, presence, frequency, status, stream
    lib.qs_apply_logit_bias.restype = _i32
    lib.qs_apply_logit_bias.argtypes = [
        _p, _i32, _i64, _i64, _i64,          # logits, dtype, B, V, row_stride
        _p, _p, _i64, _p,                    # bias ids, values, cap, count
        _p, _p]                              # row_status, stream
    lib.qs_top_logprobs.restype = _i32
    lib.qs_top_logprobs.argtypes = [
        _i64, _p, _p, _p, _i64, _i64,        # B, ids, probs, count, cap, n
        _p, _p, _p, _p]                      # top ids, top logprobs, row_status, stream
    lib.qs_version.restype = ctypes.c_char_p
    lib.qs_version.argtypes = []
    if path == LIB_PATH:
        _lib = lib
    return lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(logits):
    import torch
    if logits.dtype == torch.float32:
        return QS_F32
    if logits.dtype == torch.bfloat16:
        return QS_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {logits.dtype}")


def _check_rowvec(t, B, dtype, name):
    if t is None or t.dim() != 1 or t.shape[0] != B or t.dtype != dtype or not t.is_cuda \
            or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous CUDA tensor of shape [{B}] and {dtype}")


def _check_logits(logits, bitmask):
    if logits.dim() != 2 or not logits.is_cuda or logits.stride(1) != 1:
        raise ValueError("logits must be a CUDA tensor [B, V] with unit column stride")
    B, V = logits.shape
    if bitmask is not None:
        import torch
        if bitmask.dim() != 2 or bitmask.shape[0] != B or bitmask.dtype != torch.int32 \
                or bitmask.stride(1) != 1 or not bitmask.is_cuda:
            raise ValueError("bitmask must be an int32 CUDA tensor [B, >= ceil(V/32)] "
                             "holding the uint32 words")
    return B, V


def _status(rc, what):
    if rc != QS_OK:
        name = {QS_ERR_INVALID_ARG: "QS_ERR_INVALID_ARG", QS_ERR_WORKSPACE: "QS_ERR_WORKSPACE",
                QS_ERR_HIP: "QS_ERR_HIP"}.get(rc, rc)
        raise RuntimeError(f"{what} returned {name}")


def workspace_bytes(B, V, dtype_code, cand_cap=0):
    """Device scratch (bytes) a filter_mask / sample call on [B, V] logits needs."""
    return int(load().qs_workspace_bytes(int(B), int(V), int(dtype_code), int(cand_cap)))


def workspace_for(logits, cand_cap=0):
    """A workspace tensor (uint8, on the logits' device) sized for these logits,
    or None when the call needs none. Reuse it across calls on one stream."""
    import torch
    B, V = logits.shape
    n = workspace_bytes(B, V, _dtype_code(logits), cand_cap)
    return torch.empty(n, dtype=torch.uint8, device=logits.device) if n else None


def _workspace_args(workspace, logits, cand_cap):
    if workspace is None:
        workspace = workspace_for(logits, cand_cap)
    if workspace is None:
        return None, 0, None
    if not workspace.is_cuda or workspace.device != logits.device:
        raise ValueError("workspace must be a CUDA tensor on the logits' device")
    return _ptr(workspace), workspace.numel() * workspace.element_size(), workspace


def filter_mask(logits, temperature, top_k, top_p, bitmask=None, *, cand_cap=0,
                dense=False, debug=False, flags=0, workspace=None, processors=None):
    """Kept-candidate mask and renormalised probabilities for every row.

    logits [B, V] float32 / bfloat16 (CUDA); temperature, top_p float32 [B];
    top_k int32 [B]; bitmask int32 [B, >= ceil(V/32)] holding uint32 words, or
    None. Returns a dict of device tensors: keep_mask (int32 words [B, W]),
    status [B], and if requested cand_ids / cand_probs [B, cand_cap],
    cand_count [B], dense [B, V], debug [B, 4]. Enqueued on the current stream;
    synchronise before reading. workspace: a device buffer of at least
    workspace_bytes(...) bytes (workspace_for(logits) makes one); allocated
    per call when omitted.
    """
    import torch
    lib = load()
    B, V = _check_logits(logits, bitmask)
    dev = logits.device
    _check_rowvec(temperature, B, torch.float32, "temperature")
    _check_rowvec(top_k, B, torch.int32, "top_k")
    _check_rowvec(top_p, B, torch.float32, "top_p")
    W = (V + 31) // 32
    out = {"keep_mask": torch.empty((B, W), dtype=torch.int32, device=dev),
           "status": torch.empty(B, dtype=torch.int32, device=dev)}
    if cand_cap:
        out["cand_ids"] = torch.empty((B, cand_cap), dtype=torch.int32, device=dev)
        out["cand_probs"] = torch.empty((B, cand_cap), dtype=torch.float32, device=dev)
        out["cand_count"] = torch.empty(B, dtype=torch.int32, device=dev)
    if dense:
        out["dense"] = torch.empty((B, V), dtype=torch.float32, device=dev)
    if debug:
        out["debug"] = torch.empty((B, 4), dtype=torch.int32, device=dev)
    args = (_ptr(logits), _dtype_code(logits), B, V, logits.stride(0),
            _ptr(temperature), _ptr(top_k), _ptr(top_p),
            _ptr(bitmask), 0 if bitmask is None else bitmask.stride(0),
            _ptr(out["keep_mask"]), _ptr(out.get("cand_ids")), _ptr(out.get("cand_probs")),
            _ptr(out.get("cand_count")), int(cand_cap), _ptr(out.get("dense")),
            _ptr(out["status"]), _ptr(out.get("debug")), int(flags))
    if processors is not None:
        pr, ws = _processors_args(processors, logits, workspace)
        rc = lib.qs_filter_mask_processed(*args, ctypes.byref(pr), _ptr(ws),
                                          ws.numel() * ws.element_size(), _stream(dev))
        _status(rc, "qs_filter_mask_processed")
        return out
    ws_p, ws_n, _ws = _workspace_args(workspace, logits, cand_cap)
    rc = lib.qs_filter_mask(*args, ws_p, ws_n, _stream(dev))
    _status(rc, "qs_filter_mask")
    return out


def _processors_args(proc, logits, workspace):
    """QsProcessors from a dict of device tensors: history [B, cap] int32,
    history_count [B] int32, repetition / presence [B] float32, frequency [B]
    float32 (optional); bias_ids [B, cap] int32, bias_values [B, cap] float32,
    bias_count [B] int32. Either group may be absent. Also returns a workspace
    of processors_workspace_bytes (the given one, or a new one)."""
    import torch
    lib = load()
    B, V = int(logits.shape[0]), int(logits.shape[1])
    dev = logits.device
    pr = QsProcessors()
    keep = []
    if proc.get("history") is not None:
        h = proc["history"]
        if h.dim() != 2 or h.shape[0] != B or h.dtype != torch.int32 or not h.is_contiguous():
            raise ValueError("history: need a contiguous [B, cap] int32 tensor")
        _check_rowvec(proc["history_count"], B, torch.int32, "history_count")
        _check_rowvec(proc["repetition"], B, torch.float32, "repetition")
        _check_rowvec(proc["presence"], B, torch.float32, "presence")
        if proc.get("frequency") is not None:
            _check_rowvec(proc["frequency"], B, torch.float32, "frequency")
        pr.history, pr.history_cap = _ptr(h), int(h.shape[1])
        pr.history_count = _ptr(proc["history_count"])
        pr.repetition_penalty = _ptr(proc["repetition"])
        pr.presence_penalty = _ptr(proc["presence"])
        pr.frequency_penalty = _ptr(proc.get("frequency"))
    if proc.get("bias_ids") is not None:
        bi, bv = proc["bias_ids"], proc["bias_values"]
        if bi.dim() != 2 or bi.shape[0] != B or bi.dtype != torch.int32 or bv.shape != bi.shape \
                or bv.dtype != torch.float32 or not bi.is_contiguous() or not bv.is_contiguous():
            raise ValueError("bias_ids / bias_values: need contiguous [B, cap] int32 / float32")
        _check_rowvec(proc["bias_count"], B, torch.int32, "bias_count")
        pr.bias_ids, pr.bias_values, pr.bias_cap = _ptr(bi), _ptr(bv), int(bi.shape[1])
        pr.bias_count = _ptr(proc["bias_count"])
    need = lib.qs_processors_workspace_bytes(B, V, _dtype_code(logits))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    return pr, workspace


def processors_workspace_for(logits):
    """A device workspace for processed calls on these logits."""
    import torch
    n = load().qs_processors_workspace_bytes(int(logits.shape[0]), int(logits.shape[1]),
                                             _dtype_code(logits))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=logits.device)


def sample(logits, temperature, top_k, top_p, bitmask=None, *, seed=None, offset=None,
           uniforms=None, keep_mask=False, cand_cap=0, dense=False, debug=False,
           logprobs=False, flags=0, workspace=None, processors=None, top_n=0):
    """Filter and draw one token per row.

    seed, offset: int64 [B] CUDA tensors holding the uint64 RNG state; offset is
    advanced in place by the randomness actually consumed. uniforms: float64
    [B] to use fixed u values instead (offsets untouched). logprobs: also
    return the log-probability of each drawn token under the distribution it
    was drawn from (float32 [B]). Returns a dict with tokens [B], status [B]
    and the optional outputs of filter_mask. workspace as for filter_mask.
    processors: a dict of logit-processor tensors (see _processors_args),
    applied inside the call (qs_sample_processed); the logits are only read.
    top_n: also return each row's top_n most probable tokens (top_ids [B, n]
    int32) and their log-probabilities (top_logprobs [B, n] float32), written
    by the same launch (qs_sample_top_logprobs; needs cand_cap).
    """
    return _sample(logits, temperature, top_k, top_p, bitmask, seed, offset, uniforms,
                   keep_mask, cand_cap, dense, debug, logprobs, flags, workspace, False,
                   processors, top_n)


def sample_noalloc(logits, temperature, top_k, top_p, bitmask=None, *, seed=None,
                   offset=None, uniforms=None, keep_mask=False, cand_cap=0, dense=False,
                   debug=False, logprobs=False, flags=0):
    """sample() through qs_sample_noalloc: the library's fixed per-GPU scratch
    instead of a workspace (the outputs are still allocated here). Calls on
    one GPU must not overlap in time."""
    return _sample(logits, temperature, top_k, top_p, bitmask, seed, offset, uniforms,
                   keep_mask, cand_cap, dense, debug, logprobs, flags, None, True)


def _sample(logits, temperature, top_k, top_p, bitmask, seed, offset, uniforms, keep_mask,
            cand_cap, dense, debug, logprobs, flags, workspace, noalloc, processors=None,
            top_n=0):
    import torch
    lib = load()
    B, V = _check_logits(logits, bitmask)
    dev = logits.device
    _check_rowvec(temperature, B, torch.float32, "temperature")
    _check_rowvec(top_k, B, torch.int32, "top_k")
    _check_rowvec(top_p, B, torch.float32, "top_p")
    if uniforms is None:
        _check_rowvec(seed, B, torch.int64, "seed")
        _check_rowvec(offset, B, torch.int64, "offset")
    else:
        _check_rowvec(uniforms, B, torch.float64, "uniforms")
    W = (V + 31) // 32
    out = {"tokens": torch.empty(B, dtype=torch.int32, device=dev),
           "status": torch.empty(B, dtype=torch.int32, device=dev)}
    if logprobs:
        out["logprobs"] = torch.empty(B, dtype=torch.float32, device=dev)
    if keep_mask:
        out["keep_mask"] = torch.empty((B, W), dtype=torch.int32, device=dev)
    if cand_cap:
        out["cand_ids"] = torch.empty((B, cand_cap), dtype=torch.int32, device=dev)
        out["cand_probs"] = torch.empty((B, cand_cap), dtype=torch.float32, device=dev)
        out["cand_count"] = torch.empty(B, dtype=torch.int32, device=dev)
    if dense:
        out["dense"] = torch.empty((B, V), dtype=torch.float32, device=dev)
    if debug:
        out["debug"] = torch.empty((B, 4), dtype=torch.int32, device=dev)
    args = (
        _ptr(logits), _dtype_code(logits), B, V, logits.stride(0),
        _ptr(temperature), _ptr(top_k), _ptr(top_p),
        _ptr(bitmask), 0 if bitmask is None else bitmask.stride(0),
        _ptr(seed) if uniforms is None else None,
        _ptr(offset) if uniforms is None else None, _ptr(uniforms), _ptr(out["tokens"]),
        _ptr(out.get("logprobs")), _ptr(out.get("keep_mask")), _ptr(out.get("cand_ids")),
        _ptr(out.get("cand_probs")), _ptr(out.get("cand_count")), int(cand_cap),
        _ptr(out.get("dense")), _ptr(out["status"]), _ptr(out.get("debug")), int(flags))
    if noalloc:
        rc = lib.qs_sample_noalloc(*args, _stream(dev))
        _status(rc, "qs_sample_noalloc")
        return out
    if processors is not None:
        pr, ws = _processors_args(processors, logits, workspace)
        rc = lib.qs_sample_processed(*args, ctypes.byref(pr), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(dev))
        _status(rc, "qs_sample_processed")
        return out
    ws_p, ws_n, _ws = _workspace_args(workspace, logits, cand_cap)
    if top_n:
        out["top_ids"] = torch.empty((B, top_n), dtype=torch.int32, device=dev)
        out["top_logprobs"] = torch.empty((B, top_n), dtype=torch.float32, device=dev)
        rc = lib.qs_sample_top_logprobs(*args, int(top_n), _ptr(out["top_ids"]),
                                        _ptr(out["top_logprobs"]), ws_p, ws_n, _stream(dev))
        _status(rc, "qs_sample_top_logprobs")
        return out
    rc = lib.qs_sample(*args, ws_p, ws_n, _stream(dev))
    _status(rc, "qs_sample")
    return out


def argmax(logits, bitmask=None):
    """Greedy token per row: (tokens [B] int32, status [B] int32)."""
    import torch
    lib = load()
    B, V = _check_logits(logits, bitmask)
    dev = logits.device
    tokens = torch.empty(B, dtype=torch.int32, device=dev)
    status = torch.empty(B, dtype=torch.int32, device=dev)
    rc = lib.qs_argmax(_ptr(logits), _dtype_code(logits), B, V, logits.stride(0),
                       _ptr(bitmask), 0 if bitmask is None else bitmask.stride(0),
                       _ptr(tokens), _ptr(status), _stream(dev))
    _status(rc, "qs_argmax")
    return tokens, status


def spec_verify(target_ids, target_probs, target_count, draft_ids, draft_probs, draft_count,
                draft_tokens, u_accept, u_resample):
    """Exact speculative verification of one draft token per row over candidate
    lists (as filter_mask / sample return them). Returns a dict with tokens,
    accepted and status, int32 [B] each."""
    import torch
    lib = load()
    B = int(draft_tokens.shape[0])
    dev = draft_tokens.device
    for t, dt, name in ((target_ids, torch.int32, "target_ids"),
                        (target_probs, torch.float32, "target_probs"),
                        (draft_ids, torch.int32, "draft_ids"),
                        (draft_probs, torch.float32, "draft_probs")):
        if t.dim() != 2 or t.shape[0] != B or t.dtype != dt or not t.is_contiguous() \
                or t.device != dev:
            raise ValueError(f"{name}: need a contiguous [B, cap] {dt} tensor on {dev}")
    if target_ids.shape != target_probs.shape or draft_ids.shape != draft_probs.shape:
        raise ValueError("ids and probs of a list must have the same shape")
    _check_rowvec(target_count, B, torch.int32, "target_count")
    _check_rowvec(draft_count, B, torch.int32, "draft_count")
    _check_rowvec(draft_tokens, B, torch.int32, "draft_tokens")
    _check_rowvec(u_accept, B, torch.float64, "u_accept")
    _check_rowvec(u_resample, B, torch.float64, "u_resample")
    out = {k: torch.empty(B, dtype=torch.int32, device=dev)
           for k in ("tokens", "accepted", "status")}
    rc = lib.qs_spec_verify(
        B, _ptr(target_ids), _ptr(target_probs), _ptr(target_count), target_ids.shape[1],
        _ptr(draft_ids), _ptr(draft_probs), _ptr(draft_count), draft_ids.shape[1],
        _ptr(draft_tokens), _ptr(u_accept), _ptr(u_resample),
        _ptr(out["tokens"]), _ptr(out["accepted"]), _ptr(out["status"]), _stream(dev))
    _status(rc, "qs_spec_verify")
    return out


def apply_penalties(logits, history, history_count, repetition, presence, frequency=None):
    """Repetition, presence and (optional) frequency penalties over each row's
    history, applied to logits in place. history: int32 [B, cap];
    history_count: int32 [B]; repetition, presence, frequency: float32 [B].
    Returns the row status (int32 [B])."""
    import torch
    lib = load()
    if logits.dim() != 2 or not logits.is_cuda or logits.stride(1) != 1:
        raise ValueError("logits must be a CUDA tensor [B, V] with unit column stride")
    B, V = logits.shape
    if history.dim() != 2 or history.shape[0] != B or history.dtype != torch.int32 \
            or not history.is_contiguous() or history.device != logits.device:
        raise ValueError("history must be a contiguous int32 [B, cap] tensor on the logits' device")
    _check_rowvec(history_count, B, torch.int32, "history_count")
    _check_rowvec(repetition, B, torch.float32, "repetition")
    _check_rowvec(presence, B, torch.float32, "presence")
    if frequency is not None:
        _check_rowvec(frequency, B, torch.float32, "frequency")
    status = torch.empty(B, dtype=torch.int32, device=logits.device)
    rc = lib.qs_apply_penalties(_ptr(logits), _dtype_code(logits), B, V, logits.stride(0),
                                _ptr(history), history.shape[1], _ptr(history_count),
                                _ptr(repetition), _ptr(presence), _ptr(frequency), _ptr(status),
                                _stream(logits.device))
    _status(rc, "qs_apply_penalties")
    return status


def apply_logit_bias(logits, bias_ids, bias_values, bias_count):
    """Additive logit bias per row, applied to logits in place. bias_ids: int32
    [B, cap]; bias_values: float32 [B, cap]; bias_count: int32 [B]. Returns the
    row status (int32 [B])."""
    import torch
    lib = load()
    if logits.dim() != 2 or not logits.is_cuda or logits.stride(1) != 1:
        raise ValueError("logits must be a CUDA tensor [B, V] with unit column stride")
    B, V = logits.shape
    for t, dt, name in ((bias_ids, torch.int32, "bias_ids"), (bias_values, torch.float32,
                                                              "bias_values")):
        if t.dim() != 2 or t.shape[0] != B or t.dtype != dt or not t.is_contiguous() \
                or t.device != logits.device:
            raise ValueError(f"{name}: need a contiguous [B, cap] {dt} tensor on the logits' device")
    if bias_ids.shape != bias_values.shape:
        raise ValueError("bias_ids and bias_values must have the same shape")
    _check_rowvec(bias_count, B, torch.int32, "bias_count")
    status = torch.empty(B, dtype=torch.int32, device=logits.device)
    rc = lib.qs_apply_logit_bias(_ptr(logits), _dtype_code(logits), B, V, logits.stride(0),
                                 _ptr(bias_ids), _ptr(bias_values), bias_ids.shape[1],
                                 _ptr(bias_count), _ptr(status), _stream(logits.device))
    _status(rc, "qs_apply_logit_bias")
    return status


def top_logprobs(cand_ids, cand_probs, cand_count, n):
    """The n most probable tokens of each candidate list (as filter_mask / sample
    return them) and their log-probabilities: (ids int32 [B, n], logprobs
    float32 [B, n], status int32 [B])."""
    import torch
    lib = load()
    B = int(cand_count.shape[0])
    dev = cand_count.device
    for t, dt, name in ((cand_ids, torch.int32, "cand_ids"), (cand_probs, torch.float32,
                                                              "cand_probs")):
        if t.dim() != 2 or t.shape[0] != B or t.dtype != dt or not t.is_contiguous() \
                or t.device != dev:
            raise ValueError(f"{name}: need a contiguous [B, cap] {dt} tensor on {dev}")
    _check_rowvec(cand_count, B, torch.int32, "cand_count")
    ids = torch.empty((B, n), dtype=torch.int32, device=dev)
    lp = torch.empty((B, n), dtype=torch.float32, device=dev)
    status = torch.empty(B, dtype=torch.int32, device=dev)
    rc = lib.qs_top_logprobs(B, _ptr(cand_ids), _ptr(cand_probs), _ptr(cand_count),
                             cand_ids.shape[1], int(n), _ptr(ids), _ptr(lp), _ptr(status),
                             _stream(dev))
    _status(rc, "qs_top_logprobs")
    return ids, lp, status
