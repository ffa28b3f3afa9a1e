"""The C-ABI library without a GPU: it loads, exports every declared symbol,
and rejects bad arguments before making any HIP call."""

import ctypes
import os
import re

import pytest

from top_sampling_vocabs_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qs.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:QS_API\s+)?(?:int|const char\*|size_t)\s+(qs_\w+)\s*\(",
                                 text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libqs.so is not built: run python -m top_sampling_vocabs_amd.build")
    return _lib.load()


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.qs_version().decode().startswith("qs ")


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError):
        _lib.load(str(tmp_path / "nope.so"))


# Fake but aligned device addresses: validation must reject the call before it
# dereferences or launches anything, so no GPU is needed.
A16 = ctypes.c_void_p(0x100000)
A8 = ctypes.c_void_p(0x200000)
WS = ctypes.c_void_p(0x400000)   # a 256-byte aligned workspace address
WSN = 1 << 30                    # and a size above any requirement below


def filt(lib, **kw):
    args = dict(logits=A16, dtype=0, B=4, V=64, stride=64, T=A16, k=A16, p=A16,
                bitmask=None, bms=0, keep=A16, cids=None, cprobs=None, ccount=None,
                cap=0, dense=None, status=A16, dbg=None, flags=0, ws=WS, wsn=WSN, stream=None)
    args.update(kw)
    return lib.qs_filter_mask(args["logits"], args["dtype"], args["B"], args["V"],
                              args["stride"], args["T"], args["k"], args["p"],
                              args["bitmask"], args["bms"], args["keep"], args["cids"],
                              args["cprobs"], args["ccount"], args["cap"], args["dense"],
                              args["status"], args["dbg"], args["flags"], args["ws"],
                              args["wsn"], args["stream"])


@pytest.mark.parametrize("kw", [
    dict(logits=None), dict(dtype=2), dict(dtype=-1), dict(B=-1), dict(B=1 << 22), dict(V=0),
    dict(stride=63), dict(stride=65), dict(logits=ctypes.c_void_p(0x100004)),
    dict(T=None), dict(k=None), dict(p=None), dict(status=None), dict(keep=None),
    dict(cids=A16, ccount=None, cap=8), dict(cids=A16, ccount=A16, cap=0),
    dict(bitmask=A16, bms=1), dict(bitmask=ctypes.c_void_p(0x100002), bms=2),
    dict(flags=64), dict(T=ctypes.c_void_p(0x100001)),
    dict(dtype=1, stride=68),
])
def test_filter_rejects_bad_arguments(lib, kw):
    assert filt(lib, **kw) == _lib.QS_ERR_INVALID_ARG


def test_empty_batch_is_a_no_op(lib):
    assert filt(lib, B=0) == _lib.QS_OK
    assert filt(lib, B=0, logits=None, T=None) == _lib.QS_OK


def smp(lib, **kw):
    args = dict(logits=A16, dtype=1, B=4, V=64, stride=64, T=A16, k=A16, p=A16,
                bitmask=None, bms=0, seed=A8, offset=A8, uni=None, tokens=A16, lp=None,
                keep=None, cids=None, cprobs=None, ccount=None, cap=0, dense=None,
                status=A16, dbg=None, flags=0, ws=WS, wsn=WSN, stream=None)
    args.update(kw)
    return lib.qs_sample(args["logits"], args["dtype"], args["B"], args["V"], args["stride"],
                         args["T"], args["k"], args["p"], args["bitmask"], args["bms"],
                         args["seed"], args["offset"], args["uni"], args["tokens"],
                         args["lp"], args["keep"], args["cids"], args["cprobs"], args["ccount"],
                         args["cap"], args["dense"], args["status"], args["dbg"],
                         args["flags"], args["ws"], args["wsn"], args["stream"])


@pytest.mark.parametrize("kw", [
    dict(tokens=None), dict(seed=None), dict(offset=None), dict(seed=None, offset=None),
    dict(offset=ctypes.c_void_p(0x200004)), dict(uni=ctypes.c_void_p(0x200004)),
    dict(lp=ctypes.c_void_p(0x200002)),
    dict(stride=60), dict(V=-5),
])
def test_sample_rejects_bad_arguments(lib, kw):
    assert smp(lib, **kw) == _lib.QS_ERR_INVALID_ARG


def test_workspace_bytes(lib):
    """bf16 rows longer than the per-row kernel's register tiers (155648
    tokens) need per 4096-token segment of a row 32 bytes and 896 candidate
    entries of 4 bytes, plus 32 bytes per 16384-token chunk (each part
    rounded up to 256 bytes); shorter bf16 rows, fp32 calls and invalid
    arguments need none; cand_cap does not matter."""
    def want(B, V):
        S = -(-V // 16384)
        a256 = lambda x: -(-x // 256) * 256  # noqa: E731
        return a256(B * 4 * S * 32) + a256(B * S * 32) + B * 4 * S * 896 * 4
    for B, V in ((4, 155649), (256, 262144), (512, 200000), (3, 163840), (1, 524289),
                 (2, 64 * 16384)):
        assert lib.qs_workspace_bytes(B, V, 1, 0) == want(B, V), (B, V)
        assert lib.qs_workspace_bytes(B, V, 1, 12345) == want(B, V)
        assert lib.qs_workspace_bytes(B, V, 0, 0) == 0
    for B, V in ((4, 64), (256, 151936), (512, 155648), (3, 16384)):
        assert lib.qs_workspace_bytes(B, V, 1, 0) == 0, (B, V)
    assert lib.qs_workspace_bytes(0, 100, 1, 0) == 0
    assert lib.qs_workspace_bytes(4, 0, 1, 0) == 0
    assert lib.qs_workspace_bytes(-1, 100, 1, 0) == 0
    assert lib.qs_workspace_bytes(4, 100, 7, 0) == 0
    assert lib.qs_workspace_bytes(4, 64 * 16384 + 1, 1, 0) == 0   # rows past 64 chunks


@pytest.mark.parametrize("call", ["filter", "sample"])
def test_workspace_rejected_before_any_hip_call(lib, call):
    """A missing, misaligned or short workspace is QS_ERR_WORKSPACE; argument
    errors are still reported first; fp32 calls need no workspace."""
    V = 200000   # bf16 rows past the register tiers: the chunked pass
    f = (lambda **kw: filt(lib, dtype=1, V=V, stride=V, **kw)) if call == "filter" else \
        (lambda **kw: smp(lib, V=V, stride=V, **kw))
    need = lib.qs_workspace_bytes(4, V, 1, 0)
    assert need > 0
    assert f(ws=None, wsn=0) == _lib.QS_ERR_WORKSPACE
    assert f(ws=None, wsn=need) == _lib.QS_ERR_WORKSPACE
    assert f(ws=ctypes.c_void_p(0x400010), wsn=need) == _lib.QS_ERR_WORKSPACE
    assert f(ws=WS, wsn=need - 1) == _lib.QS_ERR_WORKSPACE
    assert f(ws=None, wsn=0, T=None) == _lib.QS_ERR_INVALID_ARG
    assert f(ws=None, wsn=0, B=0) == _lib.QS_OK


def test_argmax_rejects_bad_arguments(lib):
    def am(**kw):
        a = dict(logits=A16, dtype=0, B=2, V=10, stride=12, bitmask=None, bms=0,
                 tokens=A16, status=A16, stream=None)
        a.update(kw)
        return lib.qs_argmax(a["logits"], a["dtype"], a["B"], a["V"], a["stride"],
                             a["bitmask"], a["bms"], a["tokens"], a["status"], a["stream"])
    assert am(tokens=None) == _lib.QS_ERR_INVALID_ARG
    assert am(status=None) == _lib.QS_ERR_INVALID_ARG
    assert am(stride=10) == _lib.QS_ERR_INVALID_ARG  # 40 bytes is not a multiple of 16
    assert am(V=0) == _lib.QS_ERR_INVALID_ARG
    assert am(B=0) == _lib.QS_OK


def test_spec_verify_rejects_bad_arguments(lib):
    def sv(**kw):
        a = dict(B=2, tids=A16, tp=A16, tc=A16, tcap=8, dids=A16, dp=A16, dc=A16, dcap=8,
                 x=A16, u1=A8, u2=A8, tok=A16, acc=A16, status=A16, stream=None)
        a.update(kw)
        return lib.qs_spec_verify(a["B"], a["tids"], a["tp"], a["tc"], a["tcap"], a["dids"],
                                  a["dp"], a["dc"], a["dcap"], a["x"], a["u1"], a["u2"],
                                  a["tok"], a["acc"], a["status"], a["stream"])
    for kw in (dict(B=-1), dict(B=1 << 22), dict(tcap=0), dict(dcap=0), dict(tids=None), dict(dp=None),
               dict(x=None), dict(u1=None), dict(u2=ctypes.c_void_p(0x200004)),
               dict(acc=ctypes.c_void_p(0x200002)), dict(status=None)):
        assert sv(**kw) == _lib.QS_ERR_INVALID_ARG, kw
    assert sv(B=0) == _lib.QS_OK


def test_apply_penalties_rejects_bad_arguments(lib):
    def ap(**kw):
        a = dict(logits=A16, dtype=1, B=2, V=64, stride=64, hist=A16, cap=8, cnt=A16,
                 rep=A16, pres=A16, freq=None, status=A16, stream=None)
        a.update(kw)
        return lib.qs_apply_penalties(a["logits"], a["dtype"], a["B"], a["V"], a["stride"],
                                      a["hist"], a["cap"], a["cnt"], a["rep"], a["pres"],
                                      a["freq"], a["status"], a["stream"])
    for kw in (dict(dtype=2), dict(B=-1), dict(B=1 << 22), dict(V=0), dict(V=(1 << 20) + 1, stride=(1 << 20) + 1),
               dict(stride=63), dict(logits=ctypes.c_void_p(0x100001)),
               dict(dtype=0, logits=ctypes.c_void_p(0x100002)), dict(cap=0), dict(hist=None),
               dict(cnt=None), dict(rep=None), dict(pres=ctypes.c_void_p(0x100002)),
               dict(status=None), dict(freq=ctypes.c_void_p(0x100002))):
        assert ap(**kw) == _lib.QS_ERR_INVALID_ARG, kw
    assert ap(B=0) == _lib.QS_OK


def test_apply_logit_bias_rejects_bad_arguments(lib):
    def ab(**kw):
        a = dict(logits=A16, dtype=0, B=2, V=64, stride=64, ids=A16, vals=A16, cap=8, cnt=A16,
                 status=A16, stream=None)
        a.update(kw)
        return lib.qs_apply_logit_bias(a["logits"], a["dtype"], a["B"], a["V"], a["stride"],
                                       a["ids"], a["vals"], a["cap"], a["cnt"], a["status"],
                                       a["stream"])
    for kw in (dict(dtype=5), dict(B=-1), dict(B=1 << 22), dict(V=0), dict(V=(1 << 20) + 1, stride=(1 << 20) + 1),
               dict(stride=10), dict(logits=ctypes.c_void_p(0x100002)), dict(cap=0),
               dict(ids=None), dict(vals=ctypes.c_void_p(0x100001)), dict(cnt=None),
               dict(status=None)):
        assert ab(**kw) == _lib.QS_ERR_INVALID_ARG, kw
    assert ab(B=0) == _lib.QS_OK


def test_top_logprobs_rejects_bad_arguments(lib):
    def tp(**kw):
        a = dict(B=2, ids=A16, probs=A16, cnt=A16, cap=8, n=4, tid=A16, tlp=A16, status=A16,
                 stream=None)
        a.update(kw)
        return lib.qs_top_logprobs(a["B"], a["ids"], a["probs"], a["cnt"], a["cap"], a["n"],
                                   a["tid"], a["tlp"], a["status"], a["stream"])
    for kw in (dict(B=-1), dict(B=1 << 22), dict(cap=0), dict(n=0), dict(n=4097), dict(ids=None),
               dict(probs=ctypes.c_void_p(0x100002)), dict(cnt=None), dict(tid=None),
               dict(tlp=None), dict(status=None)):
        assert tp(**kw) == _lib.QS_ERR_INVALID_ARG, kw
    assert tp(B=0) == _lib.QS_OK


def test_sample_noalloc_rejects_before_any_hip_call(lib):
    """qs_sample_noalloc: argument errors first, then QS_ERR_WORKSPACE when the
    call's workspace would exceed the library's fixed scratch; both before any
    HIP call (no GPU here). B = 0 is a no-op."""
    assert _lib.SCRATCH_BYTES == 64 << 20

    def na(**kw):
        args = dict(logits=A16, dtype=1, B=4, V=64, stride=64, T=A16, k=A16, p=A16,
                    bitmask=None, bms=0, seed=A8, offset=A8, uni=None, tokens=A16, lp=None,
                    keep=None, cids=None, cprobs=None, ccount=None, cap=0, dense=None,
                    status=A16, dbg=None, flags=0, stream=None)
        args.update(kw)
        return lib.qs_sample_noalloc(
            args["logits"], args["dtype"], args["B"], args["V"], args["stride"], args["T"],
            args["k"], args["p"], args["bitmask"], args["bms"], args["seed"], args["offset"],
            args["uni"], args["tokens"], args["lp"], args["keep"], args["cids"],
            args["cprobs"], args["ccount"], args["cap"], args["dense"], args["status"],
            args["dbg"], args["flags"], args["stream"])
    assert na(stride=60) == _lib.QS_ERR_INVALID_ARG
    assert na(V=-5) == _lib.QS_ERR_INVALID_ARG
    assert na(B=0) == _lib.QS_OK
    # the largest batch of 262144-token bf16 rows (the chunked pass) the
    # scratch holds, and one more
    V = 262144
    per_row = lib.qs_workspace_bytes(1024, V, 1, 0) / 1024
    fit = int(_lib.SCRATCH_BYTES // per_row)
    while lib.qs_workspace_bytes(fit, V, 1, 0) > _lib.SCRATCH_BYTES:
        fit -= 1
    while lib.qs_workspace_bytes(fit + 1, V, 1, 0) <= _lib.SCRATCH_BYTES:
        fit += 1
    assert fit >= 256
    assert na(B=fit + 1, V=V, stride=V) == _lib.QS_ERR_WORKSPACE


def smp_top(lib, top_n=5, top_ids=A16, top_lp=A16, **kw):
    """qs_sample_top_logprobs with qs_sample's arguments (candidate lists on)."""
    args = dict(logits=A16, dtype=1, B=4, V=64, stride=64, T=A16, k=A16, p=A16,
                bitmask=None, bms=0, seed=A8, offset=A8, uni=None, tokens=A16, lp=None,
                keep=None, cids=A16, cprobs=A16, ccount=A16, cap=64, dense=None,
                status=A16, dbg=None, flags=0, ws=WS, wsn=WSN, stream=None)
    args.update(kw)
    return lib.qs_sample_top_logprobs(
        args["logits"], args["dtype"], args["B"], args["V"], args["stride"], args["T"],
        args["k"], args["p"], args["bitmask"], args["bms"], args["seed"], args["offset"],
        args["uni"], args["tokens"], args["lp"], args["keep"], args["cids"], args["cprobs"],
        args["ccount"], args["cap"], args["dense"], args["status"], args["dbg"], args["flags"],
        top_n, top_ids, top_lp, args["ws"], args["wsn"], args["stream"])


@pytest.mark.parametrize("kw", [
    dict(top_n=0), dict(top_n=65), dict(top_n=-3), dict(top_ids=None), dict(top_lp=None),
    dict(top_ids=ctypes.c_void_p(0x100002)), dict(cids=None), dict(cprobs=None),
    dict(tokens=None), dict(V=0),
])
def test_sample_top_logprobs_rejects_bad_arguments(lib, kw):
    """The top tokens are read off the call's candidate lists: both lists are
    required, and 1 <= top_n <= 64; checked before any launch."""
    assert smp_top(lib, **kw) == _lib.QS_ERR_INVALID_ARG


def test_processed_rejects_bad_arguments(lib):
    """qs_sample_processed needs its processor struct; a group given in part,
    or rows longer than the in-kernel table covers, are refused before any
    launch; so is a workspace smaller than a row copy per row."""
    def call(proc, V=64, wsn=WSN, ws=WS):
        return lib.qs_sample_processed(
            A16, 1, 4, V, V, A16, A16, A16, None, 0, A8, A8, None, A16, None, None, None, None,
            None, 0, None, A16, None, 0, proc, ws, wsn, None)
    assert call(None) == _lib.QS_ERR_INVALID_ARG
    full = _lib.QsProcessors(0x300000, 8, 0x300100, 0x300200, 0x300300, None,
                             None, None, 0, None)
    part = _lib.QsProcessors(0x300000, 8, None, 0x300200, 0x300300, None, None, None, 0, None)
    bias_part = _lib.QsProcessors(None, 0, None, None, None, None, 0x300000, None, 8, 0x300100)
    assert call(ctypes.byref(part)) == _lib.QS_ERR_INVALID_ARG
    assert call(ctypes.byref(bias_part)) == _lib.QS_ERR_INVALID_ARG
    assert call(ctypes.byref(full), V=155649) == _lib.QS_ERR_INVALID_ARG
    assert call(ctypes.byref(full), wsn=16) == _lib.QS_ERR_WORKSPACE
    assert call(ctypes.byref(full), ws=None) == _lib.QS_ERR_WORKSPACE
    need = lib.qs_processors_workspace_bytes(4, 64, 1)
    assert need == 4 * 256
    assert lib.qs_processors_workspace_bytes(4, 155649, 1) == 0
