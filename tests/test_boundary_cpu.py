"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

from mla_latent_cache_absorbed_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def _declared_functions():
    names = []
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmla_decode.so is not built (run __graft_entry__.build())")
    return _lib.lib()


def test_header_declares_expected_entry_points():
    names = _declared_functions()
    assert set(names) == set(_lib.SIGNATURES), names


def test_library_exports_every_declared_symbol(L):
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_abi_version_and_status_strings(L):
    assert _lib.mla_decode_abi_version() == 1
    for code, name in [(0, "MLA_OK"), (1, "MLA_ERR_NULL_POINTER"), (2, "MLA_ERR_BAD_SHAPE"),
                       (3, "MLA_ERR_UNSUPPORTED"), (4, "MLA_ERR_BAD_SCALE"),
                       (5, "MLA_ERR_WORKSPACE"), (6, "MLA_ERR_HIP"), (7, "MLA_ERR_ALIGNMENT")]:
        assert _lib.status_string(code) == name
    assert _lib.status_string(99) == "MLA_ERR_UNKNOWN"


def test_workspace_bytes(L):
    n = _lib.mla_decode_workspace_bytes(124, 128, 64, 64)
    cap = 124 + 1024
    assert n >= cap * 128 * 512 * 4 + cap * 128 * 4 + cap * 16 + 124 * 16 + 124 * 4
    assert n % 256 == 0
    assert _lib.mla_decode_workspace_bytes(2, 16, 7, 16) > 0
    # unsupported sizes give 0
    assert _lib.mla_decode_workspace_bytes(2, 129, 7, 16) == 0
    assert _lib.mla_decode_workspace_bytes(2, 0, 7, 16) == 0
    assert _lib.mla_decode_workspace_bytes(2, 128, 7, 48) == 0
    assert _lib.mla_decode_workspace_bytes(2, 128, 7, 8) == 0
    assert _lib.mla_decode_workspace_bytes(2, 128, 0, 16) == 0
    assert _lib.mla_decode_workspace_bytes(-1, 128, 7, 16) == 0
    assert _lib.mla_decode_workspace_bytes(1, 128, 1 << 24, 64) == 0  # M*BS > 2^28


FAKE = 1 << 20  # a 256-aligned non-null address; never dereferenced on these paths


def _decode(**kw):
    a = dict(q=FAKE, cache=FAKE, table=FAKE, lens=FAKE, scale=0.07, out=FAKE, lse=FAKE,
             B=2, H=128, NB=14, BS=16, M=7, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return _lib.mla_decode(a["q"], a["cache"], a["table"], a["lens"], a["scale"], a["out"],
                           a["lse"], a["B"], a["H"], a["NB"], a["BS"], a["M"], a["ws"],
                           a["wsb"], a["stream"])


def test_decode_rejects_bad_arguments_on_host(L):
    assert _decode(B=0) == _lib.MLA_OK                     # empty batch: nothing to do
    assert _decode(q=None) == _lib.MLA_ERR_NULL_POINTER
    assert _decode(cache=None) == _lib.MLA_ERR_NULL_POINTER
    assert _decode(table=None) == _lib.MLA_ERR_NULL_POINTER
    assert _decode(lens=None) == _lib.MLA_ERR_NULL_POINTER
    assert _decode(out=None) == _lib.MLA_ERR_NULL_POINTER
    assert _decode(lse=None) == _lib.MLA_ERR_NULL_POINTER
    assert _decode(ws=None) == _lib.MLA_ERR_NULL_POINTER
    assert _decode(H=0) == _lib.MLA_ERR_UNSUPPORTED
    assert _decode(H=129) == _lib.MLA_ERR_UNSUPPORTED
    assert _decode(BS=24) == _lib.MLA_ERR_UNSUPPORTED
    assert _decode(BS=2048) == _lib.MLA_ERR_UNSUPPORTED
    assert _decode(B=-1) == _lib.MLA_ERR_BAD_SHAPE
    assert _decode(M=0) == _lib.MLA_ERR_BAD_SHAPE
    assert _decode(NB=0) == _lib.MLA_ERR_BAD_SHAPE
    assert _decode(scale=float("nan")) == _lib.MLA_ERR_BAD_SCALE
    assert _decode(scale=float("inf")) == _lib.MLA_ERR_BAD_SCALE
    assert _decode(wsb=16) == _lib.MLA_ERR_WORKSPACE
    assert _decode(q=FAKE + 8) == _lib.MLA_ERR_ALIGNMENT
    assert _decode(cache=FAKE + 4) == _lib.MLA_ERR_ALIGNMENT
    assert _decode(out=FAKE + 8) == _lib.MLA_ERR_ALIGNMENT
    assert _decode(lse=FAKE + 2) == _lib.MLA_ERR_ALIGNMENT
    assert _decode(ws=FAKE + 128) == _lib.MLA_ERR_ALIGNMENT


def test_plan_attend_reject_bad_arguments_on_host(L):
    P = _lib.mla_decode_plan
    assert P(FAKE, 0, 128, 7, 16, 0, FAKE, 1 << 40, None) == _lib.MLA_OK
    assert P(None, 2, 128, 7, 16, 0, FAKE, 1 << 40, None) == _lib.MLA_ERR_NULL_POINTER
    assert P(FAKE, 2, 128, 7, 16, 0, None, 1 << 40, None) == _lib.MLA_ERR_NULL_POINTER
    assert P(FAKE, 2, 128, 7, 16, 0, FAKE, 8, None) == _lib.MLA_ERR_WORKSPACE
    assert P(FAKE, 2, 128, 7, 16, 48, FAKE, 1 << 40, None) == _lib.MLA_ERR_UNSUPPORTED
    assert P(FAKE, 2, 128, 7, 16, -32, FAKE, 1 << 40, None) == _lib.MLA_ERR_UNSUPPORTED
    # forced chunk that would need more work items than the workspace holds
    assert P(FAKE, 100, 128, 4096, 64, 32, FAKE, 1 << 40, None) == _lib.MLA_ERR_UNSUPPORTED
    A = _lib.mla_decode_attend
    assert A(None, FAKE, FAKE, 0.1, FAKE, FAKE, 2, 128, 14, 16, 7, FAKE, 1 << 40, None) \
        == _lib.MLA_ERR_NULL_POINTER
    assert A(FAKE, FAKE, FAKE, float("nan"), FAKE, FAKE, 2, 128, 14, 16, 7, FAKE, 1 << 40,
             None) == _lib.MLA_ERR_BAD_SCALE
    assert A(FAKE, FAKE, FAKE, 0.1, FAKE, FAKE, 2, 128, 0, 16, 7, FAKE, 1 << 40, None) \
        == _lib.MLA_ERR_BAD_SHAPE
    assert A(FAKE, FAKE, FAKE, 0.1, FAKE, FAKE, 2, 128, 14, 16, 7, FAKE, 4, None) \
        == _lib.MLA_ERR_WORKSPACE
    assert _lib.lib().mla_decode_read_error(None, ctypes.byref(ctypes.c_int32()), None) \
        == _lib.MLA_ERR_NULL_POINTER


def _append(**kw):
    a = dict(kv=FAKE, kvs=576, kr=FAKE + 1024, krs=576, pos=FAKE, table=FAKE, cache=FAKE,
             skipped=None, B=4, NB=14, BS=16, M=7, stream=None)
    a.update(kw)
    return _lib.mla_append_latent(a["kv"], a["kvs"], a["kr"], a["krs"], a["pos"], a["table"],
                                  a["cache"], a["skipped"], a["B"], a["NB"], a["BS"], a["M"],
                                  a["stream"])


def test_append_rejects_bad_arguments_on_host(L):
    assert _append(B=0) == _lib.MLA_OK
    assert _append(B=0, kv=None) == _lib.MLA_OK            # empty batch: nothing to do
    assert _append(kv=None) == _lib.MLA_ERR_NULL_POINTER
    assert _append(kr=None) == _lib.MLA_ERR_NULL_POINTER
    assert _append(pos=None) == _lib.MLA_ERR_NULL_POINTER
    assert _append(table=None) == _lib.MLA_ERR_NULL_POINTER
    assert _append(cache=None) == _lib.MLA_ERR_NULL_POINTER
    assert _append(B=-1) == _lib.MLA_ERR_BAD_SHAPE
    assert _append(NB=0) == _lib.MLA_ERR_BAD_SHAPE
    assert _append(M=0) == _lib.MLA_ERR_BAD_SHAPE
    assert _append(kvs=504) == _lib.MLA_ERR_BAD_SHAPE
    assert _append(krs=56) == _lib.MLA_ERR_BAD_SHAPE
    assert _append(BS=24) == _lib.MLA_ERR_UNSUPPORTED
    assert _append(BS=8) == _lib.MLA_ERR_UNSUPPORTED
    assert _append(BS=2048) == _lib.MLA_ERR_UNSUPPORTED
    assert _append(M=1 << 24, BS=64) == _lib.MLA_ERR_UNSUPPORTED  # M*BS > 2^28
    assert _append(kvs=580) == _lib.MLA_ERR_ALIGNMENT           # rows not 16-byte aligned
    assert _append(krs=68) == _lib.MLA_ERR_ALIGNMENT
    assert _append(kv=FAKE + 8) == _lib.MLA_ERR_ALIGNMENT
    assert _append(kr=FAKE + 1030) == _lib.MLA_ERR_ALIGNMENT
    assert _append(cache=FAKE + 4) == _lib.MLA_ERR_ALIGNMENT
    assert _append(pos=FAKE + 2) == _lib.MLA_ERR_ALIGNMENT
    assert _append(skipped=FAKE + 1) == _lib.MLA_ERR_ALIGNMENT


def _decode8(**kw):
    a = dict(q=FAKE, cache=FAKE, table=FAKE, lens=FAKE, scale=0.07, kv=0.0625, out=FAKE, lse=FAKE,
             B=2, H=128, NB=14, BS=64, M=7, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return _lib.mla_decode_fp8(a["q"], a["cache"], a["table"], a["lens"], a["scale"], a["kv"],
                               a["out"], a["lse"], a["B"], a["H"], a["NB"], a["BS"], a["M"],
                               a["ws"], a["wsb"], a["stream"])


def _no_device():
    """True when no HIP device is visible: then a call whose arguments pass the
    host checks stops at the first HIP call (MLA_ERR_HIP) instead of
    launching on the fake pointers these tests use."""
    import torch
    return not torch.cuda.is_available()


def test_fp8_decode_rejects_bad_arguments_on_host(L):
    assert _decode8(B=0) == _lib.MLA_OK
    assert _decode8(BS=8) == _lib.MLA_ERR_UNSUPPORTED     # as for bf16: BS is 16 .. 1024
    assert _decode8(H=129) == _lib.MLA_ERR_UNSUPPORTED
    if _no_device():
        # every head count and block size of the bf16 decode (H <= 32 by the
        # narrow kernel, BS = 16 with stages over two blocks)
        for H, BS in ((1, 64), (16, 64), (16, 16), (32, 32), (33, 32), (128, 16), (128, 256)):
            assert _decode8(H=H, BS=BS) == _lib.MLA_ERR_HIP, (H, BS)
    assert _decode8(kv=float("nan")) == _lib.MLA_ERR_BAD_SCALE
    assert _decode8(kv=float("inf")) == _lib.MLA_ERR_BAD_SCALE
    assert _decode8(scale=float("nan")) == _lib.MLA_ERR_BAD_SCALE
    assert _decode8(cache=None) == _lib.MLA_ERR_NULL_POINTER
    assert _decode8(lens=None) == _lib.MLA_ERR_NULL_POINTER
    assert _decode8(cache=FAKE + 8) == _lib.MLA_ERR_ALIGNMENT
    assert _decode8(wsb=16) == _lib.MLA_ERR_WORKSPACE
    A = _lib.mla_decode_attend_fp8
    assert A(FAKE, FAKE, FAKE, 0.1, 0.5, FAKE, FAKE, 2, 16, 14, 8, 7, FAKE, 1 << 40, None) \
        == _lib.MLA_ERR_UNSUPPORTED
    assert A(FAKE, FAKE, FAKE, 0.1, float("nan"), FAKE, FAKE, 2, 128, 14, 64, 7, FAKE, 1 << 40,
             None) == _lib.MLA_ERR_BAD_SCALE


def test_absorb_rejects_bad_arguments_on_host(L):
    P, Q, U = _lib.mla_absorb_prepare, _lib.mla_absorb_query, _lib.mla_up_project
    assert P(None, FAKE, 128, None) == _lib.MLA_ERR_NULL_POINTER
    assert P(FAKE, None, 128, None) == _lib.MLA_ERR_NULL_POINTER
    assert P(FAKE, FAKE, 0, None) == _lib.MLA_ERR_BAD_SHAPE
    assert P(FAKE, FAKE, 129, None) == _lib.MLA_ERR_UNSUPPORTED
    assert P(FAKE + 2, FAKE, 128, None) == _lib.MLA_ERR_ALIGNMENT
    for F in (Q, U):
        assert F(FAKE, FAKE, FAKE, 0, 128, None) == _lib.MLA_OK      # empty batch
        assert F(None, FAKE, FAKE, 0, 128, None) == _lib.MLA_OK
        assert F(None, FAKE, FAKE, 4, 128, None) == _lib.MLA_ERR_NULL_POINTER
        assert F(FAKE, None, FAKE, 4, 128, None) == _lib.MLA_ERR_NULL_POINTER
        assert F(FAKE, FAKE, None, 4, 128, None) == _lib.MLA_ERR_NULL_POINTER
        assert F(FAKE, FAKE, FAKE, -1, 128, None) == _lib.MLA_ERR_BAD_SHAPE
        assert F(FAKE, FAKE, FAKE, 4, 0, None) == _lib.MLA_ERR_BAD_SHAPE
        assert F(FAKE, FAKE, FAKE, 4, 129, None) == _lib.MLA_ERR_UNSUPPORTED
        assert F(FAKE, FAKE, FAKE, (1 << 24) + 1, 128, None) == _lib.MLA_ERR_UNSUPPORTED
        assert F(FAKE + 8, FAKE, FAKE, 4, 128, None) == _lib.MLA_ERR_ALIGNMENT
        assert F(FAKE, FAKE + 4, FAKE, 4, 128, None) == _lib.MLA_ERR_ALIGNMENT
        assert F(FAKE, FAKE, FAKE + 2, 4, 128, None) == _lib.MLA_ERR_ALIGNMENT


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()


def _append8(**kw):
    a = dict(kv=FAKE, kvs=576, kr=FAKE + 1024, krs=576, pos=FAKE, table=FAKE, cache=FAKE, kvsc=0.0625,
             skipped=None, B=4, NB=14, BS=16, M=7, stream=None)
    a.update(kw)
    return _lib.mla_append_latent_fp8(a["kv"], a["kvs"], a["kr"], a["krs"], a["pos"], a["table"],
                                      a["cache"], a["kvsc"], a["skipped"], a["B"], a["NB"], a["BS"],
                                      a["M"], a["stream"])


def test_append_fp8_rejects_bad_arguments_on_host(L):
    assert _append8(B=0) == _lib.MLA_OK
    for bad in (0.0, float("nan"), float("inf"), -float("inf")):
        assert _append8(kvsc=bad) == _lib.MLA_ERR_BAD_SCALE, bad
    assert _append8(kv=None) == _lib.MLA_ERR_NULL_POINTER
    assert _append8(cache=None) == _lib.MLA_ERR_NULL_POINTER
    assert _append8(B=-1) == _lib.MLA_ERR_BAD_SHAPE
    assert _append8(kvs=500) == _lib.MLA_ERR_BAD_SHAPE
    assert _append8(BS=24) == _lib.MLA_ERR_UNSUPPORTED
    assert _append8(BS=8) == _lib.MLA_ERR_UNSUPPORTED
    assert _append8(cache=FAKE + 8) == _lib.MLA_ERR_ALIGNMENT
    assert _append8(kv=FAKE + 8) == _lib.MLA_ERR_ALIGNMENT
    assert _append8(pos=FAKE + 2) == _lib.MLA_ERR_ALIGNMENT


def test_overflowing_score_factor_is_rejected_on_host(L):
    """scale and kv_scale are each finite, but the factor the kernels apply to
    raw scores (scale * kv_scale * log2 e, in fp32) overflows: rejected with
    MLA_ERR_BAD_SCALE before any launch, for both caches and both entry points."""
    big = 3.0e38  # finite in fp32; times log2(e) it overflows
    assert _decode(scale=big) == _lib.MLA_ERR_BAD_SCALE
    assert _decode(scale=-big) == _lib.MLA_ERR_BAD_SCALE
    assert _decode8(scale=1e30, kv=1e10) == _lib.MLA_ERR_BAD_SCALE
    assert _decode8(scale=-1e30, kv=1e10) == _lib.MLA_ERR_BAD_SCALE
    A = _lib.mla_decode_attend
    assert A(FAKE, FAKE, FAKE, big, FAKE, FAKE, 2, 128, 14, 16, 7, FAKE, 1 << 40, None) \
        == _lib.MLA_ERR_BAD_SCALE
    A8 = _lib.mla_decode_attend_fp8
    assert A8(FAKE, FAKE, FAKE, 1e30, 1e10, FAKE, FAKE, 2, 128, 14, 64, 7, FAKE, 1 << 40, None) \
        == _lib.MLA_ERR_BAD_SCALE
    # a large but representable factor is accepted by the host checks (it
    # only reaches the launch, which fails without a device)
    if _no_device():
        assert _decode(scale=1e30) == _lib.MLA_ERR_HIP
        assert _decode8(scale=1e20, kv=1e10) == _lib.MLA_ERR_HIP


def _noalloc(**kw):
    a = dict(q=FAKE, cache=FAKE, table=FAKE, lens=FAKE, scale=0.07, out=FAKE, lse=FAKE,
             B=2, H=128, NB=14, BS=16, M=7, stream=None)
    a.update(kw)
    return _lib.mla_decode_noalloc(a["q"], a["cache"], a["table"], a["lens"], a["scale"],
                                   a["out"], a["lse"], a["B"], a["H"], a["NB"], a["BS"], a["M"],
                                   a["stream"])


def test_noalloc_decode_rejects_bad_arguments_on_host(L):
    """The entry point without a workspace makes mla_decode's host checks,
    and rejects a batch whose plan and partials do not fit its fixed scratch
    array (at 128 heads, more than 255 requests) before any HIP call."""
    assert _noalloc(B=0) == _lib.MLA_OK
    assert _noalloc(q=None) == _lib.MLA_ERR_NULL_POINTER
    assert _noalloc(lens=None) == _lib.MLA_ERR_NULL_POINTER
    assert _noalloc(out=None) == _lib.MLA_ERR_NULL_POINTER
    assert _noalloc(H=129) == _lib.MLA_ERR_UNSUPPORTED
    assert _noalloc(BS=24) == _lib.MLA_ERR_UNSUPPORTED
    assert _noalloc(NB=0) == _lib.MLA_ERR_BAD_SHAPE
    assert _noalloc(scale=float("nan")) == _lib.MLA_ERR_BAD_SCALE
    assert _noalloc(scale=3.0e38) == _lib.MLA_ERR_BAD_SCALE
    assert _noalloc(lens=FAKE + 2) == _lib.MLA_ERR_ALIGNMENT
    assert _noalloc(out=FAKE + 8) == _lib.MLA_ERR_ALIGNMENT
    # the scratch array holds 255 requests' partials at 128 heads
    assert _noalloc(B=256, H=128) == _lib.MLA_ERR_WORKSPACE
    assert _noalloc(B=100000, H=16) == _lib.MLA_ERR_WORKSPACE
    if _no_device():
        # sizes that fit reach the device query, which fails without a GPU
        assert _noalloc(B=255, H=128) == _lib.MLA_ERR_HIP
        assert _noalloc(B=900, H=16) == _lib.MLA_ERR_HIP
