"""The Python binding rejects wrong dtypes, shapes, layouts and host tensors
before it calls into the library, so a host pointer or a short output buffer
never reaches a kernel.  Runs without a GPU: every library entry point is
replaced by a function that fails the test if it is reached."""
import pytest
import torch

import mla_latent_cache_absorbed_amd as mla
from mla_latent_cache_absorbed_amd import _lib

ENTRY_POINTS = ["mla_decode", "mla_decode_fp8", "mla_decode_plan", "mla_decode_attend",
                "mla_decode_attend_fp8", "mla_append_latent", "mla_append_latent_fp8",
                "mla_absorb_prepare", "mla_absorb_query", "mla_up_project",
                "mla_decode_workspace_bytes"]


@pytest.fixture(autouse=True)
def no_library_calls(monkeypatch):
    def reached(*a, **k):
        raise AssertionError("the library was called with arguments the binding should reject")
    for name in ENTRY_POINTS:
        monkeypatch.setattr(_lib, name, reached)


B, H, NB, BS, M = 2, 16, 14, 16, 7


def _inputs(**over):
    t = dict(q=torch.zeros(B, H, 576, dtype=torch.bfloat16),
             cache=torch.zeros(NB, BS, 576, dtype=torch.bfloat16),
             table=torch.zeros(B, M, dtype=torch.int32),
             lens=torch.zeros(B, dtype=torch.int32),
             out=torch.zeros(B, H, 512, dtype=torch.bfloat16),
             lse=torch.zeros(B, H, dtype=torch.float32))
    t.update(over)
    return t


class _FakeWs(mla.Workspace):
    """A workspace object that never touches a device (its buffer is a host tensor)."""

    def __init__(self, shape):
        self.shape = shape
        self.nbytes = 1 << 20
        self.buf = torch.zeros(16, dtype=torch.uint8)


def test_host_tensors_are_rejected():
    t = _inputs()
    with pytest.raises(ValueError, match="GPU"):
        mla.decode(t["q"], t["cache"], t["table"], t["lens"], 0.1)
    with pytest.raises(ValueError, match="GPU"):
        mla.decode(t["q"], t["cache"], t["table"], t["lens"], 0.1, out=t["out"], lse=t["lse"])
    c8 = torch.zeros(NB, BS, 576, dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU"):
        mla.decode_fp8(t["q"], c8, t["table"], t["lens"], 0.1, 0.5)
    ws = _FakeWs((B, H, M, BS))
    with pytest.raises(ValueError, match="GPU"):
        mla.plan(t["lens"], H, M, BS, ws)
    with pytest.raises(ValueError, match="GPU"):
        mla.attend(t["q"], t["cache"], t["table"], 0.1, t["out"], t["lse"], ws)
    with pytest.raises(ValueError, match="GPU"):
        mla.attend_fp8(t["q"], c8, t["table"], 0.1, 0.5, t["out"], t["lse"], ws)


@pytest.mark.parametrize("which,bad,exc", [
    ("q", torch.zeros(B, H, 576, dtype=torch.float32), TypeError),
    ("q", torch.zeros(B, H, 512, dtype=torch.bfloat16), ValueError),
    ("q", torch.zeros(B, H, 1152, dtype=torch.bfloat16)[:, :, ::2], ValueError),  # strided
    ("cache", torch.zeros(NB, BS, 576, dtype=torch.float16), TypeError),
    ("cache", torch.zeros(NB, BS, 512, dtype=torch.bfloat16), ValueError),
    ("table", torch.zeros(B, M, dtype=torch.int64), TypeError),
    ("table", torch.zeros(B + 1, M, dtype=torch.int32), ValueError),
    ("table", torch.zeros(M, B, dtype=torch.int32).t(), ValueError),  # not contiguous
    ("lens", torch.zeros(B, dtype=torch.int64), TypeError),
    ("lens", torch.zeros(B + 1, dtype=torch.int32), ValueError),
])
def test_bad_inputs_are_rejected(which, bad, exc):
    t = _inputs(**{which: bad})
    with pytest.raises(exc):
        mla.decode(t["q"], t["cache"], t["table"], t["lens"], 0.1)
    if which != "lens":
        ws = _FakeWs((B, H, M, BS))
        with pytest.raises(exc):
            mla.attend(t["q"], t["cache"], t["table"], 0.1, t["out"], t["lse"], ws)


@pytest.mark.parametrize("which,bad,exc", [
    ("out", torch.zeros(B, H, 512, dtype=torch.float32), TypeError),
    ("out", torch.zeros(B, H, 256, dtype=torch.bfloat16), ValueError),   # short buffer
    ("out", torch.zeros(B, H - 1, 512, dtype=torch.bfloat16), ValueError),
    ("out", torch.zeros(B, 512, H, dtype=torch.bfloat16).transpose(1, 2), ValueError),
    ("lse", torch.zeros(B, H, dtype=torch.float64), TypeError),
    ("lse", torch.zeros(B, H + 1, dtype=torch.float32), ValueError),
    ("lse", torch.zeros(H, B, dtype=torch.float32).t(), ValueError),
])
def test_bad_outputs_are_rejected(which, bad, exc):
    t = _inputs(**{which: bad})
    with pytest.raises(exc):
        mla.decode(t["q"], t["cache"], t["table"], t["lens"], 0.1, out=t["out"], lse=t["lse"])
    c8 = torch.zeros(NB, BS, 576, dtype=torch.uint8)
    with pytest.raises(exc):
        mla.decode_fp8(t["q"], c8, t["table"], t["lens"], 0.1, 0.5, out=t["out"], lse=t["lse"])
    ws = _FakeWs((B, H, M, BS))
    with pytest.raises(exc):
        mla.attend(t["q"], t["cache"], t["table"], 0.1, t["out"], t["lse"], ws)
    with pytest.raises(exc):
        mla.attend_fp8(t["q"], c8, t["table"], 0.1, 0.5, t["out"], t["lse"], ws)


def test_only_one_output_is_rejected():
    t = _inputs()
    with pytest.raises(ValueError, match="both"):
        mla.decode(t["q"], t["cache"], t["table"], t["lens"], 0.1, out=t["out"])


def test_fp8_cache_dtype_is_checked():
    t = _inputs()
    with pytest.raises(TypeError):
        mla.decode_fp8(t["q"], t["cache"], t["table"], t["lens"], 0.1, 0.5)  # bf16, not uint8


def test_plan_checks_lengths_and_workspace_shape():
    ws = _FakeWs((B, H, M, BS))
    with pytest.raises(TypeError):
        mla.plan(torch.zeros(B, dtype=torch.int64), H, M, BS, ws)
    with pytest.raises(ValueError):
        mla.plan(torch.zeros(B, 1, dtype=torch.int32), H, M, BS, ws)
    # a host seq_lens is caught before the workspace is looked at
    with pytest.raises(ValueError, match="GPU"):
        mla.plan(torch.zeros(B, dtype=torch.int32), H, M, BS, ws)


def test_append_rejects_host_and_misshaped_tensors():
    kv = torch.zeros(B, 512, dtype=torch.bfloat16)
    kr = torch.zeros(B, 64, dtype=torch.bfloat16)
    pos = torch.zeros(B, dtype=torch.int32)
    table = torch.zeros(B, M, dtype=torch.int32)
    cache = torch.zeros(NB, BS, 576, dtype=torch.bfloat16)
    c8 = torch.zeros(NB, BS, 576, dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU"):
        mla.append_latent(kv, kr, pos, table, cache)
    with pytest.raises(ValueError, match="GPU"):
        mla.append_latent_fp8(kv, kr, pos, table, c8, 0.5)
    with pytest.raises(ValueError, match="GPU"):
        mla.append_latent(kv, kr, pos, table, cache, skipped=torch.zeros(1, dtype=torch.int32))
    with pytest.raises(TypeError):
        mla.append_latent(kv.float(), kr, pos, table, cache)
    with pytest.raises(ValueError):
        mla.append_latent(kv[:, :256], kr, pos, table, cache)
    with pytest.raises(ValueError):
        mla.append_latent(kv, kr, pos[None], table, cache)
    with pytest.raises(TypeError):
        mla.append_latent(kv, kr, pos, table, cache, skipped=torch.zeros(1, dtype=torch.int64))


def test_absorption_rejects_host_and_misshaped_tensors():
    with pytest.raises(ValueError, match="GPU"):
        mla.absorb_prepare(torch.zeros(H, 128, 512, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        mla.absorb_prepare(torch.zeros(H, 512, 128, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        mla.absorb_query(torch.zeros(B, H, 192, dtype=torch.float32),
                         torch.zeros(H, 512, 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        mla.up_project(torch.zeros(B, H, 512, dtype=torch.bfloat16),
                       torch.zeros(H, 128, 256, dtype=torch.bfloat16))
