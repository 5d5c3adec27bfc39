"""Absorbed-form MLA decode over a paged 576-wide latent cache, for MI355X.

The computation runs in the HIP library ``libmla_decode.so`` (C ABI in
``include/mla_decode.h``); this package only marshals torch tensors into it.
PyTorch provides device memory and the current stream.

    out, lse = decode(q, latent_cache, block_table, seq_lens, scale)

q [B, H, 576] bf16, latent_cache [NB, BS, 576] bf16, block_table [B, M] int32,
seq_lens [B] int32, all on the same GPU; returns out [B, H, 512] bf16 and
lse [B, H] float32 (natural log).
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import MlaError  # noqa: F401

__all__ = ["decode", "decode_noalloc", "Workspace", "plan", "attend", "decode_fp8", "attend_fp8", "append_latent",
           "append_latent_fp8",
           "absorb_prepare", "absorb_query", "up_project", "MlaError"]


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _tensor(name, t, dtype, shape=None, ndim=None):
    """dtype, shape and contiguity of one argument (no device access)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _one_gpu(**named):
    """Every tensor lives on the same GPU; returns that device.  Checked after
    the dtype and shape checks, so that a host pointer never reaches a kernel."""
    dev = None
    for name, t in named.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor, got device {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")
    return dev


def _check_outputs(out, lse, B, H):
    _tensor("out", out, torch.bfloat16, (B, H, 512))
    _tensor("lse", lse, torch.float32, (B, H))


def _check_workspace(ws, B, H, M, BS, dev):
    if not isinstance(ws, Workspace):
        raise TypeError("workspace must be a Workspace")
    if ws.shape != (B, H, M, BS):
        raise ValueError(f"workspace was sized for (B, H, M, BS) = {ws.shape}, the call has "
                         f"{(B, H, M, BS)}")
    if ws.buf.device != dev:
        raise ValueError(f"workspace is on {ws.buf.device}, the tensors on {dev}")


def _check_inputs(q, cache, table, lens, cache_dtype=torch.bfloat16):
    """Shapes and dtypes of the decode inputs; returns B, H, NB, BS, M."""
    _tensor("q", q, torch.bfloat16, ndim=3)
    if q.shape[2] != 576:
        raise ValueError(f"q must be [B, H, 576], got {tuple(q.shape)}")
    cname = "latent_cache" if cache_dtype == torch.bfloat16 else "latent_cache_fp8"
    _tensor(cname, cache, cache_dtype, ndim=3)
    if cache.shape[2] != 576:
        raise ValueError(f"{cname} must be [NB, BS, 576], got {tuple(cache.shape)}")
    B, H = q.shape[0], q.shape[1]
    _tensor("block_table", table, torch.int32, ndim=2)
    if table.shape[0] != B:
        raise ValueError(f"block_table must be [B, M] with B = {B}, got {tuple(table.shape)}")
    if lens is not None:
        _tensor("seq_lens", lens, torch.int32, (B,))
    return B, H, cache.shape[0], cache.shape[1], table.shape[1]


class Workspace:
    """Device scratch for the plan and split partials, reusable across calls."""

    def __init__(self, B: int, H: int, M: int, BS: int, device=None):
        n = _lib.mla_decode_workspace_bytes(B, H, M, BS)
        if n == 0:
            raise ValueError(f"unsupported sizes B={B} H={H} M={M} BS={BS}")
        self.shape = (B, H, M, BS)
        self.nbytes = n
        self.buf = torch.empty(n, dtype=torch.uint8, device=device or "cuda")

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr()

    def header(self) -> list:
        """First words of the plan header: [n_items, chunk, check bits, item queue,
        n_full, n_merge_units, merge-unit queue]."""
        return self.buf[:28].view(torch.int32).tolist()

    def check_flags(self) -> int:
        return _lib.mla_decode_read_error(self.ptr, _stream())


def _ws(ws: Optional[Workspace], B, H, M, BS, device) -> Workspace:
    if ws is None or ws.shape != (B, H, M, BS):
        ws = Workspace(B, H, M, BS, device)
    return ws


def decode(q: torch.Tensor, latent_cache: torch.Tensor, block_table: torch.Tensor,
           seq_lens: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None, workspace: Optional[Workspace] = None
           ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Absorbed MLA decode of one layer (plan + attend)."""
    B, H, NB, BS, M = _check_inputs(q, latent_cache, block_table, seq_lens)
    if out is not None or lse is not None:
        if out is None or lse is None:
            raise ValueError("pass both out and lse, or neither")
        _check_outputs(out, lse, B, H)
    dev = _one_gpu(q=q, latent_cache=latent_cache, block_table=block_table, seq_lens=seq_lens,
                   out=out, lse=lse)
    if out is None:
        out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = _ws(workspace, B, H, M, BS, dev)
    _check_workspace(ws, B, H, M, BS, dev)
    st = _lib.mla_decode(q.data_ptr(), latent_cache.data_ptr(), block_table.data_ptr(),
                         seq_lens.data_ptr(), float(scale), out.data_ptr(), lse.data_ptr(),
                         B, H, NB, BS, M, ws.ptr, ws.nbytes, _stream())
    _lib._check("mla_decode", st)
    return out, lse


def decode_noalloc(q: torch.Tensor, latent_cache: torch.Tensor, block_table: torch.Tensor,
                   seq_lens: torch.Tensor, scale: float, out: torch.Tensor,
                   lse: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """decode() without a workspace: the library's own per-GPU scratch array
    holds the plan and partials, so the call allocates nothing (out and lse
    are the caller's).  Calls on one GPU must not overlap."""
    B, H, NB, BS, M = _check_inputs(q, latent_cache, block_table, seq_lens)
    _check_outputs(out, lse, B, H)
    _one_gpu(q=q, latent_cache=latent_cache, block_table=block_table, seq_lens=seq_lens,
             out=out, lse=lse)
    st = _lib.mla_decode_noalloc(q.data_ptr(), latent_cache.data_ptr(), block_table.data_ptr(),
                                 seq_lens.data_ptr(), float(scale), out.data_ptr(), lse.data_ptr(),
                                 B, H, NB, BS, M, _stream())
    _lib._check("mla_decode_noalloc", st)
    return out, lse


def decode_fp8(q: torch.Tensor, latent_cache_fp8: torch.Tensor, block_table: torch.Tensor,
               seq_lens: torch.Tensor, scale: float, kv_scale: float,
               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
               workspace: Optional[Workspace] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Absorbed MLA decode over an FP8 (e4m3) latent cache whose values are
    kv_scale * e4m3(byte); the same head counts and block sizes as decode()."""
    B, H, NB, BS, M = _check_inputs(q, latent_cache_fp8, block_table, seq_lens, torch.uint8)
    if out is not None or lse is not None:
        if out is None or lse is None:
            raise ValueError("pass both out and lse, or neither")
        _check_outputs(out, lse, B, H)
    dev = _one_gpu(q=q, latent_cache_fp8=latent_cache_fp8, block_table=block_table,
                   seq_lens=seq_lens, out=out, lse=lse)
    if out is None:
        out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = _ws(workspace, B, H, M, BS, dev)
    _check_workspace(ws, B, H, M, BS, dev)
    st = _lib.mla_decode_fp8(q.data_ptr(), latent_cache_fp8.data_ptr(), block_table.data_ptr(),
                             seq_lens.data_ptr(), float(scale), float(kv_scale), out.data_ptr(),
                             lse.data_ptr(), B, H, NB, BS, M, ws.ptr, ws.nbytes, _stream())
    _lib._check("mla_decode_fp8", st)
    return out, lse


def attend_fp8(q, latent_cache_fp8, block_table, scale, kv_scale, out, lse,
               workspace: Workspace) -> None:
    """The attend step over an FP8 cache, on a plan already in workspace."""
    B, H, NB, BS, M = _check_inputs(q, latent_cache_fp8, block_table, None, torch.uint8)
    _check_outputs(out, lse, B, H)
    dev = _one_gpu(q=q, latent_cache_fp8=latent_cache_fp8, block_table=block_table, out=out,
                   lse=lse)
    _check_workspace(workspace, B, H, M, BS, dev)
    st = _lib.mla_decode_attend_fp8(q.data_ptr(), latent_cache_fp8.data_ptr(), block_table.data_ptr(),
                                    float(scale), float(kv_scale), out.data_ptr(), lse.data_ptr(),
                                    B, H, NB, BS, M, workspace.ptr, workspace.nbytes, _stream())
    _lib._check("mla_decode_attend_fp8", st)


def plan(seq_lens: torch.Tensor, H: int, M: int, BS: int, workspace: Workspace,
         chunk_tokens: int = 0) -> None:
    """The split-KV plan of one decode step into workspace (device-side, no sync)."""
    _tensor("seq_lens", seq_lens, torch.int32, ndim=1)
    B = seq_lens.shape[0]
    dev = _one_gpu(seq_lens=seq_lens)
    _check_workspace(workspace, B, H, M, BS, dev)
    st = _lib.mla_decode_plan(seq_lens.data_ptr(), B, H, M, BS, chunk_tokens,
                              workspace.ptr, workspace.nbytes, _stream())
    _lib._check("mla_decode_plan", st)


def attend(q, latent_cache, block_table, scale, out, lse, workspace: Workspace) -> None:
    """The attend step (bf16 cache), on a plan already in workspace."""
    B, H, NB, BS, M = _check_inputs(q, latent_cache, block_table, None)
    _check_outputs(out, lse, B, H)
    dev = _one_gpu(q=q, latent_cache=latent_cache, block_table=block_table, out=out, lse=lse)
    _check_workspace(workspace, B, H, M, BS, dev)
    st = _lib.mla_decode_attend(q.data_ptr(), latent_cache.data_ptr(), block_table.data_ptr(),
                                float(scale), out.data_ptr(), lse.data_ptr(), B, H, NB, BS, M,
                                workspace.ptr, workspace.nbytes, _stream())
    _lib._check("mla_decode_attend", st)


def _check_append_args(kv_c, k_rope, positions, block_table, cache, cache_dtype, skipped):
    if kv_c.dtype != torch.bfloat16 or k_rope.dtype != torch.bfloat16:
        raise TypeError("kv_c and k_rope must be bfloat16")
    if cache.dtype != cache_dtype or cache.dim() != 3 or cache.shape[2] != 576:
        raise ValueError(f"the cache must be {cache_dtype} [NB, BS, 576]")
    if positions.dtype != torch.int32 or block_table.dtype != torch.int32:
        raise TypeError("positions and block_table must be int32")
    if positions.dim() != 1:
        raise ValueError(f"positions must be [B], got {tuple(positions.shape)}")
    B = positions.shape[0]
    if kv_c.dim() != 2 or k_rope.dim() != 2 or kv_c.shape[0] != B or k_rope.shape[0] != B:
        raise ValueError("kv_c and k_rope must be [B, n] with B = len(positions)")
    if kv_c.shape[1] < 512 or k_rope.shape[1] < 64 or kv_c.stride(1) != 1 or k_rope.stride(1) != 1:
        raise ValueError("kv_c rows need 512 and k_rope rows 64 contiguous elements")
    if block_table.dim() != 2 or block_table.shape[0] != B or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous [B, M] tensor")
    if not (cache.is_contiguous() and positions.is_contiguous()):
        raise ValueError("the cache and positions must be contiguous")
    if skipped is not None and (not isinstance(skipped, torch.Tensor) or skipped.dtype != torch.int32
                                or skipped.numel() < 1):
        raise TypeError("skipped must be an int32 device tensor")
    _one_gpu(kv_c=kv_c, k_rope=k_rope, positions=positions, block_table=block_table, cache=cache,
             skipped=skipped)


def append_latent(kv_c: torch.Tensor, k_rope: torch.Tensor, positions: torch.Tensor,
                  block_table: torch.Tensor, latent_cache: torch.Tensor,
                  skipped: Optional[torch.Tensor] = None) -> None:
    """Store each request's new token (kv_c [B, >=512], k_rope [B, >=64], bf16 rows
    with unit inner stride) at its position in the paged latent cache.
    positions [B] int32 (negative: no token); skipped: optional int32 [1]
    device counter of requests that could not be written."""
    _check_append_args(kv_c, k_rope, positions, block_table, latent_cache, torch.bfloat16, skipped)
    B = positions.shape[0]
    NB, BS, _ = latent_cache.shape
    M = block_table.shape[1]
    st = _lib.mla_append_latent(kv_c.data_ptr(), kv_c.stride(0), k_rope.data_ptr(), k_rope.stride(0),
                                positions.data_ptr(), block_table.data_ptr(),
                                latent_cache.data_ptr(),
                                skipped.data_ptr() if skipped is not None else None,
                                B, NB, BS, M, _stream())
    _lib._check("mla_append_latent", st)


def append_latent_fp8(kv_c: torch.Tensor, k_rope: torch.Tensor, positions: torch.Tensor,
                      block_table: torch.Tensor, latent_cache_fp8: torch.Tensor, kv_scale: float,
                      skipped: Optional[torch.Tensor] = None) -> None:
    """append_latent into an FP8 cache (uint8 [NB, BS, 576] of e4m3 bytes
    holding kv_scale * e4m3(byte)): each value is stored as the nearest e4m3
    code to value / kv_scale (ties to even), saturated to +-448."""
    _check_append_args(kv_c, k_rope, positions, block_table, latent_cache_fp8, torch.uint8, skipped)
    B = positions.shape[0]
    NB, BS, _ = latent_cache_fp8.shape
    M = block_table.shape[1]
    st = _lib.mla_append_latent_fp8(kv_c.data_ptr(), kv_c.stride(0), k_rope.data_ptr(), k_rope.stride(0),
                                    positions.data_ptr(), block_table.data_ptr(),
                                    latent_cache_fp8.data_ptr(), float(kv_scale),
                                    skipped.data_ptr() if skipped is not None else None,
                                    B, NB, BS, M, _stream())
    _lib._check("mla_append_latent_fp8", st)


def _bf16_contig(name, t, shape):
    _tensor(name, t, torch.bfloat16, shape)
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor, got device {t.device}")


def absorb_prepare(w_uk: torch.Tensor) -> torch.Tensor:
    """W_UK [H, 128, 512] -> its per-head transpose [H, 512, 128], the layout
    absorb_query reads (done once, when the weights are loaded)."""
    H = w_uk.shape[0]
    _bf16_contig("w_uk", w_uk, (H, 128, 512))
    w_t = torch.empty((H, 512, 128), dtype=torch.bfloat16, device=w_uk.device)
    _lib._check("mla_absorb_prepare", _lib.mla_absorb_prepare(w_uk.data_ptr(), w_t.data_ptr(), H, _stream()))
    return w_t


def absorb_query(q_in: torch.Tensor, w_uk_t: torch.Tensor, q: Optional[torch.Tensor] = None
                 ) -> torch.Tensor:
    """q_in [B, H, 192] (nope 128, then RoPE 64) -> absorbed query q [B, H, 576]."""
    B, H = q_in.shape[0], q_in.shape[1]
    _bf16_contig("q_in", q_in, (B, H, 192))
    _bf16_contig("w_uk_t", w_uk_t, (H, 512, 128))
    if q is None:
        q = torch.empty((B, H, 576), dtype=torch.bfloat16, device=q_in.device)
    _bf16_contig("q", q, (B, H, 576))
    _lib._check("mla_absorb_query",
                _lib.mla_absorb_query(q_in.data_ptr(), w_uk_t.data_ptr(), q.data_ptr(), B, H, _stream()))
    return q


def up_project(out: torch.Tensor, w_uv: torch.Tensor, o: Optional[torch.Tensor] = None
               ) -> torch.Tensor:
    """Decode output out [B, H, 512] -> value heads o [B, H, 128] = W_UV[h] out[b, h]."""
    B, H = out.shape[0], out.shape[1]
    _bf16_contig("out", out, (B, H, 512))
    _bf16_contig("w_uv", w_uv, (H, 128, 512))
    if o is None:
        o = torch.empty((B, H, 128), dtype=torch.bfloat16, device=out.device)
    _bf16_contig("o", o, (B, H, 128))
    _lib._check("mla_up_project",
                _lib.mla_up_project(out.data_ptr(), w_uv.data_ptr(), o.data_ptr(), B, H, _stream()))
    return o
