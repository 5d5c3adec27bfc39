"""ctypes binding of ``libmla_decode.so`` (C ABI in ``include/mla_decode.h``,
``include/mla_append.h`` and ``include/mla_absorb.h``).

Argument marshalling only: every step of the decode runs in the HIP library.
The library must have been built (``python -m mla_latent_cache_absorbed_amd.build``
or ``__graft_entry__.build()``); loading fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla_decode.so")

# status codes (mla_status)
MLA_OK = 0
MLA_ERR_NULL_POINTER = 1
MLA_ERR_BAD_SHAPE = 2
MLA_ERR_UNSUPPORTED = 3
MLA_ERR_BAD_SCALE = 4
MLA_ERR_WORKSPACE = 5
MLA_ERR_HIP = 6
MLA_ERR_ALIGNMENT = 7

MLA_CHECK_SEQ_LEN_RANGE = 1
MLA_CHECK_BLOCK_ID_RANGE = 2
MLA_CHECK_MERGE_WAIT = 4
MLA_CHECK_SCORE_RANGE = 8

#: every symbol the header declares, with (restype, argtypes)
_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
_S = ctypes.c_size_t
SIGNATURES = {
    "mla_decode_workspace_bytes": (_S, [_I, _I, _I, _I]),
    "mla_decode": (_I, [_P, _P, _P, _P, _F, _P, _P, _I, _I, _I, _I, _I, _P, _S, _P]),
    "mla_decode_plan": (_I, [_P, _I, _I, _I, _I, _I, _P, _S, _P]),
    "mla_decode_noalloc": (_I, [_P, _P, _P, _P, _F, _P, _P, _I, _I, _I, _I, _I, _P]),
    "mla_decode_attend": (_I, [_P, _P, _P, _F, _P, _P, _I, _I, _I, _I, _I, _P, _S, _P]),
    "mla_decode_read_error": (_I, [_P, ctypes.POINTER(ctypes.c_int32), _P]),
    "mla_status_string": (ctypes.c_char_p, [_I]),
    "mla_decode_abi_version": (_I, []),
    "mla_append_latent": (_I, [_P, _I, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "mla_append_latent_fp8": (_I, [_P, _I, _P, _I, _P, _P, _P, _F, _P, _I, _I, _I, _I, _P]),
    "mla_decode_fp8": (_I, [_P, _P, _P, _P, _F, _F, _P, _P, _I, _I, _I, _I, _I, _P, _S, _P]),
    "mla_decode_attend_fp8": (_I, [_P, _P, _P, _F, _F, _P, _P, _I, _I, _I, _I, _I, _P, _S, _P]),
    "mla_absorb_prepare": (_I, [_P, _P, _I, _P]),
    "mla_absorb_query": (_I, [_P, _P, _P, _I, _I, _P]),
    "mla_up_project": (_I, [_P, _P, _P, _I, _I, _P]),
}

_lib = None


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


def lib() -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP library not built: {LIB_PATH} is missing; run "
                "`python -m mla_latent_cache_absorbed_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().mla_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != MLA_OK:
        raise MlaError(fn, status)


# thin wrappers with the C names -------------------------------------------

def mla_decode_workspace_bytes(B: int, H: int, M: int, BS: int) -> int:
    return int(lib().mla_decode_workspace_bytes(B, H, M, BS))


def mla_decode(q, latent_cache, block_table, seq_lens, scale, out, lse,
               B, H, NB, BS, M, workspace, workspace_bytes, stream) -> int:
    return lib().mla_decode(q, latent_cache, block_table, seq_lens, scale, out, lse,
                            B, H, NB, BS, M, workspace, workspace_bytes, stream)


def mla_decode_noalloc(q, latent_cache, block_table, seq_lens, scale, out, lse,
                       B, H, NB, BS, M, stream) -> int:
    return lib().mla_decode_noalloc(q, latent_cache, block_table, seq_lens, scale, out, lse,
                                    B, H, NB, BS, M, stream)


def mla_decode_plan(seq_lens, B, H, M, BS, chunk_tokens, workspace, workspace_bytes,
                    stream) -> int:
    return lib().mla_decode_plan(seq_lens, B, H, M, BS, chunk_tokens, workspace,
                                 workspace_bytes, stream)


def mla_decode_attend(q, latent_cache, block_table, scale, out, lse, B, H, NB, BS, M,
                      workspace, workspace_bytes, stream) -> int:
    return lib().mla_decode_attend(q, latent_cache, block_table, scale, out, lse,
                                   B, H, NB, BS, M, workspace, workspace_bytes, stream)


def mla_decode_read_error(workspace, stream) -> int:
    v = ctypes.c_int32(0)
    _check("mla_decode_read_error", lib().mla_decode_read_error(workspace, ctypes.byref(v), stream))
    return int(v.value)


def mla_decode_abi_version() -> int:
    return int(lib().mla_decode_abi_version())


def mla_append_latent(kv_c, kv_c_stride, k_rope, k_rope_stride, positions, block_table,
                      latent_cache, skipped, B, NB, BS, M, stream) -> int:
    return lib().mla_append_latent(kv_c, kv_c_stride, k_rope, k_rope_stride, positions,
                                   block_table, latent_cache, skipped, B, NB, BS, M, stream)


def mla_append_latent_fp8(kv_c, kv_c_stride, k_rope, k_rope_stride, positions, block_table,
                          latent_cache_fp8, kv_scale, skipped, B, NB, BS, M, stream) -> int:
    return lib().mla_append_latent_fp8(kv_c, kv_c_stride, k_rope, k_rope_stride, positions,
                                       block_table, latent_cache_fp8, kv_scale, skipped, B, NB, BS,
                                       M, stream)


def mla_absorb_prepare(w_uk, w_uk_t, H, stream) -> int:
    return lib().mla_absorb_prepare(w_uk, w_uk_t, H, stream)


def mla_absorb_query(q_in, w_uk_t, q, B, H, stream) -> int:
    return lib().mla_absorb_query(q_in, w_uk_t, q, B, H, stream)


def mla_up_project(out, w_uv, o, B, H, stream) -> int:
    return lib().mla_up_project(out, w_uv, o, B, H, stream)


def mla_decode_fp8(q, latent_cache, block_table, seq_lens, scale, kv_scale, out, lse,
                   B, H, NB, BS, M, workspace, workspace_bytes, stream) -> int:
    return lib().mla_decode_fp8(q, latent_cache, block_table, seq_lens, scale, kv_scale, out, lse,
                                B, H, NB, BS, M, workspace, workspace_bytes, stream)


def mla_decode_attend_fp8(q, latent_cache, block_table, scale, kv_scale, out, lse, B, H, NB, BS,
                          M, workspace, workspace_bytes, stream) -> int:
    return lib().mla_decode_attend_fp8(q, latent_cache, block_table, scale, kv_scale, out, lse,
                                       B, H, NB, BS, M, workspace, workspace_bytes, stream)
