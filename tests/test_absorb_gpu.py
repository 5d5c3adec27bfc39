"""GPU parity of query absorption and value up-projection (C ABI
mla_absorb_prepare / mla_absorb_query / mla_up_project) against the oracle.

Tolerance, derived from the arithmetic: each output is a K-term dot product
of bf16 values accumulated in fp32 and rounded once to bf16, so
|gpu - ref| <= 2^-8 |ref| + K 2^-23 S with S = sum_k |w_k x_k| (bf16
round-to-nearest is within 2^-8 relative; fp32 accumulation of K products is
within K 2^-24 S, doubled for margin).  The RoPE part of q and the weight
transpose are copies and must match bit for bit.  The end-to-end chain
(absorb -> decode -> up-project) is checked against the oracle's chain on
the same inputs, which rounds to bf16 where the interfaces carry bf16 (the
absorbed query entering the decode, the decode output entering the
up-projection): lse to the decode's 1e-3, and o to the decode's gate on out
(1e-2 + 1e-2 |out|) carried through W_UV, sum_j |W_UV[i,j]| (1e-2 +
1e-2 |out_j|), plus the up-projection's own bound above.
"""
import math
import sys

import numpy as np
import pytest
import torch

from mla_latent_cache_absorbed_amd import workloads as wl
from oracle import mla_oracle as orc

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import mla_latent_cache_absorbed_amd as mla  # noqa: E402

DEV = torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True, file=sys.stderr)


def _bits(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _randn(shape, gen, std=1.0):
    return (torch.randn(shape, generator=gen) * std).to(torch.bfloat16).to(DEV)


def _gate(got, ref, S, K, what):
    bound = 2.0 ** -8 * np.abs(ref) + K * 2.0 ** -23 * S
    err = np.abs(got - ref)
    worst = float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0
    _say(f"[absorb] {what}: max |err| {err.max() if err.size else 0:.3g}, worst err/bound {worst:.3f}")
    assert np.all(err <= bound), what


def test_prepare_is_an_exact_transpose():
    gen = torch.Generator().manual_seed(1)
    for H in (1, 3, 128):
        w = _randn((H, 128, 512), gen)
        wt = mla.absorb_prepare(w)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(wt), np.swapaxes(_bits(w), 1, 2)), H


@pytest.mark.parametrize("B,H", [(1, 1), (5, 16), (33, 100), (124, 128), (300, 8)])
def test_absorb_query(B, H):
    gen = torch.Generator().manual_seed(B * 1000 + H)
    q_in = _randn((B, H, 192), gen)
    w_uk = _randn((H, 128, 512), gen, 1 / math.sqrt(128))
    q = mla.absorb_query(q_in, mla.absorb_prepare(w_uk))
    torch.cuda.synchronize()
    qb, wb = _bits(q_in), _bits(w_uk)
    ref = orc.oracle_absorb_query(qb, wb)
    S = np.einsum("bhd,hdj->bhj", np.abs(orc.bf16_bits_to_f64(qb[..., :128])),
                  np.abs(orc.bf16_bits_to_f64(wb)))
    got = orc.bf16_bits_to_f64(_bits(q))
    _gate(got[..., :512], ref[..., :512], S, 128, f"absorb B={B} H={H}")
    assert np.array_equal(_bits(q)[..., 512:], qb[..., 128:]), "RoPE part is a bit copy"


@pytest.mark.parametrize("B,H", [(1, 1), (5, 16), (33, 100), (124, 128), (300, 8)])
def test_up_project(B, H):
    gen = torch.Generator().manual_seed(B * 1000 + H + 7)
    out = _randn((B, H, 512), gen)
    w_uv = _randn((H, 128, 512), gen, 1 / math.sqrt(512))
    o = mla.up_project(out, w_uv)
    torch.cuda.synchronize()
    ob, wb = _bits(out), _bits(w_uv)
    ref = orc.oracle_up_project(ob, wb)
    S = np.einsum("bhj,hij->bhi", np.abs(orc.bf16_bits_to_f64(ob)), np.abs(orc.bf16_bits_to_f64(wb)))
    _gate(orc.bf16_bits_to_f64(_bits(o)), ref, S, 512, f"up-project B={B} H={H}")


def test_absorbed_layer_chain_against_oracle():
    """absorb -> decode -> up-project on the GPU against the oracle's chain."""
    gen = torch.Generator().manual_seed(42)
    lens = [1, 37, 200, 0, 64]
    H = 128
    w = wl.make_custom(lens, H=H, BS=16, seed=5, poison_unused=True)
    cache, table, sl = w.cache.to(DEV), w.block_table.to(DEV), w.seq_lens.to(DEV)
    B = len(lens)
    q_in = _randn((B, H, 192), gen)
    w_uk = _randn((H, 128, 512), gen, 1 / math.sqrt(128))
    w_uv = _randn((H, 128, 512), gen, 1 / math.sqrt(512) * 4)
    q = mla.absorb_query(q_in, mla.absorb_prepare(w_uk))
    out, lse = mla.decode(q, cache, table, sl, w.scale)
    o = mla.up_project(out, w_uv)
    torch.cuda.synchronize()
    q_ref = _round_bf16(orc.oracle_absorb_query(_bits(q_in), _bits(w_uk)))
    out_ref, lse_ref = orc.oracle_decode(q_ref, _bits(w.cache), w.block_table.numpy(),
                                         np.asarray(lens), w.scale)
    out_r = _round_bf16(out_ref)
    o_ref = orc.oracle_up_project(out_r, _bits(w_uv))
    Wa = np.abs(orc.bf16_bits_to_f64(_bits(w_uv)))
    carried = np.einsum("bhj,hij->bhi", 1e-2 + 1e-2 * np.abs(out_r), Wa)
    own = 2.0 ** -8 * np.abs(o_ref) + 512 * 2.0 ** -23 * np.einsum("bhj,hij->bhi", np.abs(out_r), Wa)
    got = o.float().cpu().numpy()
    err = np.abs(got - o_ref)
    lse_g = lse.cpu().numpy()
    fin = np.isfinite(lse_ref)
    lse_err = np.abs(lse_g[fin] - lse_ref[fin]).max()
    _say(f"[absorb] chain: max |err| {err.max():.3g}, worst err/bound "
         f"{(err / (carried + own)).max():.3f}, |ref| max {np.abs(o_ref).max():.3g}, "
         f"lse max err {lse_err:.3g}")
    assert np.all(err <= carried + own) and np.all(np.isfinite(got))
    assert lse_err <= 1e-3 and np.all(np.isneginf(lse_g[~fin]))
    assert np.all(got[3] == 0)  # the empty request


def _round_bf16(x):
    """float64 -> nearest bf16 value (via float32), as float64."""
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.to(torch.float64).numpy()
