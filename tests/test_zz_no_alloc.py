"""The decode without a workspace (mla_decode_noalloc, through the C ABI)
against the decode with one (mla_decode): two calls in a row on the library's
scratch array, the second with a smaller batch, each bit-identical to
mla_decode on the same inputs (same plan, same kernels) and within the parity
gate of the CPU oracle."""
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
from mla_latent_cache_absorbed_amd import _lib  # noqa: E402


def _say(*a):
    print(*a, flush=True, file=sys.stderr)


def _noalloc(w):
    out = torch.empty((w.B, w.H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
    st = _lib.mla_decode_noalloc(w.q.data_ptr(), w.cache.data_ptr(), w.block_table.data_ptr(),
                                 w.seq_lens.data_ptr(), float(w.scale), out.data_ptr(),
                                 lse.data_ptr(), w.B, w.H, w.NB, w.BS, w.M,
                                 torch.cuda.current_stream().cuda_stream)
    assert st == _lib.MLA_OK, _lib.status_string(st)
    return out, lse


def _gpu(w):
    return wl.Workload(w.name, w.q.cuda(), w.cache.cuda(), w.block_table.cuda(),
                       w.seq_lens.cuda(), w.scale)


@pytest.mark.parametrize("H", [128, 16])
def test_noalloc_matches_workspace_decode_on_two_calls(H):
    # first call: long requests (split, so the scratch holds partials and
    # counters), then a smaller batch that reuses the same scratch
    cases = [wl.make_custom([3000, 17, 2100, 64, 700, 5000], H=H, BS=64, seed=61, poison_unused=True),
             wl.make_custom([900, 33, 1], H=H, BS=16, seed=62, poison_unused=True)]
    for i, wc in enumerate(cases):
        w = _gpu(wc)
        _say(f"[noalloc] H={H} call {i}: B={w.B} lens={w.seq_lens_list()}")
        o1, l1 = _noalloc(w)
        o2, l2 = mla.decode(w.q, w.cache, w.block_table, w.seq_lens, w.scale)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"call {i}: differs from mla_decode"
        ro, rl = orc.oracle_decode(wl.bf16_bits(wc.q), wl.bf16_bits(wc.cache),
                                   wc.block_table.numpy(), wc.seq_lens.numpy(), wc.scale)
        rep = orc.parity_report(o1.float().cpu().numpy(), l1.cpu().numpy(), ro, rl)
        _say(f"[noalloc] H={H} call {i}: {rep}")
        assert rep["ok"], rep


def test_noalloc_full_size_dp_rank_sampled():
    """The DP-rank workload (124 x 4,096 tokens, 128 heads) fits the scratch
    array with the same plan as mla_decode: bit-identical outputs."""
    w = wl.make("dp_rank", device="cuda", seed=0)
    o1, l1 = _noalloc(w)
    o2, l2 = mla.decode(w.q, w.cache, w.block_table, w.seq_lens, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.isfinite(o1.float()).all() and torch.isfinite(l1).all()
    _say("[noalloc] dp_rank: bit-identical to mla_decode")


@pytest.mark.parametrize("H", [128, 16])
def test_noalloc_under_graph_capture(H):
    """The callers this entry point is for include code under HIP graph
    capture: one call captured (after a warm-up call outside the capture,
    which takes the scratch array's address), replayed four times with new
    query values, with an eager no-alloc call on another batch between the
    replays (it rewrites the shared scratch); every replay is bit-identical
    to mla_decode on the same values."""
    w = _gpu(wl.make_custom([2500, 9, 700, 64, 4100], H=H, BS=64, seed=71, poison_unused=True))
    other = _gpu(wl.make_custom([1500, 3, 333], H=H, BS=16, seed=72))
    q_in = w.q.clone()
    out = torch.empty((w.B, w.H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mla.decode_noalloc(q_in, w.cache, w.block_table, w.seq_lens, w.scale, out, lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mla.decode_noalloc(q_in, w.cache, w.block_table, w.seq_lens, w.scale, out, lse)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda")
    for rep in range(4):
        gen.manual_seed(200 + rep)
        q_new = torch.randn(w.q.shape, generator=gen, device="cuda").to(torch.bfloat16)
        q_in.copy_(q_new)
        _noalloc(other)  # eager use of the same scratch between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_e, l_e = mla.decode(q_new, w.cache, w.block_table, w.seq_lens, w.scale)
        torch.cuda.synchronize()
        assert torch.equal(out, o_e) and torch.equal(lse, l_e), rep
    _say(f"[noalloc] graph capture H={H}: 4 replays bit-identical to mla_decode")
