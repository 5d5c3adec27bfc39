"""GPU parity of the FP8-cache decode (C ABI mla_decode_fp8 / mla_decode_attend_fp8)
against the oracle, with the decode's gate: |out - ref| <= 1e-2 + 1e-2 |ref|,
|lse - ref| <= 1e-3, non-finite output where the reference is finite fails.
The caches are torch's e4m3 rounding of N(0, 1) latents over kv_scale; the
oracle decodes the same bytes."""
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


def _run(w, c8, kv, chunk=None, ws=None):
    out = torch.empty((w.B, w.H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device=DEV)
    if chunk is None:
        mla.decode_fp8(w.q, c8, w.block_table, w.seq_lens, w.scale, kv, out, lse, workspace=ws)
    else:
        ws = ws or mla.Workspace(w.B, w.H, w.M, w.BS, DEV)
        mla.plan(w.seq_lens, w.H, w.M, w.BS, ws, chunk_tokens=chunk)
        mla.attend_fp8(w.q, c8, w.block_table, w.scale, kv, out, lse, ws)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def _check(w, c8, kv, what, chunk=None, requests=None, ws=None):
    out, lse = _run(w, c8, kv, chunk, ws)
    ro, rl = orc.oracle_decode_fp8(wl.bf16_bits(w.q), c8.cpu().numpy(), w.block_table.cpu().numpy(),
                                   w.seq_lens.cpu().numpy(), w.scale, kv, requests=requests)
    if requests is not None:
        out, lse = out[requests], lse[requests]
    r = orc.parity_report(out, lse, ro, rl)
    _say(f"[fp8] {what}: {r}")
    assert r["ok"], f"{what}: {r}"


def _gpu(w):
    return wl.Workload(w.name, w.q.to(DEV), w.cache.to(DEV), w.block_table.to(DEV),
                       w.seq_lens.to(DEV), w.scale)


@pytest.mark.parametrize("H", [128, 100, 64, 48, 33, 32, 16, 5, 1])
def test_fp8_heads(H):
    """Wide kernels above 32 heads, the narrow kernel (double-buffered fp8
    stages per wave) at 32 and below."""
    w = _gpu(wl.make_custom([1, 31, 32, 33, 200, 0, 700], H=H, BS=64, seed=H, poison_unused=True))
    _check(w, wl.fp8_cache(w.cache), wl.DEFAULT_KV_SCALE, f"H={H}")


@pytest.mark.parametrize("H", [128, 48, 16])
@pytest.mark.parametrize("BS", [16, 32, 64, 128, 256, 1024])
def test_fp8_block_sizes(BS, H):
    """BS = 16 stages span two blocks (a request may end in the first)."""
    w = _gpu(wl.make_custom([5, 95, 300, 1000, 16, 17, 48], H=H, BS=BS, seed=BS + H, poison_unused=True))
    _check(w, wl.fp8_cache(w.cache), wl.DEFAULT_KV_SCALE, f"BS={BS}")


@pytest.mark.parametrize("kv", [1.0, 0.037, 3.5])
def test_fp8_scales(kv):
    w = _gpu(wl.make_custom([64, 130, 513], H=128, BS=64, seed=3))
    _check(w, wl.fp8_cache(w.cache, kv), kv, f"kv_scale={kv}")


@pytest.mark.parametrize("H,chunk", [(128, 32), (128, 96), (128, 1024), (48, 64), (48, 1024),
                                     (16, 32), (16, 96), (16, 1024), (1, 64)])
@pytest.mark.parametrize("BS", [32, 16])
def test_fp8_forced_splits(H, chunk, BS):
    """Splits of two and of three or more items: partials carry the scale."""
    w = _gpu(wl.make_custom([2000, 45, 700, 1], H=H, BS=BS, seed=chunk, poison_unused=True))
    _check(w, wl.fp8_cache(w.cache), wl.DEFAULT_KV_SCALE, f"H={H} chunk={chunk}", chunk=chunk)


@pytest.mark.parametrize("H,lens", [(128, [32 * 400, 37]), (48, [32 * 600]), (16, [32 * 400, 37])])
def test_fp8_splits_wider_than_the_staged_weights(H, lens):
    """As for the bf16 cache: more items than the merge units keep weights
    for in LDS, so every weight is recomputed from its log-sum-exp."""
    w = _gpu(wl.make_custom(lens, H=H, BS=64, seed=22, poison_unused=True))
    _check(w, wl.fp8_cache(w.cache), wl.DEFAULT_KV_SCALE, f"H={H} lens={lens} chunk=32", chunk=32)


@pytest.mark.parametrize("H", [128, 16])
def test_fp8_large_score_range_redo_path(H):
    """A key far larger than the rest late in a request forces the redo path."""
    w = wl.make_custom([600, 64], H=H, BS=64, seed=8)
    q = w.q.float()
    c = w.cache.float()
    blk = int(w.block_table[0, 500 // 64])
    c[blk, 500 % 64] = 0.0
    c[blk, 500 % 64, :512] = torch.sign(q[0, 0, :512]) * 25.0  # 400 in e4m3 units at 1/16
    w = _gpu(wl.Workload(w.name, w.q, c.to(torch.bfloat16), w.block_table, w.seq_lens, w.scale))
    _check(w, wl.fp8_cache(w.cache), wl.DEFAULT_KV_SCALE, "redo path")


def test_fp8_tiny_configuration():
    """The tiny parity shape (2 requests of 64 and 100 tokens, 128 heads,
    16-token blocks) with an fp8 cache, checked in full."""
    w = wl.make("tiny", device=DEV, seed=0)
    _check(w, wl.fp8_cache(w.cache), wl.DEFAULT_KV_SCALE, "tiny")


def test_fp8_full_size_dp_rank_sampled():
    """The DP-rank shape (124 x 4,096, 128 heads, 64-token blocks) with an fp8
    cache, in the launch configuration the benchmark times; sampled requests."""
    w = wl.make("dp_rank", device=DEV, seed=0)
    c8 = wl.fp8_cache(w.cache)
    reqs = [0, 1, 61, 122, 123]
    _check(w, c8, wl.DEFAULT_KV_SCALE, "dp_rank sampled", requests=reqs)


def test_fp8_tp_slice_full_size_sampled():
    """The TP-slice shape (159 x 4,096, 16 heads, 64-token blocks) with an fp8
    cache through the narrow kernel, as the benchmark launches it; sampled."""
    w = wl.make("tp_slice", device=DEV, seed=0)
    c8 = wl.fp8_cache(w.cache)
    reqs = [0, 1, 80, 157, 158]
    _check(w, c8, wl.DEFAULT_KV_SCALE, "tp_slice sampled", requests=reqs)


def test_fp8_ragged_full_size_sampled():
    w = wl.make("ragged", device=DEV, seed=0)
    c8 = wl.fp8_cache(w.cache)
    lens = w.seq_lens.cpu().numpy()
    reqs = [int(np.argmax(lens)), int(np.argmin(lens)), 7]
    _check(w, c8, wl.DEFAULT_KV_SCALE, "ragged sampled", requests=reqs)


@pytest.mark.parametrize("lens,H,BS", [([77, 1000, 3], 128, 64), ([2000, 45, 700, 1], 48, 32),
                                      ([77, 1000, 3, 0], 16, 64)])
def test_fp8_matches_bf16_decode_of_dequantised_cache(lens, H, BS):
    """The fp8 path against the bf16 path over the dequantised cache (e4m3
    values are exact in bf16; a power-of-two kv_scale keeps them exact).

    Every score product and every weighted-sum term is the same on both
    paths; only the order in which the score MFMAs add up the 576 products
    differs (the fp8 path reads two k-steps of 16 bytes at a time), which
    moves a score by a few fp32 ulps.  So lse agrees to 1e-5.  An output
    agrees to one bf16 rounding step of its own magnitude, 2^-7 |out|, plus,
    for a split request, one bf16 step of the split partials it merges:
    each path rounds its own partials to bf16, and two nearly equal values
    may round one step apart, 2^-7 |o_s|.  A normalised partial is a convex
    combination of the request's V rows, so |o_s| <= max_t |V[t, col]| over
    the request's tokens; 1e-4 covers the fp32 differences where terms
    cancel."""
    w = _gpu(wl.make_custom(lens, H=H, BS=BS, seed=12))
    c8 = wl.fp8_cache(w.cache, 0.0625)
    deq = (c8.view(torch.float8_e4m3fn).float() * 0.0625).to(torch.bfloat16)
    o8, l8 = _run(w, c8, 0.0625)
    wb = wl.Workload(w.name, w.q, deq, w.block_table, w.seq_lens, w.scale)
    ob = torch.empty_like(torch.from_numpy(o8)).to(DEV).to(torch.bfloat16)
    lb = torch.empty((w.B, w.H), dtype=torch.float32, device=DEV)
    mla.decode(wb.q, wb.cache, wb.block_table, wb.seq_lens, wb.scale, ob, lb)
    torch.cuda.synchronize()
    ob, lb = ob.float().cpu().numpy(), lb.cpu().numpy()
    d_out = np.abs(o8 - ob)
    fin = np.isfinite(lb)  # empty requests: lse = -inf on both paths
    d_lse = np.abs(l8[fin] - lb[fin])
    # max_t |V[t, col]| over each request's tokens, from the dequantised rows
    vmax = np.zeros((w.B, 1, 512), dtype=np.float32)
    rows = deq.float().cpu().numpy()
    table = w.block_table.cpu().numpy()
    for b, L in enumerate(lens):
        t = np.arange(int(L))
        if len(t):
            v = rows[table[b, t // BS], t % BS, :512]
            vmax[b, 0] = np.abs(v).max(axis=0)
    _say(f"[fp8] vs bf16 of the dequantised cache: max |d out| {d_out.max():.3g}, "
         f"equal {np.mean(o8 == ob):.4f}, max |d lse| {d_lse.max():.3g}")
    assert np.all(d_out <= 2.0 ** -7 * (np.maximum(np.abs(o8), np.abs(ob)) + vmax) + 1e-4)
    assert np.array_equal(np.isneginf(l8), np.isneginf(lb)) and np.all(np.isneginf(lb[~fin]))
    assert np.all(d_lse <= 1e-5 * np.maximum(1.0, np.abs(lb[fin])))


@pytest.mark.parametrize("H", [128, 16])
def test_fp8_scores_beyond_fp32_softmax_range_terminate(H):
    """A cache scale of 2^40 puts the scaled scores far beyond what the fp32
    softmax resolves: the call returns and raises at most the score-range bit."""
    w = _gpu(wl.make_custom([300, 100], H=H, BS=32, seed=2))
    ws = mla.Workspace(w.B, w.H, w.M, w.BS, DEV)
    _run(w, wl.fp8_cache(w.cache), 2.0 ** 40, ws=ws)
    flags = ws.check_flags()
    _say(f"[fp8] huge scale: flags {flags}")
    assert flags & ~mla._lib.MLA_CHECK_SCORE_RANGE == 0


@pytest.mark.parametrize("H", [128, 16])
@pytest.mark.parametrize("kv", [0.0, -0.25])
def test_fp8_zero_and_negative_cache_scale(H, kv):
    """kv_scale = 0 makes every cached value 0 (out = 0, lse = ln L); a
    negative scale negates the cache, so both scores and output change sign
    as the oracle's dequantised values do."""
    w = _gpu(wl.make_custom([1, 70, 333, 2000], H=H, BS=64, seed=32, poison_unused=True))
    c8 = wl.fp8_cache(w.cache, abs(kv) if kv != 0.0 else 0.0625)
    _check(w, c8, kv, f"H={H} kv_scale={kv}")
