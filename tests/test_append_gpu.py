"""GPU parity of the paged latent append (C ABI mla_append_latent) against the
oracle: the whole cache bit for bit, the skipped count, and a short decode
loop (append, then decode over one more token) against the oracle's."""
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
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _new_tokens(B, gen, stride=576):
    """kv_c and k_rope as views into one [B, stride] buffer (the projection's
    output layout)."""
    buf = torch.randn((B, stride), generator=gen).to(torch.bfloat16).to(DEV)
    return buf, buf[:, :512], buf[:, 512:576]


def _check(cache0, table, pos, buf, kv, kr, what):
    cache = cache0.clone()
    skipped = torch.zeros(1, dtype=torch.int32, device=DEV)
    mla.append_latent(kv, kr, pos, table, cache, skipped)
    torch.cuda.synchronize()
    bb = _bits(buf)
    want, n_skip = orc.oracle_append(_bits(cache0), table.cpu().numpy(), pos.cpu().tolist(),
                                     bb[:, :512], bb[:, 512:576])
    got = _bits(cache)
    diff = int((got != want).any(axis=-1).sum())
    _say(f"[append] {what}: rows differing {diff}, skipped {int(skipped.item())} (oracle {n_skip})")
    assert diff == 0, what
    assert int(skipped.item()) == n_skip, what


@pytest.mark.parametrize("BS", [16, 64, 256])
def test_append_small_bitwise(BS):
    gen = torch.Generator().manual_seed(BS)
    B, M = 13, 4
    NB = B * M + 3
    table = torch.randperm(NB, generator=gen)[:B * M].reshape(B, M).to(torch.int32)
    # padding, block edges, last slot, out of range, and ordinary positions
    pos = [-1, 0, BS - 1, BS, 2 * BS + 1, M * BS - 1, M * BS, M * BS + 7, 3, 5, BS + 2, -7, 1]
    table[12, 0] = NB + 4      # block id past NB: skipped and counted
    table[11, 0] = -2          # request 11 is padding (position -7): its bad entry is never read
    cache0 = torch.randn((NB, BS, 576), generator=gen).to(torch.bfloat16).to(DEV)
    buf, kv, kr = _new_tokens(B, gen)
    _check(cache0, table.to(DEV), torch.tensor(pos, dtype=torch.int32, device=DEV), buf, kv, kr,
           f"BS={BS} B={B}")


def test_append_separate_buffers_and_strides():
    gen = torch.Generator().manual_seed(5)
    B, BS, M = 9, 16, 3
    NB = B * M
    table = torch.arange(NB, dtype=torch.int32).reshape(B, M).flip(1).contiguous()
    cache0 = torch.randn((NB, BS, 576), generator=gen).to(torch.bfloat16).to(DEV)
    kv_full = torch.randn((B, 520), generator=gen).to(torch.bfloat16).to(DEV)
    kr_full = torch.randn((B, 72), generator=gen).to(torch.bfloat16).to(DEV)
    kv, kr = kv_full[:, :512], kr_full[:, :64]
    pos = torch.tensor([0, 1, 15, 16, 17, 31, 32, 47, 20], dtype=torch.int32, device=DEV)
    cache = cache0.clone()
    mla.append_latent(kv, kr, pos, table.to(DEV), cache)
    torch.cuda.synchronize()
    want, n_skip = orc.oracle_append(_bits(cache0), table.numpy(), pos.cpu().tolist(),
                                     _bits(kv_full)[:, :512], _bits(kr_full)[:, :64])
    assert n_skip == 0
    assert np.array_equal(_bits(cache), want)


def test_append_empty_batch():
    cache = torch.zeros((2, 16, 576), dtype=torch.bfloat16, device=DEV)
    e = torch.empty((0, 576), dtype=torch.bfloat16, device=DEV)
    mla.append_latent(e[:, :512], e[:, 512:], torch.empty(0, dtype=torch.int32, device=DEV),
                      torch.empty((0, 1), dtype=torch.int32, device=DEV), cache)
    torch.cuda.synchronize()
    assert int(cache.view(torch.int16).abs().sum()) == 0


def test_append_full_size_dp_rank():
    """One new token for each of the 124 requests of the DP-rank shape, written
    into its 7,936-block cache; the whole cache is compared bit for bit."""
    w = wl.make("dp_rank", device=DEV, seed=0)
    gen = torch.Generator().manual_seed(9)
    pos = torch.randint(0, w.M * w.BS, (w.B,), generator=gen, dtype=torch.int32)
    pos[:4] = torch.tensor([0, w.BS - 1, w.BS, w.M * w.BS - 1], dtype=torch.int32)
    buf, kv, kr = _new_tokens(w.B, gen)
    _check(w.cache, w.block_table, pos.to(DEV), buf, kv, kr, "dp_rank B=124")


def test_decode_loop_against_oracle():
    """Three decode steps: append one token per request at its length, decode
    over the longer sequences, compare with the oracle doing the same."""
    gen = torch.Generator().manual_seed(3)
    lens = [15, 64, 1, 0, 100]
    H, BS = 128, 16
    w = wl.make_custom([L + 3 for L in lens], H=H, BS=BS, seed=4, poison_unused=True)
    w = wl.Workload(w.name, w.q.to(DEV), w.cache.to(DEV), w.block_table.to(DEV),
                    torch.tensor(lens, dtype=torch.int32, device=DEV), w.scale)
    ref_cache = _bits(w.cache)
    table = w.block_table.cpu().numpy()
    cur = list(lens)
    for step in range(3):
        buf, kv, kr = _new_tokens(w.B, gen)
        pos = torch.tensor(cur, dtype=torch.int32, device=DEV)
        mla.append_latent(kv, kr, pos, w.block_table, w.cache)
        bb = _bits(buf)
        ref_cache, n_skip = orc.oracle_append(ref_cache, table, cur, bb[:, :512], bb[:, 512:576])
        assert n_skip == 0
        cur = [L + 1 for L in cur]
        lens_t = torch.tensor(cur, dtype=torch.int32, device=DEV)
        out, lse = mla.decode(w.q, w.cache, w.block_table, lens_t, w.scale)
        torch.cuda.synchronize()
        ro, rl = orc.oracle_decode(_bits(w.q), ref_cache, table, np.asarray(cur), w.scale)
        r = orc.parity_report(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl)
        _say(f"[append] decode loop step {step} lens {cur}: {r}")
        assert r["ok"], r


def _check8(cache0, table, pos, buf, kv, kr, kv_scale, what):
    cache = cache0.clone()
    skipped = torch.zeros(1, dtype=torch.int32, device=DEV)
    mla.append_latent_fp8(kv, kr, pos, table, cache, kv_scale, skipped)
    torch.cuda.synchronize()
    bb = _bits(buf)
    want, n_skip = orc.oracle_append_fp8(cache0.cpu().numpy(), table.cpu().numpy(), pos.cpu().tolist(),
                                         bb[:, :512], bb[:, 512:576], kv_scale)
    got = cache.cpu().numpy()
    diff = int((got != want).any(axis=-1).sum())
    _say(f"[append fp8] {what}: rows differing {diff}, skipped {int(skipped.item())} (oracle {n_skip})")
    assert diff == 0, what
    assert int(skipped.item()) == n_skip, what


@pytest.mark.parametrize("BS", [16, 64])
@pytest.mark.parametrize("kv_scale", [0.0625, 0.3, -2.0])
def test_append_fp8_bitwise(BS, kv_scale):
    """The whole fp8 cache byte for byte against the oracle: random values,
    exact midpoints between e4m3 codes (ties to even), values that saturate,
    NaN, negative zero and subnormal codes, a skipped request and one with no
    token."""
    gen = torch.Generator().manual_seed(BS + int(abs(kv_scale) * 100))
    B, M = 9, 5
    NB = B * M + 2
    table = torch.randperm(NB - 1, generator=gen)[: B * M].reshape(B, M).to(torch.int32)
    table[7, 2] = NB + 5                       # a block id outside the cache
    cache0 = torch.randint(0, 256, (NB, BS, 576), generator=gen, dtype=torch.uint8)
    pos = torch.randint(0, M * BS, (B,), generator=gen, dtype=torch.int32)
    pos[7] = 2 * BS + 1                        # lands on the bad block: skipped
    pos[8] = -1                                # no token
    buf = (torch.randn((B, 576), generator=gen) * 4 * abs(kv_scale)).to(torch.bfloat16)
    codes = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).float()
    mids = (codes[1:] + codes[:-1]) / 2
    special = torch.cat([mids, -mids, torch.tensor([449.0, 500.0, 1e4, -1e4, float("inf"), float("nan"),
                                                      -0.0, 2.0 ** -9, 3 * 2.0 ** -10])])
    buf[0, : special.numel()] = (special * kv_scale).to(torch.bfloat16)
    buf = buf.to(DEV)
    _check8(cache0.to(DEV), table.to(DEV), pos.to(DEV), buf, buf[:, :512], buf[:, 512:576], kv_scale,
            f"BS={BS} kv_scale={kv_scale}")


def test_fp8_decode_loop_against_oracle():
    """Three decode steps over an fp8 cache: append each request's token (fp8),
    decode over the longer sequences, against the oracle doing the same."""
    gen = torch.Generator().manual_seed(5)
    lens = [15, 64, 1, 0, 100]
    kv = 0.0625
    for H in (128, 16):
        w = wl.make_custom([L + 3 for L in lens], H=H, BS=32, seed=6, poison_unused=True)
        c8 = wl.fp8_cache(w.cache, kv).to(DEV)
        table_d = w.block_table.to(DEV)
        ref_cache = c8.cpu().numpy()
        table = w.block_table.numpy()
        cur = list(lens)
        q = w.q.to(DEV)
        for step in range(3):
            buf, k_c, k_r = _new_tokens(w.B, gen)
            mla.append_latent_fp8(k_c, k_r, torch.tensor(cur, dtype=torch.int32, device=DEV), table_d, c8, kv)
            bb = _bits(buf)
            ref_cache, n_skip = orc.oracle_append_fp8(ref_cache, table, cur, bb[:, :512], bb[:, 512:576], kv)
            assert n_skip == 0
            cur = [L + 1 for L in cur]
            out, lse = mla.decode_fp8(q, c8, table_d, torch.tensor(cur, dtype=torch.int32, device=DEV),
                                      w.scale, kv)
            torch.cuda.synchronize()
            assert np.array_equal(c8.cpu().numpy(), ref_cache), (H, step)
            ro, rl = orc.oracle_decode_fp8(_bits(q), ref_cache, table, np.asarray(cur), w.scale, kv)
            r = orc.parity_report(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl)
            _say(f"[append fp8] decode loop H={H} step {step}: {r}")
            assert r["ok"], r
