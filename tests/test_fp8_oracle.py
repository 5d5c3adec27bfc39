"""Pins for the oracle's FP8 latent cache (e4m3 decoding and the scale's place).

* e4m3 decoding matches torch's float8_e4m3fn for all 256 bytes, and the
  OCP definition's landmarks (1.0, the largest finite 448, the smallest
  subnormal 2^-9, NaN at S.1111.111, no infinities);
* with one token the decode has a closed form: out = kv_scale * e4m3(c[0:512])
  and lse = scale * kv_scale * q . e4m3(c);
* the fp8 decode equals the bf16 oracle over the dequantised cache, and a
  power-of-two kv_scale moves between the cache and q without changing the
  scores;
* planted mistakes (scale dropped from the output, scale squared, bias 8,
  fnuz-style decoding) each fail a pin.
"""
import math

import numpy as np
import pytest
import torch

from oracle import mla_oracle as orc

SCALE = float(np.float32(1.0 / math.sqrt(192.0)))


def _decode_ref(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def pin_decode_table(dec, rng):
    allb = np.arange(256, dtype=np.uint8)
    got, ref = dec(allb), _decode_ref(allb)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    landmarks = (dec(np.array([0x38]))[0] == 1.0 and dec(np.array([0x7E]))[0] == 448.0
                 and dec(np.array([0x01]))[0] == 2.0 ** -9 and np.isnan(dec(np.array([0x7F]))[0])
                 and np.isnan(dec(np.array([0xFF]))[0]) and dec(np.array([0xFE]))[0] == -448.0
                 and not np.isinf(dec(allb)).any())
    return bool(same.all()) and landmarks


def _case(rng, lens, BS=16, H=4):
    B = len(lens)
    need = [max(1, -(-L // BS)) for L in lens]
    M = max(need)
    NB = sum(need) + 1
    perm = rng.permutation(NB)
    table = np.full((B, M), NB - 1, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += n
    cache8 = rng.integers(0, 256, size=(NB, BS, 576), dtype=np.uint8)
    cache8[(cache8 & 0x7F) == 0x7F] = 0x11  # no NaN codes in live data
    q = rng.standard_normal((B, H, 576))
    return q, cache8, table


def pin_one_token(decode8, dec, rng):
    q, c8, t = _case(rng, [1, 1])
    kv = 0.3
    out, lse = decode8(q, c8, t, np.array([1, 1]), SCALE, kv)
    for b in range(2):
        row = dec(c8[t[b, 0], 0])
        if not (np.allclose(out[b], np.broadcast_to(kv * row[:512], out[b].shape), rtol=1e-14, atol=0)
                and np.allclose(lse[b], SCALE * kv * (q[b] @ row), rtol=1e-12, atol=1e-12)):
            return False
    return True


def pin_equals_bf16_over_dequantised(decode8, dec, rng):
    lens = [0, 5, 33, 17]
    q, c8, t = _case(rng, lens)
    kv = 0.0625
    out, lse = decode8(q, c8, t, np.array(lens), SCALE, kv)
    deq = kv * dec(c8.reshape(-1)).reshape(c8.shape)
    o2, l2 = orc.oracle_decode(q, deq, t, np.array(lens), SCALE)
    if not (np.allclose(out, o2, rtol=1e-13, atol=1e-15) and np.allclose(lse, l2, rtol=1e-13, atol=1e-13)):
        return False
    # a power-of-two scale may move from the cache to q (scores) but the
    # output carries it: out(kv=2) = 2 * out(kv=1) computed with 2q
    o_a, l_a = decode8(q, c8, t, np.array(lens), SCALE, 2.0)
    o_b, l_b = decode8(2.0 * q, c8, t, np.array(lens), SCALE, 1.0)
    fin = np.isfinite(l_b)
    return bool(np.allclose(o_a, 2.0 * o_b, rtol=1e-13, atol=1e-15)
                and np.allclose(l_a[fin], l_b[fin], rtol=1e-13, atol=1e-13))


PINS = [pin_decode_table, pin_one_token, pin_equals_bf16_over_dequantised]


def _call(pin, decode8, dec, rng):
    if pin is pin_decode_table:
        return pin(dec, rng)
    return pin(decode8, dec, rng)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_fp8_oracle_pin(pin):
    assert _call(pin, orc.oracle_decode_fp8, orc.e4m3_to_f64, np.random.default_rng(5))


def _mutant(kind):
    def dec(codes):
        b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
        sign = np.where(b & 0x80, -1.0, 1.0)
        e = (b >> 3) & 0xF
        m = (b & 0x7).astype(np.float64)
        bias = 8 if kind in ("bias8", "fnuz") else 7
        mag = np.where(e == 0, m * 2.0 ** (1 - bias - 3), (1.0 + m / 8.0) * np.exp2(e - bias))
        if kind == "fnuz":
            mag = np.where(b == 0x80, np.nan, mag)
            sign = np.where(b == 0x80, 1.0, sign)
        else:
            mag = np.where((e == 15) & (b & 0x7 == 7), np.nan, mag)
        return sign * mag

    def decode8(q, c8, table, lens, scale, kv):
        qf = orc.as_f64(q)
        BS = c8.shape[1]
        outs, lses = [], []
        for b in range(qf.shape[0]):
            L = int(lens[b])
            t = np.arange(L)
            rows = dec(c8[table[b][t // BS], t % BS]).reshape(L, 576)
            kv_rows = kv * kv if kind == "scale_squared" else kv
            o, l = orc.attend_one(qf[b], kv_rows * rows, scale)
            if kind == "output_unscaled":
                o = o / kv
            outs.append(o)
            lses.append(l)
        return np.stack(outs), np.stack(lses)
    return decode8, dec


MUTANTS = ["bias8", "fnuz", "scale_squared", "output_unscaled"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_fp8_mistake_is_caught(kind):
    d8, dec = _mutant(kind)
    caught = [p.__name__ for p in PINS if not _call(p, d8, dec, np.random.default_rng(5))]
    assert caught, f"mutant {kind} passed every pin"


def test_unmutated_fp8_copy_passes():
    d8, dec = _mutant("none")
    for p in PINS:
        assert _call(p, d8, dec, np.random.default_rng(5)), p.__name__


def test_fp8_cache_generator_is_torch_rounding():
    """The seeded fp8 caches are torch's e4m3 rounding of value / kv_scale."""
    from mla_latent_cache_absorbed_amd import workloads as wl
    w = wl.make("tiny")
    c8 = wl.fp8_cache(w.cache, 0.0625).numpy()
    v = orc.e4m3_to_f64(c8) * 0.0625
    ref = w.cache.float().numpy()
    # round to nearest with 3 mantissa bits: within 2^-4 relative (normals)
    big = np.abs(ref) >= 2.0 ** -6 * 0.0625
    assert np.all(np.abs(v[big] - ref[big]) <= 2.0 ** -4 * np.abs(ref[big]))
