"""Pins for the oracle's e4m3 encoder and FP8 append (CPU).

* encode(decode(c)) == c for all 254 finite codes (the decoder is pinned to
  torch and the OCP landmarks in test_fp8_oracle.py);
* the encoder equals torch's float8_e4m3fn rounding (an independent
  implementation) on random fp32 values of every binade in range and on the
  exact midpoints between neighbouring codes (ties to even);
* magnitudes past 448 saturate to +-448, infinities too, NaN encodes as 0x7F;
* the FP8 append stores e4m3(fp32(v) / kv_scale): decoding the row and
  multiplying by kv_scale returns v to within e4m3 rounding, exactly when v
  is kv_scale times a code value;
* planted mistakes (ties away from zero, truncation, no saturation, the
  scale multiplied instead of divided) each fail a pin.
"""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as orc


def _f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def pin_roundtrip(enc):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    return bool(np.array_equal(enc(orc.e4m3_to_f64(codes)), codes))


def pin_matches_torch(enc):
    rng = np.random.default_rng(3)
    mags = orc.e4m3_to_f64(np.arange(0x7F))
    mids = (mags[1:] + mags[:-1]) / 2
    x = np.concatenate([rng.uniform(-448, 448, 2000), rng.standard_normal(2000) * 2.0 ** rng.integers(-12, 8, 2000),
                        mids, -mids, mags, -mags])
    x = _f32(x)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return bool(np.array_equal(enc(x), ref))


def pin_saturation_and_nan(enc):
    big = _f32([449.0, 463.0, 464.0, 465.0, 1e4, 3e38, np.inf])
    return bool(np.all(enc(big) == 0x7E) and np.all(enc(-big) == 0xFE)
                and enc(np.array([np.nan]))[0] == 0x7F and enc(np.array([-0.0]))[0] == 0x80)


def pin_append_roundtrip(enc, append):
    rng = np.random.default_rng(4)
    B, NB, BS, M = 3, 5, 16, 2
    table = np.array([[3, 1], [0, 4], [2, 2]], dtype=np.int32)
    cache = np.zeros((NB, BS, 576), dtype=np.uint8)
    pos = [17, 5, 30]
    kv = 0.25
    # inputs that are kv times code values come back exactly
    codes = rng.integers(0, 0x7F, size=(B, 576)) | (rng.integers(0, 2, size=(B, 576)) << 7)
    vals = kv * orc.e4m3_to_f64(codes.astype(np.uint8))
    bits = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    new, skipped = append(cache, table, pos, bits[:, :512], bits[:, 512:], kv)
    if skipped != 0:
        return False
    for b, p in enumerate(pos):
        row = new[table[b, p // BS], p % BS]
        if not np.array_equal(kv * orc.e4m3_to_f64(row), orc.bf16_bits_to_f64(bits[b])):
            return False
    # random bf16 inputs: within e4m3 rounding (2^-4 relative for normals)
    x = rng.standard_normal((B, 576)) * 3
    bits = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    new, _ = append(cache, table, pos, bits[:, :512], bits[:, 512:], kv)
    for b, p in enumerate(pos):
        got = kv * orc.e4m3_to_f64(new[table[b, p // BS], p % BS])
        v = orc.bf16_bits_to_f64(bits[b])
        big = np.abs(v) >= kv * 2.0 ** -6
        if not (np.all(np.abs(got[big] - v[big]) <= 2.0 ** -4 * np.abs(v[big]))
                and np.all(np.abs(got[~big] - v[~big]) <= kv * 2.0 ** -10)):
            return False
    return True


PINS = [pin_roundtrip, pin_matches_torch, pin_saturation_and_nan]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_encoder_pin(pin):
    assert pin(orc.e4m3_from_f32)


def test_append_fp8_pin():
    assert pin_append_roundtrip(orc.e4m3_from_f32, orc.oracle_append_fp8)


def _mutant(kind):
    mags = orc.e4m3_to_f64(np.arange(0x7F))

    def enc(x):
        x = np.asarray(x, dtype=np.float64)
        out = np.empty(x.shape, dtype=np.uint8)
        for i, v in enumerate(x.reshape(-1)):
            if np.isnan(v):
                out.reshape(-1)[i] = 0x7F
                continue
            a = abs(v)
            j = int(np.searchsorted(mags, a))
            if j >= len(mags):
                c = 0x7F if kind == "no_saturation" and a >= 464 else 0x7E
            elif mags[j] == a or j == 0:
                c = j
            elif kind == "truncate":
                c = j - 1
            else:
                d_lo, d_hi = a - mags[j - 1], mags[j] - a
                tie = j if kind == "ties_away" else (j - 1 if (j - 1) % 2 == 0 else j)
                c = j - 1 if d_lo < d_hi else j if d_hi < d_lo else tie
            if kind == "no_saturation" and a >= 464:
                c = 0x7F
            out.reshape(-1)[i] = c | (0x80 if np.signbit(v) else 0)
        return out

    def append(cache, table, pos, kv_c, k_rope, kv_scale):
        s = np.float32(kv_scale) ** 2 if kind == "scale_multiplied" else np.float32(kv_scale)
        if kind == "scale_multiplied":
            def q(bits):
                v = orc.bf16_bits_to_f64(np.asarray(bits, dtype=np.uint16)).astype(np.float32)
                return enc((v * np.float32(kv_scale)).astype(np.float64))
        else:
            def q(bits):
                v = orc.bf16_bits_to_f64(np.asarray(bits, dtype=np.uint16)).astype(np.float32)
                return enc((v / s).astype(np.float64))
        return orc.oracle_append(cache, table, pos, [q(x) for x in kv_c], [q(x) for x in k_rope])
    return enc, append


MUTANTS = ["ties_away", "truncate", "no_saturation", "scale_multiplied"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_encoder_mistake_is_caught(kind):
    enc, append = _mutant(kind)
    caught = [p.__name__ for p in PINS if not p(enc)]
    if not pin_append_roundtrip(enc, append):
        caught.append("pin_append_roundtrip")
    assert caught, f"mutant {kind} passed every pin"


def test_unmutated_encoder_copy_passes():
    enc, append = _mutant("none")
    for p in PINS:
        assert p(enc), p.__name__
    assert pin_append_roundtrip(enc, append)
