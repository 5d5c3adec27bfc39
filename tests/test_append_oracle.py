"""Pins for the oracle of the paged latent append.

The append is pinned against the logical token sequence, built without any
paging: a decode over L + 1 tokens after appending row x at position L must
equal attention over the explicit list [rows..., x] (and torch's float64
scaled_dot_product_attention over it), every other cache row keeps its bits,
and planted indexing mistakes each fail a pin.
"""
import math

import numpy as np
import pytest
import torch

from oracle import mla_oracle as orc

SCALE = float(np.float32(1.0 / math.sqrt(192.0)))


def _bits(x):
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _setup(rng, lens, BS, spare=3):
    """Shuffled paged cache holding explicit rows per request, with room for one
    more token each.  Returns (cache bits, table, explicit rows per request)."""
    B = len(lens)
    need = [-(-(L + 1) // BS) for L in lens]
    M = max(need)
    NB = sum(need) + spare
    perm = rng.permutation(NB)
    table = np.full((B, M), NB - 1, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += n
    cache = _bits(rng.standard_normal((NB, BS, 576)))
    rows = []
    for b, L in enumerate(lens):
        t = np.arange(L)
        rows.append(cache[table[b, t // BS], t % BS].copy())
    return cache, table, rows


def pin_decode_sees_new_token_last(append, rng):
    lens = [0, 15, 16, 31, 7]  # empty, block edge from below, edge, mid
    BS = 16
    cache, table, rows = _setup(rng, lens, BS)
    B = len(lens)
    kv = _bits(rng.standard_normal((B, 512)))
    kr = _bits(rng.standard_normal((B, 64)))
    new, skipped = append(cache, table, lens, kv, kr)
    if skipped != 0:
        return False
    q = _bits(rng.standard_normal((B, 8, 576)))
    out, lse = orc.oracle_decode(q, new, table, np.asarray(lens) + 1, SCALE)
    for b in range(B):
        x = np.concatenate([kv[b], kr[b]])[None]
        explicit = orc.bf16_bits_to_f64(np.concatenate([rows[b], x]))
        qb = orc.bf16_bits_to_f64(q[b])
        o_ref, l_ref = orc.attend_one(qb, explicit, SCALE)
        # torch's float64 attention over the explicit list: one key/value head
        k = torch.from_numpy(explicit)[None, None]
        o_t = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qb)[None, :, None], k, k[..., :512], scale=SCALE)[0, :, 0]
        if not (np.allclose(out[b], o_ref, rtol=1e-12, atol=1e-13)
                and np.allclose(lse[b], l_ref, rtol=1e-12, atol=1e-12)
                and np.allclose(out[b], o_t.numpy(), rtol=1e-10, atol=1e-12)):
            return False
    return True


def pin_only_the_target_rows_change(append, rng):
    lens = [5, 16, 33]
    BS = 16
    cache, table, _ = _setup(rng, lens, BS)
    kv = _bits(rng.standard_normal((3, 512)))
    kr = _bits(rng.standard_normal((3, 64)))
    new, skipped = append(cache, table, lens, kv, kr)
    if skipped != 0:
        return False
    want = cache.copy()
    for b, p in enumerate(lens):
        r = table[b, p // BS], p % BS
        if not (np.array_equal(new[r][:512], kv[b]) and np.array_equal(new[r][512:], kr[b])):
            return False
        want[r] = new[r]
    return np.array_equal(new, want) and new.dtype == cache.dtype


def pin_skips(append, rng):
    BS = 16
    cache, table, _ = _setup(rng, [3, 3, 3, 3], BS)
    M = table.shape[1]
    table = table.copy()
    table[2, 0] = cache.shape[0]   # block id past NB
    table[3, 0] = -5               # negative block id
    kv = _bits(rng.standard_normal((4, 512)))
    kr = _bits(rng.standard_normal((4, 64)))
    new, skipped = append(cache, table, [-1, M * BS, 1, 2], kv, kr)
    return skipped == 3 and np.array_equal(new, cache)


def pin_last_slot(append, rng):
    BS = 16
    cache, table, _ = _setup(rng, [0], BS)
    M = table.shape[1]
    p = M * BS - 1
    kv = _bits(rng.standard_normal((1, 512)))
    kr = _bits(rng.standard_normal((1, 64)))
    new, skipped = append(cache, table, [p], kv, kr)
    r = table[0, M - 1], BS - 1
    return skipped == 0 and np.array_equal(new[r], np.concatenate([kv[0], kr[0]]))


PINS = [pin_decode_sees_new_token_last, pin_only_the_target_rows_change, pin_skips,
        pin_last_slot]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_append_oracle_pin(pin):
    assert pin(orc.oracle_append, np.random.default_rng(77))


def _mutant(kind):
    def append(cache, table, positions, kv_c, k_rope):
        cache = np.array(cache, copy=True)
        NB, BS, _ = cache.shape
        M = table.shape[1]
        skipped = 0
        for b, p in enumerate(int(x) for x in positions):
            if p < 0:
                continue
            if p >= M * BS or not 0 <= int(table[b, p // BS]) < NB:
                skipped += 1
                continue
            if kind == "div_mod_swapped":
                r = int(table[b, p % BS if p % BS < M else 0]), (p // BS) % BS
            elif kind == "position_plus_one":
                q_ = min(p + 1, M * BS - 1)
                r = int(table[b, q_ // BS]), q_ % BS
            elif kind == "physical_not_logical":
                r = (p // BS) % NB, p % BS
            else:
                r = int(table[b, p // BS]), p % BS
            row = np.concatenate([kv_c[b][:512], k_rope[b][:64]])
            if kind == "rope_first":
                row = np.concatenate([k_rope[b][:64], kv_c[b][:512]])
            cache[r] = row
        return cache, skipped
    return append


MUTANTS = ["div_mod_swapped", "position_plus_one", "physical_not_logical", "rope_first"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_append_mistake_is_caught(kind):
    app = _mutant(kind)
    caught = [p.__name__ for p in PINS if not p(app, np.random.default_rng(77))]
    assert caught, f"mutant {kind} passed every pin"


def test_unmutated_append_copy_passes():
    app = _mutant("none")
    for p in PINS:
        assert p(app, np.random.default_rng(77)), p.__name__
