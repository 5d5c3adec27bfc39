"""Pins for the oracle's query absorption and value up-projection.

* The chain absorb -> absorbed decode -> up-project must equal ordinary
  per-head attention with K = [W_UK kv_c ; k_rope] and V = W_UV kv_c, both the
  oracle's explicit form and torch's float64 scaled_dot_product_attention
  (page "DP attention + expert parallel: MLA KV replication", section
  "A strong answer": the absorbed form is a rewrite of that attention).
* Selector weights (identity blocks, column rotations) give exactly known
  outputs, which catch transposed weights, head mix-ups and a dropped RoPE part.
* Planted mistakes must each fail a pin.
"""
import math

import numpy as np
import pytest
import torch

from oracle import mla_oracle as orc

SCALE = float(np.float32(1.0 / math.sqrt(192.0)))


def _paged(rng, lens, BS=16):
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
    cache = rng.standard_normal((NB, BS, 576))
    rows = [cache[table[b, np.arange(L) // BS], np.arange(L) % BS] for b, L in enumerate(lens)]
    return cache, table, rows


def pin_chain_equals_explicit(absorb, up, rng):
    B, H = 3, 4
    lens = [5, 17, 1]
    cache, table, rows = _paged(rng, lens)
    q_in = rng.standard_normal((B, H, 192))
    W_UK = rng.standard_normal((H, 128, 512)) / math.sqrt(512)
    W_UV = rng.standard_normal((H, 128, 512)) / math.sqrt(512)
    q = absorb(q_in, W_UK)
    out, lse = orc.oracle_decode(q, cache, table, np.asarray(lens), SCALE)
    o = up(out, W_UV)
    for b in range(B):
        kv_c, k_rope = rows[b][:, :512], rows[b][:, 512:]
        o_e, l_e = orc.explicit_mla_decode(q_in[b, :, :128], q_in[b, :, 128:], kv_c, k_rope,
                                           W_UK, W_UV, SCALE)
        if not (np.allclose(o[b], o_e, rtol=1e-10, atol=1e-12)
                and np.allclose(lse[b], l_e, rtol=1e-12, atol=1e-12)):
            return False
        # torch: per head keys [W_UK kv_c ; k_rope], values W_UV kv_c
        kc = torch.from_numpy(kv_c)
        K = torch.stack([torch.cat([kc @ torch.from_numpy(W_UK[h]).T, torch.from_numpy(k_rope)], 1)
                         for h in range(H)])[None]
        V = torch.stack([kc @ torch.from_numpy(W_UV[h]).T for h in range(H)])[None]
        Q = torch.from_numpy(q_in[b])[None, :, None]
        o_t = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=SCALE)[0, :, 0]
        if not np.allclose(o[b], o_t.numpy(), rtol=1e-10, atol=1e-12):
            return False
    return True


def pin_selector_weights(absorb, up, rng):
    B, H = 5, 3
    q_in = rng.standard_normal((B, H, 192))
    W_UK = np.zeros((H, 128, 512))
    for h in range(H):
        # head h moves q_nope into latent columns 100h .. 100h+127
        W_UK[h, np.arange(128), 100 * h + np.arange(128)] = 1.0
    q = absorb(q_in, W_UK)
    for h in range(H):
        want = np.zeros((B, 576))
        want[:, 100 * h:100 * h + 128] = q_in[:, h, :128]
        want[:, 512:] = q_in[:, h, 128:]
        if not np.array_equal(q[:, h], want):
            return False
    out = rng.standard_normal((B, H, 512))
    W_UV = np.zeros((H, 128, 512))
    for h in range(H):
        W_UV[h, np.arange(128), (np.arange(128) * 3 + 7 * h) % 512] = 1.0
    o = up(out, W_UV)
    for h in range(H):
        if not np.array_equal(o[:, h], out[:, h, (np.arange(128) * 3 + 7 * h) % 512]):
            return False
    return True


PINS = [pin_chain_equals_explicit, pin_selector_weights]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_absorb_oracle_pin(pin):
    assert pin(orc.oracle_absorb_query, orc.oracle_up_project, np.random.default_rng(21))


def _mutants(kind):
    def absorb(q_in, W):
        q_in = np.asarray(q_in, dtype=np.float64)
        B, H, _ = q_in.shape
        q = np.zeros((B, H, 576))
        for h in range(H):
            hw = (h + 1) % H if kind == "uk_head_shift" else h
            q[:, h, :512] = q_in[:, h, :128] @ W[hw]
            if kind == "rope_dropped":
                continue
            q[:, h, 512:] = q_in[:, h, :64] if kind == "rope_from_nope" else q_in[:, h, 128:192]
        return q

    def up(out, W):
        out = np.asarray(out, dtype=np.float64)
        B, H, _ = out.shape
        o = np.zeros((B, H, 128))
        for h in range(H):
            hw = (h + 1) % H if kind == "uv_head_shift" else h
            if kind == "uv_transposed_rows":
                # reads W as if stored [512, 128] and reshaped
                o[:, h] = out[:, h] @ W[hw].reshape(512, 128)
            else:
                o[:, h] = out[:, h] @ W[hw].T
        return o
    return absorb, up


MUTANTS = ["uk_head_shift", "rope_dropped", "rope_from_nope", "uv_head_shift", "uv_transposed_rows"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_absorb_mistake_is_caught(kind):
    a, u = _mutants(kind)
    caught = [p.__name__ for p in PINS if not p(a, u, np.random.default_rng(21))]
    assert caught, f"mutant {kind} passed every pin"


def test_unmutated_absorb_copy_passes():
    a, u = _mutants("none")
    for p in PINS:
        assert p(a, u, np.random.default_rng(21)), p.__name__
