"""Pins for the CPU oracle: it is checked against things other than itself.

* brute force (pure-Python scalar loops with math.fsum) on tiny inputs;
* a textbook library routine: absorbed MLA is multi-query attention with one
  key/value head of width 576 / 512, so torch's CPU float64
  scaled_dot_product_attention and logsumexp must agree;
* the explicit, non-absorbed form with per-head K = W_UK kv_c and
  V = W_UV kv_c (page "DP attention + expert parallel: MLA KV replication",
  section "A strong answer": the absorbed query attends over the latent
  directly; page "DP 与 DPA 的区别…", section "MLA：KV 是一份共享 latent…":
  the value head size equals kv_lora_rank);
* closed forms (one token, two tokens, constant latent), invariants (physical
  block permutation, head slices of a replicated cache, token duplication),
  and the split/merge identity;
* a planted-mistake check: plausible bugs written into copies of the oracle
  must each fail at least one of these pins.
"""
import math

import numpy as np
import pytest
import torch

from oracle import mla_oracle as orc

SCALE = float(np.float32(1.0 / math.sqrt(192.0)))


def _bf16(x):
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _paged(rows, BS, rng, shuffle=True, extra=1):
    """Place rows [L, 576] into a paged cache; returns cache, table row."""
    L = rows.shape[0]
    nblk = max(1, -(-L // BS))
    NB = nblk + extra
    perm = rng.permutation(NB) if shuffle else np.arange(NB)
    cache = rng.standard_normal((NB, BS, rows.shape[1]))
    for t in range(L):
        cache[perm[t // BS], t % BS] = rows[t]
    return cache, perm[:nblk]


def _case(rng, B, H, lens, BS, shuffle=True, bf16=True):
    q = rng.standard_normal((B, H, 576)).astype(np.float32)
    M = max(1, max(-(-L // BS) for L in lens))
    need = [-(-L // BS) for L in lens]
    NB = sum(need) + 2
    perm = rng.permutation(NB) if shuffle else np.arange(NB)
    table = np.full((B, M), NB - 1, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += n
    cache = rng.standard_normal((NB, BS, 576)).astype(np.float32)
    if bf16:
        return _bf16(q), _bf16(cache), table, np.asarray(lens, np.int32)
    return q.astype(np.float64), cache.astype(np.float64), table, np.asarray(lens, np.int32)


# ---------------------------------------------------------------------------
# pin functions, parameterised by the decode function under test
# ---------------------------------------------------------------------------

def pin_brute_force(decode, rng):
    for (B, H, lens, BS) in [(2, 4, [1, 17], 16), (1, 16, [40], 32),
                             (3, 1, [2, 15, 16], 16)]:
        q, c, t, s = _case(rng, B, H, lens, BS)
        out, lse = decode(q, c, t, s, SCALE)
        bo, bl = orc.brute_force_decode(q, c, t, s, SCALE)
        bo, bl = np.asarray(bo), np.asarray(bl)
        if not np.allclose(out, bo, rtol=1e-12, atol=1e-13):
            return False
        if not np.allclose(lse, bl, rtol=1e-12, atol=1e-13):
            return False
    return True


def pin_sdpa(decode, rng):
    H, L, BS = 8, 70, 16
    q, c, t, s = _case(rng, 1, H, [L], BS)
    out, lse = decode(q, c, t, s, SCALE)
    rows = orc.gather_request_rows(c, t[0], L, BS)
    qt = torch.from_numpy(orc.as_f64(q)[0])[None, :, None, :]          # [1,H,1,576]
    kt = torch.from_numpy(rows)[None, None].expand(1, H, L, 576)       # one KV head
    vt = torch.from_numpy(rows[:, :512])[None, None].expand(1, H, L, 512)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, scale=SCALE)[0, :, 0, :].numpy()
    ref_lse = torch.logsumexp(
        SCALE * (torch.from_numpy(orc.as_f64(q)[0]) @ torch.from_numpy(rows).T),
        dim=-1).numpy()
    return (np.allclose(out[0], ref, rtol=1e-12, atol=1e-13)
            and np.allclose(lse[0], ref_lse, rtol=1e-12, atol=1e-13))


def pin_explicit(decode, rng):
    for dn in (16, 128):
        H, L, BS = 4, 37, 16
        dv = dn
        kv_c = rng.standard_normal((L, 512))
        k_rope = rng.standard_normal((L, 64))
        W_UK = rng.standard_normal((H, dn, 512)) / math.sqrt(512)
        W_UV = rng.standard_normal((H, dv, 512)) / math.sqrt(512)
        q_nope = rng.standard_normal((H, dn))
        q_rope = rng.standard_normal((H, 64))
        ex_out, ex_lse = orc.explicit_mla_decode(q_nope, q_rope, kv_c, k_rope,
                                                 W_UK, W_UV, SCALE)
        rows = np.concatenate([kv_c, k_rope], axis=1)
        cache, trow = _paged(rows, BS, rng)
        q_abs = orc.absorb_query(q_nope, q_rope, W_UK)
        out, lse = decode(q_abs[None], cache, trow[None], np.array([L]), SCALE)
        up = np.einsum("hdj,hj->hd", W_UV, out[0])
        if not (np.allclose(up, ex_out, rtol=1e-10, atol=1e-12)
                and np.allclose(lse[0], ex_lse, rtol=1e-10, atol=1e-12)):
            return False
    return True


def pin_closed_forms(decode, rng):
    # one token: out = kv_c of that token exactly, lse = its scaled score
    q, c, t, s = _case(rng, 1, 4, [1], 16)
    out, lse = decode(q, c, t, s, SCALE)
    qf, cf = orc.as_f64(q), orc.as_f64(c)
    c0 = cf[t[0, 0], 0]
    if not np.array_equal(out[0], np.broadcast_to(c0[:512], out[0].shape)):
        return False
    s0 = np.array([SCALE * math.fsum(qf[0, h, d] * c0[d] for d in range(576))
                   for h in range(4)])
    if not np.allclose(lse[0], s0, rtol=1e-13, atol=1e-13):
        return False
    # two tokens: out = sigmoid(s0 - s1) c0 + sigmoid(s1 - s0) c1
    q, c, t, s = _case(rng, 1, 4, [2], 16)
    out, lse = decode(q, c, t, s, SCALE)
    qf, cf = orc.as_f64(q), orc.as_f64(c)
    r0, r1 = cf[t[0, 0], 0], cf[t[0, 0], 1]
    for h in range(4):
        s0 = SCALE * math.fsum(qf[0, h, d] * r0[d] for d in range(576))
        s1 = SCALE * math.fsum(qf[0, h, d] * r1[d] for d in range(576))
        a = 1.0 / (1.0 + math.exp(s1 - s0))
        want = a * r0[:512] + (1.0 - a) * r1[:512]
        if not np.allclose(out[0, h], want, rtol=1e-12, atol=1e-13):
            return False
        want_lse = max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1)))
        if abs(lse[0, h] - want_lse) > 1e-12:
            return False
    # constant latent: out = c[:512] exactly, lse = scale q.c + ln L
    L, BS = 50, 16
    row = orc.as_f64(_bf16(rng.standard_normal(576)))
    rows = np.tile(row, (L, 1))
    cache, trow = _paged(rows, BS, rng)
    qb = _bf16(rng.standard_normal((1, 3, 576)))
    out, lse = decode(qb, cache, trow[None], np.array([L]), SCALE)
    if not np.array_equal(out[0], np.broadcast_to(row[:512], out[0].shape)):
        return False
    qf = orc.as_f64(qb)
    want = [SCALE * math.fsum(qf[0, h, d] * row[d] for d in range(576)) + math.log(L)
            for h in range(3)]
    return np.allclose(lse[0], want, rtol=1e-12, atol=1e-12)


def pin_empty(decode, rng):
    q, c, t, s = _case(rng, 2, 4, [0, 5], 16)
    out, lse = decode(q, c, t, s, SCALE)
    return (np.all(out[0] == 0.0) and np.all(np.isneginf(lse[0]))
            and np.all(np.isfinite(lse[1])))


def pin_duplication(decode, rng):
    L, BS = 23, 16
    rows = orc.as_f64(_bf16(rng.standard_normal((L, 576))))
    qb = _bf16(rng.standard_normal((1, 4, 576)))
    cache, trow = _paged(rows, BS, rng)
    o1, l1 = decode(qb, cache, trow[None], np.array([L]), SCALE)
    for k in (2, 3):
        dup = np.repeat(rows, k, axis=0)
        cache, trow = _paged(dup, BS, rng)
        ok, lk = decode(qb, cache, trow[None], np.array([L * k]), SCALE)
        if not np.allclose(ok, o1, rtol=1e-12, atol=1e-13):
            return False
        if not np.allclose(lk, l1 + math.log(k), rtol=0, atol=1e-12):
            return False
    return True


def pin_permutation(decode, rng):
    """Physical permutation: bitwise equal.  Logical block order: close."""
    q, c, t, s = _case(rng, 2, 8, [45, 64], 16)
    o1, l1 = decode(q, c, t, s, SCALE)
    NB = c.shape[0]
    perm = rng.permutation(NB)           # new position of old block i = perm[i]
    c2 = np.empty_like(c)
    c2[perm] = c
    t2 = perm[t].astype(np.int32)
    o2, l2 = decode(q, c2, t2, s, SCALE)
    if not (np.array_equal(o1, o2) and np.array_equal(l1, l2)):
        return False
    # full logical blocks of request 1 (64 tokens = 4 blocks) in another order
    t3 = t.copy()
    t3[1, :4] = t[1, [2, 0, 3, 1]]
    o3, l3 = decode(q, c, t3, s, SCALE)
    return (np.allclose(o3, o1, rtol=1e-12, atol=1e-13)
            and np.allclose(l3, l1, rtol=1e-12, atol=1e-13))


def pin_head_slices(decode, rng):
    q, c, t, s = _case(rng, 2, 16, [33, 20], 16)
    o_full, l_full = decode(q, c, t, s, SCALE)
    os_, ls_ = [], []
    for g in range(8):
        o, l = decode(q[:, 2 * g:2 * g + 2].copy(), c.copy(), t, s, SCALE)
        os_.append(o)
        ls_.append(l)
    return (np.allclose(np.concatenate(os_, axis=1), o_full, rtol=1e-12, atol=1e-13)
            and np.allclose(np.concatenate(ls_, axis=1), l_full, rtol=1e-12, atol=1e-13))


PINS = [pin_brute_force, pin_sdpa, pin_explicit, pin_closed_forms, pin_empty,
        pin_duplication, pin_permutation, pin_head_slices]


# ---------------------------------------------------------------------------
# the real oracle passes every pin
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    assert pin(orc.oracle_decode, np.random.default_rng(1234))


def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x3E80,
                     0x4049, 0x0001], dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, math.inf, -math.inf, 0.25, 3.140625,
            2.0 ** -133]
    got = orc.bf16_bits_to_f64(bits)
    assert got.tolist() == want
    assert np.isnan(orc.bf16_bits_to_f64(np.array([0x7FC0], np.uint16))[0])


def test_brute_force_bitwise_head_slices():
    """Scalar loops give each head on its own, so slices match bit for bit."""
    rng = np.random.default_rng(7)
    q, c, t, s = _case(rng, 1, 4, [9], 16)
    fo, fl = orc.brute_force_decode(q, c, t, s, SCALE)
    for h in range(4):
        ho, hl = orc.brute_force_decode(q[:, h:h + 1].copy(), c, t, s, SCALE)
        assert ho[0][0] == fo[0][h] and hl[0][0] == fl[0][h]


def test_split_merge_identity():
    rng = np.random.default_rng(99)
    L = 300
    q, c, t, s = _case(rng, 1, 8, [L], 64, bf16=True)
    rows = orc.gather_request_rows(c, t[0], L, 64)
    qf = orc.as_f64(q)[0]
    full_o, full_l = orc.attend_one(qf, rows, SCALE)
    for cuts in ([0, 300], [0, 1, 300], [0, 64, 128, 192, 256, 300],
                 [0, 137, 138, 299, 300], [0, 0, 150, 150, 300]):
        o, l = orc.merge_partials(orc.split_partials(qf, rows, SCALE, cuts))
        np.testing.assert_allclose(o, full_o, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(l, full_l, rtol=1e-12, atol=1e-13)
    # all-empty merge
    o, l = orc.merge_partials(orc.split_partials(qf, rows, SCALE, [0, 0, 0]))
    assert np.all(o == 0) and np.all(np.isneginf(l))


def test_parity_report_gate():
    ref = np.array([[0.5, -0.25], [0.0, 1.0]])
    lse = np.array([1.0, -np.inf])
    r = orc.parity_report(ref + 0.009, np.array([1.0009, -np.inf]), ref, lse)
    assert r["ok"]
    r = orc.parity_report(ref + 0.0201, lse, ref, lse)
    assert not r["ok"]
    bad = ref.copy()
    bad[0, 0] = np.nan
    assert not orc.parity_report(bad, lse, ref, lse)["ok"]
    assert not orc.parity_report(ref, np.array([1.0, 0.0]), ref, lse)["ok"]
    assert not orc.parity_report(ref, np.array([1.002, -np.inf]), ref, lse)["ok"]


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin
# ---------------------------------------------------------------------------

def _mutant(kind):
    def attend(q_b, rows, scale):
        H = q_b.shape[0]
        L = rows.shape[0]
        if L == 0:
            return np.zeros((H, 512)), np.full((H,), -np.inf)
        if kind == "no_rope_in_scores":
            s = scale * (q_b[:, :512] @ rows[:, :512].T)
        elif kind == "sign":
            s = -scale * (q_b @ rows.T)
        elif kind == "scale_sqrt":
            s = math.sqrt(scale) * (q_b @ rows.T)
        elif kind == "no_scale":
            s = q_b @ rows.T
        else:
            s = scale * (q_b @ rows.T)
        axis = 0 if kind == "softmax_over_heads" else 1
        m = s.max(axis=axis, keepdims=True)
        w = np.exp(s - m)
        l = w.sum(axis=axis, keepdims=True)
        if kind == "value_from_rope_side":
            v = rows[:, 64:576]
        else:
            v = rows[:, :512]
        if kind == "no_normalise":
            out = w @ v
        elif kind == "softmax_over_heads":
            out = (w / l) @ v
        else:
            out = (w @ v) / l
        if kind == "lse_log2":
            lse = m[:, 0] / math.log(2) + np.log2(l[:, 0])
        elif kind == "lse_unscaled":
            lse = m[:, 0] / scale + np.log(l[:, 0])
        elif kind == "softmax_over_heads":
            lse = np.log(np.exp(s).sum(axis=1))
        else:
            lse = m[:, 0] + np.log(l[:, 0])
        return out, lse

    def decode(q, cache, table, lens, scale):
        qf = orc.as_f64(q)
        BS = cache.shape[1]
        outs, lses = [], []
        for b in range(qf.shape[0]):
            L = int(lens[b])
            if kind == "gather_off_by_one" and L:
                t_ = np.arange(L)
                blk = np.asarray(table[b])[np.minimum((t_ + 1) // BS, table.shape[1] - 1)]
                rows = orc.as_f64(cache)[blk, t_ % BS]
            elif kind == "gather_row_major_slip" and L:
                t_ = np.arange(L)
                flat = orc.as_f64(cache).reshape(-1, cache.shape[-1])
                rows = flat[(np.asarray(table[b])[0] * BS + t_) % flat.shape[0]]
            else:
                rows = orc.gather_request_rows(cache, table[b], L, BS)
            o, l_ = attend(qf[b], rows, scale)
            outs.append(o)
            lses.append(l_)
        return np.stack(outs), np.stack(lses)
    return decode


MUTANTS = ["no_rope_in_scores", "sign", "scale_sqrt", "no_scale",
           "softmax_over_heads", "value_from_rope_side", "no_normalise",
           "lse_log2", "lse_unscaled", "gather_off_by_one",
           "gather_row_major_slip"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind):
    dec = _mutant(kind)
    caught = [p.__name__ for p in PINS if not p(dec, np.random.default_rng(1234))]
    assert caught, f"mutant {kind} passed every pin"


def test_unmutated_copy_passes():
    dec = _mutant("none")
    for p in PINS:
        assert p(dec, np.random.default_rng(1234)), p.__name__


def test_tiny_workload_brute_force_heads():
    """The oracle on the tiny workload equals scalar brute force (8 of 128 heads)."""
    from mla_latent_cache_absorbed_amd import workloads as wl
    w = wl.make("tiny")
    q = wl.bf16_bits(w.q)[:, :8].copy()
    c = wl.bf16_bits(w.cache)
    t = w.block_table.numpy()
    s = w.seq_lens.numpy()
    out, lse = orc.oracle_decode(q, c, t, s, w.scale)
    bo, bl = orc.brute_force_decode(q, c, t, s, w.scale)
    np.testing.assert_allclose(out, np.asarray(bo), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, np.asarray(bl), rtol=1e-12, atol=1e-13)
