"""The plan's split-KV chunk choice.
The plan kernel prices 256 candidate chunk sizes T (32, 64, ..., 4096, then
geometric steps of 2^(1/16) up to 32 * 32768 tokens) by
ceil(items / slots) * (T + per-item overhead), items = sum over requests of
max(1, ceil(L / T)), keeps candidates whose items fit the workspace, and
takes the cheapest, the larger chunk on ties.  The CPU test checks the
float arithmetic the kernel counts items with; the GPU test checks the
device's choice against a plain Python model of that rule.
"""

import numpy as np
import pytest

MAX_EXTRA_ITEMS = 1024  # workspace items beyond one per request


def _candidates():
    out = []
    for i in range(256):
        if i < 128:
            out.append(32 * (i + 1))
        else:
            k = 128.0 * 2.0 ** ((i - 127) / 16.0)
            # float32 exp2 on the device: the truncation below must not sit
            # on a rounding edge
            assert i % 16 == 15 or abs(k - round(k)) > 1e-3, (i, k)
            out.append(32 * int(k))
    return out


def _choose(lens, H, BS, M, slots):
    """Python model of the device chunk choice."""
    Lmax = M * BS
    lens = [min(max(int(L), 0), Lmax) for L in lens]
    cap = len(lens) + MAX_EXTRA_ITEMS
    ovh = 32 + 2 * H
    best = None
    for T in _candidates():
        n = sum(max(1, -(-L // T)) for L in lens)
        if n > cap:
            continue
        c = (-(-n // slots)) * (T + ovh)
        if best is None or c < best[0] or (c == best[0] and T > best[1]):
            best = (c, T)
    if best is None:
        return -(-Lmax // 32) * 32
    return best[1]


def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def test_float_item_count_is_exact():
    """ceil(m / d) as the kernel computes it: ceil of fma(m, 1/d, -1/(2d)) in
    float32, for every candidate d = T / 32 and m = ceil(L / 32) < 2^21,
    probed at multiples of d and one either side, with 1/d correctly rounded
    and one ulp off either way (a hardware reciprocal)."""
    ds = sorted({T // 32 for T in _candidates()})
    rng = np.random.default_rng(3)
    for d in ds:
        kmax = (1 << 21) // d
        ks = np.unique(np.concatenate([
            np.arange(0, min(kmax, 64) + 1),
            np.geomspace(1, kmax, 400).astype(np.int64),
            rng.integers(0, kmax + 1, 400), [kmax]]))
        m = np.concatenate([ks * d - 1, ks * d, ks * d + 1])
        m = m[(m >= 0) & (m < (1 << 21) + 1)]
        exact = np.maximum(1, -(-m // d))
        inv = np.float32(1.0) / np.float32(d)
        for inv_d in (inv, np.nextafter(inv, np.float32(0)), np.nextafter(inv, np.float32(1))):
            half = np.float64(inv_d) * 0.5
            # fma: the exact product and difference in float64 (49 significant
            # bits at most), then one rounding to float32
            y = _f32(m.astype(np.float64) * np.float64(inv_d) - half)
            got = np.maximum(np.float32(1), np.ceil(y)).astype(np.int64)
            bad = np.nonzero(got != exact)[0]
            assert bad.size == 0, (d, m[bad[:5]], got[bad[:5]], exact[bad[:5]])


def test_model_rule_on_textbook_cases():
    # one request of 4096 tokens, 256 slots: 128 items of 32 tokens fill one
    # round of slots, cost 1 * (32 + 288), the least any candidate reaches
    assert _choose([4096], H=128, BS=64, M=64, slots=256) == 32
    # 124 equal requests on 256 slots: two items each (248 <= 256) at 2048
    assert _choose([4096] * 124, H=128, BS=64, M=64, slots=256) == 2048
    # everything empty: every candidate gives one item per request, so the
    # cost grows with T and the smallest candidate wins
    assert _choose([0, 0, 0], H=16, BS=16, M=4, slots=1024) == 32


@pytest.mark.gpu
def test_device_choice_matches_model():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():  # pragma: no cover - CPU container
        pytest.skip("needs a GPU")
    import mla_latent_cache_absorbed_amd as mla
    from mla_latent_cache_absorbed_amd import workloads as wl

    dev = torch.device("cuda:0")
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    rng = np.random.default_rng(11)
    cases = [
        ("dp_rank", [4096] * 124, 128, 64, 64),
        ("tp_slice", [4096] * 159, 16, 64, 64),
        ("ragged", list(wl.spec("ragged").seq_lens), 128, 64, 2048),
        ("one long", [131072], 128, 64, 2048),
        ("zeros and ones", [0, 1, 0, 1, 2], 64, 16, 1),
        ("mixed", rng.integers(0, 20000, 300).tolist(), 48, 32, 625),
        ("many short", rng.integers(0, 200, 5000).tolist(), 128, 16, 13),
        ("non-resident mix", rng.integers(0, 3000, 4500).tolist(), 16, 64, 47),
    ]
    for name, lens, H, BS, M in cases:
        slots = ncu * (1 if H > 32 else 4)
        want = _choose(lens, H, BS, M, slots)
        sl = torch.tensor(lens, dtype=torch.int32, device=dev)
        ws = mla.Workspace(len(lens), H, M, BS, dev)
        mla.plan(sl, H, M, BS, ws)
        torch.cuda.synchronize()
        hdr = ws.header()
        n_items = sum(max(1, -(-min(L, M * BS) // want)) for L in lens)
        print(f"[plan] {name}: device chunk {hdr[1]} model {want} items {hdr[0]}", flush=True)
        assert hdr[1] == want, (name, hdr[:2], want)
        assert hdr[0] == n_items, (name, hdr[:2], n_items)
