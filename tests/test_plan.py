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


# ---------------------------------------------------------------------------
# The plan's whole output: header, per-request records, item list, merge-unit
# request list and counters, against a plain Python model of the layout rule.
# ---------------------------------------------------------------------------
K_HDR_BYTES = 256
K_CTR = 2
K_MERGE_MIN_ITEMS = 3


def _a256(x):
    return (x + 255) & ~255


def _layout_model(lens, chunk, nx, Lmax, units_per_req):
    """Item layout for chunk size `chunk`: requests split into exactly two
    items (pairs) first, pair j's halves nx positions apart for the first
    nx * (NP // nx) pairs and side by side after them; then every other
    request's full chunks, then their remainders, then one empty item per
    empty request.  Returns (hdr[0:7] without the check bits, req, big, items)."""
    L = [min(max(int(x), 0), Lmax) for x in lens]
    B = len(L)
    cnt = [L[b] // chunk + (1 if L[b] % chunk else 0) for b in range(B)]
    pairs = [b for b in range(B) if cnt[b] == 2]
    NP = len(pairs)
    G = NP // nx

    def pos(j, half):
        if j < G * nx:
            return 2 * nx * (j // nx) + j % nx + half * nx
        return 2 * j + half

    req = [None] * B
    items = {}
    for j, b in enumerate(pairs):
        p0, p1 = pos(j, 0), pos(j, 1)
        req[b] = (p0, 1, p1, 2)
        items[p0] = (b, 0, chunk, 2)
        items[p1] = (b, chunk, L[b], 2)
    Q0 = 2 * NP
    others = [b for b in range(B) if cnt[b] != 2]
    NF = sum(L[b] // chunk for b in others)
    NR = sum(1 for b in others if L[b] % chunk)
    NE = sum(1 for b in others if L[b] == 0)
    f = r = e = 0
    big = []
    for b in others:
        nf, nr = L[b] // chunk, (1 if L[b] % chunk else 0)
        fbeg = Q0 + f
        ritem = Q0 + NF + r if nr else -1
        req[b] = (fbeg, nf, ritem, cnt[b])
        for s in range(nf):
            items[fbeg + s] = (b, s * chunk, (s + 1) * chunk, cnt[b])
        if nr:
            items[ritem] = (b, nf * chunk, L[b], cnt[b])
        if L[b] == 0:
            items[Q0 + NF + NR + e] = (b, 0, 0, 0)
            e += 1
        if cnt[b] >= K_MERGE_MIN_ITEMS:
            big.append(b)
        f += nf
        r += nr
    n = 2 * NP + NF + NR + NE
    hdr = [n, chunk, None, 0, 2 * nx * G, len(big) * units_per_req, 0]
    return hdr, req, big, [items[i] for i in range(n)]


def test_layout_model_invariants():
    """The model covers each request's tokens exactly once, in order, with
    chunk-sized items (the last shorter), uses every position once, and puts
    the halves of the first nx * (NP // nx) pairs nx positions apart."""
    rng = np.random.default_rng(5)
    for chunk, nx in ((2048, 8), (128, 8), (96, 1), (32, 3)):
        lens = [0, 1, chunk, chunk + 1, 2 * chunk, 2 * chunk + 5, 7 * chunk] + \
            rng.integers(0, 9 * chunk, 60).tolist() + [2 * chunk] * 19
        hdr, req, big, items = _layout_model(lens, chunk, nx, 10 ** 9, 16)
        assert hdr[0] == len(items)
        for b, L in enumerate(lens):
            mine = sorted((t0, t1) for (bb, t0, t1, c) in items if bb == b)
            if L == 0:
                assert mine == [(0, 0)]
                continue
            assert mine[0][0] == 0 and mine[-1][1] == L
            assert all(a[1] == c[0] for a, c in zip(mine, mine[1:]))
            assert all(t1 - t0 == chunk for t0, t1 in mine[:-1]) and 0 < mine[-1][1] - mine[-1][0] <= chunk
            assert (b in big) == (len(mine) >= K_MERGE_MIN_ITEMS)
        pairs = [b for b in range(len(lens)) if req[b][1] == 1 and req[b][3] == 2]
        G = len(pairs) // nx
        for j, b in enumerate(pairs[:G * nx]):
            assert req[b][2] - req[b][0] == nx
    # 124 equal requests at chunk 2048 on 8 XCDs: 124 pairs, the first 120
    # in 15 groups of 16 positions, the last 4 side by side
    hdr, req, big, items = _layout_model([4096] * 124, 2048, 8, 4096, 16)
    assert hdr[0] == 248 and hdr[4] == 240 and big == []
    assert req[0] == (0, 1, 8, 2) and req[7] == (7, 1, 15, 2) and req[8] == (16, 1, 24, 2)
    assert req[120] == (240, 1, 241, 2) and req[123] == (246, 1, 247, 2)


@pytest.mark.gpu
def test_plan_layout_matches_model():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():  # pragma: no cover - CPU container
        pytest.skip("needs a GPU")
    import mla_latent_cache_absorbed_amd as mla
    from mla_latent_cache_absorbed_amd import workloads as wl

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(17)
    r1000 = rng.integers(0, 6000, 1000)
    r1000[::7] = 0
    cases = [
        ("dp_rank", [4096] * 124, 128, 64, 64, None),
        ("tp_slice", [4096] * 159, 16, 64, 64, None),
        ("ragged", list(wl.spec("ragged").seq_lens), 128, 64, 2048, None),
        ("13 pairs", [4000] * 13 + [100, 0, 9000], 128, 64, 256, 2048),
        ("forced 128", rng.integers(0, 1409, 100).tolist(), 128, 16, 88, 128),
        ("mixed H48", rng.integers(0, 20000, 300).tolist(), 48, 32, 625, None),
        ("1000", r1000.tolist(), 128, 64, 100, None),
        ("1024", rng.integers(0, 3000, 1024).tolist(), 128, 64, 50, None),
        ("1025", rng.integers(0, 3000, 1025).tolist(), 48, 64, 50, None),
        ("many short", rng.integers(0, 200, 5000).tolist(), 128, 16, 13, None),
        ("out of range", [5, -3, 70000, 64, 0, 4097], 128, 64, 64, 1024),
    ]
    for name, lens, H, BS, M, chunk in cases:
        B = len(lens)
        sl = torch.tensor(lens, dtype=torch.int32, device=dev)
        ws = mla.Workspace(B, H, M, BS, dev)
        ws.buf.fill_(0x5A)  # the plan must write every word it owns
        mla.plan(sl, H, M, BS, ws, chunk_tokens=chunk or 0)
        torch.cuda.synchronize()
        raw = ws.buf.cpu().numpy()
        words = raw.view(np.int32)
        hdr = words[:7].tolist()
        req_off = K_HDR_BYTES
        ctr_off = _a256(req_off + 16 * B)
        big_off = _a256(ctr_off + 4 * K_CTR * B)
        item_off = _a256(big_off + 4 * B)
        req = words[req_off // 4:req_off // 4 + 4 * B].reshape(B, 4)
        ctr = words[ctr_off // 4:ctr_off // 4 + K_CTR * B]
        units = 16 if H > 64 else 8 if H > 32 else 4
        Lmax = M * BS
        bad = any(L < 0 or L > Lmax for L in lens)
        # XCD placement applies to the wide kernels only; read nx back from
        # the header word that counts the XCD-paired items
        nxs = [1] if H <= 32 else [n for n in range(1, 65)
                                   if _layout_model(lens, hdr[1], n, Lmax, units)[0][4] == hdr[4]]
        want = None
        for nx in nxs:
            m = _layout_model(lens, hdr[1], nx, Lmax, units)
            items = words[item_off // 4:item_off // 4 + 4 * m[0][0]].reshape(-1, 4)
            if [tuple(x) for x in items.tolist()] == m[3]:
                want = m
                break
        print(f"[plan layout] {name}: B {B} chunk {hdr[1]} items {hdr[0]} nx {nxs[:3]}", flush=True)
        assert want is not None, (name, hdr)
        mh, mreq, mbig, _ = want
        assert hdr[0] == mh[0] and hdr[1] == mh[1] and hdr[3:7] == mh[3:7], (name, hdr, mh)
        assert hdr[2] == (mla._lib.MLA_CHECK_SEQ_LEN_RANGE if bad else 0), (name, hdr)
        assert [tuple(x) for x in req.tolist()] == mreq, name
        big = words[big_off // 4:big_off // 4 + len(mbig)].tolist()
        assert big == mbig, name
        assert (ctr == 0).all(), name
