"""CPU oracle for absorbed-form MLA decode over a paged latent cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header,
constant or helper with the HIP library; the only thing both sides see is the
seeded input bytes, which are generated elsewhere and handed to both.

What is computed (the plain definition, written out step by step):

* The cache of one layer is a paged array ``[NB, BS, 576]``: for every cached
  token one head-less vector whose elements 0..511 are ``kv_c`` (the low-rank
  latent) and 512..575 are ``k_rope`` (the decoupled RoPE key), identical for
  every attention head.  Page "MLA 的 TP 切分：为什么 8 张 GPU 存了同一份 KV
  cache" (10100.com), section 3.1 (what each rank stores) and section 一
  (kv_lora_rank = 512, qk_rope_head_dim = 64, k_rope shared MQA-style).
* In decode the engine runs MLA in its absorbed form: each head's query has
  already been projected into the 576-wide latent space and attends over the
  shared latent directly.  Page "DP attention + expert parallel: MLA KV
  replication" (inferenceinterviews.com), section "A strong answer".
* The scores therefore use all 576 dimensions (forgetting the 64-wide RoPE
  part is the first item of that page's "Common mistakes"), and the value
  vector is the ``kv_c`` part only, because the value head size equals
  ``kv_lora_rank``.  Page "DP 与 DPA 的区别：SGLang 并行部署与路由"
  (chengxuchu.com), section "MLA：KV 是一份共享 latent，没有多个 head 可切".

Readings where the pages are silent (each is listed with its reason in the
repository's design notes):

* attention form: ordinary scaled softmax of the single decode query over all
  ``L_b`` cached tokens of request ``b``; no causal mask (the query is the
  newest position and its latent is already in the cache);
* ``scale`` multiplies the raw 576-dim dot product before the softmax;
* ``lse`` is the natural logarithm of the sum of exp(scaled scores);
* ``L_b == 0`` gives ``out = 0`` and ``lse = -inf``;
* token ``t`` of request ``b`` lives at
  ``cache[block_table[b, t // BS], t % BS, :]``; block-table entries past
  ``ceil(L_b / BS)`` and rows past ``L_b`` are never read.

Everything is evaluated in float64 on the exact bf16 input values.
"""

from __future__ import annotations

import math
from typing import Iterable, List, Sequence, Tuple

import numpy as np

D_LATENT = 576  # kv_c (512) + k_rope (64), one shared vector per token
D_KVC = 512     # kv_lora_rank: the value part of the latent
D_ROPE = 64     # qk_rope_head_dim


# ---------------------------------------------------------------------------
# bf16 decoding
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Decode bf16 bit patterns (uint16 / int16 array) into float64.

    A bf16 value is the upper 16 bits of an IEEE-754 binary32 value, so the
    decode is exact: shift into the high half of a 32-bit word and reinterpret.
    """
    b = np.asarray(bits)
    if b.dtype not in (np.uint16, np.int16):
        raise TypeError(f"expected 16-bit bf16 bit patterns, got {b.dtype}")
    u32 = b.astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def as_f64(x) -> np.ndarray:
    """float64 view of an input: bf16 bit patterns are decoded, floats upcast."""
    a = np.asarray(x)
    if a.dtype in (np.uint16, np.int16):
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


# ---------------------------------------------------------------------------
# paged cache access
# ---------------------------------------------------------------------------

def gather_request_rows(latent_cache: np.ndarray, block_table_row: np.ndarray,
                        seq_len: int, block_size: int) -> np.ndarray:
    """Rows ``c_t`` for ``t = 0 .. seq_len-1`` of one request, shape [L, 576].

    Logical token t sits in physical block ``block_table_row[t // BS]`` at
    offset ``t % BS`` (page "MLA 的 TP 切分…", section 3.1: the per-layer
    cache is the rank-3 array [NB, BS, 576]).  Only the first
    ``ceil(L / BS)`` table entries are read.
    """
    L = int(seq_len)
    if L == 0:
        return np.zeros((0, latent_cache.shape[-1]), dtype=np.float64)
    t = np.arange(L)
    blocks = np.asarray(block_table_row)[t // block_size].astype(np.int64)
    return as_f64(latent_cache)[blocks, t % block_size, :]


# ---------------------------------------------------------------------------
# the definition, one request at a time
# ---------------------------------------------------------------------------

def attend_one(q_b: np.ndarray, rows: np.ndarray, scale: float
               ) -> Tuple[np.ndarray, np.ndarray]:
    """Absorbed attention of all heads of one request over its latent rows.

    q_b  [H, 576] float64 — absorbed queries (0..511 absorbed nope part,
         512..575 rope part).
    rows [L, 576] float64 — the request's cached latent rows.

    scores s[h, t] = scale * <q_b[h, :576], rows[t, :576]>   (all 576 dims)
    weights w = exp(s - max_t s), l = sum_t w
    out[h, :] = (sum_t w[h, t] * rows[t, :512]) / l           (value = kv_c)
    lse[h]    = max_t s + ln l
    """
    H = q_b.shape[0]
    L = rows.shape[0]
    if L == 0:
        return np.zeros((H, D_KVC)), np.full((H,), -np.inf)
    s = float(scale) * (q_b @ rows.T)                   # [H, L]
    m = s.max(axis=1, keepdims=True)                    # [H, 1]
    w = np.exp(s - m)                                   # [H, L]
    l = w.sum(axis=1, keepdims=True)                    # [H, 1]
    out = (w @ rows[:, :D_KVC]) / l                     # [H, 512]
    lse = m[:, 0] + np.log(l[:, 0])
    return out, lse


def oracle_decode(q, latent_cache, block_table, seq_lens, scale,
                  requests: Iterable[int] | None = None
                  ) -> Tuple[np.ndarray, np.ndarray]:
    """Reference decode for every request (or the listed ``requests``).

    q            [B, H, 576]  bf16 bits or floats
    latent_cache [NB, BS, 576] bf16 bits or floats
    block_table  [B, M] int
    seq_lens     [B] int
    scale        float (the fp32 value the GPU receives; used in fp64)

    Returns ``out`` float64 [B', H, 512] (unrounded) and ``lse`` float64
    [B', H], where B' = B or len(requests).
    """
    qf = as_f64(q)
    bt = np.asarray(block_table)
    sl = np.asarray(seq_lens)
    BS = latent_cache.shape[1]
    idx = list(range(qf.shape[0])) if requests is None else list(requests)
    outs, lses = [], []
    for b in idx:
        rows = gather_request_rows(latent_cache, bt[b], int(sl[b]), BS)
        o, l = attend_one(qf[b], rows, scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


# ---------------------------------------------------------------------------
# split-KV partials and their log-sum-exp merge
# ---------------------------------------------------------------------------

def split_partials(q_b: np.ndarray, rows: np.ndarray, scale: float,
                   boundaries: Sequence[int]
                   ) -> List[Tuple[np.ndarray, np.ndarray]]:
    """Attention over consecutive token chunks ``[boundaries[i], boundaries[i+1])``.

    Each chunk yields its own normalised output and log-sum-exp; an empty
    chunk yields ``(0, -inf)``.
    """
    parts = []
    for a, z in zip(boundaries[:-1], boundaries[1:]):
        parts.append(attend_one(q_b, rows[a:z], scale))
    return parts


def merge_partials(parts: Sequence[Tuple[np.ndarray, np.ndarray]]
                   ) -> Tuple[np.ndarray, np.ndarray]:
    """Combine chunk results by their log-sum-exps.

    With chunk outputs o_s (each normalised by its own sum) and lse_s:
    lse = ln sum_s exp(lse_s);  out = sum_s exp(lse_s - lse) * o_s.
    Chunks with lse_s = -inf carry zero weight; if every chunk is empty the
    result is out = 0, lse = -inf.
    """
    lse_s = np.stack([p[1] for p in parts])             # [S, H]
    o_s = np.stack([p[0] for p in parts])               # [S, H, 512]
    m = lse_s.max(axis=0)                               # [H]
    out = np.zeros(o_s.shape[1:])
    lse = np.full(m.shape, -np.inf)
    ok = np.isfinite(m)
    if ok.any():
        w = np.exp(lse_s[:, ok] - m[ok])                # [S, H']
        lam = w.sum(axis=0)
        lse[ok] = m[ok] + np.log(lam)
        out[ok] = np.einsum("sh,shj->hj", w / lam, o_s[:, ok])
    return out, lse


# ---------------------------------------------------------------------------
# FP8 latent cache
# ---------------------------------------------------------------------------

def e4m3_to_f64(codes) -> np.ndarray:
    """Decode OCP FP8 E4M3 bytes: sign bit, 4 exponent bits (bias 7), 3
    mantissa bits; exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN and
    there are no infinities (so S.1111.110 = 448 is the largest finite)."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    mag = np.where((e == 15) & (b & 0x7 == 7), np.nan, mag)
    return sign * mag


def oracle_decode_fp8(q, cache_fp8, block_table, seq_lens, scale, kv_scale,
                      requests: Iterable[int] | None = None
                      ) -> Tuple[np.ndarray, np.ndarray]:
    """Decode over an FP8 latent cache [NB, BS, 576] of e4m3 bytes.

    The pages give the cache as 576 bytes per token and layer in FP8 (page
    "MLA 的 TP 切分…", sections 2.3 and 5.1) and no scale convention; the
    reading taken is one scale per cache, element value = kv_scale *
    e4m3(byte).  The attention is then the bf16 definition over those values
    (:func:`attend_one`), gathered per request so that only its rows are
    decoded.
    """
    qf = as_f64(q)
    bt = np.asarray(block_table)
    sl = np.asarray(seq_lens)
    BS = cache_fp8.shape[1]
    idx = list(range(qf.shape[0])) if requests is None else list(requests)
    outs, lses = [], []
    for b in idx:
        L = int(sl[b])
        t = np.arange(L)
        rows = float(kv_scale) * e4m3_to_f64(np.asarray(cache_fp8)[np.asarray(bt[b])[t // BS], t % BS])
        rows = rows.reshape(L, D_LATENT)
        o, l = attend_one(qf[b], rows, scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


# ---------------------------------------------------------------------------
# paged append: the step that puts a new token into the cache
# ---------------------------------------------------------------------------

def oracle_append(latent_cache: np.ndarray, block_table: np.ndarray,
                  positions: Sequence[int], kv_c: np.ndarray, k_rope: np.ndarray
                  ) -> Tuple[np.ndarray, int]:
    """Cache after storing request b's new token at logical position positions[b].

    The token goes to the row the decode reads it from, block
    ``block_table[b, p // BS]``, offset ``p % BS`` (page "MLA 的 TP 切分…",
    section 3.1: per layer one [NB, BS, 576] array, elements 0..511 kv_c and
    512..575 k_rope).  The stored bits are the inputs' bits.  A negative
    position means no token; a position at or past ``M * BS`` or a block id
    outside ``[0, NB)`` is skipped and counted.  Requests are applied in
    order.  Returns (new cache, number skipped); the input cache is not
    modified.
    """
    cache = np.array(latent_cache, copy=True)
    NB, BS, _ = cache.shape
    bt = np.asarray(block_table)
    M = bt.shape[1]
    skipped = 0
    for b, p in enumerate(int(x) for x in positions):
        if p < 0:
            continue
        if p >= M * BS or not 0 <= int(bt[b, p // BS]) < NB:
            skipped += 1
            continue
        row = cache[int(bt[b, p // BS]), p % BS]
        row[:D_KVC] = kv_c[b][:D_KVC]
        row[D_KVC:] = k_rope[b][:D_ROPE]
    return cache, skipped


def e4m3_from_f32(x) -> np.ndarray:
    """Encode fp32 values as OCP FP8 E4M3 bytes: the finite code nearest to
    the value, ties to the code with an even mantissa (round to nearest
    even), magnitudes past 448 saturating to +-448 (S.1111.110), NaN to
    0x7F, and the sign kept (-0 is 0x80).

    Found by searching the 127 non-negative finite codes in order of
    magnitude, which the decoding above defines; a tie sits exactly halfway
    between two neighbouring codes, and of two neighbours the even code is
    the one whose last bit (the mantissa's last bit) is 0.
    """
    x = np.asarray(x, dtype=np.float64)
    mags = e4m3_to_f64(np.arange(0x7F))        # codes 0x00 .. 0x7E, ascending
    out = np.empty(x.shape, dtype=np.uint8)
    flat_x, flat_o = x.reshape(-1), out.reshape(-1)
    for i, v in enumerate(flat_x):
        if np.isnan(v):
            flat_o[i] = 0x7F
            continue
        a = abs(v)
        j = int(np.searchsorted(mags, a))      # first code with magnitude >= a
        if j >= len(mags):
            c = 0x7E                           # past 448: saturate
        elif mags[j] == a or j == 0:
            c = j
        else:
            d_lo, d_hi = a - mags[j - 1], mags[j] - a
            c = j - 1 if d_lo < d_hi else j if d_hi < d_lo else (j - 1 if (j - 1) % 2 == 0 else j)
        flat_o[i] = c | (0x80 if np.signbit(v) else 0)
    return out


def oracle_append_fp8(cache_fp8: np.ndarray, block_table: np.ndarray, positions: Sequence[int],
                      kv_c: np.ndarray, k_rope: np.ndarray, kv_scale: float
                      ) -> Tuple[np.ndarray, int]:
    """oracle_append for an FP8 cache [NB, BS, 576] of e4m3 bytes holding
    values kv_scale * e4m3(byte): each bf16 input value v is stored as
    e4m3_from_f32(fp32(v) / fp32(kv_scale)), the quotient rounded once to
    fp32.  The page on TP sharding prices the FP8 cache (page "MLA 的 TP
    切分…", sections 2.3 and 5.1) without a scale convention; this is the
    inverse of the one the FP8 decode reads with.  Slots, skips and order are
    those of oracle_append.
    """
    s32 = np.float32(kv_scale)

    def quant(bits):
        v = bf16_bits_to_f64(np.asarray(bits, dtype=np.uint16)).astype(np.float32)
        with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
            return e4m3_from_f32((v / s32).astype(np.float64))
    q_kv = [quant(np.asarray(kv_c[b])[:D_KVC]) for b in range(len(positions))]
    q_kr = [quant(np.asarray(k_rope[b])[:D_ROPE]) for b in range(len(positions))]
    return oracle_append(cache_fp8, block_table, positions, q_kv, q_kr)


# ---------------------------------------------------------------------------
# the explicit (non-absorbed) form, for checking the absorbed rewrite
# ---------------------------------------------------------------------------

def explicit_mla_decode(q_nope: np.ndarray, q_rope: np.ndarray,
                        kv_c: np.ndarray, k_rope: np.ndarray,
                        W_UK: np.ndarray, W_UV: np.ndarray, scale: float
                        ) -> Tuple[np.ndarray, np.ndarray]:
    """Ordinary per-head attention with keys and values expanded from the latent.

    q_nope [H, dn], q_rope [H, 64], kv_c [L, 512], k_rope [L, 64],
    W_UK [H, dn, 512], W_UV [H, dv, 512].

    Head h sees keys  k[h, t] = [W_UK[h] @ kv_c[t] ; k_rope[t]]  and values
    v[h, t] = W_UV[h] @ kv_c[t]; k_rope is the same for every head.  Returns
    out [H, dv] and lse [H].
    """
    H = q_nope.shape[0]
    L = kv_c.shape[0]
    dv = W_UV.shape[1]
    out = np.zeros((H, dv))
    lse = np.full((H,), -np.inf)
    for h in range(H):
        if L == 0:
            continue
        k_nope = kv_c @ W_UK[h].T                       # [L, dn]
        keys = np.concatenate([k_nope, k_rope], axis=1)  # [L, dn + 64]
        vals = kv_c @ W_UV[h].T                         # [L, dv]
        qh = np.concatenate([q_nope[h], q_rope[h]])
        s = float(scale) * (keys @ qh)
        m = s.max()
        w = np.exp(s - m)
        out[h] = (w @ vals) / w.sum()
        lse[h] = m + math.log(w.sum())
    return out, lse


def absorb_query(q_nope: np.ndarray, q_rope: np.ndarray, W_UK: np.ndarray
                 ) -> np.ndarray:
    """Project per-head queries into the latent: [W_UK[h]^T q_nope[h] ; q_rope[h]]."""
    q_lat = np.einsum("hdj,hd->hj", W_UK, q_nope)       # [H, 512]
    return np.concatenate([q_lat, q_rope], axis=1)     # [H, 576]


# ---------------------------------------------------------------------------
# the products either side of the absorbed decode
# ---------------------------------------------------------------------------

D_NOPE = 128    # nope part of a query head
D_VHEAD = 128   # value head width


def oracle_absorb_query(q_in, W_UK) -> np.ndarray:
    """Absorbed decode query of every request and head, float64 [B, H, 576].

    q_in [B, H, 192]: per head the 128-wide nope part, then the 64-wide RoPE
    part; W_UK [H, 128, 512]: head h's key up-projection (key = W_UK[h] kv_c).
    The score of the explicit form, q_nope . (W_UK[h] kv_c) + q_rope . k_rope,
    equals [W_UK[h]^T q_nope ; q_rope] . [kv_c ; k_rope] (page "DP attention +
    expert parallel: MLA KV replication", section "A strong answer": the query
    is moved into the latent space instead of the keys out of it).
    """
    qf = as_f64(q_in)
    W = as_f64(W_UK)
    B, H, _ = qf.shape
    q = np.zeros((B, H, D_LATENT))
    for h in range(H):
        q[:, h, :D_KVC] = qf[:, h, :D_NOPE] @ W[h]      # [B,128] @ [128,512]
        q[:, h, D_KVC:] = qf[:, h, D_NOPE:D_NOPE + D_ROPE]
    return q


def oracle_up_project(out, W_UV) -> np.ndarray:
    """Value-head outputs, float64 [B, H, 128]: o[b,h] = W_UV[h] @ out[b,h].

    out [B, H, 512] is the absorbed decode's latent-space output (attention
    weights applied to kv_c); W_UV [H, 128, 512] is head h's value
    up-projection (value = W_UV[h] kv_c), so W_UV[h] sum_t p_t kv_c_t is the
    explicit form's sum_t p_t v_t.
    """
    of = as_f64(out)
    W = as_f64(W_UV)
    B, H, _ = of.shape
    o = np.zeros((B, H, D_VHEAD))
    for h in range(H):
        o[:, h, :] = of[:, h, :] @ W[h].T               # [B,512] @ [512,128]
    return o


# ---------------------------------------------------------------------------
# scalar brute force (tiny inputs only)
# ---------------------------------------------------------------------------

def brute_force_decode(q, latent_cache, block_table, seq_lens, scale
                       ) -> Tuple[List[List[List[float]]], List[List[float]]]:
    """The same definition with plain Python loops and ``math.fsum``.

    Written independently of :func:`attend_one` (no NumPy arithmetic), for
    inputs of at most a few hundred tokens.  Returns nested lists
    out[b][h][j] and lse[b][h].
    """
    qf = as_f64(q).tolist()
    cf = as_f64(latent_cache).tolist()
    bt = np.asarray(block_table).tolist()
    sl = [int(x) for x in np.asarray(seq_lens).tolist()]
    BS = len(cf[0])
    B, H = len(qf), len(qf[0])
    sc = float(scale)
    out_all, lse_all = [], []
    for b in range(B):
        L = sl[b]
        rows = []
        for t in range(L):
            rows.append(cf[bt[b][t // BS]][t % BS])
        out_b, lse_b = [], []
        for h in range(H):
            qh = qf[b][h]
            if L == 0:
                out_b.append([0.0] * D_KVC)
                lse_b.append(-math.inf)
                continue
            scores = [sc * math.fsum(qh[d] * r[d] for d in range(D_LATENT))
                      for r in rows]
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            tot = math.fsum(w)
            o = [math.fsum(w[t] * rows[t][j] for t in range(L)) / tot
                 for j in range(D_KVC)]
            out_b.append(o)
            lse_b.append(mx + math.log(tot))
        out_all.append(out_b)
        lse_all.append(lse_b)
    return out_all, lse_all


# ---------------------------------------------------------------------------
# the tolerance the GPU result is held to
# ---------------------------------------------------------------------------

OUT_ATOL = 1e-2
OUT_RTOL = 1e-2
LSE_ATOL = 1e-3


def parity_report(out_gpu, lse_gpu, out_ref, lse_ref) -> dict:
    """Elementwise gate: |out - ref| <= 1e-2 + 1e-2*|ref|, |lse - ref| <= 1e-3.

    ``out_ref``/``lse_ref`` are the unrounded float64 oracle values.  A
    non-finite GPU value where the reference is finite fails; -inf lse must
    match -inf exactly.
    """
    og = np.asarray(out_gpu, dtype=np.float64)
    lg = np.asarray(lse_gpu, dtype=np.float64)
    orf = np.asarray(out_ref, dtype=np.float64)
    lrf = np.asarray(lse_ref, dtype=np.float64)
    out_err = np.abs(og - orf)
    out_bad = ~(out_err <= OUT_ATOL + OUT_RTOL * np.abs(orf))
    fin = np.isfinite(lrf)
    lse_bad = np.zeros(lrf.shape, dtype=bool)
    lse_bad[fin] = ~(np.abs(lg[fin] - lrf[fin]) <= LSE_ATOL)
    lse_bad[~fin] = ~(lg[~fin] == lrf[~fin])
    rms_ref = float(np.sqrt(np.mean(orf ** 2))) if orf.size else 0.0
    return {
        "ok": bool(not out_bad.any() and not lse_bad.any()),
        "out_bad": int(out_bad.sum()),
        "lse_bad": int(lse_bad.sum()),
        "out_max_abs_err": float(np.nanmax(out_err)) if out_err.size else 0.0,
        "out_rms_err_rel": (float(np.sqrt(np.nanmean(out_err ** 2))) / rms_ref
                            if rms_ref > 0 else 0.0),
        "lse_max_abs_err": (float(np.max(np.abs(lg[fin] - lrf[fin])))
                            if fin.any() else 0.0),
    }
