"""Seeded synthetic inputs for absorbed MLA decode.

This module only draws random numbers and lays them out; it contains none of
the attention arithmetic.  Both the HIP path and the CPU oracle consume the
exact tensors it returns (the oracle reads their bf16 bytes back).

Workloads follow the shapes of the DeepSeek-V3 decode step the source pages
reason about: 128 heads, a 576-wide latent (512 ``kv_c`` + 64 ``k_rope``),
61 layers, 4,096-token contexts, and 159 sequences per node under TP=8 or 996
(124 per GPU) under DP attention (page "DP attention + expert parallel: MLA
KV replication", section "A strong answer").  Values are N(0, 1) drawn in
fp32 and rounded to bf16 (round-to-nearest-even); trained weights and real
activations are not available, and the decode kernel has no data-dependent
control flow, so these values are representative for timing.

Named workloads:

* ``tiny``      batch 2, seq_lens {64, 100}, 128 heads, block 16, identity
                block table (14 blocks), generated on the CPU with seed 0.
* ``dp_rank``   batch 124 x 4,096, 128 heads, block 64, 7,936 blocks,
                randomly permuted physical blocks.
* ``tp_slice``  batch 159 x 4,096, 16 heads, block 64, 10,176 blocks,
                permuted blocks.
* ``ragged``    batch 32, seq_lens log-uniform in [256, 131,072], 128 heads,
                block 64, permuted blocks.
* ``step61``    61 layers of ``dp_rank``; one shared block table, layer l
                uses seed l for its q and cache.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np
import torch

D_LATENT = 576
D_V = 512

#: scale applied to the raw 576-dim dot product: 1/sqrt(192), the per-head
#: query/key width of the non-absorbed form (128 nope + 64 rope dims), as the
#: fp32 value handed to the kernel.
DEFAULT_SCALE = float(np.float32(1.0 / math.sqrt(192.0)))


@dataclasses.dataclass
class Workload:
    name: str
    q: torch.Tensor            # bf16 [B, H, 576]
    cache: torch.Tensor        # bf16 [NB, BS, 576]
    block_table: torch.Tensor  # int32 [B, M]
    seq_lens: torch.Tensor     # int32 [B]
    scale: float

    @property
    def B(self) -> int:
        return int(self.q.shape[0])

    @property
    def H(self) -> int:
        return int(self.q.shape[1])

    @property
    def NB(self) -> int:
        return int(self.cache.shape[0])

    @property
    def BS(self) -> int:
        return int(self.cache.shape[1])

    @property
    def M(self) -> int:
        return int(self.block_table.shape[1])

    def seq_lens_list(self) -> List[int]:
        return [int(x) for x in self.seq_lens.cpu().tolist()]


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shapes of a named workload (no tensors)."""
    name: str
    B: int
    H: int
    BS: int
    seq_lens: tuple
    M: int
    NB: int
    layers: int = 1


def _ragged_lens(B: int, lo: int, hi: int, seed: int) -> List[int]:
    """Log-uniform integer lengths: floor(exp(ln lo + u (ln hi - ln lo)))."""
    rng = np.random.default_rng(seed)
    u = rng.random(B)
    lens = np.floor(np.exp(math.log(lo) + u * (math.log(hi) - math.log(lo))))
    return [int(min(max(x, lo), hi)) for x in lens]


def spec(name: str, seed: int = 0) -> Spec:
    if name == "tiny":
        return Spec("tiny", 2, 128, 16, (64, 100), 7, 14)
    if name == "dp_rank":
        return Spec("dp_rank", 124, 128, 64, (4096,) * 124, 64, 124 * 64)
    if name == "tp_slice":
        return Spec("tp_slice", 159, 16, 64, (4096,) * 159, 64, 159 * 64)
    if name == "ragged":
        lens = _ragged_lens(32, 256, 131072, seed)
        M = max(-(-L // 64) for L in lens)
        NB = sum(-(-L // 64) for L in lens)
        return Spec("ragged", 32, 128, 64, tuple(lens), M, NB)
    if name == "step61":
        return Spec("step61", 124, 128, 64, (4096,) * 124, 64, 124 * 64, 61)
    raise KeyError(name)


NAMES = ("tiny", "dp_rank", "tp_slice", "ragged", "step61")


def _randn_bf16(shape, gen: torch.Generator, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, device=device,
                       dtype=torch.float32).to(torch.bfloat16)


def _paged_table(seq_lens: Sequence[int], BS: int, M: int, NB: int,
                 perm: Optional[torch.Tensor], fill: int) -> torch.Tensor:
    """Block table that hands out physical blocks in request order.

    Request b's j-th logical block gets physical block ``perm[off_b + j]``
    (``off_b + j`` itself when ``perm`` is None).  Unused entries hold
    ``fill``, which callers point at a real (possibly poisoned) block.
    """
    table = torch.full((len(seq_lens), M), fill, dtype=torch.int32)
    off = 0
    for b, L in enumerate(seq_lens):
        n = -(-int(L) // BS)
        ids = torch.arange(off, off + n, dtype=torch.int64)
        if perm is not None:
            ids = perm[ids]
        table[b, :n] = ids.to(torch.int32)
        off += n
    assert off <= NB
    return table


def make(name: str, device="cpu", seed: int = 0, layer: int = 0) -> Workload:
    """Generate a named workload (``layer`` selects the layer of ``step61``)."""
    s = spec(name, seed)
    dev = torch.device(device)
    if name == "tiny":
        gen = torch.Generator(device="cpu").manual_seed(seed)
        q = _randn_bf16((s.B, s.H, D_LATENT), gen, "cpu")
        cache = _randn_bf16((s.NB, s.BS, D_LATENT), gen, "cpu")
        table = torch.arange(s.NB, dtype=torch.int32).reshape(s.B, s.M)
        lens = torch.tensor(s.seq_lens, dtype=torch.int32)
        return Workload(name, q.to(dev), cache.to(dev), table.to(dev),
                        lens.to(dev), DEFAULT_SCALE)
    # The permutation is drawn on the CPU so that the table does not depend
    # on the device; q and cache are drawn on the target device.
    pgen = torch.Generator(device="cpu").manual_seed(seed)
    perm = torch.randperm(s.NB, generator=pgen)
    table = _paged_table(s.seq_lens, s.BS, s.M, s.NB, perm, fill=0)
    data_seed = seed + layer if name == "step61" else seed
    gen = torch.Generator(device=dev).manual_seed(data_seed)
    q = _randn_bf16((s.B, s.H, D_LATENT), gen, dev)
    cache = _randn_bf16((s.NB, s.BS, D_LATENT), gen, dev)
    lens = torch.tensor(s.seq_lens, dtype=torch.int32)
    return Workload(name, q, cache, table.to(dev), lens.to(dev), DEFAULT_SCALE)


def make_custom(seq_lens: Sequence[int], H: int = 128, BS: int = 64,
                seed: int = 0, device="cpu", shuffle: bool = True,
                poison_unused: bool = False, extra_blocks: int = 0,
                M: Optional[int] = None, scale: float = DEFAULT_SCALE
                ) -> Workload:
    """Arbitrary-shape workload for tests.

    Physical blocks are handed out in request order (shuffled if
    ``shuffle``).  One extra physical block (the last) is always present;
    unused table entries point at it.  With ``poison_unused`` that block and
    every row past ``seq_lens[b]`` in a request's last block are filled with
    NaN, so any read of a row the method must not use shows up in the
    result.
    """
    B = len(seq_lens)
    need = [-(-int(L) // BS) for L in seq_lens]
    if M is None:
        M = max(1, max(need) if need else 1)
    NB = sum(need) + 1 + extra_blocks
    pgen = torch.Generator(device="cpu").manual_seed(seed)
    perm = torch.randperm(NB - 1, generator=pgen) if shuffle else None
    table = _paged_table(seq_lens, BS, M, NB - 1, perm, fill=NB - 1)
    gen = torch.Generator(device="cpu").manual_seed(seed + 1)
    q = _randn_bf16((B, H, D_LATENT), gen, "cpu")
    cache = _randn_bf16((NB, BS, D_LATENT), gen, "cpu")
    if poison_unused:
        nan = torch.tensor(float("nan"), dtype=torch.bfloat16)
        cache[NB - 1] = nan
        for b, L in enumerate(seq_lens):
            L = int(L)
            if L % BS:
                last = int(table[b, L // BS])
                cache[last, L % BS:] = nan
    lens = torch.tensor(list(seq_lens), dtype=torch.int32)
    dev = torch.device(device)
    return Workload("custom", q.to(dev), cache.to(dev), table.to(dev),
                    lens.to(dev), scale)


#: default fp8 cache scale: N(0, 1) latents divided by it stay well inside
#: e4m3's range (largest finite 448) while small values keep their 3-bit
#: mantissa (smallest normal 2^-6 * 0.0625)
DEFAULT_KV_SCALE = 0.0625


def fp8_cache(cache: torch.Tensor, kv_scale: float = DEFAULT_KV_SCALE) -> torch.Tensor:
    """An fp8 cache from a bf16 one: each value divided by ``kv_scale`` and
    rounded to OCP e4m3 by torch's conversion, returned as its uint8 bytes
    (same shape, same device).  NaN stays NaN."""
    x = (cache.float() / kv_scale).to(torch.float8_e4m3fn)
    return x.view(torch.uint8)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a bf16 tensor as uint16 bit patterns (what the oracle reads)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
