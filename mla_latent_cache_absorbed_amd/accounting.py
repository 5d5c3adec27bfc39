"""Algorithmic work of one absorbed-MLA decode call (what the method must move).

Bytes counted per call (one layer):

* every cached latent row of every request once: 576 bf16 = 1,152 B per token;
* the block-table entries that are used (4 B per used block) and ``seq_lens``;
* the queries (576 bf16 per head), the outputs (512 bf16 per head) and the
  fp32 log-sum-exp per head.

With an FP8 cache a token's latent is 576 B (one byte per element).

Flops: per (request, head, token), 2*576 for the score and 2*512 for the
weighted sum of the ``kv_c`` part.  Split-KV partials are scratch traffic of
a particular kernel design and are not part of the algorithmic figure.
"""
from __future__ import annotations

from typing import Sequence

ROW_BYTES = 576 * 2     # one token's latent in bf16
Q_BYTES = 576 * 2       # one head's absorbed query
OUT_BYTES = 512 * 2     # one head's output in bf16
LSE_BYTES = 4


def cache_bytes(seq_lens: Sequence[int]) -> int:
    return ROW_BYTES * sum(int(L) for L in seq_lens)


def algorithmic_bytes(seq_lens: Sequence[int], H: int, BS: int, row_bytes: int = ROW_BYTES) -> int:
    """Bytes of one call; ``row_bytes`` = 576 for an FP8 cache."""
    B = len(seq_lens)
    per_req = sum(row_bytes * int(L) + 4 * (-(-int(L) // BS)) + 4 for L in seq_lens)
    return per_req + B * H * (Q_BYTES + OUT_BYTES + LSE_BYTES)


def algorithmic_flops(seq_lens: Sequence[int], H: int) -> int:
    return 2 * H * (576 + 512) * sum(int(L) for L in seq_lens)


def token_reads(seq_lens: Sequence[int], layers: int = 1) -> int:
    """Cached-token reads: one (request, token, layer) latent row, scored by all heads."""
    return layers * sum(int(L) for L in seq_lens)
