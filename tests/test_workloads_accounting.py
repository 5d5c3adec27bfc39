"""Workload shapes and byte accounting against the figures the pages print."""
import json
import math
import os

import numpy as np
import pytest
import torch

from mla_latent_cache_absorbed_amd import accounting as acc
from mla_latent_cache_absorbed_amd import workloads as wl

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "page_figures.json")))["entries"]
G = {e["id"]: e for e in GOLD}


def _close(x, entry, default_rel=0.01):
    rel = entry.get("rel_tol", default_rel)
    return abs(x - entry["value"]) <= rel * abs(entry["value"])


def test_bytes_per_token_closed_form():
    e = G["kv_bytes_per_token_61_layers_bf16"]
    assert 61 * acc.ROW_BYTES == e["value"] == 61 * 576 * 2
    w = G["latent_width"]
    assert w["terms"]["kv_lora_rank"] + w["terms"]["qk_rope_head_dim"] == w["value"] == 576


def test_cache_tensor_bytes_per_token():
    w = wl.make("tiny")
    per_tok = w.cache.numel() * w.cache.element_size() / (w.NB * w.BS)
    assert per_tok == acc.ROW_BYTES == 1152


def test_mha_compression_ratios():
    assert _close(576 / (128 * 128 * 2), G["mha_ratio_head_dim_128"])
    assert _close(576 / (128 * (192 + 128)), G["mha_ratio_k_head_dim_192"])


def test_capacity_arithmetic():
    per_tok = 61 * 576 * 2
    tp_tokens = G["tp8_kv_gb_per_gpu"]["value"] * 1e9 / per_tok
    dp_tokens = 8 * G["dp_kv_gb_per_gpu"]["value"] * 1e9 / per_tok
    assert _close(tp_tokens, G["tp8_capacity_tokens"])
    assert _close(dp_tokens, G["dp_capacity_tokens"])
    # the page turns its rounded capacities (652k, 4.08M) into sequences
    assert G["tp8_capacity_tokens"]["value"] // 4096 == G["tp8_sequences_at_4096"]["value"]
    assert G["dp_capacity_tokens"]["value"] // 4096 == G["dp_sequences_at_4096"]["value"]
    # the per-GPU batch of the DP-rank workload is 996 / 8 (rounded down)
    assert wl.spec("dp_rank").B == G["dp_sequences_at_4096"]["value"] // 8
    assert wl.spec("tp_slice").B == G["tp8_sequences_at_4096"]["value"]


def test_cache_read_per_step():
    s = wl.spec("tp_slice")
    per_step = 61 * acc.cache_bytes(s.seq_lens)
    assert per_step == 159 * 4096 * 70272 == 45_765_623_808
    assert round(per_step / 1e9, 1) == G["tp8_cache_read_per_step_gb"]["value"]
    assert round(per_step / 8 / 1e9, 1) == G["dp_cache_read_per_step_gb"]["value"]
    bw = G["hbm_tb_per_s_of_the_pages_gpu"]["value"] * 1e12
    assert round(per_step / bw * 1e3, 1) == G["tp8_cache_read_ms_at_4p8"]["value"]
    assert round(per_step / 8 / bw * 1e3, 1) == G["dp_cache_read_ms_at_4p8"]["value"]


def test_workload_specs():
    s = wl.spec("dp_rank")
    assert (s.B, s.H, s.BS, s.M, s.NB) == (124, 128, 64, 64, 7936)
    assert s.NB * s.BS * 1152 == 585_105_408
    assert acc.algorithmic_bytes(s.seq_lens, s.H, s.BS) == 619_738_608
    assert acc.algorithmic_flops(s.seq_lens, s.H) == 2176 * 128 * 124 * 4096
    s4 = wl.spec("step61")
    assert s4.layers * acc.cache_bytes(s4.seq_lens) == 35_691_429_888
    s2 = wl.spec("tp_slice")
    assert (s2.B, s2.H, s2.NB) == (159, 16, 10176)
    s3 = wl.spec("ragged")
    assert s3.B == 32 and all(256 <= L <= 131072 for L in s3.seq_lens)
    assert s3.NB == sum(-(-L // 64) for L in s3.seq_lens)
    assert s3.M == max(-(-L // 64) for L in s3.seq_lens)


def test_tiny_workload_layout():
    w = wl.make("tiny")
    assert w.q.dtype == torch.bfloat16 and tuple(w.q.shape) == (2, 128, 576)
    assert tuple(w.cache.shape) == (14, 16, 576)
    assert w.block_table.tolist() == [list(range(7)), list(range(7, 14))]
    assert w.seq_lens.tolist() == [64, 100]
    assert w.scale == float(np.float32(1 / math.sqrt(192)))
    # deterministic
    w2 = wl.make("tiny")
    assert torch.equal(w.q, w2.q) and torch.equal(w.cache, w2.cache)


def test_custom_poison_and_tables():
    w = wl.make_custom([5, 64, 0, 70], H=4, BS=16, poison_unused=True)
    t = w.block_table
    NB = w.NB
    assert (t[2] == NB - 1).all()                   # empty request: poison block only
    assert torch.isnan(w.cache[NB - 1].float()).all()
    last = int(t[0, 0])
    assert torch.isnan(w.cache[last, 5:].float()).all()
    assert not torch.isnan(w.cache[last, :5].float()).any()
    used = [int(x) for b, L in enumerate([5, 64, 0, 70]) for x in t[b, :-(-L // 16)]]
    assert len(set(used)) == len(used) and NB - 1 not in used
