"""The seeded input generator: bf16 rounding, frame partition, determinism (CPU only)."""
from __future__ import annotations

import numpy as np
import torch

from synthetic import CONFIGS, bf16_bits, bf16_round, frame_partition, generate, workload
from synthetic.gen import bits_to_f32


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, -3.4e38, 3.3e38], np.float32)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits(x), ref)
    assert np.array_equal(bf16_round(x), torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    assert np.array_equal(bits_to_f32(bf16_bits(x)), bf16_round(x))


def test_frame_partition_balances_frame_counts():
    rng = np.random.default_rng(1)
    fl = rng.integers(196, 325, size=500)
    bs = frame_partition(fl, 16)
    edges = np.concatenate([[0], np.cumsum(fl)])
    assert bs[0] == 0 and bs[-1] == fl.sum() and np.all(np.diff(bs) > 0)
    counts = [np.searchsorted(edges, bs[v + 1]) - np.searchsorted(edges, bs[v]) for v in range(16)]
    assert max(counts) - min(counts) <= 1 and sum(counts) == 500
    assert set(bs.tolist()) <= set(edges.tolist())          # blocks hold whole frames


def test_generator_is_deterministic_and_shaped():
    w = workload("c0")
    a, b = generate(w), generate(w)
    for k in a.bits:
        assert np.array_equal(a.bits[k], b.bits[k]), k
    assert a.bits["q_ctx"].shape == (512, 2, 64) and a.bits["k_ctx"].shape == (512, 1, 64)
    assert a.bits["q_query"].shape == (32, 2, 64) and a.bits["k_anchor"].shape == (64, 1, 64)
    assert a.block_starts.tolist() == [0, 256, 512]
    c = generate(w, keep_raw=True)
    assert np.array_equal(bf16_bits(c.raw["q_ctx"]), a.bits["q_ctx"])


def test_variable_frames_cover_context():
    w = workload("c4", total_tokens=20000, n_blocks=4, hq=2, hkv=1, head_dim=64, l_anchor=16,
                 l_query=8, l_pass=16)
    x = generate(w)
    assert x.frame_lengths.sum() == 20000
    assert np.all(x.frame_lengths[:-1] >= 196) and np.all(x.frame_lengths <= 324)
    assert x.block_starts[-1] == 20000 and len(x.block_starts) == 5


def test_frame_keys_are_correlated_within_frames():
    w = workload("c1", total_tokens=4096, n_blocks=2, block_len=2048, l_anchor=64, l_query=8,
                 l_pass=64, hq=2, hkv=1)
    k = generate(w).f32("k_ctx")[:, 0, :]
    same = np.mean(np.sum(k[0:255] * k[1:256], axis=1))       # neighbours inside frame 0
    cross = np.mean(np.sum(k[0:256] * k[256:512], axis=1))    # frame 0 vs frame 1
    assert same > 80 and abs(cross) < 40                       # E = d*1 vs 0 (d = 128)


def test_configs_match_the_headline_shapes():
    c2 = CONFIGS["c2"]
    assert (c2.hq, c2.hkv, c2.head_dim, c2.n_blocks, c2.block_len) == (28, 4, 128, 16, 8192)
    assert c2.n_buckets == 8 and c2.total_tokens == 131072
    assert CONFIGS["c3"].n_blocks == 32 and CONFIGS["c3"].l_query == 256
