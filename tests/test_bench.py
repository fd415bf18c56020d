"""Host-side arithmetic and contract of bench.py (CPU only, no kernel is launched)."""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synthetic import workload  # noqa: E402


def visible_pairs_brute(block_starts, l_anchor, l_pass, rows=None):
    """(row, key) pairs one query head attends to, counted from an explicit mask over
    [anchor | passing of every block | context]: row i of block v sees the anchor, the
    passing rows of blocks < v and its own block's keys up to i (``rows``: only these
    context rows)."""
    bs = list(block_starts)
    n = len(bs) - 1
    n_keys = l_anchor + n * l_pass + bs[-1]
    total = 0
    for v in range(n):
        for i in range(bs[v], bs[v + 1]):
            if rows is not None and i not in rows:
                continue
            mask = np.zeros(n_keys, bool)
            mask[:l_anchor] = True
            mask[l_anchor:l_anchor + v * l_pass] = True
            ctx0 = l_anchor + n * l_pass
            mask[ctx0 + bs[v]:ctx0 + i + 1] = True
            total += int(mask.sum())
    return total


def test_attention_flops_match_a_brute_force_mask_count():
    bs, la, lp, hq, d = [0, 7, 20, 26, 40], 5, 3, 6, 64
    pairs = visible_pairs_brute(bs, la, lp)
    assert bench.attention_flops(bs, la, lp, hq, d) == pairs * hq * 4 * d


def test_attention_flops_at_128k_match_the_config_arithmetic():
    # 16 blocks of 8192, anchor 2048, l_p 1024, 28 query heads, d = 128: 1.812e9 visible
    # pairs per head (anchor 0.27e9, passing 1.01e9, local 0.54e9) -> 25.98 TFLOP
    w = workload("c2")
    bs = np.arange(0, 16 * 8192 + 1, 8192)
    anchor = 16 * 8192 * 2048
    passing = sum(8192 * v * 1024 for v in range(16))
    local = 16 * (8192 * 8193 // 2)
    assert (anchor, passing, local) == (268435456, 1006632960, 536936448)
    flops = bench.attention_flops(bs, w.l_anchor, w.l_pass, w.hq, w.head_dim)
    assert flops == (anchor + passing + local) * 28 * 4 * 128
    assert abs(flops - 2.598e13) / 2.598e13 < 1e-3


def test_gather_bytes_at_128k_are_72_mib():
    class Lay:
        hkv, pre_rows = 4, 2048 + 16 * 1024
    assert bench.gather_bytes(Lay, 128) == 72 * 2**20


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_is_reported_only_for_the_profiled_kernel_source(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    f.write_text("# header\nkernel_source_sha256: %s\ntraffic_bytes_per_launch: 1.5e10\n"
                 % bench.attn_source_sha())
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.read_traffic() == pytest.approx(1.5e10)
    f.write_text("kernel_source_sha256: %s\ntraffic_bytes_per_launch: 1.5e10\n" % ("0" * 64))
    assert bench.read_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.read_traffic() is None


def test_committed_traffic_summary_matches_the_current_attention_source():
    """The committed counter summary must describe the kernel as it is now (a change to the
    attention sources needs new FETCH_SIZE / WRITE_SIZE passes)."""
    t = bench.read_traffic()
    assert t is not None and 1e9 < t < 1e11


def test_visible_pairs_of_a_row_range_match_the_brute_force_mask():
    bs, la, lp = [0, 7, 20, 26, 40], 5, 3
    n = len(bs) - 1
    whole = sum(bench.visible_pairs(bs, la, lp, v, 0, bs[v + 1] - bs[v]) for v in range(n))
    assert whole == visible_pairs_brute(bs, la, lp)
    # a range of rows counts its own prefix and causal keys: rows 3..9 of block 1 (13 rows)
    P = la + 1 * lp
    assert bench.visible_pairs(bs, la, lp, 1, 3, 10) == sum(P + r + 1 for r in range(3, 10))


def test_cpu_baseline_over_the_whole_layer_extrapolates_to_itself():
    """With every row of every (block, KV head) unit in the sample, the sampled pairs are all
    pairs of all query heads and the layer time is exactly the measured time."""
    from synthetic import generate
    x = generate(workload("c0", hq=4, hkv=2))
    rec, raw = bench.cpu_baseline(x, tiles_per_unit=None, workers=2)
    assert raw["sample_pairs"] == raw["total_pairs"]
    assert raw["total_pairs"] == visible_pairs_brute(x.block_starts, x.w.l_anchor,
                                                     x.w.l_pass) * x.w.hq
    measured = raw["sel_gather_s"] + (raw["cpu_score_s"] + raw["cpu_attn_sample_s"]) / 2
    assert raw["layer_s"] == pytest.approx(measured, rel=1e-12)
    assert rec["value"] == pytest.approx(x.N / measured, rel=1e-12)
    assert rec["cores"] == 2 and rec["blas_threads_per_worker"] == 1
    assert rec["kind"] == "oracle" and rec["unit"] == "tokens/s"


def test_cpu_baseline_sample_scales_by_all_heads():
    """A partial sample (one 256-row tile per unit) is scaled by the ratio of all visible
    pairs of all query heads to the sampled pairs of the sampled heads."""
    from synthetic import generate
    x = generate(workload("c0", hq=4, hkv=2, total_tokens=1024, n_blocks=2, block_len=512))
    rec, raw = bench.cpu_baseline(x, tiles_per_unit=1, workers=2)
    G = x.w.hq // x.w.hkv
    bs = x.block_starts
    total = sum(bench.visible_pairs(bs, x.w.l_anchor, x.w.l_pass, v, 0, bs[v + 1] - bs[v])
                for v in range(2)) * x.w.hq
    assert raw["total_pairs"] == total
    # the sampled pairs: one tile of each block, for all G heads of each of the hkv groups,
    # counted from the explicit mask
    assert [t[0] for t in raw["tiles"]] == [0, 1]
    brute = 0
    for v, a, b in raw["tiles"]:
        brute += visible_pairs_brute(bs, x.w.l_anchor, x.w.l_pass,
                                     rows=range(int(bs[v]) + a, int(bs[v]) + b))
    assert raw["sample_pairs"] == brute * G * x.w.hkv < total
    ratio = total / raw["sample_pairs"]
    est = raw["sel_gather_s"] + (raw["cpu_score_s"] + raw["cpu_attn_sample_s"] * ratio) / 2
    assert raw["layer_s"] == pytest.approx(est, rel=1e-12)
