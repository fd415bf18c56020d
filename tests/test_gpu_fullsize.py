"""Full-size GPU parity against the oracle, through the C ABI, in the launch configuration
the benchmark times (64K-256K context tokens; needs a GPU). What is compared is described in
fullsize.py: every block's scores and selection, the gather bitwise, attention teacher-forced
on whole 256-row tiles (every row of every workload; a fixed tile sample of every block in the
bucket sweep and for dense causal attention) for one query head per KV group, and the
end-to-end prefix identity.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle_pool
from fullsize import compare_attention, fullsize_check, one_head_per_group
from gpu_util import ATOL_MAX, ATOL_MEAN, dev_bf16, layout_of, say
from synthetic import generate, sweep_layouts, workload
import sequence_approximate_attention_score_amd as apbv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    apbv.lib()
    yield
    torch.cuda.synchronize()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_full_size_every_row(name):
    """64K, 128K, 256K and the variable-frame 128K layout: every row of one query head per
    KV group."""
    x = generate(workload(name))
    fullsize_check(x, layout_of(x), all_rows=True)


@pytest.mark.timeout(600)
def test_full_size_every_head_128k():
    """128K: every one of the 28 query heads on the fixed tile sample of every block (the
    every-row checks above take one head per KV group)."""
    x = generate(workload("c2"))
    fullsize_check(x, layout_of(x), all_rows=False, heads=list(range(x.w.hq)), seed=13)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["buckets_2", "buckets_4", "buckets_6", "no_passing"])
def test_sweep_128k(name):
    """The bucket-count sweep (2, 4, 6 buckets over 128K tokens; 8 is the headline layout)
    and the anchor-only baseline without passing blocks, on the same 128K context."""
    x = generate(workload("c2"))
    lay_d = [l for l in sweep_layouts(x.w) if l["name"] == name][0]
    lay = layout_of(x, block_starts=lay_d["block_starts"], l_anchor=lay_d["l_anchor"],
                    l_pass=lay_d["l_pass"])
    fullsize_check(x, lay, all_rows=False, seed=11)


@pytest.mark.timeout(600)
def test_dense_causal_128k():
    """Dense causal attention over [anchor | 128K context] (n = 1, no prefix), the comparison
    the frame-balanced 128K workload reports: tile sample, one head per KV group."""
    w = workload("c4")
    x = generate(w)
    N = x.N + w.l_anchor
    lay = apbv.Layout([0, N], l_anchor=0, l_query=0, l_pass=0, hq=w.hq, hkv=w.hkv,
                      head_dim=w.head_dim)
    q = np.concatenate([x.bits["q_anchor"], x.bits["q_ctx"]])
    k = np.concatenate([x.bits["k_anchor"], x.bits["k_ctx"]])
    v = np.concatenate([x.bits["v_anchor"], x.bits["v_ctx"]])
    out, lse = apbv.approx_attn_prefill(lay, dev_bf16(q), None, None, dev_bf16(k),
                                        dev_bf16(v), want_lse=True)
    torch.cuda.synchronize()
    out_host, lse_host = out.float().cpu().numpy(), lse.cpu().numpy().astype(np.float64)
    del out, lse
    bs = np.array([0, N])
    rows = oracle_pool.tile_sample(bs, apbv.attn_tile_rows(w.head_dim), 3)
    empty = np.zeros((w.hkv, 0, w.head_dim), np.uint16)
    heads = one_head_per_group(w.hq, w.hkv)
    res = oracle_pool.attend(q, k, v, empty, empty, bs, 0, 0, w.hq, w.hkv,
                             1 / math.sqrt(w.head_dim), rows, heads, chunk_rows=256)
    cnt, mx, mean, lmx = compare_attention(out_host, lse_host, bs, res)
    say(f"  dense causal 128K ({len(rows[0])} rows x {len(heads)} heads): max-abs {mx:.3e} "
        f"mean-abs {mean:.3e} over {cnt} values; lse max-abs {lmx:.2e}")
    assert mx <= ATOL_MAX and mean <= ATOL_MEAN and lmx <= 2e-3
