"""Rows of the query block on the GPU (partial attention over key chunks + lse merge)
against the oracle's exact attention over [anchor | context | causal query], through the C
ABI (needs a GPU)."""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import pytest
import torch

from synthetic import generate, workload
from gpu_util import check_attention, host_f64, layout_of, say, upload
import sequence_approximate_attention_score_amd as apbv
from oracle import apbv_oracle as orc

pytestmark = pytest.mark.gpu

NAMES = ("q_query", "k_query", "v_query", "k_anchor", "v_anchor", "k_ctx", "v_ctx")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    apbv.lib()
    yield
    torch.cuda.synchronize()


def run_query(x, lay, d):
    out, lse = apbv.query_forward(lay, d["q_query"], d["k_query"], d["v_query"], d["k_anchor"],
                                  d["v_anchor"], d["k_ctx"], d["v_ctx"], want_lse=True)
    torch.cuda.synchronize()
    return host_f64(out), lse.cpu().numpy().astype(np.float64)


def check_query(x, lay, heads=None):
    w = x.w
    say(f"query case {w.name}: N={x.N} hq={w.hq} hkv={w.hkv} d={w.head_dim} "
        f"l_a={lay.l_anchor} l_q={w.l_query}")
    d = upload(x, NAMES)
    out, lse = run_query(x, lay, d)
    l_a = lay.l_anchor
    o_or, l_or = orc.query_attention(x.f32("q_query"), x.f32("k_query"), x.f32("v_query"),
                                     x.f32("k_anchor")[:l_a], x.f32("v_anchor")[:l_a],
                                     x.f32("k_ctx"), x.f32("v_ctx"), w.hq, w.hkv,
                                     1 / math.sqrt(w.head_dim), heads=heads)
    check_attention(out, o_or, "query out")
    m = ~np.isnan(l_or)
    lerr = float(np.abs(lse[m] - l_or[m]).max())
    say(f"  query lse: max-abs {lerr:.2e}")
    assert lerr <= 2e-3, lerr
    return out, lse


def test_query_c0():
    x = generate(workload("c0"))
    check_query(x, layout_of(x))


VARIANTS = {
    # packed rows (G * l_q) that wrap inside a wave, ragged everything
    "g7_lq19": dict(hq=14, hkv=2, head_dim=128, total_tokens=1000, l_anchor=37, l_query=19),
    "no_anchor": dict(hq=4, hkv=2, head_dim=128, total_tokens=900, l_anchor=0, l_query=16),
    "single_row": dict(hq=7, hkv=1, head_dim=128, total_tokens=600, l_anchor=64, l_query=1),
    "big_query_d64": dict(hq=4, hkv=2, head_dim=64, total_tokens=2500, l_anchor=100,
                          l_query=300),
    # several chunks of anchor and context keys, ragged chunk ends
    "multi_chunk": dict(hq=8, hkv=2, head_dim=128, total_tokens=9000, l_anchor=4500,
                        l_query=70),
    "causal_chunks": dict(hq=2, hkv=1, head_dim=64, total_tokens=300, l_anchor=10,
                          l_query=4200),
}


@pytest.mark.parametrize("name", sorted(VARIANTS))
def test_query_variant(name):
    kw = VARIANTS[name]
    N = kw["total_tokens"]
    w = dataclasses.replace(workload("c0"), name=name, keys="iid", n_blocks=1, block_len=N,
                            l_pass=0, **kw)
    x = generate(w)
    check_query(x, layout_of(x))


def test_query_deterministic():
    x = generate(dataclasses.replace(workload("c0"), name="det", hq=8, hkv=2, head_dim=128,
                                     total_tokens=5000, n_blocks=2, block_len=2500,
                                     l_anchor=100, l_query=40))
    lay = layout_of(x)
    d = upload(x, NAMES)
    a = run_query(x, lay, d)
    b = run_query(x, lay, d)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("name", ["c2", "c3"])
def test_query_full_size(name):
    x = generate(workload(name))
    w = x.w
    check_query(x, layout_of(x), heads=sorted({0, 6, 7, w.hq // 2, w.hq - 1}))
