"""Every row of a layer in one call (apbv_layer_forward), against the oracle, through the C
ABI (needs a GPU).

The sequence is [anchor | context blocks | query block]:
  * anchor rows: dense causal attention over the anchor alone, compared with the oracle's
    attention of one block with no prefix;
  * context rows: the full oracle comparison of the three-step path (scores, selection,
    prefix, attention of every row), and bit-identity with the separate calls;
  * query rows: exact attention over the whole sequence, compared with the oracle's query
    attention, and bit-identity with apbv_query_forward.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import pytest
import torch

from fullsize import fullsize_check, one_head_per_group, three_calls
from gpu_util import check_attention, dev_bf16, host_f64, layout_of, say
from synthetic import generate, workload
import sequence_approximate_attention_score_amd as apbv
from oracle import apbv_oracle as orc

pytestmark = pytest.mark.gpu

ALL = ("q_anchor", "k_anchor", "v_anchor", "q_ctx", "k_ctx", "v_ctx", "q_query", "k_query",
       "v_query")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    apbv.lib()
    yield
    torch.cuda.synchronize()


def upload_all(x, lay):
    d = {n: dev_bf16(x.bits[n]) for n in ALL}
    for n in ("q_anchor", "k_anchor", "v_anchor"):        # the layout's anchor length
        d[n] = d[n][:lay.l_anchor].contiguous()
    return d


def call(lay, d, **kw):
    return apbv.layer_forward(lay, **{n: d[n] for n in ALL}, want_lse=True, want_scores=True,
                              **kw)


def check_anchor_rows(x, lay, r, heads):
    """Anchor rows against the oracle: one block [0, l_a), no prefix, causal."""
    w = x.w
    l_a = lay.l_anchor
    empty = np.zeros((w.hkv, 0, w.head_dim))
    o_or, l_or = orc.attend(x.f32("q_anchor")[:l_a], empty, empty, x.f32("k_anchor")[:l_a],
                            x.f32("v_anchor")[:l_a], [0, l_a], 0, 0, w.hq, w.hkv,
                            1 / math.sqrt(w.head_dim), heads=heads)
    check_attention(host_f64(r["anchor_out"]), o_or, f"anchor rows ({l_a} x {len(heads)} heads)")
    lse = r["anchor_lse"].cpu().numpy().astype(np.float64)
    m = ~np.isnan(l_or)
    lerr = float(np.abs(lse[m] - l_or[m]).max())
    say(f"  anchor lse: max-abs {lerr:.2e}")
    assert lerr <= 2e-3, lerr


def check_query_rows(x, lay, r, heads):
    w = x.w
    l_a = lay.l_anchor
    o_or, l_or = orc.query_attention(x.f32("q_query"), x.f32("k_query"), x.f32("v_query"),
                                     x.f32("k_anchor")[:l_a], x.f32("v_anchor")[:l_a],
                                     x.f32("k_ctx"), x.f32("v_ctx"), w.hq, w.hkv,
                                     1 / math.sqrt(w.head_dim), heads=heads)
    check_attention(host_f64(r["query_out"]), o_or, f"query rows ({w.l_query} x {len(heads)})")
    lse = r["query_lse"].cpu().numpy().astype(np.float64)
    m = ~np.isnan(l_or)
    lerr = float(np.abs(lse[m] - l_or[m]).max())
    say(f"  query lse: max-abs {lerr:.2e}")
    assert lerr <= 2e-3, lerr


def check_against_separate_calls(lay, d, r):
    """Context and query rows bit-identical to the separate entry points."""
    scores, sel, kp, vp, out, lse = three_calls(lay, d)
    qo, ql = apbv.query_forward(lay, d["q_query"], d["k_query"], d["v_query"], d["k_anchor"],
                                d["v_anchor"], d["k_ctx"], d["v_ctx"], want_lse=True)
    torch.cuda.synchronize()
    ref = dict(scores=scores, sel=sel, k_pre=kp, v_pre=vp, out=out, lse=lse)
    if r["query_out"] is not None:
        ref.update(query_out=qo, query_lse=ql)
    for k, t in ref.items():
        assert torch.equal(t, r[k]), k


def small(name, **kw):
    base = dict(keys="iid", n_blocks=len(kw["block_starts"]) - 1, block_len=0)
    bs = kw.pop("block_starts")
    base.update(kw)
    w = dataclasses.replace(workload("c0"), name=name, total_tokens=bs[-1], **base)
    return generate(w, block_starts=bs)


CASES = {
    "c0": lambda: generate(workload("c0")),
    # G = 7, ragged blocks, a 37-row anchor (less than one tile)
    "ragged_g7": lambda: small("ragged_g7", hq=14, hkv=2, head_dim=128, l_anchor=37,
                               l_query=19, l_pass=21,
                               block_starts=[0, 129, 300, 555, 700, 1000]),
    # an anchor of several tiles with a ragged last tile, d = 64
    "long_anchor_d64": lambda: small("long_anchor_d64", hq=8, hkv=2, head_dim=64,
                                     l_anchor=700, l_query=40, l_pass=50,
                                     block_starts=[0, 400, 800, 1200]),
    # no anchor: nothing to do for the anchor rows; no passing rows either
    "no_anchor_no_pass": lambda: small("no_anchor_no_pass", hq=4, hkv=2, head_dim=128,
                                       l_anchor=0, l_query=16, l_pass=0,
                                       block_starts=[0, 300, 600]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_layer_forward_every_row_matches_oracle(name):
    x = CASES[name]()
    lay = layout_of(x)
    held = {}

    def runner(lay, _d):
        d = upload_all(x, lay)
        held["d"] = d
        held["r"] = r = call(lay, d)
        return r["scores"], r["sel"], r["k_pre"], r["v_pre"], r["out"], r["lse"]

    fullsize_check(x, lay, all_rows=True, heads=list(range(lay.hq)), runner=runner)
    r, d = held["r"], held["d"]
    heads = list(range(lay.hq))
    if lay.l_anchor > 0:
        check_anchor_rows(x, lay, r, heads)
    else:
        assert r["anchor_out"] is None
    check_query_rows(x, lay, r, heads)
    check_against_separate_calls(lay, d, r)


def test_layer_forward_skips_rows_on_request():
    """anchor_rows / query_rows off: those outputs are absent, the context rows unchanged."""
    x = CASES["ragged_g7"]()
    lay = layout_of(x)
    d = upload_all(x, lay)
    full = call(lay, d)
    part = apbv.layer_forward(lay, q_anchor=None, k_anchor=d["k_anchor"],
                              v_anchor=d["v_anchor"], q_ctx=d["q_ctx"], k_ctx=d["k_ctx"],
                              v_ctx=d["v_ctx"], q_query=d["q_query"], k_query=None,
                              v_query=None, anchor_rows=False, query_rows=False,
                              want_lse=True, want_scores=True)
    torch.cuda.synchronize()
    assert part["anchor_out"] is None and part["query_out"] is None
    for k in ("scores", "sel", "k_pre", "v_pre", "out", "lse"):
        assert torch.equal(full[k], part[k]), k


@pytest.mark.timeout(600)
def test_layer_forward_128k():
    """The 128K layer (16 blocks of 8K, anchor 2048, query 128): anchor rows against the
    oracle for one head per KV group, context and query rows bit-identical to the separate
    calls (whose own oracle comparison at this size is in the full-size tests)."""
    x = generate(workload("c2"))
    lay = layout_of(x)
    d = upload_all(x, lay)
    r = call(lay, d)
    torch.cuda.synchronize()
    heads = one_head_per_group(lay.hq, lay.hkv)
    say(f"layer 128K: anchor {lay.l_anchor}, N {lay.n_tokens}, query {lay.l_query}")
    check_anchor_rows(x, lay, r, heads)
    check_against_separate_calls(lay, d, r)
