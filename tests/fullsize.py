"""Full-size GPU parity against the oracle (helpers of test_gpu_fullsize.py and
test_gpu_layer.py), in the launch configuration the benchmark times.

``fullsize_check`` compares, at one workload:
  * scores of every block against the oracle's (relative error <= 2e-5, each block's scores
    sum to G * l_q);
  * selection of every block: bit-exact outside the float32 near-tie band, and the exact
    selection rule (top-l_p, ties to the lower row) on the GPU's own scores;
  * gather: the prefix is bitwise the oracle's gather of the GPU selection;
  * attention, teacher-forced on that prefix, for one query head of every KV group, on
    whole 256-row tiles: every row, or every block's first, middle and last tile plus a
    seeded 5% of its other tiles;
  * end to end: for every block whose preceding blocks' selections equal the oracle's own,
    the prefix the oracle builds from its own selection is bitwise the one the GPU used, so
    the teacher-forced comparison of that block is the end-to-end comparison (every block
    up to and including the first whose own selection differs in the near-tie band); the
    count of such blocks is reported.

The oracle runs in a pool of worker processes (oracle_pool.py), started here at import when
a GPU is visible, before the GPU is initialised.
"""
from __future__ import annotations

import math
import time

import numpy as np
import torch

import oracle_pool
from gpu_util import ATOL_MAX, ATOL_MEAN, check_selection, say, upload
from synthetic import bf16_bits
import sequence_approximate_attention_score_amd as apbv
from oracle import apbv_oracle as orc

if torch.cuda.device_count() > 0:     # counting devices does not initialise the GPU
    oracle_pool.start()


def one_head_per_group(hq, hkv, shift=0):
    """One query head of every KV group, at a different position inside each group;
    ``shift`` moves every pick along its group (workloads use different shifts, so that
    together they cover more heads)."""
    G = hq // hkv
    return [g * G + (g + shift) % G for g in range(hkv)]


HEAD_SHIFT = {"c1": 0, "c2": 1, "c3": 2, "c4": 3}   # 16 distinct heads over the four


def compare_attention(out_host, lse_host, bs, results):
    """Fold the pool's oracle rows into max-abs / mean-abs error against the GPU output."""
    n, mx, tot, lmx = 0, 0.0, 0.0, 0.0
    for v, h, rows, o_or, l_or in results:
        r = int(bs[v]) + rows
        o_gpu = out_host[r, h].astype(np.float64)
        assert np.all(np.isfinite(o_gpu)), (v, h)
        err = np.abs(o_gpu - o_or)
        mx = max(mx, float(err.max()))
        tot += float(err.sum())
        n += err.size
        lmx = max(lmx, float(np.abs(lse_host[h, r] - l_or).max()))
    return n, mx, tot / max(n, 1), lmx


def three_calls(lay, d):
    """The hot path as three C-ABI calls: (scores, sel, k_pre, v_pre, out, lse)."""
    scores, sel = apbv.score_select(lay, d["q_query"], d["k_ctx"])
    kp, vp = apbv.gather_passing(lay, d["k_anchor"], d["v_anchor"], d["k_ctx"], d["v_ctx"], sel)
    out, lse = apbv.approx_attn_prefill(lay, d["q_ctx"], kp, vp, d["k_ctx"], d["v_ctx"],
                                        want_lse=True)
    return scores, sel, kp, vp, out, lse


def fullsize_check(x, lay, *, all_rows, heads=None, seed=7, runner=three_calls):
    """Run the GPU path (``runner(lay, uploaded inputs)``) and compare every output with the
    oracle as described in the module docstring."""
    w = x.w
    t0 = time.perf_counter()
    bs = np.asarray(lay.block_starts, np.int64)
    n = lay.n_blocks
    G = w.hq // w.hkv
    scale = 1.0 / math.sqrt(w.head_dim)
    if heads is None:
        heads = one_head_per_group(w.hq, w.hkv, HEAD_SHIFT.get(w.name, 0))
    say(f"case {w.name}: n={n} N={lay.n_tokens} l_a={lay.l_anchor} l_q={w.l_query} "
        f"l_p={lay.l_pass} heads={heads} rows={'all' if all_rows else 'tile sample'}")
    d = upload(x)
    scores, sel, kp, vp, out, lse = runner(lay, d)
    torch.cuda.synchronize()
    s_gpu = scores.cpu().numpy()
    sel_gpu = sel.cpu().numpy()
    kp_bits = kp.view(torch.int16).cpu().numpy().view(np.uint16)
    vp_bits = vp.view(torch.int16).cpu().numpy().view(np.uint16)
    out_host = out.float().cpu().numpy()
    lse_host = lse.cpu().numpy().astype(np.float64)
    del d, scores, sel, kp, vp, out, lse
    failures = []

    def attempt(name, fn):
        try:
            fn()
        except AssertionError as e:
            say(f"  FAILED {name}: {e}")
            failures.append(name)

    # scores and selection of every block
    s_or = oracle_pool.scores(x, bs, w.hq, w.hkv, scale, range(n))

    def score_check():
        worst = 0.0
        for v in range(n):
            lo, hi = int(bs[v]), int(bs[v + 1])
            a, b = s_gpu[:, lo:hi].astype(np.float64), s_or[:, lo:hi]
            rel = np.abs(a - b) / np.maximum(np.abs(b), 1e-30)
            worst = max(worst, float(rel.max()))
            assert rel.max() <= 2e-5, (v, float(rel.max()))
            assert np.allclose(a.sum(axis=1), G * w.l_query, rtol=1e-5), v
        say(f"  scores, all {n} blocks: max rel err {worst:.2e}")
    attempt("scores", score_check)
    s32 = s_or.astype(np.float32)
    sel_or = orc.select_passing(s32, bs, lay.l_pass)

    def sel_check():
        n_band = 0
        for v in range(n):
            lo, hi = int(bs[v]), int(bs[v + 1])
            n_band += check_selection(s32[:, lo:hi], sel_gpu[v:v + 1] - lo, [0, hi - lo],
                                      lay.l_pass)
        own = orc.select_passing(s_gpu, bs, lay.l_pass)
        assert np.array_equal(own, sel_gpu), "selection rule on the GPU's own scores"
        say(f"  selection, all {n} blocks: equal outside the tie band ({n_band} band "
            f"positions); the rule holds exactly on the GPU's scores")
    attempt("selection", sel_check)

    ka, va = x.f32("k_anchor")[:lay.l_anchor], x.f32("v_anchor")[:lay.l_anchor]
    kc, vc = x.f32("k_ctx"), x.f32("v_ctx")
    k_or, v_or = orc.gather_prefix(ka, va, kc, vc, sel_gpu)

    def gather_check():
        assert np.array_equal(bf16_bits(k_or.astype(np.float32)), kp_bits), "k_pre"
        assert np.array_equal(bf16_bits(v_or.astype(np.float32)), vp_bits), "v_pre"
    attempt("gather", gather_check)
    del k_or, v_or

    # end to end: blocks whose prefix built from the oracle's own selection is the same
    same = [bool(np.array_equal(sel_or[v], sel_gpu[v])) for v in range(n)]
    e2e = [v for v in range(n) if all(same[:v])]

    def e2e_check():
        ke, ve = orc.gather_prefix(ka, va, kc, vc, sel_or)
        P_max = lay.l_anchor + max(e2e) * lay.l_pass
        assert np.array_equal(bf16_bits(ke[:, :P_max].astype(np.float32)), kp_bits[:, :P_max])
        assert np.array_equal(bf16_bits(ve[:, :P_max].astype(np.float32)), vp_bits[:, :P_max])
    if e2e:
        attempt("end-to-end prefix", e2e_check)
    say(f"  end to end: {len(e2e)} of {n} blocks see the prefix of the oracle's own "
        f"selection ({sum(same)} of {n} selections identical)")
    del kc, vc

    rows = ({v: np.arange(int(bs[v + 1] - bs[v])) for v in range(n)} if all_rows
            else oracle_pool.tile_sample(bs, apbv.attn_tile_rows(w.head_dim), seed))
    res = oracle_pool.attend(x.bits["q_ctx"], x.bits["k_ctx"], x.bits["v_ctx"], kp_bits,
                             vp_bits, bs, lay.l_anchor, lay.l_pass, w.hq, w.hkv, scale, rows,
                             heads)
    cnt, mx, mean, lmx = compare_attention(out_host, lse_host, bs, res)
    n_rows = sum(len(r) for r in rows.values())

    def attn_check():
        say(f"  attention ({n_rows} rows x {len(heads)} heads, teacher-forced; end to end "
            f"on {len(e2e)} blocks): max-abs {mx:.3e} mean-abs {mean:.3e} over {cnt} values; "
            f"lse max-abs {lmx:.2e}")
        assert mx <= ATOL_MAX and mean <= ATOL_MEAN, (mx, mean)
        assert lmx <= 2e-3, lmx
    attempt("attention", attn_check)
    say(f"  {time.perf_counter() - t0:.1f} s")
    assert not failures, failures
    return sel_or, sel_gpu
