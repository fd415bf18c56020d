"""HIP path against the oracle, through the C ABI, on seeded synthetic inputs (needs a GPU).

Small cases, every element. Attention is teacher-forced: the oracle's attention runs on the
prefix gathered from the GPU's own selection, so a near-tie difference in selection cannot
leak into the attention comparison; where the two selections agree the end-to-end outputs
are compared too. The full-size workloads are in test_gpu_fullsize.py.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import pytest
import torch

from synthetic import bf16_bits, generate, sweep_layouts, workload
from gpu_util import (check_attention, check_selection, dev_bf16, host_f64, layout_of, say,
                      upload)
import sequence_approximate_attention_score_amd as apbv
from oracle import apbv_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    apbv.lib()
    yield
    torch.cuda.synchronize()


def run_gpu(x, lay, d):
    scores, sel = apbv.score_select(lay, d["q_query"], d["k_ctx"])
    k_pre, v_pre = apbv.gather_passing(lay, d["k_anchor"], d["v_anchor"], d["k_ctx"], d["v_ctx"], sel)
    out, lse = apbv.approx_attn_prefill(lay, d["q_ctx"], k_pre, v_pre, d["k_ctx"], d["v_ctx"],
                                        want_lse=True)
    torch.cuda.synchronize()
    return dict(scores=scores.cpu().numpy(), sel=sel.cpu().numpy(), k_pre=host_f64(k_pre),
                v_pre=host_f64(v_pre), out=host_f64(out), lse=lse.cpu().numpy().astype(np.float64))


def check_scores(s_gpu, s_or, blocks, bs, G, l_q):
    for v in blocks:
        lo, hi = bs[v], bs[v + 1]
        a, b = s_gpu[:, lo:hi].astype(np.float64), s_or[:, lo:hi]
        rel = np.abs(a - b) / np.maximum(np.abs(b), 1e-30)
        say(f"  scores block {v}: max rel err {rel.max():.2e}")
        # fp32 accumulation of G*l_q probabilities from bf16 MFMA logits
        assert rel.max() <= 2e-5, (v, rel.max())
        assert np.allclose(a.sum(axis=1), G * l_q, rtol=1e-5)


def full_check(x, lay, *, rows=None, heads=None, blocks=None):
    """Run the GPU path, then compare scores / selection / gather / attention to the oracle.
    Every sub-check runs and reports before the first failure is raised."""
    w = x.w
    bs = np.asarray(lay.block_starts)
    say(f"case {w.name}: n={lay.n_blocks} N={lay.n_tokens} hq={w.hq} hkv={w.hkv} d={w.head_dim} "
        f"l_a={lay.l_anchor} l_q={w.l_query} l_p={lay.l_pass} zigzag={lay.c.zigzag}")
    d = upload(x)
    g = run_gpu(x, lay, d)
    qq, kc, vc = x.f32("q_query"), x.f32("k_ctx"), x.f32("v_ctx")
    ka, va, qc = x.f32("k_anchor")[:lay.l_anchor], x.f32("v_anchor")[:lay.l_anchor], x.f32("q_ctx")
    blocks = range(lay.n_blocks) if blocks is None else blocks
    failures = []

    def attempt(name, fn):
        try:
            fn()
        except AssertionError as e:
            say(f"  FAILED {name}: {e}")
            failures.append(name)

    s_or = orc.passing_scores(qq, kc, bs, w.hq, w.hkv, 1 / math.sqrt(w.head_dim), blocks=blocks)
    attempt("scores", lambda: check_scores(g["scores"], s_or, blocks, bs, w.hq // w.hkv, w.l_query))
    s32 = s_or.astype(np.float32)

    def sel_check():
        n_band = sum(_sel_one(s32, g["sel"], bs, lay.l_pass, v) for v in blocks)
        say(f"  selection: equal outside the tie band ({n_band} band positions)")
    attempt("selection", sel_check)

    def sel_rule_check():
        # the selection rule itself, bit-exact whatever the score rounding: the oracle's
        # top-l_p (ties to the lower row) of the GPU's own fp32 scores gives the GPU's rows
        own = orc.select_passing(g["scores"], bs, lay.l_pass)
        for v in blocks:
            assert np.array_equal(own[v], g["sel"][v]), (v, "selection of the GPU's scores")
    attempt("selection rule", sel_rule_check)
    # gather: bitwise against the oracle's gather of the GPU's own selection
    kp, vp = orc.gather_prefix(ka, va, kc, vc, g["sel"])

    def gather_check():
        assert np.array_equal(g["k_pre"], kp) and np.array_equal(g["v_pre"], vp), "gather"
    attempt("gather", gather_check)
    # attention, teacher-forced on the GPU selection
    o_or, l_or = orc.attend(qc, kp, vp, kc, vc, bs, lay.l_anchor, lay.l_pass, w.hq, w.hkv,
                            1 / math.sqrt(w.head_dim), rows=rows, heads=heads)
    attempt("attention", lambda: check_attention(g["out"], o_or, "attention out"))

    def lse_check():
        m = ~np.isnan(l_or)
        lerr = np.abs(g["lse"][m] - l_or[m]).max()
        say(f"  lse: max-abs {lerr:.2e}")
        assert lerr <= 2e-3, lerr
    attempt("lse", lse_check)
    assert not failures, failures
    return g, s_or


def _sel_one(s32, sel, bs, l_pass, v):
    """Selection rule on block v alone (shifted to look like block 0 of one block)."""
    lo, hi = int(bs[v]), int(bs[v + 1])
    return check_selection(s32[:, lo:hi], sel[v:v + 1] - lo, [0, hi - lo], l_pass)


def small(name="c0", **kw):
    return generate(workload(name, **kw))


def test_selection_ties_go_to_the_lower_row():
    """Exact ties at the selection threshold: every block's keys repeat a 7-row pattern, so
    bitwise-equal keys give bitwise-equal scores, and the l_p-th largest score is shared by
    rows on both sides of the cut. The GPU must keep the lowest rows of the tied group,
    as the oracle's stable ranking of the same scores does."""
    x = small("c0", hq=4, hkv=2, l_query=16, l_pass=24)
    bs = np.asarray(x.block_starts)
    kb = x.bits["k_ctx"].copy()
    for v in range(len(bs) - 1):
        lo, hi = int(bs[v]), int(bs[v + 1])
        kb[lo:hi] = kb[lo + (np.arange(hi - lo) % 7)]
    x.bits["k_ctx"] = kb
    lay = layout_of(x)
    g = run_gpu(x, lay, upload(x))
    own = orc.select_passing(g["scores"], bs, lay.l_pass)
    assert np.array_equal(own, g["sel"])
    n_split = 0
    for v in range(len(bs) - 1):
        lo, hi = int(bs[v]), int(bs[v + 1])
        for kv in range(lay.hkv):
            blk = g["scores"][kv, lo:hi]
            t = np.sort(blk)[::-1][lay.l_pass - 1]
            tied = np.flatnonzero(blk == t) + lo
            chosen = np.isin(tied, g["sel"][v, kv])
            if chosen.any() and not chosen.all():
                n_split += 1
                # the chosen members of the tied group are its lowest rows
                assert np.all(tied[chosen] < tied[~chosen].min()), (v, kv)
    assert n_split > 0, "no tie straddles the threshold"


# ------------------------------------------------------------------------- small, exhaustive
def test_c0_end_to_end():
    x = small("c0")
    lay = layout_of(x)
    g, s_or = full_check(x, lay)
    sel_or = orc.select_passing(s_or.astype(np.float32), x.block_starts, lay.l_pass)
    if np.array_equal(sel_or, g["sel"]):
        ref = orc.approx_attention_prefill(x.f32("q_query"), x.f32("q_ctx"), x.f32("k_ctx"),
                                           x.f32("v_ctx"), x.f32("k_anchor"), x.f32("v_anchor"),
                                           x.block_starts, lay.l_pass, 2, 1, 1 / 8)
        check_attention(g["out"], ref["out"], "end-to-end out")


VARIANTS = {
    # name: (workload overrides, explicit block_starts or None, layout overrides)
    "ragged_odd_n_g7": (dict(hq=14, hkv=2, head_dim=128, total_tokens=1000, l_anchor=37,
                             l_query=19, l_pass=21), [0, 129, 300, 555, 700, 1000], {}),
    "no_anchor": (dict(hq=4, hkv=2, head_dim=128, total_tokens=900, l_anchor=0, l_query=16,
                       l_pass=40), [0, 300, 600, 900], {}),
    "no_passing": (dict(hq=4, hkv=4, head_dim=64, total_tokens=700, l_anchor=50, l_query=8,
                        l_pass=0), [0, 350, 700], {}),
    "lp_equals_block": (dict(hq=2, hkv=1, head_dim=64, total_tokens=384, l_anchor=16,
                             l_query=4, l_pass=128), [0, 128, 256, 384], {}),
    "single_query_row": (dict(hq=7, hkv=1, head_dim=128, total_tokens=600, l_anchor=64,
                              l_query=1, l_pass=33), [0, 200, 400, 600], {}),
    "tiny_blocks": (dict(hq=2, hkv=1, head_dim=64, total_tokens=40, l_anchor=3, l_query=3,
                         l_pass=1), [0, 5, 13, 14, 40], {}),
    "many_blocks_zigzag_off": (dict(hq=4, hkv=1, head_dim=128, total_tokens=64 * 40,
                                    l_anchor=8, l_query=8, l_pass=8),
                               list(range(0, 64 * 40 + 1, 40)), dict(zigzag=False)),
    "big_query_block": (dict(hq=4, hkv=2, head_dim=128, total_tokens=2500, l_anchor=100,
                             l_query=300, l_pass=64), [0, 1200, 2500], {}),
    "d64_several_tiles": (dict(hq=8, hkv=2, head_dim=64, total_tokens=4096, l_anchor=128,
                               l_query=32, l_pass=128), [0, 1024, 2048, 3072, 4096], {}),
    # no query block: every score is 0 and each block keeps its first l_p rows (ties go to
    # the lower row)
    "no_query_block": (dict(hq=4, hkv=2, head_dim=128, total_tokens=600, l_anchor=32,
                            l_query=0, l_pass=40), [0, 300, 600], {}),
    # G * l_q = 7 * 4600 = 32200 score rows, padded to 32256: the most the column-sum LDS
    # holds at head_dim 128 (one workgroup per CU)
    "max_score_rows": (dict(hq=28, hkv=4, head_dim=128, total_tokens=600, l_anchor=32,
                            l_query=4600, l_pass=32), [0, 300, 600], {}),
}


@pytest.mark.parametrize("name", sorted(VARIANTS))
def test_variant(name):
    wkw, bs, lkw = VARIANTS[name]
    x = generate(dataclasses.replace(workload("c0"), name=name, keys="iid", block_len=0,
                                     n_blocks=len(bs) - 1, **wkw), block_starts=bs)
    lay = layout_of(x, **lkw)
    full_check(x, lay)


def test_running_max_rescales():
    """Keys whose norm grows along the context push each row's running maximum up tile after
    tile, so the lazy rescale of the running output and sum is taken many times."""
    x = generate(dataclasses.replace(workload("c0"), name="grow", keys="iid", hq=4, hkv=2,
                                     head_dim=128, total_tokens=2048, n_blocks=4, block_len=512,
                                     l_anchor=64, l_query=16, l_pass=64))
    f = (1.0 + 4.0 * np.arange(x.N) / x.N).astype(np.float32)
    x.bits["k_ctx"] = bf16_bits(x.f32("k_ctx") * f[:, None, None])
    full_check(x, layout_of(x))


def test_single_block_is_dense_causal():
    """n = 1, no prefix: the kernel is plain causal attention (checked against the oracle,
    whose own pin ties this case to torch's causal SDPA)."""
    x = generate(dataclasses.replace(workload("c0"), name="dense", hq=8, hkv=2, head_dim=128,
                                     total_tokens=1500, n_blocks=1, block_len=1500, l_anchor=0,
                                     l_query=4, l_pass=0))
    lay = layout_of(x)
    full_check(x, lay)


def test_fused_qkv_strides():
    """q_ctx / k_ctx / v_ctx as views into one fused [N, (hq + 2 hkv) d] buffer."""
    x = small("c0", hq=4, hkv=2, head_dim=128, total_tokens=700, n_blocks=2, block_len=350,
              l_anchor=32, l_query=16, l_pass=24)
    w = x.w
    N, d = x.N, w.head_dim
    fused = np.concatenate([x.bits["q_ctx"].reshape(N, -1), x.bits["k_ctx"].reshape(N, -1),
                            x.bits["v_ctx"].reshape(N, -1)], axis=1)
    F = dev_bf16(fused)
    stride = F.shape[1]
    qv = F[:, : w.hq * d]
    kv = F[:, w.hq * d: (w.hq + w.hkv) * d]
    vv = F[:, (w.hq + w.hkv) * d:]
    lay = layout_of(x, q_row_stride=stride, kv_row_stride=stride)
    dd = upload(x, ("q_query", "k_anchor", "v_anchor"))
    _, sel = apbv.score_select(lay, dd["q_query"], kv)
    kp, vp = apbv.gather_passing(lay, dd["k_anchor"], dd["v_anchor"], kv, vv, sel)
    out, _ = apbv.approx_attn_prefill(lay, qv, kp, vp, kv, vv)
    ref_lay = layout_of(x)
    d2 = upload(x)
    ref = run_gpu(x, ref_lay, d2)
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy(), ref["sel"])
    assert np.array_equal(host_f64(out), ref["out"])


def test_largest_kv_row_stride():
    """K and V rows 2^22 - 8 elements apart, the largest stride the C ABI accepts (tile loads
    form 24-bit byte offsets: a row below 64 times a stride below 2^23 bytes). The whole
    layer equals the layer on contiguous K and V, bit for bit."""
    x = small("c0", hq=4, hkv=2, head_dim=128, total_tokens=300, n_blocks=2, block_len=150,
              l_anchor=32, l_query=16, l_pass=24)
    w = x.w
    N, d = x.N, w.head_dim
    stride = (1 << 22) - 8
    say(f"  K/V row stride {stride} elements: {2 * N * stride * 2 / 2**30:.1f} GiB of buffers")
    views = {}
    for n in ("k_ctx", "v_ctx"):
        big = torch.zeros(N * stride, dtype=torch.bfloat16, device="cuda")
        rows = big.view(N, stride)
        rows[:, : w.hkv * d] = dev_bf16(x.bits[n].reshape(N, -1))
        views[n] = rows[:, : w.hkv * d]
    lay = layout_of(x, kv_row_stride=stride)
    dd = upload(x, ("q_query", "q_ctx", "k_anchor", "v_anchor"))
    scores, sel = apbv.score_select(lay, dd["q_query"], views["k_ctx"])
    kp, vp = apbv.gather_passing(lay, dd["k_anchor"], dd["v_anchor"], views["k_ctx"],
                                 views["v_ctx"], sel)
    out, lse = apbv.approx_attn_prefill(lay, dd["q_ctx"], kp, vp, views["k_ctx"],
                                        views["v_ctx"], want_lse=True)
    torch.cuda.synchronize()
    ref = run_gpu(x, layout_of(x), upload(x))
    assert np.array_equal(scores.cpu().numpy(), ref["scores"])
    assert np.array_equal(sel.cpu().numpy(), ref["sel"])
    assert np.array_equal(host_f64(kp), ref["k_pre"]) and np.array_equal(host_f64(vp), ref["v_pre"])
    assert np.array_equal(host_f64(out), ref["out"])
    assert np.array_equal(lse.cpu().numpy().astype(np.float64), ref["lse"])
    del views
    torch.cuda.empty_cache()


def test_zigzag_ranges_and_determinism():
    """Same bits with and without ZigZag, run twice, and bucket by bucket."""
    x = small("c0", hq=4, hkv=2, head_dim=128, total_tokens=6 * 300, n_blocks=6, block_len=300,
              l_anchor=40, l_query=16, l_pass=30)
    d = upload(x)
    a = run_gpu(x, layout_of(x, zigzag=True), d)
    b = run_gpu(x, layout_of(x, zigzag=False), d)
    c = run_gpu(x, layout_of(x, zigzag=True), d)
    for k in ("scores", "sel", "k_pre", "out", "lse"):
        assert np.array_equal(a[k], b[k]), k
        assert np.array_equal(a[k], c[k]), k
    lay = layout_of(x, zigzag=True)
    _, sel = apbv.score_select(lay, d["q_query"], d["k_ctx"])
    kp, vp = apbv.gather_passing(lay, d["k_anchor"], d["v_anchor"], d["k_ctx"], d["v_ctx"], sel)
    out = torch.zeros((x.N, 4, 128), dtype=torch.bfloat16, device="cuda")
    for bkt in range(apbv.num_buckets(lay)):
        apbv.approx_attn_prefill(lay, d["q_ctx"], kp, vp, d["k_ctx"], d["v_ctx"], out=out,
                                 range_begin=bkt, range_end=bkt + 1)
    torch.cuda.synchronize()
    assert np.array_equal(host_f64(out), a["out"])


def _guarded(shape, dtype, fill):
    """A tensor view with 4096 guard elements before and after it, all set to ``fill``."""
    n = int(np.prod(shape))
    buf = torch.full((n + 8192,), fill, dtype=dtype, device="cuda")
    return buf, buf[4096:4096 + n].view(shape)


def test_outputs_stay_in_bounds():
    """Every call writes only its own outputs: guard regions around scores, selection, the
    prefix, the attention output and lse, and the query rows' output keep their fill."""
    x = generate(dataclasses.replace(workload("c0"), name="guard", keys="iid", hq=14, hkv=2,
                                     head_dim=128, total_tokens=1000, n_blocks=5, block_len=0,
                                     l_anchor=37, l_query=19, l_pass=21),
                 block_starts=[0, 129, 300, 555, 700, 1000])
    lay = layout_of(x)
    d = upload(x, ("q_query", "q_ctx", "k_ctx", "v_ctx", "k_anchor", "v_anchor", "k_query",
                   "v_query"))
    w = x.w
    bufs = {}
    bufs["scores"] = _guarded((w.hkv, x.N), torch.float32, 7.0)
    bufs["sel"] = _guarded((lay.n_blocks, w.hkv, lay.l_pass), torch.int32, -7)
    bufs["k_pre"] = _guarded((w.hkv, lay.pre_rows, w.head_dim), torch.bfloat16, 7.0)
    bufs["v_pre"] = _guarded((w.hkv, lay.pre_rows, w.head_dim), torch.bfloat16, 7.0)
    bufs["out"] = _guarded((x.N, w.hq, w.head_dim), torch.bfloat16, 7.0)
    bufs["lse"] = _guarded((w.hq, x.N), torch.float32, 7.0)
    bufs["q_out"] = _guarded((w.l_query, w.hq, w.head_dim), torch.bfloat16, 7.0)
    bufs["q_lse"] = _guarded((w.hq, w.l_query), torch.float32, 7.0)
    v = {k: b[1] for k, b in bufs.items()}
    apbv.score_select(lay, d["q_query"], d["k_ctx"], scores=v["scores"], sel=v["sel"])
    apbv.gather_passing(lay, d["k_anchor"], d["v_anchor"], d["k_ctx"], d["v_ctx"], v["sel"],
                        k_pre=v["k_pre"], v_pre=v["v_pre"])
    apbv.approx_attn_prefill(lay, d["q_ctx"], v["k_pre"], v["v_pre"], d["k_ctx"], d["v_ctx"],
                             out=v["out"], lse=v["lse"])
    apbv.query_forward(lay, d["q_query"], d["k_query"], d["v_query"], d["k_anchor"],
                       d["v_anchor"], d["k_ctx"], d["v_ctx"], out=v["q_out"], lse=v["q_lse"])
    torch.cuda.synchronize()
    for name, (buf, view) in bufs.items():
        fill = buf[0].item()
        assert torch.all(buf[:4096] == fill) and torch.all(buf[-4096:] == fill), name
        assert torch.isfinite(view.float()).all() or name == "sel", name
    say("  guards intact around every output")


def test_layer_call_stays_in_bounds():
    """The one-call layer with a second stream (block and row ranges of the scoring and the
    gather on both streams) writes only its own outputs and matches the three calls."""
    x = generate(dataclasses.replace(workload("c0"), name="guard", keys="iid", hq=14, hkv=2,
                                     head_dim=128, total_tokens=1000, n_blocks=5, block_len=0,
                                     l_anchor=37, l_query=19, l_pass=21),
                 block_starts=[0, 129, 300, 555, 700, 1000])
    lay = layout_of(x)
    d = upload(x)
    w = x.w
    bufs = {"scores": _guarded((w.hkv, x.N), torch.float32, 7.0),
            "sel": _guarded((lay.n_blocks, w.hkv, lay.l_pass), torch.int32, -7),
            "k_pre": _guarded((w.hkv, lay.pre_rows, w.head_dim), torch.bfloat16, 7.0),
            "v_pre": _guarded((w.hkv, lay.pre_rows, w.head_dim), torch.bfloat16, 7.0),
            "out": _guarded((x.N, w.hq, w.head_dim), torch.bfloat16, 7.0),
            "lse": _guarded((w.hq, x.N), torch.float32, 7.0)}
    v = {k: b[1] for k, b in bufs.items()}
    apbv.prefill_layer(lay, d["q_query"], d["q_ctx"], d["k_ctx"], d["v_ctx"], d["k_anchor"],
                       d["v_anchor"], aux_stream=torch.cuda.Stream(), **v)
    torch.cuda.synchronize()
    for name, (buf, view) in bufs.items():
        fill = buf[0].item()
        assert torch.all(buf[:4096] == fill) and torch.all(buf[-4096:] == fill), name
    g = run_gpu(x, lay, d)
    assert np.array_equal(v["sel"].cpu().numpy(), g["sel"])
    assert np.array_equal(v["scores"].cpu().numpy(), g["scores"])
    assert np.array_equal(host_f64(v["out"]), g["out"])
    say("  guards intact around every output of the one-call layer")


def test_gather_counts_selections_outside_their_block():
    """Entries of sel outside their own block are counted into sel_errors and clamped into the
    block (its first or last row); every other prefix row is the oracle's gather."""
    x = generate(dataclasses.replace(workload("c0"), name="selerr", keys="iid", hq=4, hkv=2,
                                     head_dim=128, total_tokens=900, n_blocks=3, block_len=300,
                                     l_anchor=16, l_query=8, l_pass=20))
    lay = layout_of(x)
    d = upload(x)
    _, sel = apbv.score_select(lay, d["q_query"], d["k_ctx"])
    torch.cuda.synchronize()
    bad = sel.cpu().numpy().copy()
    bs = x.block_starts
    bad[0, 0, 0] = bs[1]          # a row of the next block
    bad[1, 1, 5] = -5             # before the context
    bad[2, 0, 19] = x.N + 10      # past the context
    bad[1, 0, 0] = bs[1] - 1      # the last row of the previous block
    errs = torch.zeros(1, dtype=torch.int32, device="cuda")
    kp, vp = apbv.gather_passing(lay, d["k_anchor"], d["v_anchor"], d["k_ctx"], d["v_ctx"],
                                 torch.from_numpy(bad).cuda(), sel_errors=errs)
    torch.cuda.synchronize()
    assert int(errs.item()) == 4
    fixed = bad.copy()
    for v in range(lay.n_blocks):
        fixed[v] = np.clip(fixed[v], bs[v], bs[v + 1] - 1)
    ka, va = x.f32("k_anchor"), x.f32("v_anchor")
    k_or, v_or = orc.gather_prefix(ka, va, x.f32("k_ctx"), x.f32("v_ctx"), fixed)
    assert np.array_equal(host_f64(kp), k_or) and np.array_equal(host_f64(vp), v_or)
    # a valid selection adds nothing to the counter
    apbv.gather_passing(lay, d["k_anchor"], d["v_anchor"], d["k_ctx"], d["v_ctx"], sel,
                        sel_errors=errs)
    torch.cuda.synchronize()
    assert int(errs.item()) == 4
    say("  out-of-block selections counted (4) and clamped into their blocks")
