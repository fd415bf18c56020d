"""The one-call layer (apbv_prefill_layer). With an aux stream, the scoring, selection and
gather of later blocks run beside the attention of the buckets that no longer need them.
Every output must be bit-identical to the three separate calls on the same inputs: the
same kernels compute every value, only the launch order and streams differ."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import layout_of, say, upload
from synthetic import generate, workload
import sequence_approximate_attention_score_amd as apbv
from sequence_approximate_attention_score_amd import _lib

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    apbv.lib()
    yield
    torch.cuda.synchronize()


def three_calls(lay, d):
    scores, sel = apbv.score_select(lay, d["q_query"], d["k_ctx"])
    k_pre, v_pre = apbv.gather_passing(lay, d["k_anchor"], d["v_anchor"], d["k_ctx"],
                                       d["v_ctx"], sel)
    out, lse = apbv.approx_attn_prefill(lay, d["q_ctx"], k_pre, v_pre, d["k_ctx"], d["v_ctx"],
                                        want_lse=True)
    return dict(out=out, lse=lse, sel=sel, scores=scores, k_pre=k_pre, v_pre=v_pre)


def one_call(lay, d, aux):
    shape = (lay.hkv, lay.pre_rows, lay.head_dim)
    k_pre = torch.full(shape, 7.0, dtype=torch.bfloat16, device=d["k_ctx"].device)
    v_pre = torch.full(shape, 7.0, dtype=torch.bfloat16, device=d["k_ctx"].device)
    out, lse, sel, scores = apbv.prefill_layer(lay, d["q_query"], d["q_ctx"], d["k_ctx"],
                                               d["v_ctx"], d["k_anchor"], d["v_anchor"],
                                               aux_stream=aux, k_pre=k_pre, v_pre=v_pre,
                                               want_scores=True, want_lse=True)
    return dict(out=out, lse=lse, sel=sel, scores=scores, k_pre=k_pre, v_pre=v_pre)


CASES = {
    # name: (workload, overrides, explicit block_starts or None, layout overrides)
    "c0": ("c0", {}, None, {}),
    "ragged_odd_n": ("c0", dict(hq=14, hkv=2, head_dim=128, total_tokens=1000, l_anchor=37,
                                l_query=19, l_pass=21), [0, 129, 300, 555, 700, 1000], {}),
    "no_passing": ("c0", dict(hq=4, hkv=4, head_dim=64, total_tokens=700, l_anchor=50,
                              l_query=8, l_pass=0), [0, 350, 700], {}),
    "zigzag_off": ("c0", dict(hq=4, hkv=2, head_dim=128, total_tokens=900, l_anchor=64,
                              l_query=16, l_pass=40), [0, 300, 600, 900], dict(zigzag=False)),
    "64k": ("c1", {}, None, {}),
    "128k": ("c2", {}, None, {}),
}


@pytest.mark.parametrize("name", list(CASES))
def test_layer_is_bit_identical_to_three_calls(name):
    wl, over, bs, lay_over = CASES[name]
    x = generate(workload(wl, **over))
    lay = layout_of(x, block_starts=bs, **lay_over)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    late, early = _lib.prefill_layer_plan(lay, cus)
    say(f"case {name}: n={lay.n_blocks} N={lay.n_tokens} buckets={apbv.num_buckets(lay)} "
        f"plan on {cus} CUs: late buckets from {late}, early blocks {early}")
    d = upload(x)
    ref = three_calls(lay, d)
    aux = torch.cuda.Stream()
    for trial, stream in enumerate((None, aux, aux)):
        got = one_call(lay, d, stream)
        torch.cuda.synchronize()
        for k in ("scores", "sel", "k_pre", "v_pre", "out", "lse"):
            assert torch.equal(ref[k], got[k]), (name, trial, k)


def test_128k_plan_splits_on_this_device():
    """At 128K on a 256-CU device the layer runs buckets 6 and 7 (7 whole rounds) beside the
    selections of blocks 9..15."""
    x = generate(workload("c2"))
    lay = layout_of(x)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    late, early = _lib.prefill_layer_plan(lay, cus)
    if cus == 256:
        assert (late, early) == (6, 9)
    assert 0 <= late < apbv.num_buckets(lay) and early == lay.n_blocks - 1 - late


def _random_case(seed):
    import dataclasses
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(2, 9))
    lens = rng.integers(40, 700, size=n)
    bs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 3, 7]))
    w = dataclasses.replace(workload("c0"), name=f"random{seed}", keys="iid", hq=hq, hkv=hkv,
                            head_dim=int(rng.choice([64, 128])), total_tokens=int(bs[-1]),
                            n_blocks=n, block_len=0, l_anchor=int(rng.choice([0, 33, 64])),
                            l_query=int(rng.integers(1, 24)),
                            l_pass=int(rng.integers(0, lens.min() + 1)))
    return generate(w, block_starts=bs.tolist()), rng


@pytest.mark.parametrize("seed", range(12))
def test_layer_split_on_random_layouts(seed):
    """Random ragged layouts with a CU count chosen so that the plan really splits the
    attention (late > 0): the two-stream layer is bit-identical to the three calls."""
    x, rng = _random_case(seed)
    lay = layout_of(x)
    nb = apbv.num_buckets(lay)
    cus = 0
    if nb > 1 and lay.l_pass > 0:
        b = int(rng.integers(1, nb))
        cus = apbv.schedule(lay, b, nb).shape[0] * lay.hq
    late, early = _lib.prefill_layer_plan(lay, cus)
    say(f"seed {seed}: n={lay.n_blocks} N={lay.n_tokens} hq={lay.hq} hkv={lay.hkv} "
        f"d={lay.head_dim} l_a={lay.l_anchor} l_p={lay.l_pass} buckets={nb} cus={cus} "
        f"-> late {late}, early {early}")
    if cus:
        assert late >= 1 and early == lay.n_blocks - 1 - late
    d = upload(x)
    ref = three_calls(lay, d)
    shape = (lay.hkv, lay.pre_rows, lay.head_dim)
    k_pre = torch.full(shape, 7.0, dtype=torch.bfloat16, device="cuda")
    v_pre = torch.full(shape, 7.0, dtype=torch.bfloat16, device="cuda")
    out, lse, sel, scores = apbv.prefill_layer(lay, d["q_query"], d["q_ctx"], d["k_ctx"],
                                               d["v_ctx"], d["k_anchor"], d["v_anchor"],
                                               aux_stream=torch.cuda.Stream(), k_pre=k_pre,
                                               v_pre=v_pre, want_scores=True, want_lse=True,
                                               compute_units=cus)
    torch.cuda.synchronize()
    got = dict(out=out, lse=lse, sel=sel, scores=scores, k_pre=k_pre, v_pre=v_pre)
    for k in ("scores", "sel", "k_pre", "v_pre", "out", "lse"):
        assert torch.equal(ref[k], got[k]), (seed, k)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["c0", "ragged_odd_n", "zigzag_off", "64k"])
def test_layer_matches_oracle(name):
    """The one-call layer with its second stream, against the oracle (not only against the
    three calls): every block's scores and selection, the prefix bitwise, and every row of
    one query head per KV group. Small layouts get a CU count that makes the plan split the
    attention into two launches around the second stream's selections."""
    from fullsize import fullsize_check
    wl, over, bs, lay_over = CASES[name]
    x = generate(workload(wl, **over))
    lay = layout_of(x, block_starts=bs, **lay_over)
    nb = apbv.num_buckets(lay)
    cus = 0
    if wl == "c0" and nb > 1 and lay.l_pass > 0 and lay.c.zigzag:
        cus = apbv.schedule(lay, nb // 2, nb).shape[0] * lay.hq
    late, early = _lib.prefill_layer_plan(
        lay, cus or torch.cuda.get_device_properties(0).multi_processor_count)
    say(f"layer {name}: buckets={nb} late buckets from {late}, early blocks {early}")

    def runner(lay, d):
        shape = (lay.hkv, lay.pre_rows, lay.head_dim)
        k_pre = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        v_pre = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        out, lse, sel, scores = apbv.prefill_layer(
            lay, d["q_query"], d["q_ctx"], d["k_ctx"], d["v_ctx"], d["k_anchor"], d["v_anchor"],
            aux_stream=torch.cuda.Stream(), k_pre=k_pre, v_pre=v_pre, want_scores=True,
            want_lse=True, compute_units=cus)
        return scores, sel, k_pre, v_pre, out, lse

    heads = list(range(lay.hq)) if wl == "c0" else None
    fullsize_check(x, lay, all_rows=True, heads=heads, runner=runner)
