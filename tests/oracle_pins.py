"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Every pin is a function ``pin_*(orc)`` taking an oracle module, so that the same pins run
against the real oracle (they must all hold) and against deliberately broken copies of it
(each broken copy must fail at least one pin). Pins never recompute the oracle's formula
the same way: they use an explicit full-sequence mask, torch's scaled-dot-product
attention as an independent softmax, closed forms, hand-worked rational examples or the
definition of a top-k set.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------- helpers
def tiny_problem(seed=0, hq=4, hkv=2, d=8, block_starts=(0, 7, 12, 20), l_a=3, l_q=5, l_p=3,
                 key_scale=1.0):
    rng = np.random.default_rng(seed)
    N = block_starts[-1]
    f = lambda *s: rng.standard_normal(s)
    return dict(q_query=f(l_q, hq, d), q_ctx=f(N, hq, d), k_ctx=key_scale * f(N, hkv, d),
                v_ctx=f(N, hkv, d), k_anchor=f(l_a, hkv, d), v_anchor=f(l_a, hkv, d),
                block_starts=np.asarray(block_starts, np.int32), l_pass=l_p, hq=hq, hkv=hkv,
                scale=1.0 / math.sqrt(d))


def run(orc, p, **kw):
    return orc.approx_attention_prefill(p["q_query"], p["q_ctx"], p["k_ctx"], p["v_ctx"],
                                        p["k_anchor"], p["v_anchor"], p["block_starts"],
                                        p["l_pass"], p["hq"], p["hkv"], p["scale"], **kw)


def sdpa(q, k, v, scale, causal=False):
    """torch's scaled-dot-product attention in float64 on rows q [R, d], keys k [K, d]."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float64))[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal,
                                                         scale=scale)
    return o[0, 0].numpy()


def brute_force_masked(p, sel):
    """Attention of every context row with an explicit mask over the whole sequence
    [anchor | context]: anchor visible; context key j visible iff it lies in an earlier
    block and is in that block's passing set for the row's KV head, or lies in the row's own
    block at or before the row. Returns (out [N, hq, d], lse [hq, N])."""
    bs = list(p["block_starts"])
    N, hq, hkv = bs[-1], p["hq"], p["hkv"]
    G = hq // hkv
    l_a = p["k_anchor"].shape[0]
    block_of = np.searchsorted(np.asarray(bs), np.arange(N), side="right") - 1
    out = np.zeros((N, hq, p["q_ctx"].shape[2]))
    lse = np.zeros((hq, N))
    for h in range(hq):
        g = h // G
        K = np.concatenate([p["k_anchor"][:, g], p["k_ctx"][:, g]])
        V = np.concatenate([p["v_anchor"][:, g], p["v_ctx"][:, g]])
        chosen = np.zeros(N, bool)
        for u in range(len(bs) - 1):
            chosen[sel[u, g]] = True
        for i in range(N):
            vi = block_of[i]
            vis = np.zeros(l_a + N, bool)
            vis[:l_a] = True
            for j in range(N):
                if block_of[j] < vi and chosen[j]:
                    vis[l_a + j] = True
                elif block_of[j] == vi and j <= i:
                    vis[l_a + j] = True
            z = p["scale"] * (K[vis] @ p["q_ctx"][i, h])
            w = np.exp(z - z.max())
            out[i, h] = (w / w.sum()) @ V[vis]
            lse[h, i] = z.max() + math.log(w.sum())
    return out, lse


def is_topk_set(scores_block, chosen_positions, k):
    """Definition of the selected set: k distinct positions such that every chosen position
    beats every unchosen one (higher score, or equal score and lower position)."""
    s = np.asarray(scores_block, np.float32)
    chosen = set(int(c) for c in chosen_positions)
    if len(chosen) != k:
        return False
    for j in chosen:
        for jj in range(s.size):
            if jj in chosen:
                continue
            if not (s[j] > s[jj] or (s[j] == s[jj] and j < jj)):
                return False
    return True


# ----------------------------------------------------------------------------- pins
def pin_bruteforce_mask(orc):
    """Block-wise attention == explicit-mask attention over the whole sequence."""
    for seed in (0, 1):
        p = tiny_problem(seed)
        r = run(orc, p)
        bo, bl = brute_force_masked(p, r["sel"])
        assert np.allclose(r["out"], bo, atol=1e-12, rtol=0), "output vs explicit mask"
        assert np.allclose(r["lse"], bl, atol=1e-12, rtol=0), "lse vs explicit mask"


def pin_single_block_is_dense_causal(orc):
    """One block (one host): attention is plain causal attention over [anchor | block]."""
    p = tiny_problem(2, block_starts=(0, 13))
    r = run(orc, p)
    l_a, G = p["k_anchor"].shape[0], p["hq"] // p["hkv"]
    for h in range(p["hq"]):
        g = h // G
        q = np.concatenate([np.zeros((l_a, p["q_ctx"].shape[2])), p["q_ctx"][:, h]])
        k = np.concatenate([p["k_anchor"][:, g], p["k_ctx"][:, g]])
        v = np.concatenate([p["v_anchor"][:, g], p["v_ctx"][:, g]])
        ref = sdpa(q, k, v, p["scale"], causal=True)[l_a:]
        assert np.allclose(r["out"][:, h], ref, atol=1e-12, rtol=0), "n=1 vs causal SDPA"


def pin_full_passing_is_dense_causal(orc):
    """l_p equal to the block length passes every earlier key: dense causal attention."""
    p = tiny_problem(3, block_starts=(0, 6, 12, 18), l_p=6)
    r = run(orc, p)
    l_a, G = p["k_anchor"].shape[0], p["hq"] // p["hkv"]
    for h in range(p["hq"]):
        g = h // G
        q = np.concatenate([np.zeros((l_a, p["q_ctx"].shape[2])), p["q_ctx"][:, h]])
        k = np.concatenate([p["k_anchor"][:, g], p["k_ctx"][:, g]])
        v = np.concatenate([p["v_anchor"][:, g], p["v_ctx"][:, g]])
        ref = sdpa(q, k, v, p["scale"], causal=True)[l_a:]
        assert np.allclose(r["out"][:, h], ref, atol=1e-12, rtol=0), "l_p=L vs causal SDPA"


def pin_probability_mass(orc):
    """Attention weights sum to one and put exactly no mass on masked keys: future keys of
    the row's own block, unselected keys of earlier blocks and every key of later blocks."""
    p = tiny_problem(4)
    sel = run(orc, p)["sel"]
    bs = p["block_starts"]
    N, hkv, G = bs[-1], p["hkv"], p["hq"] // p["hkv"]
    ones = dict(p, v_ctx=np.ones_like(p["v_ctx"]), v_anchor=np.ones_like(p["v_anchor"]))
    assert np.allclose(run(orc, ones)["out"], 1.0, atol=1e-13), "V = 1 must give O = 1"
    va = np.zeros_like(p["v_anchor"]); va[:, :, 0] = 1
    for v in range(len(bs) - 1):
        for i in range(bs[v], bs[v + 1]):
            vc = np.zeros_like(p["v_ctx"])
            for g in range(hkv):
                picked = np.zeros(N, bool)
                for u in range(v):
                    picked[sel[u, g]] = True
                earlier = np.arange(N) < bs[v]
                vc[picked, g, 1] = 1                              # passing keys of earlier blocks
                vc[earlier & ~picked, g, 3] = 1                   # unselected earlier keys
                vc[bs[v]:i + 1, g, 2] = 1                         # own block, at or before i
                vc[i + 1:bs[v + 1], g, 5] = 1                     # own block, after i
                vc[bs[v + 1]:, g, 4] = 1                          # later blocks
            o = run(orc, dict(p, v_ctx=vc, v_anchor=va))["out"][i]
            assert np.all(o[:, 3] == 0) and np.all(o[:, 4] == 0) and np.all(o[:, 5] == 0), \
                "mass on a masked key"
            assert np.allclose(o[:, 0] + o[:, 1] + o[:, 2], 1.0, atol=1e-13)
            assert np.all(o[:, 0] > 0) and np.all(o[:, 2] > 0), "anchor and diagonal visible"
            if v > 0 and p["l_pass"] > 0:
                assert np.all(o[:, 1] > 0), "earlier passing keys visible"


def pin_scores_are_library_softmax_sums(orc):
    """s[g, j] equals the column sums of torch's softmax probabilities (SDPA with V = I)
    over the heads of g's group and the query rows; every block sums to G * l_q."""
    p = tiny_problem(5)
    s = orc.passing_scores(p["q_query"], p["k_ctx"], p["block_starts"], p["hq"], p["hkv"],
                           p["scale"])
    bs, G, l_q = p["block_starts"], p["hq"] // p["hkv"], p["q_query"].shape[0]
    ref = np.zeros_like(s)
    for v in range(len(bs) - 1):
        lo, hi = bs[v], bs[v + 1]
        for h in range(p["hq"]):
            g = h // G
            P = sdpa(p["q_query"][:, h], p["k_ctx"][lo:hi, g], np.eye(hi - lo), p["scale"])
            ref[g, lo:hi] += P.sum(axis=0)
        for g in range(p["hkv"]):
            assert math.isclose(s[g, lo:hi].sum(), G * l_q, rel_tol=1e-12), "block sum G*l_q"
    assert np.allclose(s, ref, atol=1e-12, rtol=0), "scores vs SDPA probabilities"


def pin_score_query_permutation(orc):
    """Scores do not depend on the order of the query rows or of the heads within a group."""
    p = tiny_problem(6)
    args = (p["k_ctx"], p["block_starts"], p["hq"], p["hkv"], p["scale"])
    s0 = orc.passing_scores(p["q_query"], *args)
    perm = np.random.default_rng(1).permutation(p["q_query"].shape[0])
    s1 = orc.passing_scores(p["q_query"][perm], *args)
    G = p["hq"] // p["hkv"]
    hp = np.concatenate([np.arange(g * G, (g + 1) * G)[::-1] for g in range(p["hkv"])])
    s2 = orc.passing_scores(p["q_query"][:, hp], *args)
    assert np.allclose(s0, s1, atol=1e-12) and np.allclose(s0, s2, atol=1e-12)


def pin_needles_rank_first(orc):
    """Keys planted along the query direction with decreasing strength are selected first,
    in order of strength, and a key orthogonal to every query never outranks them."""
    rng = np.random.default_rng(7)
    d, L = 16, 40
    u = rng.standard_normal(d); u /= np.linalg.norm(u)
    q = np.tile(u, (6, 2, 1))                               # l_q=6, hq=2 (one group)
    k = 0.3 * rng.standard_normal((2 * L, 1, d))
    needles = {3: 9.0, 17: 7.0, 30: 5.0, 44: 9.5, 70: 8.0, 52: 6.0}
    for j, a in needles.items():
        k[j, 0] = a * u
    bs = np.array([0, L, 2 * L], np.int32)
    s = orc.passing_scores(q, k, bs, 2, 1, 1.0)
    sel = orc.select_passing(s.astype(np.float32), bs, 3)
    assert sel[0, 0].tolist() == [3, 17, 30] and sel[1, 0].tolist() == [44, 52, 70], sel
    assert s[0, 3] > s[0, 17] > s[0, 30] and s[0, 44] > s[0, 70] > s[0, 52]


def pin_selection_definition(orc):
    """Selected sets satisfy the top-k definition with ties to the lower position, on scores
    full of exact ties; output ascending, absolute rows, inside the block."""
    rng = np.random.default_rng(8)
    for trial in range(60):
        L = int(rng.integers(1, 12))
        n = int(rng.integers(1, 4))
        bs = np.arange(n + 1, dtype=np.int32) * L
        s = rng.integers(0, 4, size=(2, n * L)).astype(np.float32) / 4
        k = int(rng.integers(0, L + 1))
        sel = orc.select_passing(s, bs, k)
        for v in range(n):
            for g in range(2):
                row = sel[v, g]
                assert np.all(np.diff(row) > 0) and np.all(row >= bs[v]) and np.all(row < bs[v + 1])
                assert is_topk_set(s[g, bs[v]:bs[v + 1]], row - bs[v], k), (s, row)


def pin_no_passing_is_anchor_plus_local(orc):
    """l_p = 0: each row sees only the anchor and its own block's past (explicit mask)."""
    p = tiny_problem(9, l_p=0)
    r = run(orc, p)
    bo, bl = brute_force_masked(p, r["sel"])
    assert r["sel"].shape[2] == 0
    assert np.allclose(r["out"], bo, atol=1e-12, rtol=0)


def pin_hand_worked_golden(orc):
    """Hand-worked rational examples (tests/golden/hand_worked.json)."""
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        gold = json.load(f)
    c = gold["common"]
    bs = np.asarray(c["block_starts"], np.int32)
    N = int(bs[-1])
    fr = lambda m: np.array([[float(Fraction(x)) for x in row] for row in m])
    for case in gold["cases"]:
        q_query = np.asarray(case["q_query"], float)[:, None, :]
        k_ctx = np.asarray(case["k_ctx"], float)[:, None, :]
        v_ctx = np.asarray(c["v_ctx"], float)[:, None, :]
        ka = np.asarray(c["k_anchor"], float)[:, None, :]
        va = np.asarray(c["v_anchor"], float)[:, None, :]
        q_ctx = np.zeros((N, 1, c["head_dim"]))
        r = orc.approx_attention_prefill(q_query, q_ctx, k_ctx, v_ctx, ka, va, bs, c["l_pass"],
                                         1, 1, 1 / math.sqrt(c["head_dim"]))
        assert r["sel"][:, 0, :].tolist() == case["expected_sel"], case["name"]
        assert np.allclose(r["out"][:, 0, :], fr(case["expected_out"]), atol=1e-14), case["name"]
        assert np.allclose(np.exp(r["lse"][0]), case["expected_visible_keys"], rtol=1e-13)
        if "expected_scores" in case:
            exp_s = np.array([float(Fraction(x)) for x in case["expected_scores"]])
            assert np.allclose(r["scores"][0], exp_s, atol=1e-15)


def query_problem(seed, **kw):
    p = tiny_problem(seed, **kw)
    rng = np.random.default_rng(seed + 1000)
    l_q, hkv, d = p["q_query"].shape[0], p["hkv"], p["q_query"].shape[2]
    p["k_query"] = rng.standard_normal((l_q, hkv, d))
    p["v_query"] = rng.standard_normal((l_q, hkv, d))
    return p


def run_query(orc, p, **over):
    a = dict(p, **over)
    return orc.query_attention(a["q_query"], a["k_query"], a["v_query"], a["k_anchor"],
                               a["v_anchor"], a["k_ctx"], a["v_ctx"], a["hq"], a["hkv"],
                               a["scale"])


def pin_query_rows_are_dense_causal_tail(orc):
    """The query block closes the sequence: its rows equal the last l_q rows of dense causal
    attention (torch SDPA) over [anchor | context | query block]; lse equals the
    log-sum-exp (scipy) of each row's visible logits, enumerated one key at a time."""
    from scipy.special import logsumexp
    p = query_problem(11)
    out, lse = run_query(orc, p)
    rng = np.random.default_rng(12)
    l_q, hq, d = p["q_query"].shape
    G = hq // p["hkv"]
    for h in range(hq):
        g = h // G
        K = np.concatenate([p["k_anchor"][:, g], p["k_ctx"][:, g], p["k_query"][:, g]])
        V = np.concatenate([p["v_anchor"][:, g], p["v_ctx"][:, g], p["v_query"][:, g]])
        Q = np.concatenate([rng.standard_normal((K.shape[0] - l_q, d)), p["q_query"][:, h]])
        ref = sdpa(Q, K, V, p["scale"], causal=True)[-l_q:]
        assert np.allclose(out[:, h], ref, atol=1e-12, rtol=0), "query rows vs dense causal"
        for i in range(l_q):
            visible = [p["scale"] * float(K[j] @ p["q_query"][i, h])
                       for j in range(K.shape[0] - l_q + i + 1)]
            assert math.isclose(lse[h, i], logsumexp(visible), rel_tol=0, abs_tol=1e-12)


def pin_query_merge_of_split_keys(orc):
    """Attention over a union of key sets is recovered from the parts through their lse:
    context split at a random row into [anchor | ctx[:m] | query] and [ctx[m:]]; a part in
    which no key is visible (lse -inf, output NaN) changes nothing; V = const gives const."""
    p = query_problem(13)
    whole_o, whole_l = run_query(orc, p)
    N = p["k_ctx"].shape[0]
    for m in (1, 7, N - 1):
        a_o, a_l = run_query(orc, p, k_ctx=p["k_ctx"][:m], v_ctx=p["v_ctx"][:m])
        b_o, b_l = run_query(orc, p, k_ctx=p["k_ctx"][m:], v_ctx=p["v_ctx"][m:],
                             k_anchor=p["k_anchor"][:0], v_anchor=p["v_anchor"][:0],
                             k_query=p["k_query"][:0], v_query=p["v_query"][:0])
        o, l = orc.merge_partials([a_o, b_o], [a_l, b_l])
        assert np.allclose(o, whole_o, atol=1e-12, rtol=0) and np.allclose(l, whole_l, atol=1e-12)
    empty_o = np.full_like(whole_o, np.nan)
    empty_l = np.full_like(whole_l, -np.inf)
    o, l = orc.merge_partials([whole_o, empty_o], [whole_l, empty_l])
    assert np.allclose(o, whole_o, atol=1e-14) and np.allclose(l, whole_l, atol=1e-14)
    c = np.full_like(p["v_ctx"], 0.75)
    o, _ = run_query(orc, p, v_ctx=c, v_anchor=np.full_like(p["v_anchor"], 0.75),
                     v_query=np.full_like(p["v_query"], 0.75))
    assert np.allclose(o, 0.75, atol=1e-14, rtol=0)


PINS = [pin_bruteforce_mask, pin_single_block_is_dense_causal, pin_full_passing_is_dense_causal,
        pin_probability_mass, pin_scores_are_library_softmax_sums, pin_score_query_permutation,
        pin_needles_rank_first, pin_selection_definition, pin_no_passing_is_anchor_plus_local,
        pin_hand_worked_golden, pin_query_rows_are_dense_causal_tail,
        pin_query_merge_of_split_keys]
