"""Plain CPU oracle for the APB-V / Spava approximate-attention prefill (float64 numpy).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import or run this module. It shares no code with the HIP path.

Sources (the method is described only in prose; no formula or listing is printed):

* "Riepilogo Tecnico: APB-V" (gist.science), section Metodologia, part 1 "Design del
  Framework": the context is split into an anchor block B_a, a query block B_qr and
  context blocks B^(h) (sub-part "Suddivisione del Contesto e Disposizione ZigZag"); the
  approximate attention (sub-part "Meccanismo di Attenzione Approssimata") keeps the anchor,
  picks for every host the most important key/value pairs of the preceding hosts by
  query-to-context attention scores and collects them as passing blocks, and computes
  attention over anchor, local context and the collected passing blocks.
* Same page, part 2 "Ottimizzazioni a Livello di Sistema": ZigZag pairing of virtual hosts
  h and 2H-1-h balances the passing-block length per physical host; the fused forward of
  context and query ("Forward Fuso di Contesto e Query") runs the query block's rows with
  the context and merges their partial results over different key sets through the
  log-sum-exp that flash attention returns.
* Same page, "Limitazioni": with a single block the method is plain (flash) attention.

Readings taken where the pages are silent (each one is listed with its reason in the design
notes of the repository):

* score of context key j of block v for KV head g:
  s[g, j] = sum over the G query heads h of group g and the l_q rows i of the query block of
  softmax over the keys of block v of (scale * q[i, h] . k[j, g]); scale = 1/sqrt(d);
* head h uses KV head h // G (G = hq / hkv);
* the anchor is its own prefix, attended by every context row and never selectable;
* block v's passing prefix is the anchor followed by the passing blocks of blocks 0..v-1 in
  sequence order, each in ascending position order;
* selection keeps the l_p largest scores of a block, ties to the lower position, decided on
  the float32-rounded scores (the precision of the GPU kernel's scores);
* mask: anchor and passing keys fully visible, local keys causal (j <= i);
* the query block's rows are exact: they see the anchor, all N context keys and the query
  block's keys up to their own position.

Parity pins are in ``tests/test_oracle.py``; none of the pages prints a worked example,
so agreement with the paper's own outputs is unpinned.
"""
from __future__ import annotations

import numpy as np


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _softmax_rows(z: np.ndarray) -> np.ndarray:
    """Row softmax with the row maximum subtracted first (float64)."""
    m = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def kv_head(h: int, hq: int, hkv: int) -> int:
    """KV head shared by query head h (contiguous groups of G = hq / hkv heads)."""
    return h // (hq // hkv)


# --------------------------------------------------------------------------------------
# Step 1 - query-to-context scores of every block (the passing-block criterion).
# --------------------------------------------------------------------------------------
def passing_scores(q_query, k_ctx, block_starts, hq: int, hkv: int, scale: float,
                   blocks=None) -> np.ndarray:
    """Scores s[g, j] of every context key, float64 ``[hkv, N]``.

    For block v (rows bs[v]..bs[v+1]) and KV head g, every query-block row i of every head h
    in g's group spreads a softmax over block v's keys; s is the sum of those distributions
    (heads ascending, then rows ascending). Each block's scores sum to G * l_q.
    ``blocks`` restricts the work to some blocks (the others are left as NaN).
    """
    q = _as64(q_query)             # [l_q, hq, d]
    bs = np.asarray(block_starts, np.int64)
    s = np.full((hkv, np.asarray(k_ctx).shape[0]), np.nan)
    for v in (range(bs.size - 1) if blocks is None else blocks):
        lo, hi = int(bs[v]), int(bs[v + 1])
        k = _as64(k_ctx[lo:hi])    # [L_v, hkv, d]
        s[:, lo:hi] = 0.0
        for h in range(hq):
            g = kv_head(h, hq, hkv)
            z = scale * (q[:, h, :] @ k[:, g, :].T)             # [l_q, L_v]
            s[g, lo:hi] += _softmax_rows(z).sum(axis=0)
    return s


# --------------------------------------------------------------------------------------
# Step 2 - top-l_p selection per (block, KV head) -> passing block indices.
# --------------------------------------------------------------------------------------
def select_passing(scores32, block_starts, l_pass: int) -> np.ndarray:
    """int32 ``[n, hkv, l_pass]``: the l_pass highest-scoring context rows of each block.

    ``scores32`` are float32 scores; ties go to the lower position; the result is written as
    absolute context rows in ascending order.
    """
    s = np.asarray(scores32, np.float32)
    bs = np.asarray(block_starts, np.int64)
    n, hkv = bs.size - 1, s.shape[0]
    sel = np.empty((n, hkv, l_pass), np.int32)
    for v in range(n):
        lo, hi = int(bs[v]), int(bs[v + 1])
        if l_pass > hi - lo:
            raise ValueError("l_pass exceeds the block length")
        for g in range(hkv):
            order = np.argsort(-s[g, lo:hi], kind="stable")      # descending, ties keep order
            sel[v, g] = np.sort(order[:l_pass]) + lo
    return sel


# --------------------------------------------------------------------------------------
# Step 3 - collect the anchor and every block's passing block in one prefix per KV head.
# --------------------------------------------------------------------------------------
def gather_prefix(k_anchor, v_anchor, k_ctx, v_ctx, sel):
    """``K_pre, V_pre`` float64 ``[hkv, l_a + n * l_pass, d]``: anchor, then passing 0..n-1."""
    ka, va = _as64(k_anchor), _as64(v_anchor)
    kc, vc = np.asarray(k_ctx), np.asarray(v_ctx)   # rows are widened once gathered
    sel = np.asarray(sel, np.int64)
    n, hkv, _ = sel.shape
    k_pre, v_pre = [], []
    for g in range(hkv):
        k_parts = [ka[:, g, :]] + [_as64(kc[sel[v, g], g, :]) for v in range(n)]
        v_parts = [va[:, g, :]] + [_as64(vc[sel[v, g], g, :]) for v in range(n)]
        k_pre.append(np.concatenate(k_parts, axis=0))
        v_pre.append(np.concatenate(v_parts, axis=0))
    return np.stack(k_pre), np.stack(v_pre)


# --------------------------------------------------------------------------------------
# Step 4 - attention of each context row over [anchor | passing of earlier blocks | local].
# --------------------------------------------------------------------------------------
def attend(q_ctx, k_pre, v_pre, k_ctx, v_ctx, block_starts, l_anchor: int, l_pass: int,
           hq: int, hkv: int, scale: float, rows=None, heads=None, row_chunk: int = 512):
    """Approximate attention of context rows; returns (out ``[N, hq, d]``, lse ``[hq, N]``).

    Row i of block v and head h sees key set K_pre[g, : l_a + v * l_pass] (all visible) then
    block v's own keys bs[v] .. i (causal, diagonal included). lse is the natural-log
    log-sum-exp of the scaled logits. ``rows`` (sorted absolute rows) and ``heads`` restrict
    the work to a sample; entries outside the sample are left as NaN.
    """
    kp, vp = _as64(k_pre), _as64(v_pre)
    bs = np.asarray(block_starts, np.int64)
    N, d = np.asarray(q_ctx).shape[0], np.asarray(q_ctx).shape[2]
    out = np.full((N, hq, d), np.nan)
    lse = np.full((hq, N), np.nan)
    all_rows = np.arange(N) if rows is None else np.asarray(rows, np.int64)
    heads = range(hq) if heads is None else heads
    for v in range(bs.size - 1):
        lo, hi = int(bs[v]), int(bs[v + 1])
        mine = all_rows[(all_rows >= lo) & (all_rows < hi)]
        if mine.size == 0:
            continue
        P = l_anchor + v * l_pass
        kc, vc = _as64(k_ctx[lo:hi]), _as64(v_ctx[lo:hi])
        for h in heads:
            g = kv_head(h, hq, hkv)
            keys = np.concatenate([kp[g, :P], kc[:, g]], axis=0)
            vals = np.concatenate([vp[g, :P], vc[:, g]], axis=0)
            local_pos = np.arange(hi - lo)
            for c in range(0, mine.size, row_chunk):
                r = mine[c:c + row_chunk]
                z = scale * (_as64(q_ctx[r, h, :]) @ keys.T)          # [rows, P + L_v]
                z[:, P:][local_pos[None, :] > (r - lo)[:, None]] = -np.inf
                m = np.max(z, axis=1, keepdims=True)
                e = np.exp(z - m)
                l = np.sum(e, axis=1, keepdims=True)
                out[r, h, :] = (e @ vals) / l
                lse[h, r] = (m + np.log(l))[:, 0]
    return out, lse


def approx_attention_prefill(q_query, q_ctx, k_ctx, v_ctx, k_anchor, v_anchor, block_starts,
                             l_pass: int, hq: int, hkv: int, scale: float, rows=None, heads=None):
    """Whole hot path: scores -> selection -> passing prefix -> attention. Returns a dict."""
    l_anchor = np.asarray(k_anchor).shape[0]
    s = passing_scores(q_query, k_ctx, block_starts, hq, hkv, scale)
    s32 = s.astype(np.float32)
    sel = select_passing(s32, block_starts, l_pass)
    k_pre, v_pre = gather_prefix(k_anchor, v_anchor, k_ctx, v_ctx, sel)
    out, lse = attend(q_ctx, k_pre, v_pre, k_ctx, v_ctx, block_starts, l_anchor, l_pass,
                      hq, hkv, scale, rows=rows, heads=heads)
    return {"scores": s, "scores32": s32, "sel": sel, "k_pre": k_pre, "v_pre": v_pre,
            "out": out, "lse": lse}


# --------------------------------------------------------------------------------------
# Step 5 - rows of the query block (fused query forward).
# --------------------------------------------------------------------------------------
def query_attention(q_query, k_query, v_query, k_anchor, v_anchor, k_ctx, v_ctx, hq: int,
                    hkv: int, scale: float, heads=None):
    """Attention of the query block's rows; returns (out ``[l_q, hq, d]``, lse ``[hq, l_q]``).

    The query block closes the sequence [anchor | context | query block] and its rows are
    not approximated: row i of head h sees every anchor key, every context key and the query
    block's keys 0..i. ``k_query`` may hold fewer rows than ``q_query`` (query key j is
    visible to query row i iff j <= i). Entries of heads outside ``heads`` are NaN.
    """
    q = _as64(q_query)
    l_q, d = q.shape[0], q.shape[2]
    n_q = np.asarray(k_query).shape[0]
    out = np.full((l_q, hq, d), np.nan)
    lse = np.full((hq, l_q), np.nan)
    rows = np.arange(l_q)
    for h in (range(hq) if heads is None else heads):
        g = kv_head(h, hq, hkv)
        keys = np.concatenate([_as64(k_anchor[:, g]), _as64(k_ctx[:, g]), _as64(k_query[:, g])])
        vals = np.concatenate([_as64(v_anchor[:, g]), _as64(v_ctx[:, g]), _as64(v_query[:, g])])
        n_before = keys.shape[0] - n_q
        z = scale * (q[:, h, :] @ keys.T)                         # [l_q, l_a + N + n_q]
        z[:, n_before:][np.arange(n_q)[None, :] > rows[:, None]] = -np.inf
        m = np.max(z, axis=1, keepdims=True)
        e = np.exp(z - m)
        l = np.sum(e, axis=1, keepdims=True)
        out[:, h, :] = (e @ vals) / l
        lse[h, :] = (m + np.log(l))[:, 0]
    return out, lse


def merge_partials(outs, lses):
    """Attention over a union of disjoint key sets from the attention over each set
    (the fused forward's merge of partial query results through their log-sum-exp).

    ``outs[s]`` ``[rows, heads, d]`` and ``lses[s]`` ``[heads, rows]`` are the normalised
    output and natural-log lse of part s; a part in which a row sees no key has lse -inf and
    contributes nothing. Returns (out, lse) of the union.
    """
    L = np.stack([_as64(x) for x in lses])                         # [S, heads, rows]
    top = np.max(L, axis=0)
    w = np.exp(L - top[None])                                      # weight of each part
    total = np.sum(w, axis=0)
    lse = top + np.log(total)
    wt = np.transpose(w / total[None], (0, 2, 1))[..., None]      # [S, rows, heads, 1]
    o = np.stack([np.nan_to_num(_as64(x)) for x in outs])
    return np.sum(wt * o, axis=0), lse


# --------------------------------------------------------------------------------------
# Selection comparison rule (ties and near-ties).
# --------------------------------------------------------------------------------------
def ambiguous_positions(scores32_block, l_pass: int, rel: float = 1e-5) -> np.ndarray:
    """Boolean mask of block positions whose float32 score lies within ``rel`` (relative) of
    the l_pass-th largest score: two correct float32 evaluations may order these differently.
    """
    s = np.asarray(scores32_block, np.float64)
    if l_pass == 0 or l_pass >= s.size:
        return np.zeros(s.shape, bool)
    t = np.sort(s)[::-1][l_pass - 1]
    return np.abs(s - t) < rel * abs(t)
