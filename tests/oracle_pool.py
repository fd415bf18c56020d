"""A process pool that runs the oracle for the full-size GPU parity tests.

The full-size workloads (64K-256K context tokens) need seconds to minutes of float64 oracle
work, split here into independent units run by spawned worker processes (BLAS at one thread
each): the scores of one block, and the attention of some rows of one block for one query
head. The workers import numpy and the oracle only; they never touch the GPU. The pool is
started before the GPU is initialised (``start()`` at import of the full-size test modules)
and shut down at interpreter exit.

Inputs travel to the workers as bf16 bit patterns (uint16), the exact values both the GPU
and the oracle compute on.
"""
from __future__ import annotations

import atexit
import concurrent.futures
import math
import multiprocessing
import os

import numpy as np

MAX_WORKERS = 16   # host cores of one GPU's share of the box
_pool = None


def _init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # noqa: BLE001
        pass


def _ping(_):
    from oracle import apbv_oracle  # noqa: F401
    return os.getpid()


def start() -> None:
    """Start the pool (idempotent)."""
    global _pool
    if _pool is None:
        n = max(1, min(MAX_WORKERS, len(os.sched_getaffinity(0))))
        _pool = concurrent.futures.ProcessPoolExecutor(
            n, mp_context=multiprocessing.get_context("spawn"), initializer=_init)
        list(_pool.map(_ping, range(n)))
        atexit.register(_pool.shutdown)


def pool():
    start()
    return _pool


def _f32(bits):
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _score_task(t):
    """Scores of block v for every KV head (the oracle's step 1 on one block)."""
    from oracle import apbv_oracle as orc
    k = _f32(t["k_block"])
    s = orc.passing_scores(_f32(t["q_query"]), k, [0, k.shape[0]], t["hq"], t["hkv"],
                           t["scale"])
    return t["v"], s


def _attend_task(t):
    """Attention of the given rows (offsets inside the block) of one block for one query
    head, over the block's prefix and its causal local keys (the oracle's step 4)."""
    from oracle import apbv_oracle as orc
    rows = np.asarray(t["rows"], np.int64)
    b = int(rows.max()) + 1
    d = t["q"].shape[-1]
    q = np.zeros((b, 1, d), np.float32)
    q[rows, 0] = _f32(t["q"])
    kp, vp = _f32(t["k_pre"])[None], _f32(t["v_pre"])[None]          # [1, P, d]
    kc, vc = _f32(t["k_loc"])[:, None], _f32(t["v_loc"])[:, None]     # [b, 1, d]
    out, lse = orc.attend(q, kp, vp, kc, vc, [0, b], kp.shape[1], 0, 1, 1, t["scale"],
                          rows=rows)
    return t["key"], out[rows, 0], lse[0, rows]


def scores(x, bs, hq, hkv, scale, blocks):
    """Oracle scores ``[hkv, N]`` (float64; NaN outside ``blocks``)."""
    qq, kc = x.bits["q_query"], x.bits["k_ctx"]
    tasks = [dict(v=v, hq=hq, hkv=hkv, scale=scale, q_query=qq,
                  k_block=kc[int(bs[v]):int(bs[v + 1])]) for v in blocks]
    s = np.full((hkv, kc.shape[0]), np.nan)
    for v, sv in pool().map(_score_task, tasks):
        s[:, int(bs[v]):int(bs[v + 1])] = sv
    return s


def attend(q_bits, kc_bits, vc_bits, kp_bits, vp_bits, bs, l_anchor, l_pass, hq, hkv, scale,
           rows_of_block, heads, chunk_rows=None):
    """Oracle attention of the listed rows: ``rows_of_block[v]`` are row offsets inside block
    v; every such row is computed for every head of ``heads``. ``kp_bits`` / ``vp_bits`` are
    the gathered prefix ``[hkv, l_a + n*l_p, d]`` as bf16 bits. Yields ``(v, h, rows, out,
    lse)`` with ``out`` ``[len(rows), d]`` float64."""
    G = hq // hkv
    tasks = []
    for v, rows in rows_of_block.items():
        rows = np.asarray(sorted(rows), np.int64)
        if rows.size == 0:
            continue
        lo = int(bs[v])
        P = l_anchor + v * l_pass
        parts = [rows] if chunk_rows is None else [rows[i:i + chunk_rows]
                                                   for i in range(0, rows.size, chunk_rows)]
        for part in parts:
            b = int(part.max()) + 1
            for h in heads:
                g = h // G
                tasks.append(dict(key=(v, h), rows=part, scale=scale,
                                  q=q_bits[lo + part, h], k_pre=kp_bits[g, :P],
                                  v_pre=vp_bits[g, :P], k_loc=kc_bits[lo:lo + b, g],
                                  v_loc=vc_bits[lo:lo + b, g]))
    for t, (key, out, lse) in zip(tasks, pool().map(_attend_task, tasks)):
        yield key[0], key[1], t["rows"], out, lse


def tile_sample(bs, tile_rows, seed, frac=0.05):
    """Row offsets per block of a fixed tile sample: every block's first, middle (the ZigZag
    pairing centre) and last ``tile_rows``-row tile, plus a seeded ``frac`` of its other
    tiles. Returns ``{v: row offsets}``."""
    rng = np.random.default_rng(seed)
    out = {}
    for v in range(len(bs) - 1):
        L = int(bs[v + 1] - bs[v])
        T = (L + tile_rows - 1) // tile_rows
        fixed = {0, T // 2, T - 1}
        others = [t for t in range(T) if t not in fixed]
        k = int(math.ceil(frac * len(others))) if others else 0
        pick = fixed | set(int(t) for t in rng.choice(others, size=k, replace=False))
        out[v] = np.concatenate([np.arange(t * tile_rows, min(L, (t + 1) * tile_rows))
                                 for t in sorted(pick)])
    return out
