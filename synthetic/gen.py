"""Seeded input generator (numpy PCG64) for the approximate-attention workloads.

Recipe (one ``numpy.random.default_rng(seed)`` stream, draws in this order, all standard
normal float32 unless noted):

1. variable frame lengths (only when ``frame_range`` is set): ``ceil(N / lo) + 1`` integers
   from UniformInt[lo, hi] in one call; frames are taken in order until they cover N
   tokens, the last one truncated;
2. anchor block B_a: Q ``[l_a, hq, d]``, K ``[l_a, hkv, d]``, V ``[l_a, hkv, d]``;
3. context keys: for ``keys == "frame"`` a per-(frame, KV head) mean ``[F, hkv, d]`` ~ N(0, 1)
   followed by per-token noise ``[N, hkv, d]`` scaled by 0.5 (standard deviation 0.5);
   for ``keys == "iid"`` a single ``[N, hkv, d]`` draw;
4. context Q ``[N, hq, d]``;  5. context V ``[N, hkv, d]``;
6. query block B_qr (the text question): Q ``[l_q, hq, d]``, K and V ``[l_q, hkv, d]``.

Every tensor is then rounded to bf16 (round to nearest, ties to even); the kernels receive
the bf16 bit patterns and the oracle receives the same values widened back to float.
Frames tile the context from row 0; blocks are whole frames, split by frame count
(the first ``F mod n`` blocks get one extra frame).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

from .configs import Workload

_CHUNK = 1 << 24


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even. Inputs must be finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, np.uint16)
    for s in range(0, flat.size, _CHUNK):
        u = flat[s:s + _CHUNK].view(np.uint32)
        r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        out[s:s + _CHUNK] = r.astype(np.uint16)
    return out.reshape(x.shape)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact)."""
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value, returned as float32."""
    return bits_to_f32(bf16_bits(x))


def frame_partition(frame_lengths: np.ndarray, n_blocks: int) -> np.ndarray:
    """Whole frames split over ``n_blocks`` by frame count -> int32 block_starts ``[n+1]``."""
    frame_lengths = np.asarray(frame_lengths, np.int64)
    F = frame_lengths.size
    if F < n_blocks:
        raise ValueError("fewer frames than blocks")
    per = np.full(n_blocks, F // n_blocks, np.int64)
    per[: F % n_blocks] += 1
    frame_edges = np.concatenate([[0], np.cumsum(per)])
    token_edges = np.concatenate([[0], np.cumsum(frame_lengths)])
    return token_edges[frame_edges].astype(np.int32)


@dataclasses.dataclass
class Inputs:
    """bf16 bit patterns of every input, plus the layout integers."""
    w: Workload
    block_starts: np.ndarray           # int32 [n+1]
    frame_lengths: np.ndarray | None   # int64 [F] or None
    bits: dict                         # name -> uint16 array
    raw: dict | None = None            # name -> float32 array before rounding (only if kept)

    def f32(self, name: str) -> np.ndarray:
        return bits_to_f32(self.bits[name])

    @property
    def N(self) -> int:
        return int(self.block_starts[-1])


def _normal(rng, shape, scale=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def generate(w: Workload, *, keep_raw: bool = False, seed: int | None = None,
             block_starts=None) -> Inputs:
    """Draw every input of workload ``w``. ``block_starts`` overrides the block layout (any
    strictly increasing offsets from 0 to N) for test cases with ragged blocks."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    N, hq, hkv, d = w.total_tokens, w.hq, w.hkv, w.head_dim

    frame_lengths = None
    if block_starts is not None:
        block_starts = np.asarray(block_starts, np.int32)
        if block_starts[0] != 0 or block_starts[-1] != N or np.any(np.diff(block_starts) <= 0):
            raise ValueError("block_starts must increase strictly from 0 to N")
        if w.keys == "frame":
            F = math.ceil(N / w.frame_len)
            frame_lengths = np.full(F, w.frame_len, np.int64)
            frame_lengths[-1] = N - w.frame_len * (F - 1)
    elif w.frame_range:
        lo, hi = w.frame_range
        draw = rng.integers(lo, hi + 1, size=math.ceil(N / lo) + 1)
        cum = np.cumsum(draw)
        F = int(np.searchsorted(cum, N) + 1)
        frame_lengths = draw[:F].copy()
        frame_lengths[-1] -= int(cum[F - 1] - N)
        block_starts = frame_partition(frame_lengths, w.n_blocks)
    else:
        block_starts = w.uniform_block_starts()
        if w.keys == "frame":
            F = math.ceil(N / w.frame_len)
            frame_lengths = np.full(F, w.frame_len, np.int64)
            frame_lengths[-1] = N - w.frame_len * (F - 1)

    raw = {}
    raw["q_anchor"] = _normal(rng, (w.l_anchor, hq, d))
    raw["k_anchor"] = _normal(rng, (w.l_anchor, hkv, d))
    raw["v_anchor"] = _normal(rng, (w.l_anchor, hkv, d))
    if w.keys == "frame":
        means = _normal(rng, (frame_lengths.size, hkv, d))
        k = _normal(rng, (N, hkv, d), 0.5)
        frame_of_token = np.repeat(np.arange(frame_lengths.size), frame_lengths)
        for s in range(0, N, 1 << 16):
            k[s:s + (1 << 16)] += means[frame_of_token[s:s + (1 << 16)]]
        raw["k_ctx"] = k
    else:
        raw["k_ctx"] = _normal(rng, (N, hkv, d))
    raw["q_ctx"] = _normal(rng, (N, hq, d))
    raw["v_ctx"] = _normal(rng, (N, hkv, d))
    raw["q_query"] = _normal(rng, (w.l_query, hq, d))
    raw["k_query"] = _normal(rng, (w.l_query, hkv, d))
    raw["v_query"] = _normal(rng, (w.l_query, hkv, d))

    bits = {}
    for name in list(raw):
        bits[name] = bf16_bits(raw[name])
        if not keep_raw:
            del raw[name]
    return Inputs(w=w, block_starts=block_starts, frame_lengths=frame_lengths, bits=bits,
                  raw=raw if keep_raw else None)
