"""Helpers of the GPU parity tests: upload bf16 inputs, run the three C-ABI calls, and
compare with the oracle by the acceptance rules (bit-exact selection outside the float32
near-tie band; attention max-abs <= 2e-2 and mean-abs <= 2e-3 on bf16 inputs)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import sequence_approximate_attention_score_amd as apbv
from oracle import apbv_oracle as orc

ATOL_MAX = 2e-2
ATOL_MEAN = 2e-3


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def layout_of(x, *, zigzag=True, l_pass=None, l_anchor=None, block_starts=None, **kw):
    w = x.w
    return apbv.Layout(x.block_starts if block_starts is None else block_starts,
                       l_anchor=w.l_anchor if l_anchor is None else l_anchor, l_query=w.l_query,
                       l_pass=w.l_pass if l_pass is None else l_pass, hq=w.hq, hkv=w.hkv,
                       head_dim=w.head_dim, zigzag=zigzag, **kw)


def upload(x, names=("q_query", "q_ctx", "k_ctx", "v_ctx", "k_anchor", "v_anchor")):
    return {n: dev_bf16(x.bits[n]) for n in names}


def check_selection(scores32_oracle, sel_gpu, block_starts, l_pass):
    """Selection rule: outside the near-tie band (|s - t| < 1e-5 |t| around the oracle's
    l_pass-th score) the GPU and oracle sets are equal; the GPU set is l_pass strictly
    ascending rows inside the block. Returns the number of band positions seen."""
    bs = np.asarray(block_starts)
    n_band = 0
    for v in range(sel_gpu.shape[0]):
        lo, hi = int(bs[v]), int(bs[v + 1])
        for g in range(sel_gpu.shape[1]):
            row = sel_gpu[v, g].astype(np.int64)
            assert row.size == l_pass
            if l_pass == 0:
                continue
            assert np.all(np.diff(row) > 0), (v, g, "not strictly ascending")
            assert row.min() >= lo and row.max() < hi, (v, g, "outside the block")
            blk = scores32_oracle[g, lo:hi]
            amb = orc.ambiguous_positions(blk, l_pass)
            n_band += int(amb.sum())
            o_order = np.argsort(-blk.astype(np.float32), kind="stable")[:l_pass]
            o_set = set(int(j) for j in o_order if not amb[j])
            g_set = set(int(j - lo) for j in row if not amb[j - lo])
            assert o_set == g_set, (v, g, sorted(o_set ^ g_set)[:10])
    return n_band


def check_attention(out_gpu: np.ndarray, out_ref: np.ndarray, what: str):
    m = ~np.isnan(out_ref)
    assert m.any(), what
    err = np.abs(out_gpu[m] - out_ref[m])
    mx, mean = float(err.max()), float(err.mean())
    say(f"  {what}: max-abs {mx:.3e} mean-abs {mean:.3e} over {int(m.sum())} values")
    assert np.all(np.isfinite(out_gpu[m])), what
    assert mx <= ATOL_MAX and mean <= ATOL_MEAN, (what, mx, mean)
    return mx, mean
