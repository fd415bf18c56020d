"""The five synthetic workloads of the approximate-attention prefill.

The pages give no layer shapes or hyper-parameters, so the shapes are fixed here:

* ``c0``  tiny correctness case: 2 query heads / 1 KV head, head_dim 64, two virtual
  blocks of 256 context tokens, anchor 64, query block 32, passing length 32,
  i.i.d. N(0, 1) inputs generated in fp32.
* ``c1``  Qwen2.5-VL-7B-shaped layer (28 query heads / 4 KV heads, head_dim 128), 64K
  visual tokens as 8 work buckets of 8K, i.e. 16 virtual blocks of 4K (ZigZag pairs),
  anchor 1024, query 128, passing 512; frame-correlated keys, 256 tokens per frame.
* ``c2``  same layer, 128K visual tokens as 16 virtual blocks of 8K on 8 ZigZag buckets,
  anchor 2048, query 128, passing 1024.  This is the headline 128K workload.
* ``c3``  same layer, 256K tokens as 32 virtual blocks of 8K on 16 buckets, anchor 2048,
  query 256, passing 1024.
* ``c4``  same layer, 128K tokens made of frames of UniformInt[196, 324] tokens, split by
  frame count over 16 virtual blocks (8 buckets), anchor 2048, query 128, passing 1024.

Reading of "H blocks of S": H names the work buckets (physical hosts in the method's
sequence-parallel layout), each holding a ZigZag pair of virtual blocks of S/2 tokens
(APB-V, gist.science summary, Metodologia section 1, context splitting and ZigZag
arrangement: host h pairs virtual hosts h and 2H-1-h).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

SEED_BASE = 20260129


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    description: str
    hq: int
    hkv: int
    head_dim: int
    n_blocks: int               # virtual blocks (sequence order)
    block_len: int              # uniform virtual-block length, 0 for frame-balanced blocks
    total_tokens: int           # N, context tokens (anchor and query block not counted)
    l_anchor: int
    l_query: int
    l_pass: int
    keys: str                   # "iid" or "frame"
    frame_len: int = 0          # fixed frame length for "frame" keys (0 = variable)
    frame_range: tuple = ()     # (lo, hi) inclusive frame-length range when variable
    input_dtype: str = "bf16"   # arithmetic inputs handed to the kernels are bf16 always
    seed: int = SEED_BASE

    @property
    def n_buckets(self) -> int:
        return (self.n_blocks + 1) // 2

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def uniform_block_starts(self) -> np.ndarray:
        assert self.block_len > 0
        return (np.arange(self.n_blocks + 1, dtype=np.int64) * self.block_len).astype(np.int32)


CONFIGS = {
    "c0": Workload("c0", "tiny fp32: 2/1 heads, d64, 2 x 256, anchor 64, query 32, l_p 32",
                   hq=2, hkv=1, head_dim=64, n_blocks=2, block_len=256, total_tokens=512,
                   l_anchor=64, l_query=32, l_pass=32, keys="iid", input_dtype="fp32",
                   seed=SEED_BASE + 0),
    "c1": Workload("c1", "28/4 heads, d128, 64K = 16 x 4K (8 buckets), anchor 1024, query 128, l_p 512",
                   hq=28, hkv=4, head_dim=128, n_blocks=16, block_len=4096, total_tokens=65536,
                   l_anchor=1024, l_query=128, l_pass=512, keys="frame", frame_len=256,
                   seed=SEED_BASE + 1),
    "c2": Workload("c2", "28/4 heads, d128, 128K = 16 x 8K (8 buckets), anchor 2048, query 128, l_p 1024",
                   hq=28, hkv=4, head_dim=128, n_blocks=16, block_len=8192, total_tokens=131072,
                   l_anchor=2048, l_query=128, l_pass=1024, keys="frame", frame_len=256,
                   seed=SEED_BASE + 2),
    "c3": Workload("c3", "28/4 heads, d128, 256K = 32 x 8K (16 buckets), anchor 2048, query 256, l_p 1024",
                   hq=28, hkv=4, head_dim=128, n_blocks=32, block_len=8192, total_tokens=262144,
                   l_anchor=2048, l_query=256, l_pass=1024, keys="frame", frame_len=256,
                   seed=SEED_BASE + 3),
    "c4": Workload("c4", "28/4 heads, d128, 128K of 196-324-token frames over 16 frame-balanced blocks, "
                         "anchor 2048, query 128, l_p 1024",
                   hq=28, hkv=4, head_dim=128, n_blocks=16, block_len=0, total_tokens=131072,
                   l_anchor=2048, l_query=128, l_pass=1024, keys="frame", frame_range=(196, 324),
                   seed=SEED_BASE + 4),
}


def workload(name: str, **overrides) -> Workload:
    """Return a named workload, optionally with fields replaced (for scaled-down test cases)."""
    w = CONFIGS[name]
    return dataclasses.replace(w, **overrides) if overrides else w


def sweep_layouts(w: Workload):
    """Layouts of the bucket-count sweep and the no-passing baseline over the same context as
    a fixed-frame workload (the pages evaluate 2, 4, 6 and 8 hosts, and name an anchor-only
    method without passing blocks among the baselines). Each entry is a dict with ``name``,
    ``block_starts`` (whole frames split evenly by count over 2H virtual blocks), ``l_anchor``
    and ``l_pass``."""
    from .gen import frame_partition
    assert w.keys == "frame" and w.frame_len > 0 and w.total_tokens % w.frame_len == 0
    frames = np.full(w.total_tokens // w.frame_len, w.frame_len, np.int64)
    out = []
    for h in (2, 4, 6, 8):
        out.append(dict(name=f"buckets_{h}", block_starts=frame_partition(frames, 2 * h),
                        l_anchor=w.l_anchor, l_pass=w.l_pass))
    out.append(dict(name="no_passing", block_starts=frame_partition(frames, w.n_blocks),
                    l_anchor=w.l_anchor, l_pass=0))
    return out

