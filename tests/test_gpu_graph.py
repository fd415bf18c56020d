"""One layer replayed from a HIP graph (needs a GPU).

The allocation-free scoring entry point exists for callers that cannot allocate, such as code
under graph capture. Here the whole layer runs through it: scoring and selection in the
library's scratch, then the gather and the attention into preallocated buffers. The layer is
captured once through torch and replayed on several input sets. Each set is copied into the
captured input buffers by ordinary eager work between replays, and every replay must equal,
bit for bit, the same layer run eagerly on that set. No call in the captured region allocates
or clears memory.
"""
from __future__ import annotations

import dataclasses

import pytest
import torch

from gpu_util import dev_bf16, layout_of, say
from synthetic import generate, workload
import sequence_approximate_attention_score_amd as apbv

pytestmark = pytest.mark.gpu

NAMES = ("q_query", "q_ctx", "k_ctx", "v_ctx", "k_anchor", "v_anchor")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    apbv.lib()
    yield
    torch.cuda.synchronize()


def inputs(seed):
    bs = [0, 700, 1500, 2304, 3000, 4096]
    w = dataclasses.replace(workload("c0"), name=f"graph{seed}", keys="iid", hq=14, hkv=2,
                            head_dim=128, total_tokens=bs[-1], n_blocks=len(bs) - 1,
                            block_len=0, l_anchor=96, l_query=40, l_pass=160,
                            seed=1000 + seed)
    return generate(w, block_starts=bs)


class Buffers:
    def __init__(self, lay, dev):
        d = lay.head_dim
        self.sel = torch.empty((lay.n_blocks, lay.hkv, lay.l_pass), dtype=torch.int32,
                               device=dev)
        self.kp = torch.empty((lay.hkv, lay.pre_rows, d), dtype=torch.bfloat16, device=dev)
        self.vp = torch.empty_like(self.kp)
        self.out = torch.empty((lay.n_tokens, lay.hq, d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((lay.hq, lay.n_tokens), dtype=torch.float32, device=dev)


def layer(lay, d, b):
    apbv.score_select_noalloc(lay, d["q_query"], d["k_ctx"], sel=b.sel, want_scores=False)
    apbv.gather_passing(lay, d["k_anchor"], d["v_anchor"], d["k_ctx"], d["v_ctx"], b.sel,
                        k_pre=b.kp, v_pre=b.vp)
    apbv.approx_attn_prefill(lay, d["q_ctx"], b.kp, b.vp, d["k_ctx"], d["v_ctx"], out=b.out,
                             lse=b.lse)


def test_layer_replays_from_a_hip_graph():
    x0 = inputs(0)
    lay = layout_of(x0)
    dev = torch.device("cuda:0")
    static = {n: dev_bf16(x0.bits[n]) for n in NAMES}
    captured = Buffers(lay, dev)
    # warm-up on a side stream (first calls look up the scratch address), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer(lay, static, captured)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer(lay, static, captured)
    torch.cuda.synchronize()

    eager = Buffers(lay, dev)
    for seed in (1, 2, 0, 3):
        x = inputs(seed)
        fresh = {n: dev_bf16(x.bits[n]) for n in NAMES}
        for n in NAMES:
            static[n].copy_(fresh[n])
        captured.out.fill_(7.0)            # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        layer(lay, fresh, eager)           # the same layer, eager, other buffers
        torch.cuda.synchronize()
        for k in ("sel", "kp", "vp", "out", "lse"):
            assert torch.equal(getattr(captured, k), getattr(eager, k)), (seed, k)
        assert bool(torch.isfinite(captured.out.float()).all())
        say(f"  replay on input set {seed}: selection, prefix, output and lse equal to eager")
    # the replays really computed new results: two input sets give different selections
    sels = []
    for seed in (1, 2):
        x = inputs(seed)
        for n in NAMES:
            static[n].copy_(dev_bf16(x.bits[n]))
        graph.replay()
        torch.cuda.synchronize()
        sels.append(captured.sel.clone())
    assert not torch.equal(sels[0], sels[1])
