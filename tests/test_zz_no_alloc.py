"""The allocation-free scoring entry point (apbv_score_select_noalloc) against the workspace
entry point (apbv_score_select), through the C ABI (needs a GPU). Both run the same kernels,
so scores and selections must be bitwise equal; the calls follow one another on one device,
the later ones smaller, so that whatever an earlier call left in the shared scratch cannot
leak into a later result."""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

from gpu_util import layout_of, say, upload
from synthetic import generate, workload
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


def _cases():
    yield "128k", generate(workload("c2")), None
    bs = [0, 129, 300, 555, 700, 1000]
    yield "ragged", generate(dataclasses.replace(
        workload("c0"), name="ragged", keys="iid", hq=14, hkv=2, head_dim=128,
        total_tokens=1000, n_blocks=5, block_len=0, l_anchor=37, l_query=19, l_pass=21),
        block_starts=bs), bs
    yield "tiny", generate(workload("c0")), None


def test_noalloc_matches_the_workspace_entry_point():
    for name, x, bs in _cases():
        lay = layout_of(x, block_starts=bs)
        d = upload(x, ("q_query", "k_ctx"))
        ref_s, ref_sel = apbv.score_select(lay, d["q_query"], d["k_ctx"])
        # scores kept in the scratch (no score buffer), then scores written to the caller's
        _, sel_a = apbv.score_select_noalloc(lay, d["q_query"], d["k_ctx"], want_scores=False)
        s_b, sel_b = apbv.score_select_noalloc(lay, d["q_query"], d["k_ctx"])
        torch.cuda.synchronize()
        assert torch.equal(sel_a, ref_sel), name
        assert torch.equal(sel_b, ref_sel), name
        assert torch.equal(s_b, ref_s), name
        # and the selection rule holds exactly on those scores
        own = orc.select_passing(s_b.cpu().numpy(), lay.block_starts, lay.l_pass)
        assert np.array_equal(own, sel_b.cpu().numpy()), name
        say(f"  {name}: N={lay.n_tokens} blocks={lay.n_blocks}: no-alloc scores and selection "
            f"bitwise equal to the workspace entry point")


def test_noalloc_rejects_layouts_beyond_its_scratch():
    x = generate(workload("c0"))
    big = apbv.Layout(list(range(0, 64 * 2048 + 1, 2048)), l_anchor=0, l_query=2000,
                      l_pass=16, hq=64, hkv=8, head_dim=128)
    q = torch.zeros((2000, 64, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((64 * 2048, 8, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(apbv.ApbvError) as e:
        apbv.score_select_noalloc(big, q, k)
    assert e.value.status == 2 and "scratch" in str(e.value)
