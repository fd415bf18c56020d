"""MI355X (gfx950) approximate-attention prefill of APB-V / Spava.

The hot path is three C-ABI calls backed by hand-written HIP kernels (``libapbv.so``):
``score_select`` (query-to-context scores + per-KV-head top-l_p passing selection),
``gather_passing`` (anchor + passing blocks into one prefix per KV head) and
``approx_attn_prefill`` (bf16 MFMA attention over [anchor | passing | causal local] with a
ZigZag work schedule), ``prefill_layer`` (the three in one call, optionally with the
selection of later blocks on a second stream beside the attention), plus ``query_forward``
for the rows of the query block (exact attention over the whole sequence, partial results
merged through their lse), and ``layer_forward`` (every row of a layer in one call: anchor
rows, context rows, query rows). This package is the thin Python binding over that library.
"""
from ._lib import (ApbvError, Layout, approx_attn_prefill, attn_tile_rows, gather_passing,
                   layer_forward, layer_workspace, lib, num_buckets, prefill_layer,
                   prefill_layer_plan, query_forward, query_forward_workspace, schedule, score_select, score_select_noalloc,
                   score_select_workspace, version)

__all__ = ["ApbvError", "Layout", "approx_attn_prefill", "attn_tile_rows", "gather_passing",
           "layer_forward", "layer_workspace", "lib", "num_buckets", "prefill_layer",
           "prefill_layer_plan", "query_forward", "query_forward_workspace", "schedule",
           "score_select", "score_select_noalloc", "score_select_workspace", "version",
           "run_layer"]


def run_layer(layout: Layout, q_query, q_ctx, k_ctx, v_ctx, k_anchor, v_anchor, *, workspace=None,
              want_lse: bool = False):
    """One layer of the hot path: score_select -> gather_passing -> approx_attn_prefill."""
    _, sel = score_select(layout, q_query, k_ctx, workspace=workspace, want_scores=False)
    k_pre, v_pre = gather_passing(layout, k_anchor, v_anchor, k_ctx, v_ctx, sel)
    out, lse = approx_attn_prefill(layout, q_ctx, k_pre, v_pre, k_ctx, v_ctx, want_lse=want_lse)
    return out, lse, sel
