"""CPU oracle of the approximate-attention prefill (float64 numpy).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; never by the library or its binding.
"""
from . import apbv_oracle
from .apbv_oracle import (ambiguous_positions, approx_attention_prefill, attend, gather_prefix,
                          kv_head, merge_partials, passing_scores, query_attention,
                          select_passing)

__all__ = ["apbv_oracle", "ambiguous_positions", "approx_attention_prefill", "attend",
           "gather_prefix", "kv_head", "merge_partials", "passing_scores", "query_attention",
           "select_passing"]
