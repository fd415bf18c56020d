"""The oracle against its pins, and the pins against planted mistakes (CPU only)."""
from __future__ import annotations

import importlib.util
import os
import sys
import types

import numpy as np
import pytest

from oracle import apbv_oracle
import oracle_pins as pins  # noqa: E402  (tests/ is on sys.path under pytest)

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "apbv_oracle.py")


@pytest.mark.parametrize("pin", pins.PINS, ids=lambda f: f.__name__)
def test_pin_holds(pin):
    pin(apbv_oracle)


# A plausible mistake anywhere in the oracle must break at least one pin. Each mutation is a
# textual replacement in the oracle source; the mutated copy is loaded as its own module.
MUTATIONS = {
    "causal mask excludes the diagonal":
        ("local_pos[None, :] > (r - lo)[:, None]", "local_pos[None, :] >= (r - lo)[:, None]"),
    "block sees its own passing block":
        ("P = l_anchor + v * l_pass", "P = l_anchor + (v + 1) * l_pass"),
    "anchor dropped from the visible prefix":
        ("P = l_anchor + v * l_pass\n", "P = l_anchor + v * l_pass\n        kp = kp[:, l_anchor:]; vp = vp[:, l_anchor:]; P -= l_anchor\n"),
    "attention scale dropped":
        ("z = scale * (_as64(q_ctx[r, h, :]) @ keys.T)", "z = (_as64(q_ctx[r, h, :]) @ keys.T)"),
    "score softmax over the queries instead of the keys":
        ("s[g, lo:hi] += _softmax_rows(z).sum(axis=0)", "s[g, lo:hi] += _softmax_rows(z.T).sum(axis=1)"),
    "score scale dropped":
        ("z = scale * (q[:, h, :] @ k[:, g, :].T)", "z = (q[:, h, :] @ k[:, g, :].T)"),
    "ties go to the higher position":
        ('order = np.argsort(-s[g, lo:hi], kind="stable")',
         'order = (hi - lo - 1) - np.argsort(-s[g, lo:hi][::-1], kind="stable")'),
    "lowest scores selected":
        ('np.argsort(-s[g, lo:hi], kind="stable")', 'np.argsort(s[g, lo:hi], kind="stable")'),
    "interleaved head -> KV head map":
        ("return h // (hq // hkv)", "return h % hkv"),
    "lse without the log":
        ("lse[h, r] = (m + np.log(l))[:, 0]", "lse[h, r] = (m + l)[:, 0]"),
    "values gathered from the keys":
        ("v_parts = [va[:, g, :]] + [_as64(vc[sel[v, g], g, :]) for v in range(n)]",
         "v_parts = [va[:, g, :]] + [_as64(kc[sel[v, g], g, :]) for v in range(n)]"),
    "passing rows off by one":
        ("k_parts = [ka[:, g, :]] + [_as64(kc[sel[v, g], g, :]) for v in range(n)]",
         "k_parts = [ka[:, g, :]] + [_as64(kc[np.minimum(sel[v, g] + 1, kc.shape[0] - 1), g, :]) for v in range(n)]"),
    "softmax without normalisation":
        ("return e / np.sum(e, axis=-1, keepdims=True)", "return e"),
    "selection indices relative to the block":
        ("sel[v, g] = np.sort(order[:l_pass]) + lo", "sel[v, g] = np.sort(order[:l_pass])"),
    "query rows see the next query key":
        ("np.arange(n_q)[None, :] > rows[:, None]] = -np.inf",
         "np.arange(n_q)[None, :] > rows[:, None] + 1] = -np.inf"),
    "query rows ignore the anchor keys":
        ("keys = np.concatenate([_as64(k_anchor[:, g]),", "keys = np.concatenate([0 * _as64(k_anchor[:, g]),"),
    "query rows use the interleaved KV head":
        ("g = kv_head(h, hq, hkv)\n        keys = np.concatenate([_as64(k_anchor",
         "g = h % hkv\n        keys = np.concatenate([_as64(k_anchor"),
    "merge weights not normalised":
        ("wt = np.transpose(w / total[None], (0, 2, 1))", "wt = np.transpose(w, (0, 2, 1))"),
    "merged lse without the log":
        ("lse = top + np.log(total)", "lse = top + total"),
}


def _mutant(old: str, new: str) -> types.ModuleType:
    src = open(ORACLE_SRC).read()
    assert old in src, f"mutation anchor vanished from the oracle: {old!r}"
    mod = types.ModuleType("apbv_oracle_mutant")
    exec(compile(src.replace(old, new, 1), "apbv_oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    mod = _mutant(*MUTATIONS[name])
    caught = []
    for pin in pins.PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught the planted mistake: {name}"


def test_ambiguity_band():
    s = np.array([1.0, 0.5, 0.5 * (1 + 5e-6), 0.25, 0.5 * (1 - 2e-5)], np.float32)
    amb = apbv_oracle.ambiguous_positions(s, 2)
    assert amb.tolist() == [False, True, True, False, False]
    assert not apbv_oracle.ambiguous_positions(s, 5).any()
    assert not apbv_oracle.ambiguous_positions(s, 0).any()
