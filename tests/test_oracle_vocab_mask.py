"""Pins of the vocabulary-mask oracle (oracle/vocab_mask.py) against a
hand-worked fixture, the trivial masks, and the sampling steps downstream."""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "vocab_mask.json")


def _fixture():
    with open(GOLDEN) as f:
        g = json.load(f)
    v = g["vocab"]
    words = np.array([[int(w, 16) for w in m["words"]] for m in g["masks"]], dtype=np.int64)
    allowed = [list(range(v)) if m["allowed"] == "all" else m["allowed"] for m in g["masks"]]
    return g, v, words, allowed


def test_hand_worked_masks():
    g, v, words, allowed = _fixture()
    x = np.arange(len(words) * v, dtype=np.float64).reshape(len(words), v) * 0.25 - 3.0
    out = oracle.apply_vocab_mask(x, words)
    for r, keep in enumerate(allowed):
        finite = np.flatnonzero(np.isfinite(out[r])).tolist()
        assert finite == keep, r
        assert np.all(out[r, keep] == x[r, keep])          # allowed entries unchanged
        assert np.all(out[r][~np.isin(np.arange(v), keep)] == -np.inf)


def test_mask_index_shares_rows():
    g, v, words, allowed = _fixture()
    case = g["mask_index_case"]
    x = np.ones((3, v))
    out = oracle.apply_vocab_mask(x, words, mask_index=case["mask_index"])
    for r, want in enumerate(case["allowed_rows"]):
        keep = allowed[0] if want == "mask0" else want
        assert np.flatnonzero(np.isfinite(out[r])).tolist() == keep


def test_trivial_masks_and_no_aliasing():
    rng = np.random.default_rng(3)
    x = rng.normal(size=(4, 100))
    ones = np.full((4, 4), 0xFFFFFFFF, dtype=np.int64)
    zeros = np.zeros((4, 4), dtype=np.int64)
    assert np.array_equal(oracle.apply_vocab_mask(x, ones), x)
    assert np.all(oracle.apply_vocab_mask(x, zeros) == -np.inf)
    y = x.copy()
    oracle.apply_vocab_mask(x, zeros)
    assert np.array_equal(x, y)                              # a copy, not in place


@pytest.mark.parametrize("k,p,t", [(0, 1.0, 1.0), (5, 1.0, 0.7), (0, 0.5, 1.3), (3, 0.2, 0.9)])
def test_single_allowed_entry_is_always_sampled(k, p, t):
    # with one allowed entry, P = {that entry} under every filter: the sample is
    # that entry and its log-prob is 0, whatever the seed
    rng = np.random.default_rng(11)
    v = 300
    x = rng.normal(size=(6, v)) * 3
    words = np.zeros((6, (v + 31) // 32), dtype=np.int64)
    keep = rng.integers(0, v, size=6)
    for r, j in enumerate(keep):
        words[r, j // 32] |= 1 << (j % 32)
    xm = oracle.apply_vocab_mask(x, words)
    params = {"temperature": np.full(6, t), "top_k": np.full(6, k, dtype=np.int64),
              "top_p": np.full(6, p), "seed": np.arange(6, dtype=np.int64) * 7 + 1}
    res = oracle.sample(xm, 6, params, step_offset=5)
    for r in range(6):
        assert res[r].token == keep[r]
        assert res[r].logprob == 0.0
