"""Vocabulary mask applied to logits (CPU oracle).

Test infrastructure (see the package docstring): never imported by the HIP path.

Page: the TokenSpeed Triton sampling backend source page, methods ``sample``
and ``verify`` of ``TritonSamplingBackend``: after the NaN guard and before
the greedy argmax or any Gumbel kernel, the logits pass through
``apply_vocab_mask(logits, vocab_mask)`` whenever the batch carries a mask.
The page prints neither the mask's layout nor that function's body.

Reading taken: the mask of a row is a packed bit set of 32-bit words, bit
(j mod 32) of word j // 32 standing for vocabulary entry j; a set bit allows the
entry, a clear bit sets its logit to -inf, so that no later step can select
it.  Rows may share a mask through ``mask_index`` (mask row ``mask_index[r]``
for logits row r).  Entries at or past the vocabulary size are never touched.

Pins: ``tests/test_oracle_vocab_mask.py`` checks this against a hand-worked
fixture (``tests/golden/vocab_mask.json``), the all-set and all-clear masks,
and the sampling steps downstream: a row left with one allowed entry samples
it with log-prob 0 under every filter.
"""

from __future__ import annotations

import numpy as np


def entry_allowed(words, j: int) -> bool:
    """Whether vocabulary entry j is allowed by one row's mask words."""
    return (int(words[j // 32]) >> (j % 32)) & 1 == 1


def apply_vocab_mask(logits, mask_words, mask_index=None) -> np.ndarray:
    """A fp64 copy of ``logits`` [rows, V] with every entry whose mask bit is clear
    set to -inf.  ``mask_words``: integer array [mask rows, >= ceil(V / 32)] (only
    the low 32 bits of each word count)."""
    x = np.array(logits, dtype=np.float64, copy=True)
    words = np.asarray(mask_words, dtype=np.int64) & 0xFFFFFFFF
    rows, v = x.shape
    for r in range(rows):
        m = r if mask_index is None else int(mask_index[r])
        row_words = words[m]
        for j in range(v):
            if not entry_allowed(row_words, j):
                x[r, j] = -np.inf
    return x
