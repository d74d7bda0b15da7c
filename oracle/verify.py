"""Chain verification of speculative drafts against target samples (CPU oracle).

Test infrastructure (see the package docstring): never imported by the HIP path.

Page: the TokenSpeed Triton sampling backend source page, method ``verify`` of
``TritonSamplingBackend``.  It samples one target token per row of the
speculative layout (``num_tokens_per_req`` = 1 + S rows per request, request
``b`` owning rows b * N .. b * N + N - 1), then calls
``verify_chain_target_sampled(predicts, accept_index, accept_token_num,
candidates, target_sampled)`` with ``candidates`` of shape [bs, N], an
``accept_index`` of shape [bs, N] filled with -1 beforehand, and afterwards adds
one to ``accept_token_num``.  The page does not print that kernel's arithmetic.

Reading taken (parity unpinned: no page prints a value or the steps):

* ``candidates[b, 0]`` is the request's last verified token and
  ``candidates[b, 1:]`` its S drafts in chain order; ``target_sampled[b * N + i]``
  is the target model's sample after the chain prefix up to ``candidates[b, i]``.
* Draft i + 1 is accepted while every earlier draft was and
  ``candidates[b, i + 1] == target_sampled[b * N + i]`` (plain integer equality).
  ``accept_length[b]`` is the number of accepted drafts (0 .. S); the page's
  caller adds one for the token the target contributes after them.
* The emitted positions are i = 0 .. accept_length[b]: ``predicts[b * N + i] =
  target_sampled[b * N + i]`` (equal to the accepted draft where one was
  accepted, the target's own sample at the last one), and
  ``accept_index[b, i] = b * N + i``.  Every other position of ``predicts`` and
  ``accept_index`` is -1.
"""

from __future__ import annotations

import numpy as np


def verify_chain(candidates, target_sampled):
    """Returns (predicts [bs * N], accept_index [bs, N], accept_length [bs]),
    all int64, for candidates [bs, N] and target_sampled [bs * N]."""
    cand = np.asarray(candidates, dtype=np.int64)
    if cand.ndim != 2:
        raise ValueError("candidates must be [bs, N]")
    bs, n = cand.shape
    tgt = np.asarray(target_sampled, dtype=np.int64).reshape(-1)
    if tgt.shape[0] != bs * n:
        raise ValueError("target_sampled must hold bs * N entries")
    predicts = np.full(bs * n, -1, dtype=np.int64)
    accept_index = np.full((bs, n), -1, dtype=np.int64)
    accept_length = np.zeros(bs, dtype=np.int64)
    for b in range(bs):
        accepted = 0
        while accepted + 1 < n and cand[b, accepted + 1] == tgt[b * n + accepted]:
            accepted += 1
        accept_length[b] = accepted
        for i in range(accepted + 1):
            predicts[b * n + i] = tgt[b * n + i]
            accept_index[b, i] = b * n + i
    return predicts, accept_index, accept_length
