"""Plain fp64 CPU oracle for batched categorical token sampling.

This package is test infrastructure.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The HIP library in
``token_sampling_scaled_amd`` never imports it, calls it or shares code with it:
the two are independent implementations of the same definition, and the tests
compare them element by element.

What it follows (page titles as printed at the top of each page):

* "core.inference.sampling.base" (Megatron-Core API docs), class ``Sampling``:
  ``sample_kernel`` (rows selected by ``gather_indices``, parameters gathered per
  token by ``token_to_request_index``) and ``sample_speculative`` (decode
  requests contribute 1 + num_speculative_tokens rows, prefill requests 1).
* "core.inference.sampling.flashinfer_sampling" (Megatron-Core API docs), class
  ``FlashInferSampling``: top-k / top-p / joint filtering, seeded Philox noise
  that advances per step, and ``log_probs_kernel`` (log-probs of the processed
  distribution).
* the TokenSpeed Triton sampling backend source page
  (``runtime/sampling/backends/triton.py``): per-request seed pools, Gumbel-max
  sampling, the "top-p disabled when p is within eps of 1" test, and the
  vocabulary mask applied before sampling (``oracle/vocab_mask.py``).

Every floating-point step is fp64.  Where the pages leave a step open, the
reading taken is stated in the docstring of the function that takes it.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
something other than itself (two independent Philox libraries, brute-force
enumeration on tiny vocabularies, closed forms, chi-square frequency tests,
scipy's log_softmax), except ``verify_chain`` (``oracle/verify.py``): the page
names that step and its outputs but prints neither its arithmetic nor a value,
so it is "parity unpinned" -- pinned only to hand-worked cases of the reading
stated there and to invariants.
"""

from .philox import philox4x32_10, noise_words, uniform_from_words, gumbel_from_uniform
from .sampler import (
    RowParams,
    RowResult,
    order_key_sort,
    top_k_mask,
    top_p_mask,
    process_row,
    sample_row,
    sample,
    raw_log_probs_at,
    log_probs,
    build_spec_map,
    GREEDY_T_MAX,
    TOP_P_EPS,
    NEAR_TIE_REL,
)
from .verify import verify_chain
from .vocab_mask import apply_vocab_mask

__all__ = [
    "philox4x32_10", "noise_words", "uniform_from_words", "gumbel_from_uniform",
    "RowParams", "RowResult", "order_key_sort", "top_k_mask", "top_p_mask",
    "process_row", "sample_row", "sample", "raw_log_probs_at", "log_probs", "build_spec_map",
    "GREEDY_T_MAX", "TOP_P_EPS", "NEAR_TIE_REL", "verify_chain", "apply_vocab_mask",
]
