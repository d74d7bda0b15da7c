"""The oracle's rows spread over a pool of CPU processes.

Test infrastructure (see the package docstring): never imported by the HIP path.

Rows are independent (every step of ``oracle.sampler`` works on one output row
at a time), so a batch can be split into chunks of rows, each chunk computed by
``oracle.sample`` / ``oracle.log_probs`` in a worker process exactly as it would
be in one process.  Nothing here does any of the method's arithmetic: the
parent only picks, for each chunk, the source rows its output rows read (so a
worker receives those rows alone) and rewrites the gather indices to point into
that smaller array.  Workers are started with the "spawn" method: fresh
interpreters that import numpy and this package only, so a parent that has
already initialised a GPU is never forked.
"""
from __future__ import annotations

import multiprocessing
import os
from concurrent.futures import ProcessPoolExecutor
from typing import List, Optional, Sequence

import numpy as np

from . import sampler

# A machine with one GPU per process typically gives a process about 16 host
# cores; more workers than that only compete for them.
MAX_WORKERS = 16


def host_cores() -> int:
    """Cores this process may run on."""
    return len(os.sched_getaffinity(0))


def default_workers() -> int:
    return max(1, min(MAX_WORKERS, host_cores()))


def _light(res: sampler.RowResult) -> sampler.RowResult:
    """Drop the per-entry arrays of an unflagged row (only the id and log-prob
    are compared there); flagged rows keep them for the alternative sets."""
    if res.flagged:
        return res
    return sampler.RowResult(res.token, res.logprob, None, None, None,
                             res.flag_sample, res.flag_topp,
                             [sampler.Outcome(o.token, o.logprob, None, None) for o in res.alternatives])


def _chunk_worker(kind, x_sub, n, params, gather_local, req, step_offset, no_top_k, no_top_p,
                  rows, token_ids, light):
    if kind == "sample":
        out = sampler.sample(x_sub, n, params, gather_indices=gather_local,
                             token_to_request_index=req, step_offset=step_offset,
                             no_top_k=no_top_k, no_top_p=no_top_p, rows=rows)
        return [_light(r) for r in out] if light else out
    return sampler.log_probs(x_sub, n, params, gather_indices=gather_local,
                             token_to_request_index=req, no_top_k=no_top_k, no_top_p=no_top_p,
                             token_ids=token_ids, rows=rows)


class Pool:
    """A process pool for the oracle; use as a context manager."""

    def __init__(self, workers: Optional[int] = None):
        self.workers = workers or default_workers()
        self._ex = ProcessPoolExecutor(max_workers=self.workers,
                                       mp_context=multiprocessing.get_context("spawn"))

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def close(self):
        self._ex.shutdown(wait=True)

    def warm(self):
        """Start every worker (interpreter start and imports) before anything is timed."""
        list(self._ex.map(_noop, range(self.workers * 2)))

    def run(self, kind: str, logits, n: int, params: dict, *, gather_indices=None,
            token_to_request_index=None, step_offset: int = 0, no_top_k: bool = False,
            no_top_p: bool = False, token_ids=None, rows: Optional[Sequence[int]] = None,
            light: bool = False, chunks_per_worker: int = 4):
        """``oracle.sample`` (kind "sample") or ``oracle.log_probs`` (kind
        "log_probs") over ``rows`` (default: all n), in row order."""
        logits = np.asarray(logits)
        rows = list(range(n)) if rows is None else [int(r) for r in rows]
        if not rows:
            return [] if kind == "sample" else np.zeros((0,))
        nchunks = max(1, min(len(rows), self.workers * chunks_per_worker))
        futs = []
        for part in np.array_split(np.asarray(rows), nchunks):
            part = part.tolist()
            src = [int(gather_indices[r]) if gather_indices is not None else r for r in part]
            uniq = sorted(set(src))
            where = {s: i for i, s in enumerate(uniq)}
            gather_local = np.full(n, -1, dtype=np.int64)
            for r, s in zip(part, src):
                gather_local[r] = where[s]
            futs.append(self._ex.submit(_chunk_worker, kind, logits[uniq], n, params, gather_local,
                                        token_to_request_index, step_offset, no_top_k, no_top_p,
                                        part, token_ids, light))
        outs = [f.result() for f in futs]
        if kind == "sample":
            return [r for o in outs for r in o]
        return np.concatenate(outs, axis=0)


def _noop(i):
    return i
