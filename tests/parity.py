"""Helpers that run the HIP sampler and compare it with the oracle."""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

import oracle
import token_sampling_scaled_amd as tsa

LP_ATOL = 1e-4


def to_device(wl, device="cuda"):
    """Device copies of a synth.Workload's tensors."""
    d = {
        "logits": wl.logits.to(device),
        "params": tsa.SamplingParams(
            temperature=wl.temperature.to(device), seed=wl.seed.to(device),
            top_k=wl.top_k.to(device), top_p=wl.top_p.to(device),
            step_offsets=None if wl.step_offsets is None else wl.step_offsets.to(device)),
        "gather": None if wl.gather_indices is None else wl.gather_indices.to(device),
        "req": None if wl.token_to_request_index is None else wl.token_to_request_index.to(device),
    }
    return d


def gpu_sample(wl, sampler=None, dev=None, step_offset=None):
    dev = dev or to_device(wl)
    s = sampler or tsa.Sampler(wl.vocab, max(wl.n, 1))
    ids, lp = s.sample(dev["logits"], wl.n, dev["params"], no_top_k=wl.no_top_k,
                       no_top_p=wl.no_top_p, gather_indices=dev["gather"],
                       token_to_request_index=dev["req"],
                       step_offset=wl.step_offset if step_offset is None else step_offset,
                       return_logprobs=True)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), lp.cpu().numpy()


def gpu_log_probs(wl, sampler=None, dev=None, token_ids=None):
    dev = dev or to_device(wl)
    s = sampler or tsa.Sampler(wl.vocab, max(wl.n, 1))
    out = s.log_probs(dev["logits"], dev["params"], n=wl.n, no_top_k=wl.no_top_k,
                      no_top_p=wl.no_top_p, gather_indices=dev["gather"],
                      token_to_request_index=dev["req"],
                      token_ids=None if token_ids is None else token_ids.to(dev["logits"].device))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_sample(wl, rows: Optional[Sequence[int]] = None, step_offset=None):
    return oracle.sample(
        wl.logits_f64(), wl.n, wl.params_numpy(),
        gather_indices=None if wl.gather_indices is None else wl.gather_indices.numpy(),
        token_to_request_index=None if wl.token_to_request_index is None
        else wl.token_to_request_index.numpy(),
        step_offset=wl.step_offset if step_offset is None else step_offset,
        no_top_k=wl.no_top_k, no_top_p=wl.no_top_p, rows=rows)


def oracle_log_probs(wl, rows: Optional[Sequence[int]] = None):
    return oracle.log_probs(
        wl.logits_f64(), wl.n, wl.params_numpy(),
        gather_indices=None if wl.gather_indices is None else wl.gather_indices.numpy(),
        token_to_request_index=None if wl.token_to_request_index is None
        else wl.token_to_request_index.numpy(),
        no_top_k=wl.no_top_k, no_top_p=wl.no_top_p, rows=rows)


def _oracle_kwargs(wl, step_offset=None):
    return dict(gather_indices=None if wl.gather_indices is None else wl.gather_indices.numpy(),
                token_to_request_index=None if wl.token_to_request_index is None
                else wl.token_to_request_index.numpy(),
                no_top_k=wl.no_top_k, no_top_p=wl.no_top_p)


def oracle_sample_pool(pool, wl, rows: Optional[Sequence[int]] = None, step_offset=None,
                       light: bool = True):
    """oracle.sample over a process pool (oracle.parallel.Pool)."""
    return pool.run("sample", wl.logits_f64(), wl.n, wl.params_numpy(), rows=rows,
                    step_offset=wl.step_offset if step_offset is None else step_offset,
                    light=light, **_oracle_kwargs(wl))


def oracle_log_probs_pool(pool, wl, rows: Optional[Sequence[int]] = None):
    """oracle.log_probs (full rows) over a process pool."""
    return pool.run("log_probs", wl.logits_f64(), wl.n, wl.params_numpy(), rows=rows,
                    **_oracle_kwargs(wl))


def _lp_close(a: float, b: float) -> bool:
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return abs(a - b) <= LP_ATOL


# Every checked report, in order; tests/conftest.py prints them as JSON lines
# at the end of the session (they survive ``pytest -q``).
RECORDS: List[dict] = []


@dataclass
class Report:
    rows: int = 0
    flagged: int = 0            # rows the oracle flags as near ties
    diverged_flagged: int = 0   # flagged rows where the GPU took an admissible alternative
    mismatches: List[str] = field(default_factory=list)

    def record(self, label: str) -> dict:
        return {"case": label, "rows": self.rows, "flagged": self.flagged,
                "took_alternative": self.diverged_flagged, "mismatches": len(self.mismatches)}

    def check(self, label: Optional[str] = None):
        print(f"[parity] rows={self.rows} flagged={self.flagged} "
              f"took_alternative={self.diverged_flagged} mismatches={len(self.mismatches)}",
              flush=True)
        if label is not None:
            RECORDS.append(self.record(label))
        assert not self.mismatches, "\n".join(self.mismatches[:20])


def compare_samples(ids, lps, results, rows: Optional[Sequence[int]] = None) -> Report:
    rep = Report()
    rows = list(range(len(results))) if rows is None else list(rows)
    for res, r in zip(results, rows):
        rep.rows += 1
        gid, glp = int(ids[r]), float(lps[r])
        rep.flagged += int(res.flagged)
        if gid == res.token and _lp_close(glp, res.logprob):
            continue
        if res.flagged and any(o.token == gid and _lp_close(glp, o.logprob) for o in res.alternatives):
            rep.diverged_flagged += 1
            continue
        rep.mismatches.append(f"row {r}: gpu ({gid}, {glp:.6f}) oracle ({res.token}, "
                              f"{res.logprob:.6f}) flagged={res.flagged}")
    return rep


def compare_log_probs(gpu, ref, results=None, rows: Optional[Sequence[int]] = None) -> Report:
    """Full-row log-probs: identical -inf pattern (exact sets) and values within LP_ATOL.
    Rows the oracle flags for a top-p near tie may differ by the boundary tie group."""
    rep = Report()
    rows = list(range(ref.shape[0])) if rows is None else list(rows)
    for i, r in enumerate(rows):
        rep.rows += 1
        g, o = gpu[r], ref[i]
        if np.all(np.isnan(o)):
            if not np.all(np.isnan(g)):
                rep.mismatches.append(f"row {r}: expected NaN row")
            continue
        same_set = np.array_equal(np.isneginf(g), np.isneginf(o))
        fin = ~np.isneginf(o)
        if same_set and np.all(np.abs(g[fin] - o[fin]) <= LP_ATOL):
            continue
        res = results[i] if results is not None else None
        if res is not None and res.flag_topp:
            # a top-p near tie: the GPU may keep the other side of the boundary
            # group, and then its row must be that set's log-probs
            rep.flagged += 1
            ok = False
            for alt in res.alternatives:
                if alt.lp_row is None or not np.array_equal(~np.isneginf(g), alt.keep):
                    continue
                if np.all(np.abs(g[alt.keep] - alt.lp_row[alt.keep]) <= LP_ATOL):
                    ok = True
            if ok:
                rep.diverged_flagged += 1
                continue
        bad = np.nonzero(np.isneginf(g) != np.isneginf(o))[0][:5]
        err = float(np.max(np.abs(np.where(fin & ~np.isneginf(g), g - o, 0.0))))
        rep.mismatches.append(f"row {r}: set_equal={same_set} first_diff={bad.tolist()} max_err={err:.3g}")
    return rep
