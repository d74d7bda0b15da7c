"""fp64 reference for one sampling step: filters, Gumbel-max draw, log-probs.

Test infrastructure (see the package docstring): never imported by the HIP path.

Per output row r (all arithmetic in fp64, one row at a time, no blocking):

1. Row and parameters.  The source row is ``gather_indices[r]`` when given,
   else r ("core.inference.sampling.base", ``sample_kernel``, parameter
   ``gather_indices``: sample only from ``logits[gather_indices[:n], :]``).  The
   parameter slot is ``token_to_request_index[r]`` when given, else r (same page,
   parameter ``token_to_request_index``: parameters gathered per token).
2. NaN logits are read as -inf and -0 as +0 (reading: the TokenSpeed page names
   a NaN guard without printing it; -inf keeps a NaN out of every filtered set).
3. Top-k ("core.inference.sampling.flashinfer_sampling": exact top-k kernel).
   Reading: k is active when 1 <= k < V; K is the first min(k, #finite) indices
   in the order (x descending, index ascending) on the raw logits.  Temperature
   is a positive scale, so it cannot change this set.
4. Temperature: s = x / T.  Reading: a temperature below GREEDY_T_MAX means
   greedy (the TokenSpeed page routes all-greedy batches to an argmax); the
   greedy pick is the first index in the order of step 3 and its log-prob is 0
   (a point mass).  Parameters arrive as fp32 values, and both thresholds
   (GREEDY_T_MAX here, 1 - TOP_P_EPS in step 5) are compared in fp32: a row is
   greedy unless fp32(T) >= fp32(1e-5), and top-p is on only when
   fp32(p) < fp32(1) - fp32(1e-6) (an fp32 subtraction), so a parameter that
   equals a threshold falls on the same side for every implementation.
5. Top-p on the top-k distribution (joint filtering, top-k first; reading of
   "top-k / top-p sampling distribution" in ``log_probs_kernel``).  With
   pi = softmax(s) over K, index j is kept when the mass of the members of K
   whose logit is strictly larger than x_j is below p.  Equal logits are kept or
   dropped together.  p >= 1 - TOP_P_EPS disables the filter (the TokenSpeed
   page's "|p - 1| <= eps" test; eps is not printed, 1e-6 is the reading); the
   top tie group is always kept, so p <= 0 keeps exactly that group.
6. Noise: g_j from ``oracle.philox`` keyed on (seed, r, j, step offset).
7. Sample: j* = argmax over P of s_j + g_j, smallest j on exact ties
   (Gumbel-max; every TokenSpeed kernel is a ``gumbel_sample_*`` kernel).
8. Log-prob of the processed distribution ("flashinfer_sampling",
   ``log_probs_kernel``): lp_j = s_j - logsumexp_P(s) for j in P, -inf elsewhere.

Near ties (``NEAR_TIE_REL``): when the two best perturbed scores differ by at
most 1e-5 * max(1, |z1|, |z2|), or a kept/dropped tie group's cumulative mass
is within 1e-5 * p of p, an fp32 implementation may take the other branch.
Such rows are flagged, and every alternative outcome is listed, so a test can
accept it while counting it.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

from .philox import noise_words, uniform_from_words, gumbel_from_uniform

GREEDY_T_MAX = 1e-5
TOP_P_EPS = 1e-6
NEAR_TIE_REL = 1e-5


@dataclass
class RowParams:
    temperature: float
    top_k: int
    top_p: float
    seed: int


@dataclass
class Outcome:
    """One admissible result of a row: the sampled id, its log-prob and the kept set P."""
    token: int
    logprob: float
    keep: np.ndarray  # bool [V], the set P this outcome samples from
    # float64 [V]: log-probs of the processed distribution over ``keep`` (set for
    # the alternatives of a top-p near tie, whose kept set differs from the row's)
    lp_row: Optional[np.ndarray] = None


@dataclass
class RowResult:
    token: int
    logprob: float
    keep: np.ndarray                      # bool [V]: the kept set P
    topk: np.ndarray                      # bool [V]: the top-k set K (all finite when inactive)
    lp_row: np.ndarray                    # float64 [V]: log-probs of the processed distribution
    flag_sample: bool = False             # perturbed-score near tie
    flag_topp: bool = False               # top-p cumulative-mass near tie
    alternatives: List[Outcome] = field(default_factory=list)

    @property
    def flagged(self) -> bool:
        return self.flag_sample or self.flag_topp


def is_greedy(t: float) -> bool:
    """Greedy unless fp32(t) >= fp32(GREEDY_T_MAX) (a NaN temperature is greedy too)."""
    return not (np.float32(t) >= np.float32(GREEDY_T_MAX))


def top_p_active(p: float) -> bool:
    """Top-p filters only when fp32(p) < fp32(1) - fp32(TOP_P_EPS), evaluated in fp32."""
    return bool(np.float32(p) < np.float32(1.0) - np.float32(TOP_P_EPS))


def canonical_logits(x) -> np.ndarray:
    """fp64 copy with NaN -> -inf and -0 -> +0."""
    x = np.array(x, dtype=np.float64, copy=True)
    x[np.isnan(x)] = -np.inf
    return x + 0.0


def order_key_sort(x: np.ndarray) -> np.ndarray:
    """Indices of x in the order (value descending, index ascending)."""
    j = np.arange(x.size)
    return np.lexsort((j, -x))


def top_k_mask(x: np.ndarray, k: int) -> np.ndarray:
    """K: the first min(k, #finite) indices in the order, or all finite when k is inactive."""
    finite = x > -np.inf
    v = x.size
    if not (1 <= k < v):
        return finite
    take = min(int(k), int(finite.sum()))
    keep = np.zeros(v, dtype=bool)
    keep[order_key_sort(x)[:take]] = True
    return keep


def _tie_groups(x: np.ndarray, members: np.ndarray):
    """Members of a set grouped by equal logit, groups in descending logit order."""
    idx = np.nonzero(members)[0]
    vals = x[idx]
    order = np.argsort(-vals, kind="stable")
    idx, vals = idx[order], vals[order]
    starts = np.concatenate(([0], np.nonzero(np.diff(vals) != 0)[0] + 1, [idx.size]))
    return [idx[starts[g]:starts[g + 1]] for g in range(starts.size - 1)]


def top_p_mask(x: np.ndarray, s: np.ndarray, topk: np.ndarray, p: float):
    """P inside K, plus the cumulative masses that decided it.

    Returns (keep, groups, cum) where groups are K's tie groups in descending
    logit order and cum[g] is the normalised mass of groups 0..g.  The number of
    kept groups is the count of g with cum[g-1] < p (cum[-1] = 0), at least 1.
    """
    groups = _tie_groups(x, topk)
    if not groups:
        return np.zeros_like(topk), groups, np.zeros(0), 0
    m = np.max(s[topk])
    w = np.exp(s - m)
    z = np.sum(w[topk])
    cum = np.cumsum([np.sum(w[g]) for g in groups]) / z
    if not top_p_active(p):
        kept = len(groups)
    else:
        before = np.concatenate(([0.0], cum[:-1]))
        kept = max(1, int(np.sum(before < p)))
    keep = np.zeros_like(topk)
    for g in groups[:kept]:
        keep[g] = True
    return keep, groups, cum, kept


def _lp_row(s: np.ndarray, keep: np.ndarray) -> np.ndarray:
    out = np.full(s.size, -np.inf)
    if keep.any():
        m = np.max(s[keep])
        out[keep] = s[keep] - m - np.log(np.sum(np.exp(s[keep] - m)))
    return out


def _draw(s: np.ndarray, keep: np.ndarray, seed: int, r: int, step_offset: int):
    """argmax over the kept set of s + g (smallest index on exact ties) and all near-tie ids."""
    j = np.nonzero(keep)[0]
    g = gumbel_from_uniform(uniform_from_words(noise_words(seed, r, step_offset, j)))
    z = s[j] + g
    best = int(np.argmax(z))                          # first maximum = smallest index
    z1 = z[best]
    band = NEAR_TIE_REL * np.maximum(np.maximum(1.0, abs(z1)), np.abs(z))
    near = j[(z1 - z <= band)]
    return int(j[best]), near


def process_row(x, params: RowParams, use_top_k: bool = True, use_top_p: bool = True):
    """Steps 2-5 and 8 for one row: (x, s, K, P, groups, cum, kept, lp_row, greedy)."""
    x = canonical_logits(x)
    v = x.size
    k = int(params.top_k) if use_top_k else 0
    p = float(params.top_p) if use_top_p else 1.0
    t = float(params.temperature)
    topk = top_k_mask(x, k)
    if not topk.any():
        return dict(x=x, s=None, topk=topk, keep=topk, groups=[], cum=np.zeros(0), kept=0,
                    lp_row=np.full(v, np.nan), greedy=False)
    if is_greedy(t):
        keep = np.zeros(v, dtype=bool)
        keep[order_key_sort(x)[0]] = True
        lp_row = np.where(keep, 0.0, -np.inf)
        return dict(x=x, s=None, topk=topk, keep=keep, groups=[], cum=np.zeros(0), kept=1,
                    lp_row=lp_row, greedy=True)
    s = x / t
    keep, groups, cum, kept = top_p_mask(x, s, topk, p)
    return dict(x=x, s=s, topk=topk, keep=keep, groups=groups, cum=cum, kept=kept,
                lp_row=_lp_row(s, keep), greedy=False)


def sample_row(x, params: RowParams, r: int, step_offset: int = 0,
               use_top_k: bool = True, use_top_p: bool = True) -> RowResult:
    """Steps 1-8 for one already-selected row ``x`` sampled as output row ``r``."""
    d = process_row(x, params, use_top_k, use_top_p)
    keep, lp_row = d["keep"], d["lp_row"]
    if not keep.any():
        return RowResult(-1, float("nan"), keep, d["topk"], lp_row)
    if d["greedy"]:
        tok = int(np.nonzero(keep)[0][0])
        return RowResult(tok, 0.0, keep, d["topk"], lp_row)
    s = d["s"]
    tok, near = _draw(s, keep, params.seed, r, step_offset)
    res = RowResult(tok, float(lp_row[tok]), keep, d["topk"], lp_row)
    res.flag_sample = near.size > 1
    for alt in near:
        res.alternatives.append(Outcome(int(alt), float(lp_row[alt]), keep))
    # Top-p near ties: the last kept group may be dropped, or the next one kept.
    p = float(params.top_p) if use_top_p else 1.0
    groups, cum, kept = d["groups"], d["cum"], d["kept"]
    if top_p_active(p) and groups:
        alt_sets = []
        if kept >= 2 and abs(cum[kept - 2] - p) <= NEAR_TIE_REL * p:
            a = keep.copy()
            a[groups[kept - 1]] = False
            alt_sets.append(a)
        if kept < len(groups) and abs(cum[kept - 1] - p) <= NEAR_TIE_REL * p:
            a = keep.copy()
            a[groups[kept]] = True
            alt_sets.append(a)
        for a in alt_sets:
            res.flag_topp = True
            lp_a = _lp_row(s, a)
            t_a, near_a = _draw(s, a, params.seed, r, step_offset)
            for alt in near_a:
                res.alternatives.append(Outcome(int(alt), float(lp_a[alt]), a, lp_a))
    return res


def _row_params(r, params, token_to_request_index):
    q = int(token_to_request_index[r]) if token_to_request_index is not None else r
    return RowParams(float(params["temperature"][q]),
                     int(params["top_k"][q]) if params.get("top_k") is not None else 0,
                     float(params["top_p"][q]) if params.get("top_p") is not None else 1.0,
                     int(params["seed"][q]))


def sample(logits, n: int, params: dict, *, gather_indices=None, token_to_request_index=None,
           step_offset: int = 0, no_top_k: bool = False, no_top_p: bool = False,
           rows: Optional[Sequence[int]] = None) -> List[RowResult]:
    """One sampling step over n output rows (or the listed subset ``rows``).

    ``logits`` is a 2-D array [rows_in_buffer, V]; ``params`` maps
    temperature / top_k / top_p / seed (and optionally step_offsets, a
    per-request offset pool added to ``step_offset``) to per-request arrays.
    ``no_top_k`` and ``no_top_p`` are the batch-level promises of
    "flashinfer_sampling" ``sample_kernel``: when set, that filter is off for
    every row.
    """
    logits = np.asarray(logits)
    offsets = params.get("step_offsets")
    out = []
    for r in (range(n) if rows is None else rows):
        src = int(gather_indices[r]) if gather_indices is not None else r
        rp = _row_params(r, params, token_to_request_index)
        out.append(sample_row(logits[src], rp, r, _row_offset(r, step_offset, offsets,
                                                               token_to_request_index),
                              not no_top_k, not no_top_p))
    return out


def _row_offset(r, step_offset, offsets, token_to_request_index) -> int:
    """Philox offset of output row r: the call's offset plus, when given, its
    request's entry of a per-request offset pool, modulo 2^64 (the TokenSpeed
    Triton sampling backend page passes such a pool, ``offsets_pool``, to every
    Gumbel kernel)."""
    if offsets is None:
        return int(step_offset) % (1 << 64)
    q = int(token_to_request_index[r]) if token_to_request_index is not None else r
    return (int(step_offset) + (int(offsets[q]) % (1 << 64))) % (1 << 64)


def log_probs(logits, n: int, params: dict, *, gather_indices=None, token_to_request_index=None,
              no_top_k: bool = False, no_top_p: bool = False, token_ids=None,
              rows: Optional[Sequence[int]] = None):
    """Log-probs of the processed distribution: [n, V], or [n] at ``token_ids``."""
    logits = np.asarray(logits)
    out = []
    for r in (range(n) if rows is None else rows):
        src = int(gather_indices[r]) if gather_indices is not None else r
        rp = _row_params(r, params, token_to_request_index)
        lp = process_row(logits[src], rp, not no_top_k, not no_top_p)["lp_row"]
        out.append(lp if token_ids is None else lp[int(token_ids[r])])
    return np.array(out)


def raw_log_probs_at(logits, n: int, token_ids, *, gather_indices=None,
                     rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Log-softmax of the raw row (no temperature, no filter) at token_ids[r]:
    the selected-token log-probs that the TokenSpeed Triton sampling backend
    page writes from the logits and the sampled ids.  NaN reads as -inf; a -inf
    entry at the id gives -inf; an id outside the row or a row with no finite
    logit gives NaN."""
    logits = np.asarray(logits)
    out = []
    for r in (range(n) if rows is None else rows):
        src = int(gather_indices[r]) if gather_indices is not None else r
        x = canonical_logits(logits[src])
        j = int(token_ids[r])
        fin = x > -np.inf
        if not fin.any() or j < 0 or j >= x.size:
            out.append(np.nan)
            continue
        m = np.max(x[fin])
        lse = m + np.log(np.sum(np.exp(x[fin] - m)))
        out.append(x[j] - lse if x[j] > -np.inf else -np.inf)
    return np.array(out)


def build_spec_map(num_decode: int, num_prefill: int, num_spec: int) -> np.ndarray:
    """Per-row request index of the speculative-verify layout.

    "core.inference.sampling.base", ``sample_speculative``: each decode request
    contributes 1 + num_speculative_tokens rows, each prefill request one row.
    Reading: decode requests come first, each in a contiguous block, then the
    prefill requests; request indices are 0..num_decode+num_prefill-1 in that order.
    """
    rows = []
    for d in range(num_decode):
        rows.extend([d] * (1 + num_spec))
    for i in range(num_prefill):
        rows.append(num_decode + i)
    return np.array(rows, dtype=np.int32)
