"""Pins of the oracle's filters, draw and log-probs against brute force,
closed forms, frequency tests and scipy."""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy import special, stats

import oracle
from oracle import RowParams
from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))


def _order_by_python_sort(x):
    return sorted(range(len(x)), key=lambda j: (-x[j], j))


def _tiny_rows(count, v, seed):
    """Small integer-valued rows with many ties, some -inf, NaN and -0."""
    rng = np.random.default_rng(seed)
    rows = []
    for _ in range(count):
        x = rng.integers(-2, 3, size=v).astype(np.float64)
        if rng.random() < 0.3:
            x[rng.integers(v)] = -np.inf
        if rng.random() < 0.2:
            x[rng.integers(v)] = np.nan
        if rng.random() < 0.3:
            x[x == 0] = -0.0
        rows.append(x)
    return rows


# ---------------------------------------------------------------- top-k


def test_top_k_matches_brute_force_subsets():
    for x in _tiny_rows(300, 7, 1):
        xc = oracle.sampler.canonical_logits(x)
        finite = [j for j in range(7) if xc[j] > -np.inf]
        for k in range(0, 9):
            got = set(np.nonzero(oracle.top_k_mask(xc, k))[0])
            if not (1 <= k < 7):
                assert got == set(finite)
                continue
            size = min(k, len(finite))
            pos = {j: i for i, j in enumerate(_order_by_python_sort(list(xc)))}
            valid = [set(c) for c in itertools.combinations(finite, size)
                     if all(pos[a] < pos[b] for a in c for b in finite if b not in c)]
            assert len(valid) == 1 and got == valid[0]


def test_top_k_ignores_temperature_and_breaks_ties_by_index():
    x = np.array([1.0, 3.0, 3.0, 2.0, 3.0, -0.0, 0.0])
    m = oracle.top_k_mask(oracle.sampler.canonical_logits(x), 2)
    assert list(np.nonzero(m)[0]) == [1, 2]
    m = oracle.top_k_mask(oracle.sampler.canonical_logits(x), 6)
    assert list(np.nonzero(m)[0]) == [0, 1, 2, 3, 4, 5]      # -0 == +0, lower index first


# ---------------------------------------------------------------- top-p


def _brute_top_p(x, s, topk, p):
    """Per-element definition: j kept iff the K-mass of strictly larger logits is < p."""
    kk = [j for j in range(len(x)) if topk[j]]
    w = {j: math.exp(s[j] - max(s[i] for i in kk)) for j in kk}
    z = math.fsum(w.values())
    keep = set()
    for j in kk:
        above = math.fsum(w[i] for i in kk if x[i] > x[j]) / z
        if above < p:
            keep.add(j)
    top = max(x[j] for j in kk)
    keep |= {j for j in kk if x[j] == top}
    return keep


def _smallest_upper_set(x, s, topk, p):
    """Textbook nucleus: the smallest union of leading tie groups whose mass reaches p."""
    kk = [j for j in range(len(x)) if topk[j]]
    vals = sorted({x[j] for j in kk}, reverse=True)
    w = {j: math.exp(s[j]) for j in kk}
    z = math.fsum(w.values())
    keep = set()
    for v in vals:
        keep |= {j for j in kk if x[j] == v}
        if math.fsum(w[j] for j in keep) / z >= p:
            break
    return keep


@pytest.mark.parametrize("p", [0.0, 0.1, 0.35, 0.5, 0.8, 0.95, 0.999999, 1.0])
def test_top_p_matches_brute_force(p):
    for x in _tiny_rows(150, 8, 2):
        xc = oracle.sampler.canonical_logits(x)
        for k in (0, 3, 5):
            topk = oracle.top_k_mask(xc, k)
            if not topk.any():
                continue
            for t in (0.5, 1.0, 2.0):
                s = xc / t
                keep, _, _, _ = oracle.top_p_mask(xc, s, topk, p)
                got = set(np.nonzero(keep)[0])
                if p >= 1 - oracle.TOP_P_EPS:
                    assert got == set(np.nonzero(topk)[0])
                    continue
                assert got == _brute_top_p(list(xc), list(s), topk, p)
                if p > 0:
                    assert got == _smallest_upper_set(list(xc), list(s), topk, p)


def _zipf_nucleus_closed_form(v, p, a=1.1):
    """Smallest R with H_R(a) >= p * H_V(a), where H_R(a) = sum_{i<=R} i^-a."""
    terms = np.arange(1, v + 1, dtype=np.float64) ** -a
    total = math.fsum(terms)
    r = int(np.searchsorted(np.cumsum(terms), p * total))   # approximate, then exact check
    for cand in range(max(1, r - 3), r + 4):
        if math.fsum(terms[:cand]) >= p * total:
            return cand
    raise AssertionError("closed form search failed")


@pytest.mark.parametrize("p", [0.5, 0.6, 0.7, 0.8, 0.9, 0.95, 0.99])
def test_top_p_zipf_closed_form(p):
    v = 151936
    rng = np.random.default_rng(4)
    perm = rng.permutation(v)
    base = -1.1 * np.log(np.arange(1, v + 1, dtype=np.float64))
    x = np.empty(v)
    x[perm] = base
    d = oracle.process_row(x, RowParams(1.0, 0, p, 0))
    r = _zipf_nucleus_closed_form(v, p)
    assert d["keep"].sum() == r
    assert set(np.nonzero(d["keep"])[0]) == set(perm[:r])


# ---------------------------------------------------------------- draw + log-probs


def _tempered_filtered_softmax(x, t, k, p):
    d = oracle.process_row(x, RowParams(t, k, p, 0))
    keep = d["keep"]
    return keep, special.softmax(np.where(keep, d["x"] / t, -np.inf))


@pytest.mark.parametrize("t,k,p", [(1.0, 0, 1.0), (0.7, 4, 1.0), (1.3, 0, 0.8), (0.9, 5, 0.7)])
def test_sample_frequencies_chi_square(t, k, p):
    x = np.array([0.3, -1.0, 1.2, 0.0, 0.9, 1.2, -0.4])
    keep, prob = _tempered_filtered_softmax(x, t, k, p)
    draws = 30000
    counts = np.zeros(x.size)
    for off in range(draws):
        counts[oracle.sample_row(x, RowParams(t, k, p, 1234), 3, off).token] += 1
    assert counts[~keep].sum() == 0
    chi = stats.chisquare(counts[keep], prob[keep] * draws)
    assert chi.pvalue > 1e-4, chi


def test_log_prob_matches_scipy_log_softmax():
    rng = np.random.default_rng(3)
    for trial in range(40):
        v = int(rng.integers(1, 300))
        x = rng.normal(0, 3, size=v)
        t = float(rng.uniform(0.3, 2.0))
        k = int(rng.integers(0, v + 2))
        p = float(rng.uniform(0.2, 1.0))
        res = oracle.sample_row(x, RowParams(t, k, p, trial), trial, 0)
        ref = special.log_softmax(np.where(res.keep, x / t, -np.inf))
        assert np.allclose(res.lp_row[res.keep], ref[res.keep], atol=1e-12)
        assert np.all(np.isneginf(res.lp_row[~res.keep]))
        assert res.keep[res.token] and math.isclose(res.logprob, ref[res.token], abs_tol=1e-12)
        assert abs(np.exp(res.lp_row[res.keep]).sum() - 1.0) < 1e-12
        assert res.logprob <= 0.0


def test_special_cases():
    x = np.array([0.5, 2.0, -1.0, 2.0, 1.9])
    # k = 1 is the argmax, whatever the seed
    for seed in range(20):
        assert oracle.sample_row(x, RowParams(1.0, 1, 1.0, seed), 0, seed).token == 1
    # V = 1
    r = oracle.sample_row(np.array([3.0]), RowParams(0.8, 0, 1.0, 9), 0, 0)
    assert r.token == 0 and r.logprob == 0.0
    # no filter: log-prob is log_softmax(x / T)
    r = oracle.sample_row(x, RowParams(0.6, 0, 1.0, 5), 2, 7)
    assert math.isclose(r.logprob, special.log_softmax(x / 0.6)[r.token], abs_tol=1e-12)
    # p <= 0 keeps exactly the top tie group
    r = oracle.sample_row(x, RowParams(1.0, 0, 0.0, 5), 0, 0)
    assert list(np.nonzero(r.keep)[0]) == [1, 3]
    assert math.isclose(r.logprob, math.log(0.5), abs_tol=1e-12)
    # all -inf / NaN row
    r = oracle.sample_row(np.array([-np.inf, np.nan]), RowParams(1.0, 0, 1.0, 0), 0, 0)
    assert r.token == -1 and math.isnan(r.logprob)
    # NaN behaves as -inf
    a = oracle.sample_row(np.array([1.0, np.nan, 0.5]), RowParams(1.0, 0, 1.0, 4), 0, 3)
    b = oracle.sample_row(np.array([1.0, -np.inf, 0.5]), RowParams(1.0, 0, 1.0, 4), 0, 3)
    assert a.token == b.token and a.token != 1
    # greedy: first maximum, log-prob 0
    r = oracle.sample_row(x, RowParams(0.0, 0, 1.0, 0), 0, 0)
    assert r.token == 1 and r.logprob == 0.0


def test_step_offset_and_seed_reproducibility():
    x = np.random.default_rng(8).normal(0, 1, size=500)
    a = [oracle.sample_row(x, RowParams(1.0, 0, 1.0, 77), 5, off).token for off in range(64)]
    b = [oracle.sample_row(x, RowParams(1.0, 0, 1.0, 77), 5, off).token for off in range(64)]
    assert a == b
    assert len(set(a)) > 10


def test_per_request_offsets_add_to_the_call_offset():
    """A row sampled with a per-request offset pool draws the noise of a plain
    call made at (step_offset + pool[q]) mod 2^64, q being the row's request."""
    rng = np.random.default_rng(12)
    logits = rng.normal(0, 2, size=(10, 48))
    params = {"temperature": np.full(4, 0.9), "top_k": np.array([0, 7, 0, 12]),
              "top_p": np.array([1.0, 1.0, 0.8, 0.6]),
              "seed": np.array([5, 6, 7, 8], dtype=np.uint64),
              "step_offsets": np.array([0, 3, 2**64 - 1, 2**40], dtype=np.uint64)}
    req = np.array([0, 1, 2, 3, 0, 1, 2, 3, 1, 2])
    base = 2**64 - 2
    got = oracle.sample(logits, 10, params, token_to_request_index=req, step_offset=base)
    plain = {k: v for k, v in params.items() if k != "step_offsets"}
    for r in range(10):
        off = (base + int(params["step_offsets"][req[r]])) % 2**64
        want = oracle.sample(logits, 10, plain, token_to_request_index=req, step_offset=off,
                             rows=[r])[0]
        assert got[r].token == want.token and got[r].logprob == want.logprob
    # the pool reaches the noise: over many pools the unfiltered row changes its draw
    draws = {oracle.sample(logits, 10, dict(plain, step_offsets=np.full(4, o, dtype=np.uint64)),
                           token_to_request_index=req, rows=[0])[0].token for o in range(40)}
    assert len(draws) > 5


def test_raw_log_probs_at_pins():
    """Log-softmax of the raw row: a worked example, normalisation, shift
    invariance, the special cases, and agreement with the processed
    distribution when no filter and T = 1 leave the row as it is."""
    x = np.array([[0.0, math.log(3.0)]])
    got = oracle.raw_log_probs_at(np.repeat(x, 2, 0), 2, [1, 0])
    assert np.allclose(got, [math.log(0.75), -math.log(4.0)], rtol=0, atol=1e-15)
    rng = np.random.default_rng(21)
    row = rng.normal(0, 3, size=(1, 200))
    every = np.array([oracle.raw_log_probs_at(row, 1, [j])[0] for j in range(200)])
    assert abs(np.sum(np.exp(every)) - 1.0) < 1e-12
    shifted = np.array([oracle.raw_log_probs_at(row + 123.25, 1, [j])[0] for j in range(200)])
    assert np.allclose(shifted, every, rtol=0, atol=1e-11)
    params = {"temperature": np.ones(1), "top_k": np.zeros(1, dtype=np.int64),
              "top_p": np.ones(1), "seed": np.zeros(1, dtype=np.uint64)}
    assert np.allclose(oracle.log_probs(row, 1, params)[0], every, rtol=0, atol=1e-12)
    odd = np.array([[1.0, np.nan, -np.inf, 2.0]] * 5 + [[-np.inf] * 4])
    got = oracle.raw_log_probs_at(odd, 6, [0, 1, 2, -1, 4, 3])
    want0 = 1.0 - math.log(math.e + math.e ** 2)
    assert abs(got[0] - want0) < 1e-15 and got[1] == -np.inf and got[2] == -np.inf
    assert np.isnan(got[3]) and np.isnan(got[4]) and np.isnan(got[5])


def test_near_tie_is_flagged_with_both_alternatives():
    j = np.arange(6)
    g = philox.gumbel_from_uniform(philox.uniform_from_words(philox.noise_words(3, 0, 0, j)))
    x = np.full(6, -30.0)
    x[1] = 5.0 - g[1]
    x[4] = 5.0 - g[4]
    r = oracle.sample_row(x, RowParams(1.0, 0, 1.0, 3), 0, 0)
    assert r.flag_sample and {o.token for o in r.alternatives} == {1, 4}


# Rows with exactly known softmax masses for the top-p near-tie pins: logits
# x = T ln(w), so s = x / T = ln(w) and pi = w / sum(w).  Tie groups (in
# descending logit order): {0} 0.3, {1, 2} 0.4, {3, 4, 5} 0.3, so the
# cumulative masses through each group are 0.3, 0.7 and 1.0.
_TP_W = np.array([0.3, 0.2, 0.2, 0.1, 0.1, 0.1])
_TP_ALL, _TP_01, _TP_0 = {0, 1, 2, 3, 4, 5}, {0, 1, 2}, {0}


def _tp_expect_lp(members):
    w = np.where(np.isin(np.arange(6), sorted(members)), _TP_W, 0.0)
    with np.errstate(divide="ignore"):
        return np.where(w > 0, np.log(w / w.sum()), -np.inf)


def _tp_expect_token(members, seed, r, off):
    """Brute force: argmax over the set of ln(w) + g (lowest index on ties)."""
    g = philox.gumbel_from_uniform(philox.uniform_from_words(philox.noise_words(seed, r, off, np.arange(6))))
    return max(sorted(members), key=lambda j: (math.log(_TP_W[j]) + g[j], -j))


@pytest.mark.parametrize("t", [1.0, 0.7])
@pytest.mark.parametrize("p,kept,alts", [
    (0.7 * (1 + 4e-6), _TP_ALL, [_TP_01]),   # just above C(1) = 0.7: group 2 kept, may drop
    (0.7 * (1 - 4e-6), _TP_01, [_TP_ALL]),   # just below C(1): group 2 dropped, may be kept
    (0.3 * (1 + 4e-6), _TP_01, [_TP_0]),     # just above C(0) = 0.3: group 1 kept, may drop
    (0.3 * (1 - 4e-6), _TP_0, [_TP_01]),     # just below C(0): group 1 dropped, may be kept
    (0.7 * (1 + 3e-5), _TP_ALL, []),         # outside the 1e-5 * p band: not flagged
    (0.7 * (1 - 3e-5), _TP_01, []),
    (0.3 * (1 + 3e-5), _TP_01, []),
])
def test_top_p_near_tie_flag_and_alternative_sets(t, p, kept, alts):
    """Top-p near ties: a cumulative tie-group mass within 1e-5 * p of p flags
    the row, and the listed alternatives sample from exactly the set with that
    boundary group toggled (whole tie groups), with that set's log-probs."""
    x = t * np.log(_TP_W)
    for seed in (3, 8, 21):
        r = oracle.sample_row(x, RowParams(t, 0, p, seed), 2, 5)
        assert set(np.nonzero(r.keep)[0]) == kept
        assert r.token == _tp_expect_token(kept, seed, 2, 5)
        assert np.allclose(r.lp_row, _tp_expect_lp(kept), rtol=0, atol=1e-12)
        assert r.flag_topp == bool(alts)
        topp_alts = [o for o in r.alternatives if o.lp_row is not None]
        assert sorted({tuple(np.nonzero(o.keep)[0]) for o in topp_alts}) == \
            sorted(tuple(sorted(a)) for a in alts)
        for o in topp_alts:
            members = set(np.nonzero(o.keep)[0])
            assert o.token == _tp_expect_token(members, seed, 2, 5)
            assert np.allclose(o.lp_row, _tp_expect_lp(members), rtol=0, atol=1e-12)
            assert abs(o.logprob - o.lp_row[o.token]) < 1e-15


def test_top_p_near_tie_inside_top_k():
    """Joint: with k = 4 the top-k set cuts the group {3, 4, 5} at index 3, and
    the renormalised K-masses are 0.375, 0.5, 0.125 (cumulative 0.375, 0.875,
    1).  A p just above 0.875 keeps index 3 and lists the set without it."""
    x = np.log(_TP_W)
    r = oracle.sample_row(x, RowParams(1.0, 4, 0.875 * (1 + 4e-6), 9), 0, 0)
    assert set(np.nonzero(r.topk)[0]) == {0, 1, 2, 3}
    assert set(np.nonzero(r.keep)[0]) == {0, 1, 2, 3} and r.flag_topp
    alt = [o for o in r.alternatives if o.lp_row is not None]
    assert {tuple(np.nonzero(o.keep)[0]) for o in alt} == {(0, 1, 2)}
    assert np.allclose(alt[0].lp_row[:3], np.log(np.array([0.3, 0.2, 0.2]) / 0.7), rtol=0, atol=1e-12)
    r = oracle.sample_row(x, RowParams(1.0, 4, 0.875 * (1 + 3e-5), 9), 0, 0)
    assert not r.flag_topp


def test_thresholds_are_compared_in_fp32():
    """A temperature equal to fp32(1e-5) samples and anything below it is
    greedy; a top-p equal to fp32(1) - fp32(1e-6) (= fp32(0.999999)) is off and
    the next fp32 value below it filters."""
    t_thr = float(np.float32(1e-5))
    assert not oracle.sampler.is_greedy(t_thr)
    assert oracle.sampler.is_greedy(float(np.nextafter(np.float32(t_thr), np.float32(0))))
    assert oracle.sampler.is_greedy(float("nan")) and oracle.sampler.is_greedy(0.0)
    p_thr = float(np.float32(1.0) - np.float32(1e-6))
    assert p_thr == float(np.float32(0.999999))
    assert not oracle.sampler.top_p_active(p_thr)
    assert oracle.sampler.top_p_active(float(np.nextafter(np.float32(p_thr), np.float32(0))))
    assert not oracle.sampler.top_p_active(float("nan"))
    # end to end: at the temperature threshold the row is sampled, not greedy
    x = np.array([2.0, 2.0, 1.0])
    r = oracle.sample_row(x, RowParams(t_thr, 0, 1.0, 4), 0, 0)
    assert r.keep.sum() == 3


def test_gather_map_and_spec_layout():
    rng = np.random.default_rng(2)
    logits = rng.normal(0, 2, size=(12, 64))
    params = {"temperature": np.full(4, 0.8), "top_k": np.array([0, 5, 0, 9]),
              "top_p": np.array([1.0, 1.0, 0.7, 0.9]), "seed": np.arange(4) + 100}
    gather = np.array([11, 3, 0, 7, 7, 2])
    req = np.array([0, 0, 1, 2, 3, 3])
    got = oracle.sample(logits, 6, params, gather_indices=gather, token_to_request_index=req, step_offset=4)
    # gather identity: sampling the gathered rows directly gives the same results
    p2 = {kk: np.asarray(v)[req] for kk, v in params.items()}
    ref = oracle.sample(logits[gather], 6, p2, step_offset=4)
    assert [a.token for a in got] == [b.token for b in ref]
    assert [a.logprob for a in got] == [b.logprob for b in ref]
    # identity map is the same as no map
    ident = oracle.sample(logits, 4, params, token_to_request_index=np.arange(4))
    none = oracle.sample(logits, 4, params)
    assert [a.token for a in ident] == [b.token for b in none]
    # batch-level promises switch the filters off
    off = oracle.sample(logits, 4, params, no_top_k=True, no_top_p=True)
    assert all(r.keep.sum() == 64 for r in off)


def test_spec_map_golden():
    with open(os.path.join(HERE, "golden", "spec_layout.json")) as f:
        doc = json.load(f)
    for c in doc["cases"]:
        got = oracle.build_spec_map(c["num_decode"], c["num_prefill"], c["num_spec"])
        assert got.tolist() == c["map"]


def test_log_probs_at_token_ids_and_full_rows():
    rng = np.random.default_rng(5)
    logits = rng.normal(0, 3, size=(5, 40))
    params = {"temperature": np.array([1.0, 0.5, 2.0, 1.0, 1.0]), "top_k": np.array([0, 3, 10, 0, 1]),
              "top_p": np.array([0.9, 1.0, 0.5, 1.0, 1.0]), "seed": np.arange(5)}
    full = oracle.log_probs(logits, 5, params)
    ids = np.array([int(np.argmax(full[r])) for r in range(5)])
    at = oracle.log_probs(logits, 5, params, token_ids=ids)
    assert np.array_equal(at, full[np.arange(5), ids])
    samples = oracle.sample(logits, 5, params)
    for r, s in enumerate(samples):
        assert s.logprob == full[r, s.token]


# ---------------------------------------------------------------------------
# Chain verification of speculative drafts (TokenSpeed page, TritonSamplingBackend.verify).
# Parity unpinned: the page prints neither the kernel's steps nor a value; the
# pins are hand-worked cases of the stated reading and invariants.

def test_verify_chain_golden_cases():
    with open(os.path.join(HERE, "golden", "verify_chain.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        pred, idx, acc = oracle.verify_chain(np.array(c["candidates"]), np.array(c["target"]))
        assert pred.tolist() == c["predicts"], c
        assert idx.tolist() == c["accept_index"], c
        assert acc.tolist() == c["accept_length"], c


def test_verify_chain_invariants():
    rng = np.random.default_rng(5)
    for n in (1, 2, 4, 7):
        bs = 50
        cand = rng.integers(0, 3, size=(bs, n))
        tgt = rng.integers(0, 3, size=bs * n)
        pred, idx, acc = oracle.verify_chain(cand, tgt)
        for b in range(bs):
            a = int(acc[b])
            assert 0 <= a <= n - 1
            # every accepted draft equals the target sample before it, and the
            # first rejected one does not
            for i in range(a):
                assert cand[b, i + 1] == tgt[b * n + i]
            if a < n - 1:
                assert cand[b, a + 1] != tgt[b * n + a]
            assert idx[b].tolist() == [b * n + i for i in range(a + 1)] + [-1] * (n - 1 - a)
            assert pred[b * n:(b + 1) * n].tolist() == tgt[b * n:b * n + a + 1].tolist() + [-1] * (n - 1 - a)


def test_verify_chain_accepts_everything_when_drafts_are_the_target_samples():
    # drafts taken from the target samples themselves (shifted by one) are all
    # accepted: the chain emits every target sample
    rng = np.random.default_rng(9)
    bs, n = 8, 5
    tgt = rng.integers(0, 1000, size=bs * n)
    cand = np.empty((bs, n), dtype=np.int64)
    cand[:, 0] = rng.integers(0, 1000, size=bs)
    cand[:, 1:] = tgt.reshape(bs, n)[:, :-1]
    pred, idx, acc = oracle.verify_chain(cand, tgt)
    assert np.all(acc == n - 1)
    assert np.array_equal(pred, tgt)
    assert np.array_equal(idx.reshape(-1), np.arange(bs * n))


def test_process_pool_gives_the_single_process_results():
    """oracle.parallel splits rows over worker processes; every row's result is
    the one oracle.sample / oracle.log_probs computes in one process (gather,
    request map and step offset included)."""
    import synth
    from oracle.parallel import Pool
    wl = synth.make("spec_mix", rows=30, vocab=777)
    x, prm = wl.logits_f64(), wl.params_numpy()
    kw = dict(gather_indices=wl.gather_indices.numpy(),
              token_to_request_index=wl.token_to_request_index.numpy())
    one = oracle.sample(x, wl.n, prm, step_offset=3, **kw)
    lp1 = oracle.log_probs(x, wl.n, prm, **kw)
    with Pool(workers=3) as pool:
        many = pool.run("sample", x, wl.n, prm, step_offset=3, light=True, **kw)
        lpm = pool.run("log_probs", x, wl.n, prm, **kw)
        sub = pool.run("sample", x, wl.n, prm, step_offset=3, rows=[29, 4, 4], **kw)
    assert [(a.token, a.logprob, a.flagged) for a in one] == \
        [(b.token, b.logprob, b.flagged) for b in many]
    assert np.array_equal(lp1, lpm)
    assert [a.token for a in sub] == [one[29].token, one[4].token, one[4].token]
    # the synthetic speculative workload uses the oracle's layout
    wl = synth.make("spec_mix")
    assert np.array_equal(wl.token_to_request_index.numpy(), oracle.build_spec_map(64, 32, 3))
