"""GPU parity: the HIP sampler against the fp64 oracle on the same seeded inputs.

Bars: top-k sets bit-exact; top-p sets and sampled ids exact except rows the
oracle flags as near ties within 1e-5 relative (counted, and the GPU must take
one of the listed alternatives); log-probs within 1e-4 absolute.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import token_sampling_scaled_amd as tsa
from tests import parity

pytestmark = pytest.mark.gpu

SMALL = [
    ("tiny_joint", None, None),
    ("none_32k", 16, 32000),
    ("topk_128k", 12, 20011),      # odd vocab: rows not vector aligned, ragged tail
    ("joint_128k", 12, 20000),
    ("joint_128k_shifted", 24, 20000),   # thresholds of every sign
    ("topp_152k", 8, 30000),
    ("spec_mix", 24, 16384),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tsa.library()


@pytest.mark.parametrize("name,rows,vocab", SMALL)
def test_sample_parity_small(name, rows, vocab):
    wl = synth.make(name, rows=rows, vocab=vocab)
    print(f"[case] sample {name} rows={wl.n} vocab={wl.vocab} dtype={wl.logits.dtype}", flush=True)
    ids, lps = parity.gpu_sample(wl)
    parity.compare_samples(ids, lps, parity.oracle_sample(wl)).check()


@pytest.mark.parametrize("name,rows,vocab", SMALL)
def test_log_probs_parity_small(name, rows, vocab):
    wl = synth.make(name, rows=rows, vocab=vocab)
    print(f"[case] log_probs {name} rows={wl.n} vocab={wl.vocab}", flush=True)
    gpu = parity.gpu_log_probs(wl)
    ref = parity.oracle_log_probs(wl)
    res = parity.oracle_sample(wl)
    parity.compare_log_probs(gpu, ref, res).check()
    # log-probs at the sampled ids equal the fused log-prob of sample()
    ids, lps = parity.gpu_sample(wl)
    at = parity.gpu_log_probs(wl, token_ids=torch.from_numpy(ids.astype(np.int32)))
    fin = ids >= 0
    assert np.allclose(at[fin], lps[fin], atol=1e-5, rtol=0)


def test_bf16_top_p_route_log_probs():
    """bf16 rows on the top-p-only route: full log-probs and log-probs at the
    sampled ids come from the register-resident body (exact key histogram)."""
    wl = synth.make("topp_152k", rows=8, vocab=30000)
    wl.logits = wl.logits.to(torch.bfloat16)
    print(f"[case] log_probs bf16 top-p rows={wl.n} vocab={wl.vocab}", flush=True)
    gpu = parity.gpu_log_probs(wl)
    res = parity.oracle_sample(wl)
    parity.compare_log_probs(gpu, parity.oracle_log_probs(wl), res).check("log_probs bf16 top-p")
    ids, lps = parity.gpu_sample(wl)
    parity.compare_samples(ids, lps, res).check("sample bf16 top-p")
    at = parity.gpu_log_probs(wl, token_ids=torch.from_numpy(ids.astype(np.int32)))
    fin = ids >= 0
    assert np.allclose(at[fin], lps[fin], atol=1e-5, rtol=0)


@pytest.fixture(scope="module")
def oracle_pool():
    from oracle.parallel import Pool
    with Pool() as pool:
        pool.warm()
        yield pool


FULL = ["tiny_joint", "none_32k", "topk_128k", "joint_128k", "joint_128k_shifted", "topp_152k",
        "spec_mix"]


@pytest.mark.parametrize("name", FULL)
def test_sample_parity_full_size_every_row(name, oracle_pool):
    """Every row of every workload at its full size, in the launch configuration
    the benchmark times: ids and fused log-probs against the oracle (run over a
    process pool)."""
    wl = synth.make(name)
    print(f"[case] full {name} rows={wl.n} vocab={wl.vocab}", flush=True)
    ids, lps = parity.gpu_sample(wl)
    rep = parity.compare_samples(ids, lps, parity.oracle_sample_pool(oracle_pool, wl))
    rep.check(f"sample {name} full")
    assert np.all((ids >= 0) & (ids < wl.vocab))


@pytest.mark.parametrize("name", FULL)
def test_log_probs_full_size_every_row(name, oracle_pool):
    """Full [n, V] log-probs of every row at the full sizes (the register-resident
    bf16 kernel on the top-k and joint routes, the general kernel elsewhere),
    then the same at the sampled ids."""
    wl = synth.make(name)
    print(f"[case] log_probs full {name} rows={wl.n} vocab={wl.vocab}", flush=True)
    gpu = parity.gpu_log_probs(wl)
    ref = parity.oracle_log_probs_pool(oracle_pool, wl)
    res = parity.oracle_sample_pool(oracle_pool, wl)
    parity.compare_log_probs(gpu, ref, res).check(f"log_probs {name} full")
    del ref
    # at the sampled ids: the log-prob kernel's value equals its own full row;
    # the sampling kernel's fused value (another kernel on some routes, with
    # its own fp32 sums) agrees within the parity tolerance
    ids, lps = parity.gpu_sample(wl)
    at = parity.gpu_log_probs(wl, token_ids=torch.from_numpy(ids.astype(np.int32)))
    assert np.allclose(at, gpu[np.arange(wl.n), ids], atol=1e-5, rtol=0)
    assert np.allclose(at, lps, atol=parity.LP_ATOL, rtol=0)


@pytest.mark.parametrize("name,rows,vocab", SMALL)
def test_per_request_step_offsets(name, rows, vocab):
    """Per-request offsets read on the device, added to the call's offset."""
    wl = synth.make(name, rows=rows, vocab=vocab)
    q = wl.temperature.numel()
    wl.step_offsets = torch.from_numpy(
        np.random.default_rng(31).integers(0, 2**63 - 1, q, dtype=np.int64))
    wl.step_offset = 5
    print(f"[case] step_offsets {name} rows={wl.n} vocab={wl.vocab}", flush=True)
    ids, lps = parity.gpu_sample(wl)
    parity.compare_samples(ids, lps, parity.oracle_sample(wl)).check()


@pytest.mark.parametrize("name,rows,vocab", [("joint_128k", 16, 20000), ("topp_152k", 8, 30000),
                                             ("none_32k", 16, 32000), ("spec_mix", 24, 16384)])
def test_graph_replay_with_device_offsets(name, rows, vocab):
    """One call captured in a graph, replayed four times; between replays the
    per-request offsets advance on the device.  Every replay must equal an eager
    call at the same offsets (bitwise) and the oracle, and the replays must not
    all draw the same ids."""
    wl = synth.make(name, rows=rows, vocab=vocab)
    q = wl.temperature.numel()
    dev = parity.to_device(wl)
    offs = torch.zeros(q, dtype=torch.int64, device="cuda")
    dev["params"].step_offsets = offs
    s = tsa.Sampler(wl.vocab, wl.n)
    ids = torch.empty(wl.n, dtype=torch.int32, device="cuda")
    lps = torch.empty(wl.n, dtype=torch.float32, device="cuda")

    def call():
        s.sample(dev["logits"], wl.n, dev["params"], no_top_k=wl.no_top_k, no_top_p=wl.no_top_p,
                 gather_indices=dev["gather"], token_to_request_index=dev["req"],
                 step_offset=wl.step_offset, output=ids, logprob_output=lps)

    print(f"[case] graph {name} rows={wl.n} vocab={wl.vocab}", flush=True)
    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    check_rows = sorted(set(np.linspace(0, wl.n - 1, 6).astype(int).tolist()))
    seen = set()
    for step in range(4):
        offs.fill_(7 * step + 1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_ids, got_lps = ids.cpu().numpy().copy(), lps.cpu().numpy().copy()
        call()
        torch.cuda.synchronize()
        assert np.array_equal(got_ids, ids.cpu().numpy())
        assert np.array_equal(got_lps.view(np.int32), lps.cpu().numpy().view(np.int32))
        wl.step_offsets = offs.cpu()
        rep = parity.compare_samples(got_ids, got_lps, parity.oracle_sample(wl, rows=check_rows),
                                     rows=check_rows)
        rep.check()
        seen.add(tuple(got_ids.tolist()))
    assert len(seen) > 1


@pytest.mark.parametrize("name,rows,vocab", [("tiny_joint", None, None), ("none_32k", 16, 32000),
                                             ("topk_128k", 12, 20011), ("topp_152k", 8, 30000),
                                             ("spec_mix", 24, 16384), ("joint_128k", None, None)])
def test_raw_log_probs_at(name, rows, vocab):
    """Log-softmax of the raw rows at given ids (sampled ids, random ids, and
    ids outside the row), against the oracle within 1e-4."""
    wl = synth.make(name, rows=rows, vocab=vocab)
    print(f"[case] raw log-probs {name} rows={wl.n} vocab={wl.vocab}", flush=True)
    dev = parity.to_device(wl)
    s = tsa.Sampler(wl.vocab, wl.n)
    ids, _ = parity.gpu_sample(wl, s, dev)
    rng = np.random.default_rng(7)
    for tok in (ids, rng.integers(0, wl.vocab, wl.n).astype(np.int32),
                np.where(np.arange(wl.n) % 3 == 0, -1, wl.vocab).astype(np.int32)):
        got = s.raw_log_probs_at(dev["logits"], torch.from_numpy(tok).cuda(), n=wl.n,
                                 gather_indices=dev["gather"])
        got = got.cpu().numpy()
        gi = None if wl.gather_indices is None else wl.gather_indices.numpy()
        want = oracle.raw_log_probs_at(wl.logits_f64(), wl.n, tok, gather_indices=gi)
        assert np.array_equal(np.isnan(got), np.isnan(want))
        assert np.array_equal(np.isneginf(got), np.isneginf(want))
        fin = np.isfinite(want)
        assert np.max(np.abs(got[fin] - want[fin]), initial=0.0) <= parity.LP_ATOL


def test_raw_log_probs_at_odd_rows():
    rows = [[1.0, np.nan, -np.inf, 2.0, 0.5, -1.0, 3.0, 0.0]] * 5 + [[-np.inf] * 8]
    for dtype in (torch.float32, torch.bfloat16):
        x = torch.tensor(np.array(rows, dtype=np.float32)).to(dtype)
        tok = np.array([0, 1, 2, -1, 6, 3], dtype=np.int32)
        s = tsa.Sampler(8, 6)
        got = s.raw_log_probs_at(x.cuda(), torch.from_numpy(tok).cuda()).cpu().numpy()
        want = oracle.raw_log_probs_at(x.float().numpy().astype(np.float64), 6, tok)
        assert np.array_equal(np.isnan(got), np.isnan(want))
        assert np.array_equal(np.isneginf(got), np.isneginf(want))
        fin = np.isfinite(want)
        assert np.max(np.abs(got[fin] - want[fin])) <= parity.LP_ATOL


def _custom(rows, dtype=torch.float32, k=0, p=1.0, t=1.0, no_top_k=None, no_top_p=None,
            stride_pad=0):
    x = torch.tensor(np.array(rows, dtype=np.float32)).to(dtype)
    n, v = x.shape
    wl = synth.Workload("custom", x, n, torch.full((n,), float(t)), torch.full((n,), int(k), dtype=torch.int32),
                        torch.full((n,), float(p)), torch.arange(n, dtype=torch.int64) + 11)
    wl.no_top_k = (k == 0) if no_top_k is None else no_top_k
    wl.no_top_p = (p >= 1.0) if no_top_p is None else no_top_p
    wl.stride_pad = stride_pad
    return wl


def _device_logits(wl):
    pad = getattr(wl, "stride_pad", 0)
    if not pad:
        return wl.logits.cuda()
    buf = torch.full((wl.n, wl.vocab + pad), 7.0, dtype=wl.logits.dtype, device="cuda")
    buf[:, :wl.vocab] = wl.logits.cuda()
    return buf[:, :wl.vocab]


def _run_custom(wl):
    dev = {"logits": _device_logits(wl), "gather": None, "req": None,
           "params": tsa.SamplingParams(wl.temperature.cuda(), wl.seed.cuda(), wl.top_k.cuda(),
                                        wl.top_p.cuda())}
    s = tsa.Sampler(wl.vocab, wl.n)
    ids, lps = parity.gpu_sample(wl, s, dev)
    parity.compare_samples(ids, lps, parity.oracle_sample(wl)).check()
    gpu = parity.gpu_log_probs(wl, s, dev)
    parity.compare_log_probs(gpu, parity.oracle_log_probs(wl), parity.oracle_sample(wl)).check()
    return ids, lps


EDGE_ROWS = {
    "ties": [[1.0, 3.0, 3.0, 2.0, 3.0, -0.0, 0.0, 3.0]] * 3,
    "neg_inf_nan": [[-np.inf, 1.0, np.nan, 2.0, -np.inf, 0.5, np.nan, -1.0]],
    "all_neg_inf": [[-np.inf] * 5, [np.nan] * 5],
    "single": [[0.25]],
    "three": [[0.1, 0.1, 0.1]],
}


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("case", sorted(EDGE_ROWS))
@pytest.mark.parametrize("k,p,t", [(0, 1.0, 1.0), (2, 1.0, 0.8), (0, 0.5, 1.3), (3, 0.7, 1.0),
                                   (1, 1.0, 1.0), (0, 0.0, 1.0), (0, 1.0, 0.0), (100, 0.9, 1.0),
                                   (2, 0.9, 0.0)])
def test_edge_rows(case, dtype, k, p, t):
    wl = _custom(EDGE_ROWS[case], dtype=dtype, k=k, p=p, t=t)
    print(f"[case] edge {case} {dtype} k={k} p={p} t={t}", flush=True)
    _run_custom(wl)


NOK_ROWS = [
    [1.0, 3.0, 3.0, 2.0, 3.0, -0.0, 0.0, 3.0] * 2,                       # ties at the top
    [-np.inf, 1.0, np.nan, 2.0, -np.inf, 0.5, -np.nan, -1.0] * 2,        # NaN of both signs
    [-np.inf] * 16,                                                      # nothing finite
    [-1.0, -0.0, -2.0, -0.5] * 4,                                        # the maximum is -0
    [0.5] + [-20.0] * 15,                                                # flat at T = 100
    [-np.nan, 1.0, 0.5, -0.0, 0.0, 2.0, -np.nan, -3.0] * 2,              # negative NaN only
    [-0.0, 0.0, -0.0, -8.0] * 4,                                         # -0 and +0 in the top group
]


@pytest.mark.parametrize("p,t", [(1.0, 1.0), (0.9, 1.0), (0.99, 100.0), (0.0, 0.7), (0.9, 0.0)])
def test_joint_route_rows_without_top_k(p, t):
    """bf16 rows on the joint route whose own top-k is off: the register-resident
    body (unfiltered, or top-p by an exact key histogram); a cutoff below its key
    window (the flat row at T = 100) takes the general body."""
    wl = _custom(NOK_ROWS, torch.bfloat16, k=0, p=p, t=t, no_top_k=False, no_top_p=False)
    print(f"[case] joint route without top-k p={p} t={t}", flush=True)
    _run_custom(wl)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_bf16_like_ties_and_misaligned_stride(dtype):
    rng = np.random.default_rng(12)
    rows = np.round(rng.normal(0, 3, size=(6, 3001)) * 4) / 4     # heavy ties
    for k, p in [(50, 1.0), (700, 0.8), (0, 0.6), (1, 0.9), (0, 1.0)]:
        wl = _custom(rows, dtype=dtype, k=k, p=p, t=0.9, stride_pad=3)
        print(f"[case] ties k={k} p={p} {dtype}", flush=True)
        _run_custom(wl)


def _signed_bf16_rows(v, seed):
    """bf16 rows whose top-k cut is at or below zero: all negative, crossing
    zero, signed zeros at the cut, values inside |x| < 2^-64 (the zone the
    register-resident kernel's second pass cannot cut in: general body), and
    negatives mixed with -inf and NaN of both signs."""
    rng = np.random.default_rng(seed)
    rows = np.empty((6, v), dtype=np.float32)
    rows[0] = rng.normal(-20.0, 3.0, v)
    rows[1] = rng.normal(0.0, 1.0, v)
    rows[2] = np.where(rng.random(v) < 0.5, -0.0, 0.0)
    rows[2, rng.choice(v, 20, replace=False)] = rng.normal(2.0, 1.0, 20)
    rows[3] = rng.normal(0.0, 1.0, v) * 1e-25
    rows[4] = rng.normal(-3.0, 2.0, v)
    rows[4, rng.choice(v, 5, replace=False)] = 6.0
    rows[5] = -rng.exponential(1.0, v)
    rows[5, rng.choice(v, v // 16, replace=False)] = -np.inf
    rows[5, rng.choice(v, 7, replace=False)] = np.nan
    rows[5, rng.choice(v, 7, replace=False)] = -np.nan
    return rows


@pytest.mark.parametrize("k,p,t", [(1, 1.0, 1.0), (60, 0.9, 0.8), (700, 0.95, 1.2), (1024, 1.0, 1.0),
                                   (2500, 0.5, 1.0)])
def test_bf16_rows_cut_at_or_below_zero(k, p, t):
    """The signed-order second pass of the register-resident kernel (and the
    rows it sends on to the general body)."""
    rows = _signed_bf16_rows(4096, 7 + k)
    wl = _custom(rows, torch.bfloat16, k=k, p=p, t=t)
    print(f"[case] signed bf16 k={k} p={p} t={t}", flush=True)
    _run_custom(wl)


def _binade_rows(v, seed):
    """bf16 rows whose 172 largest entries lie one per binary exponent, from
    +2^60 (+2^20 in the last row) down through the signed zero region to
    -2^-10 (-2^30), over a floor of -2^100 that stays outside every top-k
    below: the signed-order pass's window holds 60 to 90 occupied 256-key
    blocks above the k-th value (its scan's block index past 64 blocks)."""
    rng = np.random.default_rng(seed)
    rows = np.full((5, v), -2.0 ** 100, dtype=np.float32)
    for r in range(5):
        top_e, low_e = (60, -10) if r < 4 else (20, 30)
        pos = np.ldexp(1.0 + rng.integers(0, 128, top_e + 61) / 128.0, np.arange(-60, top_e + 1))
        neg = -np.ldexp(1.0 + rng.integers(0, 128, low_e + 61) / 128.0, np.arange(-60, low_e + 1))
        vals = np.concatenate([pos, neg])
        rows[r, rng.choice(v, vals.size, replace=False)] = vals
    return rows


@pytest.mark.parametrize("k,p,t", [(150, 1.0, 2.0 ** 57), (150, 0.99, 2.0 ** 57), (100, 0.9, 2.0 ** 56),
                                   (172, 0.999, 2.0 ** 58)])
def test_bf16_rows_top_k_spanning_many_binades(k, p, t):
    """The signed-order pass on a window whose occupied blocks above the k-th
    value (and above the top-p cutoff) number more than one wave's lanes."""
    rows = _binade_rows(16384, 91 + k)
    wl = _custom(rows, torch.bfloat16, k=k, p=p, t=t)
    print(f"[case] binade bf16 k={k} p={p} t={t}", flush=True)
    _run_custom(wl)


def _small_f32_rows(v, seed):
    """fp32 rows for the short-row kernel: heavy ties, signed zeros, -inf and
    NaN sprinkled in, one row with fewer finite entries than most k, one flat
    row (a single histogram bin: more candidates than the kernel keeps, so the
    general body) and one of coarse ties (large tie groups at the cut)."""
    rng = np.random.default_rng(seed)
    rows = np.round(rng.normal(0, 2, size=(8, v)) * 8) / 8
    rows[1, rng.choice(v, v // 8, replace=False)] = -np.inf
    rows[1, rng.choice(v, 9, replace=False)] = np.nan
    rows[2, : v // 2] = -0.0
    rows[2, v // 2:] = 0.0
    rows[2, rng.choice(v, 40, replace=False)] = rng.normal(0, 1, 40)
    rows[3, :] = -np.inf
    rows[3, rng.choice(v, 30, replace=False)] = rng.normal(0, 1, 30)
    rows[4, :] = 1.5
    rows[5] = np.round(rows[5])
    rows[6] -= 30.0
    return rows


@pytest.mark.parametrize("v", [4096, 8192])
@pytest.mark.parametrize("k,p,t", [(1, 1.0, 1.0), (50, 0.9, 0.7), (256, 0.95, 1.3), (257, 0.9, 1.0),
                                   (50, 1.0, 0.0), (200, 0.3, 0.5)])
def test_short_fp32_rows_with_top_k(v, k, p, t):
    """The register-resident fp32 kernel for short rows (joint and top-k routes),
    with the rows it hands to the general body (k above 256, greedy, +inf, more
    than 1024 candidates, nothing finite)."""
    rows = _small_f32_rows(v, 100 + k)
    wl = _custom(rows, torch.float32, k=k, p=p, t=t)
    print(f"[case] short fp32 v={v} k={k} p={p} t={t}", flush=True)
    _run_custom(wl)
    wl = _custom(rows, torch.float32, k=k, p=p, t=t, stride_pad=4)   # padded rows, still aligned
    _run_custom(wl)


@pytest.mark.parametrize("name,rows,vocab", [("tiny_joint", None, None), ("joint_128k", 6, 16384),
                                             ("topp_152k", 4, 8192), ("none_32k", 4, 8192)])
def test_full_log_probs_into_an_unaligned_output(name, rows, vocab):
    """Full-row log-probs into an output 4 bytes past a 16-byte boundary: the
    kernels that store 16 bytes at a time are not chosen, the rows match the
    oracle all the same."""
    wl = synth.make(name, rows=rows, vocab=vocab)
    print(f"[case] unaligned log_probs {name} rows={wl.n} vocab={wl.vocab}", flush=True)
    dev = parity.to_device(wl)
    s = tsa.Sampler(wl.vocab, wl.n)
    buf = torch.empty(wl.n * wl.vocab + 4, dtype=torch.float32, device="cuda")
    out = buf[1:1 + wl.n * wl.vocab].view(wl.n, wl.vocab)
    assert out.data_ptr() % 16 == 4
    s.log_probs(dev["logits"], dev["params"], n=wl.n, no_top_k=wl.no_top_k, no_top_p=wl.no_top_p,
                gather_indices=dev["gather"], token_to_request_index=dev["req"], output=out)
    torch.cuda.synchronize()
    parity.compare_log_probs(out.cpu().numpy(), parity.oracle_log_probs(wl),
                             parity.oracle_sample(wl)).check()


def test_determinism_and_step_offset():
    wl = synth.make("spec_mix", rows=24, vocab=16384)
    dev = parity.to_device(wl)
    s = tsa.Sampler(wl.vocab, wl.n)
    a = parity.gpu_sample(wl, s, dev)
    b = parity.gpu_sample(wl, s, dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    c = parity.gpu_sample(wl, s, dev, step_offset=1)
    assert not np.array_equal(a[0], c[0])
    parity.compare_samples(*c, parity.oracle_sample(wl, step_offset=1)).check()


def test_gather_identity_and_int64_indices():
    wl = synth.make("spec_mix", rows=24, vocab=4096)
    dev = parity.to_device(wl)
    s = tsa.Sampler(wl.vocab, wl.n)
    ids, lps = s.sample(dev["logits"], wl.n, dev["params"], gather_indices=dev["gather"].long(),
                        token_to_request_index=dev["req"].long(), return_logprobs=True)
    pre = dev["logits"][dev["gather"].long()].contiguous()
    ids2, lps2 = s.sample(pre, wl.n, dev["params"], token_to_request_index=dev["req"],
                          return_logprobs=True)
    assert torch.equal(ids, ids2) and torch.equal(lps, lps2)
    with pytest.raises(ValueError):
        s.sample(dev["logits"], wl.n, dev["params"], gather_indices=dev["gather"].float())


def test_sample_speculative_matches_explicit_map():
    wl = synth.make("spec_mix")
    dev = parity.to_device(wl)
    s = tsa.Sampler(wl.vocab, wl.n)
    a = s.sample_speculative(dev["logits"], 64, 32, 3, dev["params"], gather_indices=dev["gather"])
    b = s.sample(dev["logits"], wl.n, dev["params"], gather_indices=dev["gather"],
                 token_to_request_index=dev["req"])
    assert torch.equal(a, b)
    m, n = tsa.build_spec_map(64, 32, 3, device="cuda")
    assert n == 288 and np.array_equal(m.cpu().numpy(), oracle.build_spec_map(64, 32, 3))


def test_argument_errors_on_gpu_handle():
    s = tsa.Sampler(100, 4)
    x = torch.zeros(4, 100, device="cuda")
    prm = tsa.SamplingParams(torch.ones(4, device="cuda"), torch.zeros(4, dtype=torch.int64, device="cuda"),
                             torch.zeros(4, dtype=torch.int32, device="cuda"), torch.ones(4, device="cuda"))
    with pytest.raises(ValueError):
        s.sample(x, 5, prm)                       # n > max_rows
    with pytest.raises(TypeError):
        s.sample(x.half(), 4, prm)
    out = s.sample(x, 0, prm)
    assert out.numel() == 0
    # caller-supplied outputs are checked before any kernel is launched
    bad_outputs = [dict(output=torch.empty(4, dtype=torch.int32)),               # host memory
                   dict(output=torch.empty(3, dtype=torch.int32, device="cuda")),  # too short
                   dict(output=torch.empty(4, dtype=torch.int64, device="cuda")),  # wrong dtype
                   dict(output=torch.empty(8, dtype=torch.int32, device="cuda")[::2]),
                   dict(logprob_output=torch.empty(4, dtype=torch.bfloat16, device="cuda")),
                   dict(logprob_output=torch.empty(2, dtype=torch.float32, device="cuda")),
                   dict(logprob_output=torch.empty(4, dtype=torch.float32))]
    for kw in bad_outputs:
        with pytest.raises(ValueError):
            s.sample(x, 4, prm, **kw)
    with pytest.raises(ValueError):
        s.sample(x.cpu(), 4, prm)                                                # host logits
    with pytest.raises(ValueError):
        s.log_probs(x, prm, output=torch.empty(4, 100))                          # host output
    with pytest.raises(ValueError):
        s.log_probs(x, prm, output=torch.empty(4, 99, device="cuda"))
    ids = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        s.log_probs(x, prm, token_ids=ids, output=torch.empty(4))
    with pytest.raises(ValueError):
        s.raw_log_probs_at(x, ids, output=torch.empty(4, device="cuda", dtype=torch.float16))
    with pytest.raises(ValueError):
        s.raw_log_probs_at(x, ids, output=torch.empty(4))
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("route", ["joint", "topk", "topp", "none"])
def test_parameters_at_the_fp32_thresholds(dtype, route):
    """Temperatures at fp32(1e-5) and the next fp32 below it, top-p at
    fp32(1) - fp32(1e-6) and the next fp32 below it: the kernels and the oracle
    take the same side of both thresholds (rows with a tied maximum, so a
    greedy row and a sampled one differ)."""
    t_thr = float(np.float32(1e-5))
    t_below = float(np.nextafter(np.float32(t_thr), np.float32(0)))
    p_thr = float(np.float32(1.0) - np.float32(1e-6))
    p_below = float(np.nextafter(np.float32(p_thr), np.float32(0)))
    rng = np.random.default_rng(5)
    rows = rng.normal(0, 1e-4, size=(8, 2048)).astype(np.float32)
    rows[:, [3, 700, 1500]] = 1e-3                     # a tied maximum
    t = [t_thr, t_below, t_thr, t_below, 1.0, 1.0, 0.5, 2.0]
    p = [p_thr, p_thr, p_below, p_below, p_thr, p_below, p_below, p_thr]
    k = 0 if route in ("topp", "none") else 1500
    wl = _custom(rows, dtype=dtype, k=k, p=1.0, t=1.0,
                 no_top_k=route in ("topp", "none"), no_top_p=route in ("topk", "none"))
    wl.temperature = torch.tensor(t, dtype=torch.float32)
    wl.top_p = torch.tensor(p, dtype=torch.float32)
    print(f"[case] thresholds {route} {dtype}", flush=True)
    _run_custom(wl)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("vocab,stride_pad", [(4099, 0), (20011, 5), (32000, 0), (262147, 1)])
def test_no_filter_rows_split_over_workgroups(dtype, vocab, stride_pad):
    """No-filter route: each row is spread over many workgroups whose partial
    argmax / log-sum-exp results are merged by the last one (odd vocab, padded
    stride, the largest split)."""
    rng = np.random.default_rng(vocab)
    n = 5
    x = rng.normal(0, 3, size=(n, vocab)).astype(np.float32)
    x[1, rng.integers(0, vocab, 50)] = -np.inf
    x[2, :] = 0.5                                     # one big tie group
    wl = _custom(x, dtype=dtype, k=0, p=1.0, t=1.0, stride_pad=stride_pad)
    wl.temperature = torch.tensor([1.0, 0.7, 1.3, 0.0, 2.0])
    print(f"[case] split none {dtype} vocab={vocab} pad={stride_pad}", flush=True)
    dev = {"logits": _device_logits(wl), "gather": None, "req": None,
           "params": tsa.SamplingParams(wl.temperature.cuda(), wl.seed.cuda(), wl.top_k.cuda(),
                                        wl.top_p.cuda())}
    s = tsa.Sampler(wl.vocab, wl.n)
    ids, lps = parity.gpu_sample(wl, s, dev)
    parity.compare_samples(ids, lps, parity.oracle_sample(wl)).check()
    # the per-row counters are back at zero: a second call gives the same result
    ids2, lps2 = parity.gpu_sample(wl, s, dev)
    assert np.array_equal(ids, ids2) and np.array_equal(lps, lps2, equal_nan=True)
    # another step offset: fresh noise, still the oracle's draw
    wl.step_offset = 1
    ids3, lps3 = parity.gpu_sample(wl, s, dev)
    parity.compare_samples(ids3, lps3, parity.oracle_sample(wl)).check()


def _mixed_rows_workload(n, vocab, frac_unfiltered, seed, n_req=None, gather_pool=0):
    """bf16 N(0, 3^2) rows on the joint route; each request is unfiltered with
    probability frac_unfiltered, else top-k, top-p or both (k ~ U{1..1024},
    p ~ U[0.5, 0.99], T ~ U[0.5, 1.5]).  With n_req, rows map onto requests."""
    rng = np.random.default_rng(seed)
    rows_in_buf = n + gather_pool
    x = torch.from_numpy(rng.normal(0.0, 3.0, size=(rows_in_buf, vocab)).astype(np.float32)).to(torch.bfloat16)
    q = n if n_req is None else n_req
    mode = np.where(rng.random(q) < frac_unfiltered, 0, rng.integers(1, 4, size=q))
    k = np.where((mode == 1) | (mode == 3), rng.integers(1, 1025, size=q), 0).astype(np.int32)
    p = np.where(mode >= 2, rng.uniform(0.5, 0.99, size=q), 1.0).astype(np.float32)
    t = rng.uniform(0.5, 1.5, size=q).astype(np.float32)
    wl = synth.Workload("mixed", x, n, torch.from_numpy(t), torch.from_numpy(k), torch.from_numpy(p),
                        torch.arange(q, dtype=torch.int64) * 7 + 3)
    if n_req is not None:
        wl.token_to_request_index = torch.from_numpy(rng.integers(0, q, size=n).astype(np.int32))
    if gather_pool:
        wl.gather_indices = torch.from_numpy(rng.permutation(rows_in_buf)[:n].astype(np.int32))
    wl.no_top_k = False
    wl.no_top_p = False
    return wl


@pytest.mark.parametrize("n,vocab,frac,n_req,pool", [
    (40, 20000, 0.4, None, 0),       # rows not a multiple of the 16-vector stride
    (48, 131072, 1.0, None, 0),      # every row unfiltered, the largest register-resident row
    (96, 65536, 0.3, 32, 16),        # request map and gather
    (1100, 2048, 0.3, None, 0),      # more rows than a workgroup has threads
    (300, 8192, 0.4, 100, 20),       # more rows than CUs: heavy rows are started first
])
def test_unfiltered_rows_in_mixed_batches(n, vocab, frac, n_req, pool):
    """Joint-route bf16 calls whose rows mix unfiltered, top-k-only,
    top-p-only and joint requests (ragged last vectors, request maps, gather,
    more rows than one workgroup has threads).  Calls in a row on one handle,
    with step offsets 0, 1, 0, each write every output (the buffers are
    filled with sentinels first) and give the oracle's results for their
    offset, so no state carries over between calls."""
    wl = _mixed_rows_workload(n, vocab, frac, seed=n + vocab, n_req=n_req, gather_pool=pool)
    print(f"[case] mixed unfiltered n={n} vocab={vocab} frac={frac}", flush=True)
    dev = parity.to_device(wl)
    s = tsa.Sampler(wl.vocab, wl.n)
    refs = {off: parity.oracle_sample(wl, step_offset=off) for off in (0, 1)}
    out = torch.empty(n, dtype=torch.int32, device="cuda")
    lp = torch.empty(n, dtype=torch.float32, device="cuda")
    got = {}
    for off in (0, 1, 0):
        out.fill_(-7)
        lp.fill_(123.0)
        s.sample(dev["logits"], n, dev["params"], no_top_k=False, no_top_p=False,
                 gather_indices=dev["gather"], token_to_request_index=dev["req"],
                 step_offset=off, output=out, logprob_output=lp)
        torch.cuda.synchronize()
        ids, lps = out.cpu().numpy(), lp.cpu().numpy()
        assert not np.any(ids == -7), "rows left unwritten"
        parity.compare_samples(ids, lps, refs[off]).check()
        if off in got:
            assert np.array_equal(ids, got[off][0])
            assert np.array_equal(lps, got[off][1], equal_nan=True)
        got[off] = (ids, lps)
    assert not np.array_equal(got[0][0], got[1][0])


def test_log_probs_with_more_rows_than_cus():
    """Full-row log-probs on the joint route with more rows than the device has
    CUs (the workgroups take the rows without a top-k body first)."""
    wl = _mixed_rows_workload(300, 4096, 0.3, seed=77, n_req=120, gather_pool=10)
    print(f"[case] log_probs mixed rows={wl.n} vocab={wl.vocab}", flush=True)
    gpu = parity.gpu_log_probs(wl)
    parity.compare_log_probs(gpu, parity.oracle_log_probs(wl), parity.oracle_sample(wl)).check()


def _draft_chains(bs, n, rng, target):
    """Drafts that follow the target samples for a random number of steps, then
    diverge (a draft that equals the target by chance is accepted too)."""
    tgt = target.reshape(bs, n)
    cand = rng.integers(0, 50, size=(bs, n)).astype(np.int32)
    stop = rng.integers(0, n, size=bs)             # drafts copied before this position
    for b in range(bs):
        for i in range(1, n):
            if i <= stop[b]:
                cand[b, i] = tgt[b, i - 1]
    return cand


@pytest.mark.parametrize("bs,n", [(1, 1), (5, 2), (64, 4), (300, 8), (2048, 3)])
def test_verify_chain_matches_oracle(bs, n):
    rng = np.random.default_rng(bs * 31 + n)
    target = rng.integers(0, 50, size=bs * n).astype(np.int32)
    cand = _draft_chains(bs, n, rng, target)
    print(f"[case] verify_chain bs={bs} n={n}", flush=True)
    pred, idx, acc = tsa.verify_chain(torch.from_numpy(cand).cuda(), torch.from_numpy(target).cuda())
    torch.cuda.synchronize()
    want_p, want_i, want_a = oracle.verify_chain(cand, target)
    assert np.array_equal(pred.cpu().numpy(), want_p)
    assert np.array_equal(idx.cpu().numpy(), want_i)
    assert np.array_equal(acc.cpu().numpy(), want_a)


def test_verify_chain_on_sampled_speculative_rows():
    """The speculative layout end to end: sample the decode rows of the mixed
    workload, draft chains that follow those samples part of the way, verify;
    int64 inputs are converted, and an empty batch is a no-op."""
    wl = synth.make("spec_mix", rows=24, vocab=16384)
    ids, lps = parity.gpu_sample(wl)
    ref = parity.oracle_sample(wl)
    parity.compare_samples(ids, lps, ref).check()
    n = 4                                           # 1 + 3 rows per decode request
    bs = int(np.sum(np.bincount(wl.token_to_request_index.numpy()) == n))   # decode requests
    rows = bs * n                                   # the decode rows come first
    rng = np.random.default_rng(3)
    target = ids[:rows].astype(np.int32)
    cand = _draft_chains(bs, n, rng, target)
    print(f"[case] verify_chain on sampled rows bs={bs}", flush=True)
    pred, idx, acc = tsa.verify_chain(torch.from_numpy(cand.astype(np.int64)).cuda(),
                                      torch.from_numpy(target.astype(np.int64)).cuda())
    torch.cuda.synchronize()
    # against the oracle's own samples where no row is a flagged near tie
    # (those are counted by compare_samples above and may differ by design)
    if not any(r.flagged for r in ref[:rows]):
        want_p, want_i, want_a = oracle.verify_chain(cand, np.array([r.token for r in ref[:rows]]))
        assert np.array_equal(pred.cpu().numpy(), want_p)
        assert np.array_equal(idx.cpu().numpy(), want_i)
        assert np.array_equal(acc.cpu().numpy(), want_a)
    e = tsa.verify_chain(torch.empty((0, 4), dtype=torch.int32, device="cuda"),
                         torch.empty(0, dtype=torch.int32, device="cuda"))
    assert e[0].numel() == 0 and e[2].numel() == 0


@pytest.mark.parametrize("n", [1, 63, 1000, 300001])
def test_check_indices_flags_out_of_range_entries(n):
    """The debug index check against the definition: the gather bit is set iff
    some gather index falls outside [0, rows), the request bit iff some request
    index falls outside [0, Q); arrays left out are not checked."""
    rng = np.random.default_rng(n)
    rows, q = 2 * n + 3, max(1, n // 3)
    print(f"[case] check_indices n={n}", flush=True)
    for trial in range(6):
        g = rng.integers(0, rows, n).astype(np.int32)
        m = rng.integers(0, q, n).astype(np.int32)
        if trial in (1, 3):
            g[rng.integers(0, n)] = rows if trial == 1 else -1
        if trial in (2, 3):
            m[rng.integers(0, n)] = q if trial == 2 else -7
        if trial == 4:
            g[-1] = np.iinfo(np.int32).max
            m[0] = np.iinfo(np.int32).min
        want = (tsa.INDEX_GATHER_OUT if ((g < 0) | (g >= rows)).any() else 0) | \
               (tsa.INDEX_REQUEST_OUT if ((m < 0) | (m >= q)).any() else 0)
        gd, md = torch.from_numpy(g).cuda(), torch.from_numpy(m).cuda()
        got = tsa.check_indices(n, gather_indices=gd, rows_in_buffer=rows,
                                token_to_request_index=md, num_requests=q)
        assert int(got.item()) == want, (trial, int(got.item()), want)
        only_g = tsa.check_indices(n, gather_indices=gd, rows_in_buffer=rows)
        only_m = tsa.check_indices(n, token_to_request_index=md.long(), num_requests=q)
        assert int(only_g.item()) == want & tsa.INDEX_GATHER_OUT
        assert int(only_m.item()) == want & tsa.INDEX_REQUEST_OUT
    assert int(tsa.check_indices(0, device="cuda").item()) == 0
