"""Seeded random configurations against the oracle: dtype, vocabulary size,
value law, ties, -inf and NaN, per-row temperature / top-k / top-p (greedy and
inactive filters included), gather, request maps and offsets all drawn at
random, so that every kernel (register-resident bf16, short fp32, top-p route,
no-filter split, general body) and their fallbacks meet inputs no hand-written
case chose.  Ids and fused log-probs, and full log-prob rows, are compared row
by row."""
import numpy as np
import pytest
import torch

import synth
import token_sampling_scaled_amd as tsa
from tests import parity

pytestmark = pytest.mark.gpu

VOCABS = [8, 64, 1000, 4096, 8192, 20011, 65536]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tsa.library()


def _random_workload(case: int) -> synth.Workload:
    rng = np.random.default_rng(5000 + case)
    dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float32
    v = int(rng.choice(VOCABS))
    n = int(rng.integers(1, 13))
    q = n if rng.random() < 0.5 else int(rng.integers(1, n + 1))
    buf_rows = n + int(rng.integers(0, 4))
    mu = rng.uniform(-20.0, 5.0, size=(buf_rows, 1))
    sigma = rng.choice([0.1, 1.0, 3.0, 10.0], size=(buf_rows, 1))
    x = rng.normal(0.0, 1.0, size=(buf_rows, v)) * sigma + mu
    if rng.random() < 0.4:                                   # heavy ties
        x = np.round(x * 4.0) / 4.0
    if rng.random() < 0.4:                                   # spikes
        for r in range(buf_rows):
            x[r, rng.choice(v, min(5, v), replace=False)] += 8.0
    if rng.random() < 0.3:                                   # -inf and NaN entries
        m = rng.random(x.shape)
        x[m < 0.05] = -np.inf
        x[(m >= 0.05) & (m < 0.06)] = np.nan
    t = rng.choice([0.0, 0.3, 1.0, 2.0], size=q).astype(np.float32)
    k = np.where(rng.random(q) < 0.3, 0,
                 np.where(rng.random(q) < 0.5, rng.integers(1, 1025, q), rng.integers(1, v + 1, q)))
    p = np.where(rng.random(q) < 0.3, 1.0, rng.uniform(0.05, 0.999, q)).astype(np.float32)
    wl = synth.Workload(f"random{case}", torch.from_numpy(x.astype(np.float32)).to(dtype), n,
                        torch.from_numpy(t), torch.from_numpy(k.astype(np.int32)),
                        torch.from_numpy(p), torch.from_numpy(rng.integers(0, 2**62, q)))
    if buf_rows > n or rng.random() < 0.3:
        wl.gather_indices = torch.from_numpy(rng.integers(0, buf_rows, n).astype(np.int32))
    if q < n or rng.random() < 0.3:
        wl.token_to_request_index = torch.from_numpy(rng.integers(0, q, n).astype(np.int32))
    wl.no_top_k = bool(np.all(k == 0)) and rng.random() < 0.8
    wl.no_top_p = bool(np.all(p >= 1.0)) and rng.random() < 0.8
    if wl.no_top_k:
        wl.top_k.zero_()
    if wl.no_top_p:
        wl.top_p.fill_(1.0)
    wl.step_offset = int(rng.integers(0, 2**40))
    return wl


@pytest.mark.parametrize("case", range(64))
def test_random_configuration(case):
    wl = _random_workload(case)
    print(f"[case] random {case}: {wl.logits.dtype} rows={wl.n} vocab={wl.vocab} "
          f"gather={wl.gather_indices is not None} map={wl.token_to_request_index is not None} "
          f"no_top_k={wl.no_top_k} no_top_p={wl.no_top_p}", flush=True)
    s = tsa.Sampler(wl.vocab, wl.n)
    dev = parity.to_device(wl)
    ids, lps = parity.gpu_sample(wl, s, dev)
    res = parity.oracle_sample(wl)
    parity.compare_samples(ids, lps, res).check()
    gpu = parity.gpu_log_probs(wl, s, dev)
    parity.compare_log_probs(gpu, parity.oracle_log_probs(wl), res).check()
