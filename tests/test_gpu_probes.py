"""GPU checks of the measurement probes and of the device noise transform.

The sampling kernels turn a Philox word w into Gumbel noise with the hardware
base-2 logarithm and no log1p branch next to u = 1 (device_common.hpp,
gumbel_from_word / gumbel2_from_word).  The probe library evaluates exactly
those functions for every one of the 2^23 uniforms u = (i + 1/2) 2^-23 they
can see; here they are held to the oracle's fp64 transform
(oracle.philox.gumbel_from_uniform, which takes -ln u through log1p for
u > 1/2).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from token_sampling_scaled_amd import probes

pytestmark = pytest.mark.gpu

# |g_device - g_fp64| <= GUMBEL_REL_BOUND * max(1, |g_fp64|) for every u: ten
# times inside the 1e-5 relative band within which the parity tests accept
# either of two near-tied perturbed scores.
GUMBEL_REL_BOUND = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    probes.library()


def test_device_gumbel_transform_on_every_uniform():
    print("[case] gumbel table 2^23", flush=True)
    g, g2 = probes.gumbel_table()
    torch.cuda.synchronize()
    g = g.cpu().numpy().astype(np.float64)
    g2 = g2.cpu().numpy().astype(np.float64)
    i = np.arange(1 << 23, dtype=np.uint64)
    ref = oracle.gumbel_from_uniform(oracle.uniform_from_words(i << np.uint64(9)))
    ref2 = (ref + math.log(math.log(2.0))) / math.log(2.0)
    scale = np.maximum(1.0, np.abs(ref))
    err = np.abs(g - ref) / scale
    err2 = np.abs(g2 - ref2) / np.maximum(1.0, np.abs(ref2))
    hi = i >= (1 << 22)                                   # u > 1/2, where the winners come from
    print(f"[gumbel] max rel err natural {err.max():.3e} (u>1/2: {err[hi].max():.3e}, "
          f"at u index {int(np.argmax(err))}); base-2 {err2.max():.3e} "
          f"(u>1/2: {err2[hi].max():.3e})", flush=True)
    assert np.all(np.isfinite(g)) and np.all(np.isfinite(g2))
    assert err.max() <= GUMBEL_REL_BOUND
    assert err2.max() <= GUMBEL_REL_BOUND
    # the endpoints: u = 2^-24 gives the smallest noise, u = 1 - 2^-24 the largest
    assert abs(g[0] - ref[0]) <= GUMBEL_REL_BOUND * abs(ref[0])
    assert abs(g[-1] - ref[-1]) <= GUMBEL_REL_BOUND * abs(ref[-1])


def test_read_probe_reads_every_vector():
    """The read-ceiling probe touches every 16-byte vector of each row: its
    per-row xor equals the host's."""
    rng = np.random.default_rng(4)
    rows, row_bytes = 5, 16 * 16032
    host = rng.integers(0, 2**32, size=(rows, row_bytes // 4 + 12), dtype=np.uint64).astype(np.uint32)
    data = torch.from_numpy(host.view(np.int32)).cuda()
    out = torch.zeros(rows, dtype=torch.int32, device="cuda")
    print("[case] read probe", flush=True)
    probes.read_rows(data, rows, row_bytes, 16, out)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host[:, :row_bytes // 4], axis=1)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want)
