"""GPU parity of ts_apply_vocab_mask: the masked logits bit for bit against the
oracle's mask, and mask-then-sample against the oracle on the masked logits."""
import copy

import numpy as np
import pytest
import torch

import oracle
import synth
import token_sampling_scaled_amd as tsa
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tsa.library()


def _masks(rng, rows, v, densities):
    """int32 mask words [rows, ceil(v / 32)]: row r allows each entry with
    probability densities[r % len(densities)]."""
    w = (v + 31) // 32
    bits = np.zeros((rows, w * 32), dtype=bool)
    for r in range(rows):
        bits[r, :v] = rng.random(v) < densities[r % len(densities)]
    words = np.packbits(bits.reshape(rows, w, 4, 8), axis=-1, bitorder="little").reshape(rows, w * 4)
    return words.view(np.uint32).astype(np.int64), torch.from_numpy(words.view(np.int32).copy())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,v,pad,use_index", [(5, 1003, 0, False), (3, 4096, 0, True),
                                                  (4, 777, 5, False), (7, 131072, 0, False),
                                                  (2, 33, 3, True)])
def test_mask_is_bit_exact(dtype, rows, v, pad, use_index):
    print(f"[case] vocab_mask dtype={dtype} rows={rows} v={v} pad={pad} index={use_index}", flush=True)
    rng = np.random.default_rng(rows * 1000 + v)
    buf = torch.from_numpy(rng.normal(size=(rows, v + pad)).astype(np.float32) * 4).to(dtype)
    dens = [0.0, 0.02, 0.5, 0.97, 1.0]
    nmask = 3 if use_index else rows
    words, mask_t = _masks(rng, nmask, v, dens)
    index = rng.integers(0, nmask, size=rows).astype(np.int32) if use_index else None
    dev = buf.to("cuda")
    tsa.apply_vocab_mask(dev[:, :v], mask_t.to("cuda"),
                         None if index is None else torch.from_numpy(index).to("cuda"))
    torch.cuda.synchronize()
    got = dev.cpu()
    want = oracle.apply_vocab_mask(buf[:, :v].double().numpy(), words, mask_index=index)
    # bit for bit: allowed entries unchanged, masked entries the -inf pattern
    assert np.array_equal(got[:, :v].double().numpy(), want)
    assert torch.equal(got[:, v:], buf[:, v:])             # padding untouched


def test_mask_then_sample_matches_oracle():
    rng = np.random.default_rng(5)
    for name, rows, vocab in [("joint_128k", 12, 20000), ("topp_152k", 6, 30000),
                              ("none_32k", 8, 32000), ("topk_128k", 8, 20011)]:
        wl = synth.make(name, rows=rows, vocab=vocab)
        print(f"[case] mask+sample {name} rows={wl.n} vocab={wl.vocab}", flush=True)
        nb = wl.logits.shape[0]
        words, mask_t = _masks(rng, nb, wl.vocab, [0.3, 0.9, 0.05])
        dev = parity.to_device(wl)
        tsa.apply_vocab_mask(dev["logits"], mask_t.to("cuda"))
        masked = copy.copy(wl)
        xm = oracle.apply_vocab_mask(wl.logits.double().numpy(), words)
        masked.logits = torch.from_numpy(xm).to(wl.logits.dtype)
        ids, lps = parity.gpu_sample(wl, dev=dev)
        res = parity.oracle_sample(masked)
        for r in range(wl.n):
            src = r if wl.gather_indices is None else int(wl.gather_indices[r])
            if ids[r] >= 0:
                assert oracle.vocab_mask.entry_allowed(words[src], int(ids[r])), (name, r)
        parity.compare_samples(ids, lps, res).check(f"vocab_mask {name}")


def test_argument_errors():
    lib = tsa.library()
    x = torch.zeros(2, 64, device="cuda")
    m = torch.zeros(2, 2, dtype=torch.int32, device="cuda")
    p = x.data_ptr()
    assert lib.ts_apply_vocab_mask(64, p, tsa.TS_F32, 2, 64, None, 2, None, None) == tsa.TS_E_ARG
    assert lib.ts_apply_vocab_mask(64, p, tsa.TS_F32, 2, 64, m.data_ptr(), 1, None, None) == tsa.TS_E_SIZE
    assert lib.ts_apply_vocab_mask(64, p, tsa.TS_F32, 2, 63, m.data_ptr(), 2, None, None) == tsa.TS_E_SIZE
    assert lib.ts_apply_vocab_mask(64, p, 7, 2, 64, m.data_ptr(), 2, None, None) == tsa.TS_E_DTYPE
    assert lib.ts_apply_vocab_mask(0, p, tsa.TS_F32, 2, 64, m.data_ptr(), 2, None, None) == tsa.TS_E_ARG
    assert lib.ts_apply_vocab_mask(64, None, tsa.TS_F32, 0, 64, None, 2, None, None) == tsa.TS_OK
    with pytest.raises(ValueError):
        tsa.apply_vocab_mask(x, m[:, :1])
