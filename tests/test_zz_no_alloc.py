"""ts_sample_noalloc against ts_sample through the C ABI: the same ids and
log-probs, bit for bit, on every route whose kernels use scratch memory (the
split no-filter kernel, the top-p cutoff and draw kernels) and on the joint
route, on two calls in a row, the second with a smaller input."""
import ctypes

import numpy as np
import pytest
import torch

import synth
import token_sampling_scaled_amd as tsa

pytestmark = pytest.mark.gpu


def _noalloc():
    lib = tsa.library()
    c_i32, c_i64, c_u64, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p
    f = lib.ts_sample_noalloc
    f.argtypes = [c_i64, c_vp, c_i32, c_i64, c_i64, c_i32, c_vp, c_vp, ctypes.POINTER(tsa._Params),
                  c_u64, c_i32, c_i32, c_vp, c_vp, c_vp]
    f.restype = c_i32
    return f


def _call_both(wl, step_offset):
    dev = torch.device("cuda", torch.cuda.current_device())
    x = wl.logits.to(dev)
    prm = tsa.SamplingParams(wl.temperature.to(dev), wl.seed.to(dev), wl.top_k.to(dev),
                             wl.top_p.to(dev))
    gather = None if wl.gather_indices is None else wl.gather_indices.to(dev)
    req = None if wl.token_to_request_index is None else wl.token_to_request_index.to(dev)
    s = tsa.Sampler(wl.vocab, wl.n)
    ids, lps = s.sample(x, wl.n, prm, no_top_k=wl.no_top_k, no_top_p=wl.no_top_p,
                        gather_indices=gather, token_to_request_index=req,
                        step_offset=step_offset, return_logprobs=True)
    ids2 = torch.full((wl.n,), -7, dtype=torch.int32, device=dev)
    lps2 = torch.full((wl.n,), 123.0, dtype=torch.float32, device=dev)
    p = prm._struct(dev)
    dt = tsa.TS_F32 if x.dtype == torch.float32 else tsa.TS_BF16
    st = _noalloc()(wl.vocab, ctypes.c_void_p(x.data_ptr()), dt, x.shape[0], x.stride(0), wl.n,
                    None if gather is None else ctypes.c_void_p(gather.data_ptr()),
                    None if req is None else ctypes.c_void_p(req.data_ptr()), ctypes.byref(p),
                    step_offset, int(wl.no_top_k), int(wl.no_top_p),
                    ctypes.c_void_p(ids2.data_ptr()), ctypes.c_void_p(lps2.data_ptr()),
                    ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    assert st == tsa.TS_OK, st
    torch.cuda.synchronize()
    return (ids.cpu().numpy(), lps.cpu().numpy()), (ids2.cpu().numpy(), lps2.cpu().numpy())


@pytest.mark.parametrize("name,sizes", [
    ("none_32k", [(None, None), (9, 4099)]),
    ("topp_152k", [(64, 40000), (5, 30011)]),
    ("joint_128k", [(None, None), (12, 20000)]),
    ("spec_mix", [(None, None), (24, 16384)]),
])
def test_noalloc_matches_ts_sample(name, sizes):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    for i, (rows, vocab) in enumerate(sizes):
        wl = synth.make(name, rows=rows, vocab=vocab)
        print(f"[case] noalloc {name} call {i} rows={wl.n} vocab={wl.vocab}", flush=True)
        (a_ids, a_lp), (b_ids, b_lp) = _call_both(wl, step_offset=3 + i)
        assert np.array_equal(a_ids, b_ids)
        assert np.array_equal(a_lp.view(np.int32), b_lp.view(np.int32))


def test_noalloc_rejects_sizes_beyond_its_maximum():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    f = _noalloc()
    x = torch.zeros(8, 100, device="cuda")
    prm = tsa.SamplingParams(torch.ones(2000, device="cuda"),
                             torch.zeros(2000, dtype=torch.int64, device="cuda")
                             )._struct(x.device)
    out = torch.empty(2000, dtype=torch.int32, device="cuda")
    st = f(100, ctypes.c_void_p(x.data_ptr()), tsa.TS_F32, 8, 100, 1025, ctypes.c_void_p(x.data_ptr()),
           None, ctypes.byref(prm), 0, 1, 1, ctypes.c_void_p(out.data_ptr()), None, None)
    assert st == tsa.TS_E_SIZE
    assert tsa.library().ts_status_str(st)
