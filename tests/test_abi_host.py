"""Host-side tests of the C ABI: the library loads, exports what the header
declares, routes flags, and rejects bad arguments before touching a GPU."""
import ctypes
import json
import os
import re

import pytest

import token_sampling_scaled_amd as tsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tssample.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tsa.LIB_PATH):
        from token_sampling_scaled_amd import build
        build.build()
    return tsa.library()


def _declared(header=HEADER, prefix="ts_"):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(" + prefix + r"[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert "ts_sample" in names and "ts_log_probs" in names
    for name in names:
        assert hasattr(lib, name), name


def test_probe_library_exports_and_checks_arguments(lib):
    from token_sampling_scaled_amd import probes
    plib = probes.library()
    names = _declared(os.path.join(ROOT, "include", "tsprobe.h"), "tsp_")
    assert names == ["tsp_empty", "tsp_gumbel_table", "tsp_noise_rate", "tsp_read_rows",
                     "tsp_read_rows_ring"]
    for name in names:
        assert hasattr(plib, name), name
    # argument errors come back before any HIP call
    assert plib.tsp_empty(0, None) == 1
    assert plib.tsp_gumbel_table(None, None, None) == 1
    assert plib.tsp_noise_rate(0, 1, 0, FAKE, None) == 1
    assert plib.tsp_noise_rate(4, 0, 1, FAKE, None) == 1
    assert plib.tsp_noise_rate(4, 1, 1, None, None) == 1
    assert plib.tsp_read_rows_ring(FAKE, 4, 256, 256, 128, 1, 0, FAKE, None) == 1   # bad block
    assert plib.tsp_read_rows_ring(FAKE, 4, 256, 256, 256, 65, 0, FAKE, None) == 1  # parts > 64
    assert plib.tsp_read_rows(None, 4, 256, 256, 1, FAKE, None) == 1
    assert plib.tsp_read_rows(FAKE, 4, 250, 256, 1, FAKE, None) == 1       # not 16-byte rows
    assert plib.tsp_read_rows(FAKE, 4, 16 * 1024 * 2, 16 * 1024 * 2, 1, FAKE, None) == 1
    assert plib.tsp_read_rows(FAKE, 4, 256, 256, 3, FAKE, None) == 1
    assert plib.tsp_read_rows(FAKE, 0, 256, 256, 1, FAKE, None) == 1


def test_status_strings_and_routes(lib):
    for code in range(6):
        assert lib.ts_status_str(code)
    # "flashinfer_sampling": dedicated kernels for one filter, joint for mixed batches
    assert lib.ts_select_route(1, 1) == tsa.ROUTE_NONE
    assert lib.ts_select_route(0, 1) == tsa.ROUTE_TOPK
    assert lib.ts_select_route(1, 0) == tsa.ROUTE_TOPP
    assert lib.ts_select_route(0, 0) == tsa.ROUTE_JOINT


def test_create_argument_errors(lib):
    h = ctypes.c_void_p()
    assert lib.ts_create(0, 4, -1, ctypes.byref(h)) == tsa.TS_E_ARG
    assert lib.ts_create(100, 0, -1, ctypes.byref(h)) == tsa.TS_E_ARG
    assert lib.ts_create(2**31, 4, -1, ctypes.byref(h)) == tsa.TS_E_ARG
    assert lib.ts_create(100, 4, -2, ctypes.byref(h)) == tsa.TS_E_ARG
    assert lib.ts_create(100, 4, -1, None) == tsa.TS_E_ARG


FAKE = 0x10000   # never dereferenced: a validation-only handle enqueues nothing


def _params(temperature=FAKE, top_k=FAKE, top_p=FAKE, seed=FAKE, q=8):
    return tsa._Params(temperature, top_k, top_p, seed, q)


def test_sample_argument_checks_on_validation_handle(lib):
    h = ctypes.c_void_p()
    assert lib.ts_create(100, 8, -1, ctypes.byref(h)) == tsa.TS_OK
    try:
        def call(logits=FAKE, dtype=tsa.TS_BF16, rows=8, stride=100, n=8, gather=None, req=None,
                 params=None, nk=0, np_=0, out=FAKE, lp=None):
            p = params if params is not None else _params()
            return lib.ts_sample(h, logits, dtype, rows, stride, n, gather, req, ctypes.byref(p),
                                 0, nk, np_, out, lp, None)
        assert call() == tsa.TS_E_HIP                      # all checks pass, no GPU on this handle
        assert call(n=0) == tsa.TS_OK                      # nothing to do
        assert call(dtype=7) == tsa.TS_E_DTYPE
        assert call(n=9) == tsa.TS_E_SIZE                  # above max_rows
        assert call(n=-1) == tsa.TS_E_ARG
        assert call(stride=99) == tsa.TS_E_SIZE            # stride below vocab
        assert call(rows=4) == tsa.TS_E_SIZE               # fewer rows than n, no gather
        assert call(rows=4, gather=FAKE) == tsa.TS_E_HIP   # gathered rows may repeat
        assert call(logits=None) == tsa.TS_E_ARG
        assert call(out=None) == tsa.TS_E_ARG
        assert call(params=_params(top_k=None)) == tsa.TS_E_ARG           # k used, array missing
        assert call(params=_params(top_k=None), nk=1) == tsa.TS_E_HIP     # flag promises no top-k
        assert call(params=_params(top_p=None)) == tsa.TS_E_ARG
        assert call(params=_params(top_p=None), np_=1) == tsa.TS_E_HIP
        assert call(params=_params(temperature=None)) == tsa.TS_E_ARG
        assert call(params=_params(seed=None)) == tsa.TS_E_ARG
        assert call(params=_params(q=4)) == tsa.TS_E_SIZE                 # q = r needs >= n slots
        assert call(params=_params(q=4), req=FAKE) == tsa.TS_E_HIP
        assert call(params=_params(q=0), req=FAKE) == tsa.TS_E_ARG
        p = _params()
        assert lib.ts_log_probs(h, FAKE, tsa.TS_F32, 8, 100, 8, None, None, ctypes.byref(p),
                                0, 0, None, None, None) == tsa.TS_E_ARG   # no output
        assert lib.ts_log_probs(h, FAKE, tsa.TS_F32, 8, 100, 8, None, None, ctypes.byref(p),
                                0, 0, None, FAKE, None) == tsa.TS_E_HIP
        assert lib.ts_sample(None, FAKE, 0, 8, 100, 8, None, None, ctypes.byref(p), 0, 0, 0,
                             FAKE, None, None) == tsa.TS_E_ARG
    finally:
        lib.ts_destroy(h)


def test_spec_map_on_host(lib):
    with open(os.path.join(ROOT, "tests", "golden", "spec_layout.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        m, n = tsa.build_spec_map(c["num_decode"], c["num_prefill"], c["num_spec"])
        assert n == len(c["map"]) and m.tolist() == c["map"]
    got = ctypes.c_int32()
    buf = (ctypes.c_int32 * 4)()
    assert lib.ts_build_spec_map(2, 2, 3, buf, 4, 0, None, ctypes.byref(got)) == tsa.TS_E_SIZE
    assert got.value == 10
    assert lib.ts_build_spec_map(-1, 2, 3, buf, 4, 0, None, ctypes.byref(got)) == tsa.TS_E_ARG


def test_raw_log_probs_argument_checks_on_validation_handle(lib):
    h = ctypes.c_void_p()
    assert lib.ts_create(100, 8, -1, ctypes.byref(h)) == tsa.TS_OK
    try:
        def call(logits=FAKE, dtype=tsa.TS_BF16, rows=8, stride=100, n=8, gather=None, ids=FAKE,
                 out=FAKE):
            return lib.ts_raw_log_probs_at(h, logits, dtype, rows, stride, n, gather, ids, out, None)
        assert call() == tsa.TS_E_HIP                      # all checks pass, no GPU on this handle
        assert call(n=0) == tsa.TS_OK
        assert call(dtype=7) == tsa.TS_E_DTYPE
        assert call(n=9) == tsa.TS_E_SIZE
        assert call(stride=99) == tsa.TS_E_SIZE
        assert call(rows=4) == tsa.TS_E_SIZE
        assert call(rows=4, gather=FAKE) == tsa.TS_E_HIP
        assert call(logits=None) == tsa.TS_E_ARG
        assert call(ids=None) == tsa.TS_E_ARG
        assert call(out=None) == tsa.TS_E_ARG
        assert lib.ts_raw_log_probs_at(None, FAKE, 0, 8, 100, 8, None, FAKE, FAKE,
                                       None) == tsa.TS_E_ARG
    finally:
        lib.ts_destroy(h)


def test_check_indices_argument_checks(lib):
    # every argument error returns before any GPU call
    assert lib.ts_check_indices(-1, FAKE, 8, None, 0, FAKE, None) == tsa.TS_E_ARG
    assert lib.ts_check_indices(4, FAKE, 8, None, 0, None, None) == tsa.TS_E_ARG
    assert lib.ts_check_indices(4, FAKE, 0, None, 0, FAKE, None) == tsa.TS_E_ARG
    assert lib.ts_check_indices(4, None, 0, FAKE, 0, FAKE, None) == tsa.TS_E_ARG
    assert lib.ts_check_indices(4, FAKE, -3, FAKE, 2, FAKE, None) == tsa.TS_E_ARG


def test_verify_chain_argument_checks(lib):
    # error paths and the empty batch return before any GPU call
    assert lib.ts_verify_chain(0, 4, None, None, None, None, None, None) == tsa.TS_OK
    assert lib.ts_verify_chain(-1, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None) == tsa.TS_E_ARG
    assert lib.ts_verify_chain(2, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == tsa.TS_E_ARG
    assert lib.ts_verify_chain(1 << 20, 1 << 12, FAKE, FAKE, FAKE, FAKE, FAKE, None) == tsa.TS_E_SIZE
    for k in range(5):
        ptrs = [FAKE] * 5
        ptrs[k] = None
        assert lib.ts_verify_chain(2, 4, *ptrs, None) == tsa.TS_E_ARG


def test_stage_marks_only_in_the_marks_build(lib):
    # the product library compiles the stage marks out; the marks build
    # (python -m token_sampling_scaled_amd.build --stage-marks) exports them
    from token_sampling_scaled_amd import build
    assert not hasattr(lib, "tss_stage_marks")
    if not os.path.exists(build.MARKS_LIB):
        pytest.skip("libtssample_marks.so not built")
    marks = ctypes.CDLL(build.MARKS_LIB)
    assert hasattr(marks, "tss_stage_marks") and hasattr(marks, "tss_stage_marks_clear")
    marks.tss_stage_marks.argtypes = [ctypes.c_void_p, ctypes.c_int]
    # argument errors return 0 before any HIP call
    assert marks.tss_stage_marks(None, 4) == 0
    assert marks.tss_stage_marks(ctypes.c_void_p(FAKE), 0) == 0
    assert marks.tss_stage_marks(ctypes.c_void_p(FAKE), 1025) == 0
