"""ctypes binding of the measurement probes in ``libtsprobe.so`` (declared in
``include/tsprobe.h``): the streaming-read ceiling at the sampling kernel's
launch shape, an empty launch, and the device noise transforms evaluated on
their whole domain.  Used by ``bench.py`` and the GPU tests; the sampling path
never calls them."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(_HERE, "libtsprobe.so")

_lib = None


def library() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(PROBE_LIB_PATH):
        raise RuntimeError(f"{PROBE_LIB_PATH} is missing: build it with "
                           "`python -m token_sampling_scaled_amd.build`")
    lib = ctypes.CDLL(PROBE_LIB_PATH)
    c_i32, c_i64, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.tsp_read_rows.argtypes = [c_vp, c_i64, c_i64, c_i64, c_i32, c_vp, c_vp]
    lib.tsp_read_rows_ring.argtypes = [c_vp, c_i64, c_i64, c_i64, c_i32, c_i32, c_i32, c_vp, c_vp]
    lib.tsp_empty.argtypes = [c_i32, c_vp]
    lib.tsp_gumbel_table.argtypes = [c_vp, c_vp, c_vp]
    lib.tsp_noise_rate.argtypes = [c_i32, c_i32, c_i32, c_vp, c_vp]
    for name in ("tsp_read_rows", "tsp_read_rows_ring", "tsp_empty", "tsp_gumbel_table",
                 "tsp_noise_rate"):
        getattr(lib, name).restype = c_i32
    _lib = lib
    return lib


def _check(st: int, what: str) -> None:
    if st != 0:
        raise (ValueError if st == 1 else RuntimeError)(f"{what} failed with status {st}")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def read_rows_args(data: torch.Tensor, n: int, row_bytes: int, loads_per_thread: int,
                   out: torch.Tensor):
    """Argument list of one tsp_read_rows call over the first n rows of ``data``
    (a 2-D GPU tensor), built once so a timing loop only calls the library."""
    stride = data.stride(0) * data.element_size()
    return [ctypes.c_void_p(data.data_ptr()), int(n), int(row_bytes), int(stride),
            int(loads_per_thread), ctypes.c_void_p(out.data_ptr()), _stream(data.device)]


def read_rows(data: torch.Tensor, n: int, row_bytes: int, loads_per_thread: int,
              out: torch.Tensor) -> None:
    _check(library().tsp_read_rows(*read_rows_args(data, n, row_bytes, loads_per_thread, out)),
           "tsp_read_rows")


def read_rows_ring_args(data: torch.Tensor, n: int, row_bytes: int, threads: int, parts: int,
                       nontemporal: bool, out: torch.Tensor):
    """Argument list of one tsp_read_rows_ring call over the first n rows of ``data``."""
    stride = data.stride(0) * data.element_size()
    return [ctypes.c_void_p(data.data_ptr()), int(n), int(row_bytes), int(stride), int(threads),
            int(parts), int(bool(nontemporal)), ctypes.c_void_p(out.data_ptr()),
            _stream(data.device)]


def empty(blocks: int, device) -> None:
    _check(library().tsp_empty(int(blocks), _stream(device)), "tsp_empty")


def noise_rate(blocks: int, per_thread: int, with_gumbel: bool, out: torch.Tensor) -> None:
    """Launch the noise throughput probe on the current stream (out: int32 [blocks * 256])."""
    if out.dtype != torch.int32 or not out.is_cuda or out.numel() < blocks * 256:
        raise ValueError("out must be a CUDA int32 tensor of at least blocks * 256 elements")
    _check(library().tsp_noise_rate(blocks, per_thread, 1 if with_gumbel else 0,
                                    ctypes.c_void_p(out.data_ptr()), _stream(out.device)),
           "tsp_noise_rate")


def gumbel_table(device="cuda"):
    """(g, g2): the device's -ln(-ln u) and -log2(-log2 u) for every one of the
    2^23 uniforms u_i = (i + 1/2) 2^-23, as float32 GPU tensors."""
    g = torch.empty(1 << 23, dtype=torch.float32, device=device)
    g2 = torch.empty_like(g)
    _check(library().tsp_gumbel_table(ctypes.c_void_p(g.data_ptr()), ctypes.c_void_p(g2.data_ptr()),
                                      _stream(g.device)), "tsp_gumbel_table")
    return g, g2
