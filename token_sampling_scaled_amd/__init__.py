"""Batched categorical token sampling on MI355X (gfx950).

Thin Python binding over the C ABI of ``libtssample.so`` (declared in
``include/tssample.h``).  This module only marshals arguments: torch tensors
supply device memory and the current HIP stream, and every step of the
sampling path runs in the library's HIP kernels.  There is no CPU fallback:
importing works without the library, but any call raises if it is missing.

API (after "core.inference.sampling.base" and
"core.inference.sampling.flashinfer_sampling", Megatron-Core API docs):

    params = SamplingParams(temperature, top_k, top_p, seed)     # per request
    s = Sampler(vocab_size, max_rows)
    ids = s.sample(logits, n, params, no_top_k=False, no_top_p=False,
                   gather_indices=None, token_to_request_index=None, step_offset=0)
    ids, lp = s.sample(..., return_logprobs=True)
    ids = s.sample_speculative(required_logits, num_decode, num_prefill,
                               num_speculative_tokens, params, gather_indices=None, ...)
    lp = s.log_probs(logits, params, ...)          # [n, V], or [n] with token_ids
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtssample.so")

TS_OK, TS_E_ARG, TS_E_DTYPE, TS_E_SIZE, TS_E_HIP, TS_E_NOMEM = range(6)
TS_F32, TS_BF16 = 0, 1
ROUTE_NONE, ROUTE_TOPK, ROUTE_TOPP, ROUTE_JOINT = range(4)

_STATUS_ERRORS = {TS_E_ARG: ValueError, TS_E_DTYPE: TypeError, TS_E_SIZE: ValueError,
                  TS_E_HIP: RuntimeError, TS_E_NOMEM: MemoryError}


class _Params(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_void_p), ("top_k", ctypes.c_void_p),
                ("top_p", ctypes.c_void_p), ("seed", ctypes.c_void_p),
                ("num_requests", ctypes.c_int32), ("step_offsets", ctypes.c_void_p)]


_lib = None


def library() -> ctypes.CDLL:
    """Load libtssample.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m token_sampling_scaled_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    c_i32, c_i64, c_u64, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p
    lib.ts_create.argtypes = [c_i64, c_i32, c_i32, ctypes.POINTER(c_vp)]
    lib.ts_destroy.argtypes = [c_vp]
    lib.ts_sample.argtypes = [c_vp, c_vp, c_i32, c_i64, c_i64, c_i32, c_vp, c_vp,
                              ctypes.POINTER(_Params), c_u64, c_i32, c_i32, c_vp, c_vp, c_vp]
    lib.ts_log_probs.argtypes = [c_vp, c_vp, c_i32, c_i64, c_i64, c_i32, c_vp, c_vp,
                                 ctypes.POINTER(_Params), c_i32, c_i32, c_vp, c_vp, c_vp]
    lib.ts_raw_log_probs_at.argtypes = [c_vp, c_vp, c_i32, c_i64, c_i64, c_i32, c_vp, c_vp,
                                        c_vp, c_vp]
    lib.ts_build_spec_map.argtypes = [c_i32, c_i32, c_i32, c_vp, c_i32, c_i32, c_vp,
                                      ctypes.POINTER(c_i32)]
    lib.ts_verify_chain.argtypes = [c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]
    lib.ts_apply_vocab_mask.argtypes = [c_i64, c_vp, c_i32, c_i64, c_i64, c_vp, c_i64, c_vp, c_vp]
    lib.ts_check_indices.argtypes = [c_i32, c_vp, c_i64, c_vp, c_i32, c_vp, c_vp]
    lib.ts_select_route.argtypes = [c_i32, c_i32]
    lib.ts_status_str.argtypes = [c_i32]
    lib.ts_status_str.restype = ctypes.c_char_p
    for name in ("ts_create", "ts_destroy", "ts_sample", "ts_log_probs", "ts_raw_log_probs_at",
                 "ts_build_spec_map", "ts_verify_chain", "ts_apply_vocab_mask", "ts_select_route",
                 "ts_check_indices"):
        getattr(lib, name).restype = ctypes.c_int32
    _lib = lib
    return lib


def _check(status: int, what: str) -> None:
    if status != TS_OK:
        msg = library().ts_status_str(status).decode()
        raise _STATUS_ERRORS.get(status, RuntimeError)(f"{what}: {msg} (status {status})")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _index_i32(t: Optional[torch.Tensor], name: str, n: int, device) -> Optional[torch.Tensor]:
    """int32 index arrays pass through; int64 is converted; other dtypes are rejected
    (the TokenSpeed Triton backend page applies the same rule to request-pool indices)."""
    if t is None:
        return None
    if t.dtype not in (torch.int32, torch.int64):
        raise ValueError(f"{name} must be int32 or int64, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dim() != 1 or t.numel() < n:
        raise ValueError(f"{name} must be 1-D with at least n={n} entries")
    t = t[:n]
    if t.dtype == torch.int64:
        t = t.to(torch.int32)
    return t.contiguous()


@dataclass
class SamplingParams:
    """Per-request parameter arrays (device tensors), indexed by request slot."""
    temperature: torch.Tensor            # float32 [Q]
    seed: torch.Tensor                   # int64 [Q] (read as uint64)
    top_k: Optional[torch.Tensor] = None  # int32 [Q]; k <= 0 or k >= V: off
    top_p: Optional[torch.Tensor] = None  # float32 [Q]; p >= 1 - 1e-6: off
    # int64 [Q] (read as uint64): per-request Philox offsets added to the call's
    # step_offset; read on the device, so a captured call can be advanced
    step_offsets: Optional[torch.Tensor] = None

    def _struct(self, device) -> _Params:
        q = self.temperature.numel()
        for name, t, dt in (("temperature", self.temperature, torch.float32),
                            ("seed", self.seed, torch.int64),
                            ("top_k", self.top_k, torch.int32),
                            ("top_p", self.top_p, torch.float32),
                            ("step_offsets", self.step_offsets, torch.int64)):
            if t is None:
                continue
            if t.dtype != dt or t.device != device or not t.is_contiguous() or t.numel() != q:
                raise ValueError(f"params.{name} must be a contiguous {dt} tensor of {q} "
                                 f"entries on {device}")
        return _Params(_ptr(self.temperature), _ptr(self.top_k), _ptr(self.top_p),
                       _ptr(self.seed), q, _ptr(self.step_offsets))


def select_route(no_top_k: bool, no_top_p: bool) -> int:
    return int(library().ts_select_route(int(bool(no_top_k)), int(bool(no_top_p))))


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_out(t: torch.Tensor, dtype, numel: int, device, name: str,
               shape: Optional[tuple] = None) -> None:
    """A caller-supplied output buffer: right dtype and device, contiguous, large enough
    (the kernels write through its raw pointer)."""
    ok = (t.dtype == dtype and t.device == device and t.is_contiguous()
          and (t.numel() >= numel if shape is None else tuple(t.shape) == shape))
    if not ok:
        want = f"shape {shape}" if shape is not None else f">= {numel} entries"
        raise ValueError(f"{name} must be a contiguous {dtype} tensor with {want} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def _logits_args(logits: torch.Tensor, vocab: int, device=None):
    if device is not None and logits.device != device:
        raise ValueError(f"logits must be on the sampler's device {device}, got {logits.device}")
    if logits.device.type != "cuda":
        raise ValueError(f"logits must be a GPU tensor, got {logits.device}")
    if logits.dim() != 2:
        raise ValueError("logits must be 2-D [rows, vocab]")
    if logits.dtype == torch.float32:
        dt = TS_F32
    elif logits.dtype == torch.bfloat16:
        dt = TS_BF16
    else:
        raise TypeError(f"logits must be float32 or bfloat16, got {logits.dtype}")
    if logits.shape[1] != vocab:
        raise ValueError(f"logits have {logits.shape[1]} columns, sampler vocab is {vocab}")
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous (stride(1) == 1)")
    return dt, logits.shape[0], logits.stride(0)


class Sampler:
    """A sampler handle for one vocabulary size and a maximum row count."""

    def __init__(self, vocab_size: int, max_rows: int, device=None):
        lib = library()
        dev = torch.device("cuda") if device is None else torch.device(device)
        if dev.type != "cuda":
            raise ValueError(f"a Sampler lives on a GPU, got {dev}")
        self.device = dev if dev.index is not None else torch.device("cuda", torch.cuda.current_device())
        self.vocab = int(vocab_size)
        self.max_rows = int(max_rows)
        h = ctypes.c_void_p()
        _check(lib.ts_create(self.vocab, self.max_rows, self.device.index or 0, ctypes.byref(h)),
               "ts_create")
        self._h = h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            library().ts_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def sample(self, logits: torch.Tensor, n: int, params: SamplingParams, *,
               no_top_k: bool = False, no_top_p: bool = False,
               gather_indices: Optional[torch.Tensor] = None,
               token_to_request_index: Optional[torch.Tensor] = None,
               step_offset: int = 0, output: Optional[torch.Tensor] = None,
               logprob_output: Optional[torch.Tensor] = None, return_logprobs: bool = False):
        """Sample n ids from rows of ``logits`` (``logits[gather_indices[:n]]`` when given)."""
        dt, rows, stride = _logits_args(logits, self.vocab, self.device)
        dev = logits.device
        gather = _index_i32(gather_indices, "gather_indices", n, dev)
        req = _index_i32(token_to_request_index, "token_to_request_index", n, dev)
        if output is None:
            output = torch.empty(n, dtype=torch.int32, device=dev)
        else:
            _check_out(output, torch.int32, n, dev, "output")
        lp = logprob_output
        if lp is None and return_logprobs:
            lp = torch.empty(n, dtype=torch.float32, device=dev)
        elif lp is not None:
            _check_out(lp, torch.float32, n, dev, "logprob_output")
        p = params._struct(dev)
        _check(library().ts_sample(self._h, _ptr(logits), dt, rows, stride, int(n), _ptr(gather),
                                   _ptr(req), ctypes.byref(p), int(step_offset) & (2**64 - 1),
                                   int(bool(no_top_k)), int(bool(no_top_p)), _ptr(output),
                                   _ptr(lp), _stream(dev)), "ts_sample")
        if return_logprobs:
            return output[:n], lp[:n]
        return output[:n]

    def sample_speculative(self, required_logits: torch.Tensor, num_decode: int, num_prefill: int,
                           num_speculative_tokens: int, params: SamplingParams, *,
                           gather_indices: Optional[torch.Tensor] = None, **kw):
        """Speculative-verify sampling: builds the per-row request map, then samples.

        With ``gather_indices`` the rows are ``required_logits[gather_indices[:n]]``;
        without, ``required_logits`` is already in the layout (decode blocks, then prefill)."""
        req, n = build_spec_map(num_decode, num_prefill, num_speculative_tokens,
                                device=required_logits.device)
        return self.sample(required_logits, n, params, gather_indices=gather_indices,
                           token_to_request_index=req, **kw)

    def log_probs(self, logits: torch.Tensor, params: SamplingParams, *, n: Optional[int] = None,
                  no_top_k: bool = False, no_top_p: bool = False,
                  gather_indices: Optional[torch.Tensor] = None,
                  token_to_request_index: Optional[torch.Tensor] = None,
                  token_ids: Optional[torch.Tensor] = None,
                  output: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Log-probs of the processed distribution: [n, V], or [n] at ``token_ids``."""
        dt, rows, stride = _logits_args(logits, self.vocab, self.device)
        dev = logits.device
        n = rows if n is None else int(n)
        gather = _index_i32(gather_indices, "gather_indices", n, dev)
        req = _index_i32(token_to_request_index, "token_to_request_index", n, dev)
        ids = _index_i32(token_ids, "token_ids", n, dev)
        shape = (n,) if ids is not None else (n, self.vocab)
        if output is None:
            output = torch.empty(shape, dtype=torch.float32, device=dev)
        else:
            _check_out(output, torch.float32, 0, dev, "output", shape=shape)
        p = params._struct(dev)
        _check(library().ts_log_probs(self._h, _ptr(logits), dt, rows, stride, n, _ptr(gather),
                                      _ptr(req), ctypes.byref(p), int(bool(no_top_k)),
                                      int(bool(no_top_p)), _ptr(ids), _ptr(output), _stream(dev)),
               "ts_log_probs")
        return output


    def raw_log_probs_at(self, logits: torch.Tensor, token_ids: torch.Tensor, *,
                         n: Optional[int] = None, gather_indices: Optional[torch.Tensor] = None,
                         output: Optional[torch.Tensor] = None) -> torch.Tensor:
        """[n] log-softmax of the raw rows (no temperature, no filter) at token_ids."""
        dt, rows, stride = _logits_args(logits, self.vocab, self.device)
        dev = logits.device
        n = rows if n is None else int(n)
        gather = _index_i32(gather_indices, "gather_indices", n, dev)
        ids = _index_i32(token_ids, "token_ids", n, dev)
        if ids is None:
            raise ValueError("token_ids is required")
        if output is None:
            output = torch.empty(n, dtype=torch.float32, device=dev)
        else:
            _check_out(output, torch.float32, n, dev, "output")
        _check(library().ts_raw_log_probs_at(self._h, _ptr(logits), dt, rows, stride, n,
                                             _ptr(gather), _ptr(ids), _ptr(output), _stream(dev)),
               "ts_raw_log_probs_at")
        return output[:n]


def build_spec_map(num_decode: int, num_prefill: int, num_spec: int, device=None):
    """(map, n): request index per row of the speculative-verify layout, on ``device``
    (host memory when device is None or "cpu")."""
    lib = library()
    n = max(0, int(num_decode) * (1 + int(num_spec)) + int(num_prefill))
    on_dev = device is not None and torch.device(device).type == "cuda"
    out = torch.empty(n, dtype=torch.int32, device=device if on_dev else "cpu")
    got = ctypes.c_int32()
    stream = _stream(out.device) if on_dev else None
    _check(lib.ts_build_spec_map(int(num_decode), int(num_prefill), int(num_spec),
                                 _ptr(out) if n else None, n, int(on_dev), stream,
                                 ctypes.byref(got)), "ts_build_spec_map")
    return out, int(got.value)


def verify_chain(candidates: torch.Tensor, target_sampled: torch.Tensor, *,
                 predicts: Optional[torch.Tensor] = None,
                 accept_index: Optional[torch.Tensor] = None,
                 accept_length: Optional[torch.Tensor] = None):
    """(predicts [bs * N], accept_index [bs, N], accept_length [bs]) for the
    draft chains ``candidates`` [bs, N] (column 0 the last verified token) against
    the target samples ``target_sampled`` [bs * N], on their device and current
    stream.  A request emits accept_length + 1 tokens (ts_verify_chain)."""
    if candidates.dim() != 2:
        raise ValueError("candidates must be [bs, N]")
    bs, n = int(candidates.shape[0]), int(candidates.shape[1])
    dev = candidates.device
    if dev.type != "cuda":
        raise ValueError("candidates must be on a GPU")
    cand = _index_i32(candidates.reshape(-1).contiguous(), "candidates", bs * n, dev)
    tgt = _index_i32(target_sampled.reshape(-1).contiguous(), "target_sampled", bs * n, dev)

    def _out(t, shape, name):
        if t is None:
            return torch.empty(shape, dtype=torch.int32, device=dev)
        if t.dtype != torch.int32 or tuple(t.shape) != shape or not t.is_contiguous() or t.device != dev:
            raise ValueError(f"{name} must be a contiguous int32 tensor of shape {shape} on {dev}")
        return t

    predicts = _out(predicts, (bs * n,), "predicts")
    accept_index = _out(accept_index, (bs, n), "accept_index")
    accept_length = _out(accept_length, (bs,), "accept_length")
    _check(library().ts_verify_chain(bs, n, _ptr(cand), _ptr(tgt), _ptr(predicts),
                                     _ptr(accept_index), _ptr(accept_length), _stream(dev)),
           "ts_verify_chain")
    return predicts, accept_index, accept_length


def apply_vocab_mask(logits: torch.Tensor, mask: torch.Tensor,
                     mask_index: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Set to -inf, in place, every entry of ``logits`` [rows, V] (bf16 or fp32, on a
    GPU) whose bit in the row's mask is 0: bit (j % 32) of word j // 32 of mask row
    ``mask_index[r]`` (or r), ``mask`` int32/uint32 bits as an int32 tensor
    [mask rows, >= ceil(V / 32)] on the same device (ts_apply_vocab_mask).  Returns
    ``logits``."""
    dt, rows, stride = _logits_args(logits, int(logits.shape[1]) if logits.dim() == 2 else -1)
    dev = logits.device
    if mask.dtype != torch.int32 or mask.device != dev or mask.dim() != 2 or mask.stride(1) != 1:
        raise ValueError(f"mask must be a 2-D int32 tensor with contiguous rows on {dev}")
    if mask.shape[1] < (int(logits.shape[1]) + 31) // 32:
        raise ValueError(f"mask rows need at least ceil(V / 32) = {(int(logits.shape[1]) + 31) // 32} words")
    idx = _index_i32(mask_index, "mask_index", rows, dev)
    if idx is None and mask.shape[0] < rows:
        raise ValueError(f"mask has {mask.shape[0]} rows, logits have {rows}")
    _check(library().ts_apply_vocab_mask(int(logits.shape[1]), _ptr(logits), dt, rows, stride,
                                         _ptr(mask), int(mask.stride(0)), _ptr(idx), _stream(dev)),
           "ts_apply_vocab_mask")
    return logits


INDEX_GATHER_OUT, INDEX_REQUEST_OUT = 1, 2


def check_indices(n: int, *, gather_indices: Optional[torch.Tensor] = None,
                  rows_in_buffer: int = 0,
                  token_to_request_index: Optional[torch.Tensor] = None,
                  num_requests: int = 0, device=None) -> torch.Tensor:
    """Debug check of the index arrays a sampling call would read through
    unguarded: a device int32 [1] holding 0, or INDEX_GATHER_OUT (a gather index
    outside [0, rows_in_buffer)) | INDEX_REQUEST_OUT (a request index outside
    [0, num_requests)), enqueued on the current stream (ts_check_indices)."""
    src = gather_indices if gather_indices is not None else token_to_request_index
    dev = torch.device(device) if device is not None else (src.device if src is not None else None)
    if dev is None or dev.type != "cuda":
        raise ValueError("check_indices needs a GPU device (or an index tensor on one)")
    g = _index_i32(gather_indices, "gather_indices", n, dev)
    q = _index_i32(token_to_request_index, "token_to_request_index", n, dev)
    word = torch.empty(1, dtype=torch.int32, device=dev)
    _check(library().ts_check_indices(int(n), _ptr(g), int(rows_in_buffer), _ptr(q),
                                      int(num_requests), _ptr(word), _stream(dev)),
           "ts_check_indices")
    return word


__all__ = ["Sampler", "SamplingParams", "build_spec_map", "verify_chain", "select_route",
           "apply_vocab_mask", "check_indices", "INDEX_GATHER_OUT", "INDEX_REQUEST_OUT",
           "library", "LIB_PATH"]
