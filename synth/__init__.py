"""Seeded synthetic inputs for the sampling workloads.

This module only draws inputs: logits matrices, per-request parameters and
index arrays.  It holds none of the sampling arithmetic, and both the HIP path
(through its tests and the benchmark) and the CPU oracle consume exactly the
tensors it returns.

Workloads (shapes, value laws and parameter laws):

  tiny_joint    8 x 4096 fp32, N(0, 2^2); T = 0.7 on even rows, 1.0 on odd rows;
                top_k = 50, top_p = 0.9, seed = row; joint filtering.
  none_32k      64 x 32000 bf16, N(0, 3^2); T = 1; no filter; seed = row.
  topk_128k     256 x 128256 bf16, N(0, 3^2) plus +8 added at 20 distinct uniform
                positions per row (before rounding to bf16); top_k ~ U{1..1024},
                T ~ U[0.5, 1.5]; top-k only.
  joint_128k    topk_128k's logits, k and T, plus top_p ~ U[0.5, 0.99]; joint.
  joint_128k_shifted
                joint_128k with row r's fp32 logits shifted by s_r ~ U[-16, 0]
                before rounding to bf16 (the same distributions; most rows, or
                all of their top-k, below zero).
  topp_152k     256 x 151936 fp32, x[r, perm_r(i)] = -1.1 ln i for i = 1..V
                (Zipf(1.1) log-probabilities up to a constant, one random
                permutation per row); T = 1, top_p ~ U[0.5, 0.99]; top-p only.
  spec_mix      320 x 128256 bf16 buffer, N(0, 3^2); 288 rows gathered (a random
                288-of-320 choice without replacement) in the speculative layout
                64 decode requests x (1 + 3) rows + 32 prefill rows = 96 requests;
                each request is none / top-k / top-p / joint (24 of each, random
                order), k ~ U{1..1024}, p ~ U[0.5, 0.99], T = 1, seed = request.

Each workload draws from numpy.random.default_rng(1000 + its id) in fp32; bf16
logits are rounded from those fp32 draws by torch (round to nearest even).
``rows`` and ``vocab`` overrides give smaller instances with the same laws.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

WORKLOAD_IDS = {
    "tiny_joint": 1,
    "none_32k": 2,
    "topk_128k": 3,
    "topp_152k": 4,
    "spec_mix": 5,
    "joint_128k": 6,
    "joint_128k_shifted": 7,
}

FULL_SHAPES = {
    "tiny_joint": (8, 4096, torch.float32),
    "none_32k": (64, 32000, torch.bfloat16),
    "topk_128k": (256, 128256, torch.bfloat16),
    "joint_128k": (256, 128256, torch.bfloat16),
    "joint_128k_shifted": (256, 128256, torch.bfloat16),
    "topp_152k": (256, 151936, torch.float32),
    "spec_mix": (288, 128256, torch.bfloat16),
}


@dataclass
class Workload:
    name: str
    logits: torch.Tensor                 # [rows_in_buffer, V], CPU, bf16 or fp32
    n: int                               # output rows
    temperature: torch.Tensor            # f32 [Q]
    top_k: torch.Tensor                  # i32 [Q]
    top_p: torch.Tensor                  # f32 [Q]
    seed: torch.Tensor                   # i64 [Q]
    gather_indices: Optional[torch.Tensor] = None          # i32 [n]
    token_to_request_index: Optional[torch.Tensor] = None  # i32 [n]
    no_top_k: bool = False
    no_top_p: bool = False
    step_offset: int = 0
    step_offsets: Optional[torch.Tensor] = None              # i64 [Q], read as u64

    @property
    def vocab(self) -> int:
        return int(self.logits.shape[1])

    def params_numpy(self) -> dict:
        return {
            "temperature": self.temperature.numpy().astype(np.float64),
            "top_k": self.top_k.numpy().astype(np.int64),
            "top_p": self.top_p.numpy().astype(np.float64),
            "seed": self.seed.numpy().astype(np.int64).view(np.uint64),
            "step_offsets": None if self.step_offsets is None
            else self.step_offsets.numpy().astype(np.int64).view(np.uint64),
        }

    def logits_f64(self) -> np.ndarray:
        return self.logits.float().numpy().astype(np.float64)


def _to_dtype(a: np.ndarray, dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dtype)


def _spec_layout(num_decode: int, num_prefill: int, num_spec: int) -> np.ndarray:
    """Request index of each row: decode blocks of 1 + num_spec rows, then prefill rows."""
    req = [d for d in range(num_decode) for _ in range(1 + num_spec)]
    req += [num_decode + i for i in range(num_prefill)]
    return np.array(req, dtype=np.int32)


def make(name: str, rows: Optional[int] = None, vocab: Optional[int] = None) -> Workload:
    """Build one workload (optionally a smaller instance with the same laws)."""
    wid = WORKLOAD_IDS[name]
    full_rows, full_vocab, dtype = FULL_SHAPES[name]
    n = full_rows if rows is None else int(rows)
    v = full_vocab if vocab is None else int(vocab)
    rng = np.random.default_rng(1000 + wid)

    if name == "tiny_joint":
        x = rng.normal(0.0, 2.0, size=(n, v)).astype(np.float32)
        t = np.where(np.arange(n) % 2 == 0, 0.7, 1.0).astype(np.float32)
        return Workload(name, _to_dtype(x, dtype), n, torch.from_numpy(t),
                        torch.full((n,), 50, dtype=torch.int32),
                        torch.full((n,), 0.9, dtype=torch.float32),
                        torch.arange(n, dtype=torch.int64))

    if name == "none_32k":
        x = rng.normal(0.0, 3.0, size=(n, v)).astype(np.float32)
        return Workload(name, _to_dtype(x, dtype), n, torch.ones(n, dtype=torch.float32),
                        torch.zeros(n, dtype=torch.int32), torch.ones(n, dtype=torch.float32),
                        torch.arange(n, dtype=torch.int64), no_top_k=True, no_top_p=True)

    if name in ("topk_128k", "joint_128k", "joint_128k_shifted"):
        rng = np.random.default_rng(1000 + WORKLOAD_IDS["topk_128k"])
        x = rng.normal(0.0, 3.0, size=(n, v)).astype(np.float32)
        spikes = min(20, v)
        for r in range(n):
            x[r, rng.choice(v, size=spikes, replace=False)] += np.float32(8.0)
        k = rng.integers(1, 1025, size=n).astype(np.int32)
        t = rng.uniform(0.5, 1.5, size=n).astype(np.float32)
        if name == "joint_128k_shifted":
            shift = np.random.default_rng(1000 + wid).uniform(-16.0, 0.0, size=n)
            x += shift.astype(np.float32)[:, None]
        wl = Workload(name, _to_dtype(x, dtype), n, torch.from_numpy(t), torch.from_numpy(k),
                      torch.ones(n, dtype=torch.float32), torch.arange(n, dtype=torch.int64),
                      no_top_p=True)
        if name != "topk_128k":
            prng = np.random.default_rng(1000 + WORKLOAD_IDS["joint_128k"])
            wl.top_p = torch.from_numpy(prng.uniform(0.5, 0.99, size=n).astype(np.float32))
            wl.no_top_p = False
        return wl

    if name == "topp_152k":
        base = (-1.1 * np.log(np.arange(1, v + 1, dtype=np.float64))).astype(np.float32)
        x = np.empty((n, v), dtype=np.float32)
        for r in range(n):
            x[r, rng.permutation(v)] = base
        p = rng.uniform(0.5, 0.99, size=n).astype(np.float32)
        return Workload(name, _to_dtype(x, dtype), n, torch.ones(n, dtype=torch.float32),
                        torch.zeros(n, dtype=torch.int32), torch.from_numpy(p),
                        torch.arange(n, dtype=torch.int64), no_top_k=True)

    if name == "spec_mix":
        num_decode, num_spec, num_prefill = 64, 3, 32
        if rows is not None:   # smaller instance: keep the 2:1 decode:prefill request mix
            num_decode = max(1, n // 6)
            num_prefill = max(1, n - num_decode * (1 + num_spec))
        req = _spec_layout(num_decode, num_prefill, num_spec)
        n = int(req.size)
        buf_rows = n + max(1, n // 9)
        x = rng.normal(0.0, 3.0, size=(buf_rows, v)).astype(np.float32)
        gather = rng.choice(buf_rows, size=n, replace=False).astype(np.int32)
        q = num_decode + num_prefill
        modes = np.repeat(np.arange(4), (q + 3) // 4)[:q]
        rng.shuffle(modes)
        k = np.where((modes == 1) | (modes == 3), rng.integers(1, 1025, size=q), 0).astype(np.int32)
        p = np.where((modes == 2) | (modes == 3), rng.uniform(0.5, 0.99, size=q), 1.0).astype(np.float32)
        return Workload(name, _to_dtype(x, dtype), n, torch.ones(q, dtype=torch.float32),
                        torch.from_numpy(k), torch.from_numpy(p), torch.arange(q, dtype=torch.int64),
                        gather_indices=torch.from_numpy(gather),
                        token_to_request_index=torch.from_numpy(req))

    raise KeyError(name)
