"""Stage times of the register-resident bf16 kernel, from its stage marks.

    python -m token_sampling_scaled_amd.build --stage-marks
    python -m token_sampling_scaled_amd.stage_times --workload joint_128k

Loads libtssample_marks.so (the sampler built with TSS_STAGE_MARKS: thread 0
of each workgroup records the device's wall clock at each stage of the top-k
body and of the sampling body of rows without top-k), samples the workload a
few times, and prints over the workgroups of the last call the median of each
stage, the spread of the starts, the median and the last end, and the slowest
workgroups' stages.  Times are in microseconds
from the first workgroup's start.  The library must exist: nothing here
builds it or falls back to another.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys

import numpy as np

STAGES = ["threshold", "data offered", "counted + barrier", "scanned + barrier",
          "listed + barrier", "drawn + picked"]
NOK_STAGES = ["row maximum + barrier", "Z + barrier", "histogram + barrier", "cutoff + barrier",
              "draw", "pick"]
NMARKS = 16


def _setup(workload: str):
    import torch
    import synth
    import token_sampling_scaled_amd as tsa
    from token_sampling_scaled_amd import build

    if not os.path.exists(build.MARKS_LIB):
        raise RuntimeError(f"{build.MARKS_LIB} is missing: build it with "
                           "`python -m token_sampling_scaled_amd.build --stage-marks`")
    tsa.LIB_PATH = build.MARKS_LIB     # before the binding loads a library
    lib = tsa.library()
    marks = ctypes.CDLL(build.MARKS_LIB)
    marks.tss_stage_marks.argtypes = [ctypes.c_void_p, ctypes.c_int]
    marks.tss_stage_marks.restype = ctypes.c_int
    marks.tss_stage_marks_clear.restype = ctypes.c_int
    wl = synth.make(workload)
    dev = "cuda"
    params = tsa.SamplingParams(
        temperature=wl.temperature.to(dev), seed=wl.seed.to(dev), top_k=wl.top_k.to(dev),
        top_p=wl.top_p.to(dev),
        step_offsets=None if wl.step_offsets is None else wl.step_offsets.to(dev))
    logits = wl.logits.to(dev)
    gather = None if wl.gather_indices is None else wl.gather_indices.to(dev)
    req = None if wl.token_to_request_index is None else wl.token_to_request_index.to(dev)
    sampler = tsa.Sampler(wl.vocab, wl.n)

    def call():
        sampler.sample(logits, wl.n, params, no_top_k=wl.no_top_k, no_top_p=wl.no_top_p,
                       gather_indices=gather, token_to_request_index=req,
                       step_offset=wl.step_offset, return_logprobs=True)

    return wl, marks, call, torch, lib


def stage_table(workload: str, calls: int = 5, slowest: int = 6) -> dict:
    wl, marks, call, torch, _ = _setup(workload)
    rows = min(wl.n, 1024)
    if not marks.tss_stage_marks_clear():
        raise RuntimeError("tss_stage_marks_clear failed")
    for _ in range(calls):
        call()
    torch.cuda.synchronize()
    buf = np.zeros((rows, NMARKS), dtype=np.uint64)
    khz = marks.tss_stage_marks(buf.ctypes.data, rows)
    if khz <= 0:
        raise RuntimeError("tss_stage_marks failed")
    t = buf.astype(np.float64) / (khz / 1000.0)          # microseconds
    seen = buf[:, 6] > 0                                 # workgroups that finished the top-k body
    t0 = t[buf[:, 0] > 0, 0].min()
    out = {"workload": workload, "workgroups": int(rows), "through_top_k_body": int(seen.sum()),
           "signed_pass": int((buf[:, 7] > 0).sum())}
    if seen.any():
        # a row that took the signed-order pass: its stages are the second
        # pass's (from mark 7), the first pass is reported on its own
        start = np.where(buf[:, 7] > 0, t[:, 7], t[:, 0])
        st = t.copy()
        st[:, 0] = start
        out["stage_median_us"] = {name: round(float(np.median(st[seen, i + 1] - st[seen, i])), 2)
                                  for i, name in enumerate(STAGES)}
        sg = seen & (buf[:, 7] > 0)
        if sg.any():
            out["first_pass_median_us"] = round(float(np.median(t[sg, 7] - t[sg, 0])), 2)
        ends = t[seen, 6] - t0
        out["start_spread_p95_us"] = round(float(np.percentile(t[seen, 0] - t0, 95)), 2)
        out["end_median_us"] = round(float(np.median(ends)), 2)
        out["end_max_us"] = round(float(ends.max()), 2)
        order = np.argsort(-(t[:, 6] - t0) * seen)[:slowest]
        out["slowest"] = [{"workgroup": int(b), "end_us": round(float(t[b, 6] - t0), 2),
                           "stages_us": [round(float(st[b, i + 1] - st[b, i]), 2) for i in range(6)]}
                          for b in order if seen[b]]
    # rows without top-k (sampling): top-p rows pass marks 8 to 13, the race
    # rows (no top-p) 8, 12 and 13
    nok = buf[:, 13] > 0
    topp = nok & (buf[:, 11] > 0)
    race = nok & ~topp
    if topp.any():
        marks = [0, 8, 9, 10, 11, 12, 13]
        out["top_p_rows"] = int(topp.sum())
        out["top_p_stage_median_us"] = {
            name: round(float(np.median(t[topp, marks[i + 1]] - t[topp, marks[i]])), 2)
            for i, name in enumerate(NOK_STAGES)}
        out["top_p_end_max_us"] = round(float((t[topp, 13] - t0).max()), 2)
    if race.any():
        out["race_rows"] = int(race.sum())
        out["race_stage_median_us"] = {
            "row maximum + barrier": round(float(np.median(t[race, 8] - t[race, 0])), 2),
            "Z and the race": round(float(np.median(t[race, 12] - t[race, 8])), 2),
            "pick": round(float(np.median(t[race, 13] - t[race, 12])), 2)}
        out["race_end_max_us"] = round(float((t[race, 13] - t0).max()), 2)
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="joint_128k")
    ap.add_argument("--calls", type=int, default=5)
    args = ap.parse_args(argv)
    print(json.dumps(stage_table(args.workload, args.calls), indent=1), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
