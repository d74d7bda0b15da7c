"""Throughput of one sampling step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--call sample|log_probs] [--gpus 1]

A step is one ts_sample call over the whole batch (every row: filters, noise,
draw and the fused log-prob), on synthetic logits already resident in HBM.
The default workload is 256 rows x 128256 bf16 logits with per-row top-k and
top-p (joint route).  Inputs rotate over enough copies to exceed the 256 MB
Infinity Cache, so each step reads its logits from HBM.

Prints one JSON line: rows/s (value), logits-read GB/s, % of the 8 TB/s HBM
peak, the roofline record of the sampling kernel (HIP events on the launch
stream) and the CPU oracle's rate on a bounded sample of the same rows.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import synth  # noqa: E402
import token_sampling_scaled_amd as tsa  # noqa: E402

HBM_PEAK_GBPS = 8000.0
METRIC = "sampled rows/s + logits-read GB/s, 256x128256 bf16 top-k+top-p (% HBM peak)"
DESCRIPTIONS = {
    "joint_128k": "256x128256 bf16 logits N(0,3^2)+spikes, per-row top-k U{1..1024} + top-p U[0.5,0.99], T U[0.5,1.5]",
    "topk_128k": "256x128256 bf16 logits N(0,3^2)+spikes, per-row top-k U{1..1024}, T U[0.5,1.5]",
    "none_32k": "64x32000 bf16 logits N(0,3^2), no filter",
    "topp_152k": "256x151936 fp32 Zipf(1.1) logits, per-row top-p U[0.5,0.99]",
    "spec_mix": "288 of 320 rows x 128256 bf16, speculative layout, mixed none/top-k/top-p/joint + log-probs",
    "tiny_joint": "8x4096 fp32 logits, top-k 50 + top-p 0.9",
}


def logits_bytes(wl) -> int:
    return wl.n * wl.vocab * wl.logits.element_size()


def algorithmic_bytes(wl, call: str = "sample") -> int:
    """HBM bytes one step must move: every selected logit read once, plus per
    row its gather and request indices, the request's parameters (T 4 B, k 4 B,
    p 4 B, seed 8 B) and the outputs: id 4 B and log-prob 4 B for a sample
    call; the full fp32 row of log-probs (4 B per entry) for a log_probs call.
    A raw_log_probs call reads only the logits, the gather index and the token
    id (4 B) and writes one fp32 per row."""
    if call == "raw_log_probs":
        per_row = 4 + 4 + (0 if wl.gather_indices is None else 4)
        return logits_bytes(wl) + wl.n * per_row
    per_row = 4 + 8 + (8 if call == "sample" else 4 * wl.vocab)
    per_row += 0 if wl.no_top_k else 4
    per_row += 0 if wl.no_top_p else 4
    per_row += 0 if wl.gather_indices is None else 4
    per_row += 0 if wl.token_to_request_index is None else 4
    return logits_bytes(wl) + wl.n * per_row


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed counter summaries, or None when
    none matches this workload and the current kernel sources."""
    from token_sampling_scaled_amd import profiling
    digest = profiling.source_digest()
    for rec in profiling.read_records(os.path.join(ROOT, "profiles")):
        if rec.get("workload") == workload and rec.get("source_sha256") == digest:
            return rec["bytes_per_launch"]
    return None


def cpu_baseline(wl, budget_s: float, call: str = "sample"):
    """The fp64 oracle, single process, on the leading rows of the same workload."""
    import oracle
    x = wl.logits_f64()
    params = wl.params_numpy()
    gather = None if wl.gather_indices is None else wl.gather_indices.numpy()
    req = None if wl.token_to_request_index is None else wl.token_to_request_index.numpy()
    t0 = time.perf_counter()
    done = 0
    while done < wl.n and time.perf_counter() - t0 < budget_s:
        if call == "sample":
            oracle.sample(x, wl.n, params, gather_indices=gather, token_to_request_index=req,
                          step_offset=wl.step_offset, no_top_k=wl.no_top_k, no_top_p=wl.no_top_p,
                          rows=[done])
        elif call == "raw_log_probs":
            oracle.raw_log_probs_at(x, wl.n, np.zeros(wl.n, dtype=np.int32),
                                    gather_indices=gather, rows=[done])
        else:
            oracle.log_probs(x, wl.n, params, gather_indices=gather, token_to_request_index=req,
                             no_top_k=wl.no_top_k, no_top_p=wl.no_top_p, rows=[done])
        done += 1
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"first {done} of {wl.n} rows of the same workload, fp64 numpy, "
                      f"one process ({dt:.1f} s)"}


def verify_inputs(wl, sampler, logits, params, gather, req, dev):
    """Chain-verification inputs on the speculative workload: the decode
    requests (those owning 1 + S rows, first in the layout) with one sampled
    target token per row, and seeded draft chains that follow those samples for
    a random number of steps before diverging."""
    counts = np.bincount(wl.token_to_request_index.numpy())
    n = int(counts.max())
    bs = int(np.sum(counts == n))
    ids, _ = sampler.sample(logits, wl.n, params, no_top_k=wl.no_top_k, no_top_p=wl.no_top_p,
                            gather_indices=gather, token_to_request_index=req,
                            return_logprobs=True)
    tgt = ids[:bs * n].contiguous()
    t = tgt.cpu().numpy().reshape(bs, n)
    rng = np.random.default_rng(17)
    cand = rng.integers(0, wl.vocab, size=(bs, n)).astype(np.int32)
    stop = rng.integers(0, n, size=bs)
    for b in range(bs):
        cand[b, 1:stop[b] + 1] = t[b, :stop[b]]
    return {"bs": bs, "n": n, "tgt": tgt, "cand": torch.from_numpy(cand.reshape(-1)).to(dev)}


def verify_cpu_baseline(verify, budget_s: float):
    """The oracle's chain verification on the same requests, repeated for the budget."""
    import oracle
    cand = verify["cand"].cpu().numpy().reshape(verify["bs"], verify["n"])
    tgt = verify["tgt"].cpu().numpy()
    t0 = time.perf_counter()
    reps = 0
    while reps < 1 or (time.perf_counter() - t0 < min(budget_s, 2.0) and reps < 1000):
        oracle.verify_chain(cand, tgt)
        reps += 1
    dt = time.perf_counter() - t0
    rows = verify["bs"] * verify["n"]
    return {"value": rows * reps / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} passes over the {verify['bs']} decode requests, python loops, "
                      f"one process ({dt:.2f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="joint_128k", choices=sorted(synth.WORKLOAD_IDS))
    ap.add_argument("--copies", type=int, default=0, help="input copies to rotate (0: auto)")
    ap.add_argument("--call", default="sample",
                    choices=("sample", "log_probs", "raw_log_probs", "verify_chain"),
                    help="time ts_sample (default), ts_log_probs with full [n, V] rows, "
                         "ts_raw_log_probs_at at the sampled ids, or ts_verify_chain over the "
                         "decode requests of the speculative workload (spec_mix)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the sampler is single-GPU (rows shard with no "
              "exchange); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if not os.path.exists(tsa.LIB_PATH):
        from token_sampling_scaled_amd import build
        build.build()

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    wl = synth.make(args.workload)
    nbytes = algorithmic_bytes(wl, args.call)
    buf_bytes = wl.logits.numel() * wl.logits.element_size()
    copies = args.copies or max(2, int(np.ceil(400e6 / buf_bytes)))
    logits = [wl.logits.to(dev) for _ in range(copies)]
    params = tsa.SamplingParams(wl.temperature.to(dev), wl.seed.to(dev), wl.top_k.to(dev),
                                wl.top_p.to(dev))
    gather = None if wl.gather_indices is None else wl.gather_indices.to(dev)
    req = None if wl.token_to_request_index is None else wl.token_to_request_index.to(dev)
    sampler = tsa.Sampler(wl.vocab, wl.n)
    ids = torch.empty(wl.n, dtype=torch.int32, device=dev)
    lps = torch.empty(wl.n, dtype=torch.float32, device=dev)

    def step_checked(i):
        sampler.sample(logits[i % copies], wl.n, params, no_top_k=wl.no_top_k,
                       no_top_p=wl.no_top_p, gather_indices=gather, token_to_request_index=req,
                       step_offset=i, output=ids, logprob_output=lps)

    # Timed steps call the C ABI directly with argument lists built once, so
    # the host issues a step in a few microseconds and the GPU never waits on
    # Python; the checked wrapper above runs the warm-up steps.
    lib = tsa.library()
    prm = params._struct(dev)
    prm_ref = ctypes.byref(prm)
    stream_ptr = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    dt_code = tsa.TS_F32 if wl.logits.dtype == torch.float32 else tsa.TS_BF16
    call_args = [[sampler._h, ctypes.c_void_p(lg.data_ptr()), dt_code, lg.shape[0], lg.stride(0),
                  wl.n, None if gather is None else ctypes.c_void_p(gather.data_ptr()),
                  None if req is None else ctypes.c_void_p(req.data_ptr()), prm_ref, 0,
                  int(wl.no_top_k), int(wl.no_top_p), ctypes.c_void_p(ids.data_ptr()),
                  ctypes.c_void_p(lps.data_ptr()), stream_ptr] for lg in logits]
    ts_sample = lib.ts_sample

    def step(i):
        cargs = call_args[i % copies]
        cargs[9] = i
        st = ts_sample(*cargs)
        if st != tsa.TS_OK:
            raise RuntimeError(f"ts_sample failed with status {st}")

    if args.call == "log_probs":
        full = torch.empty((wl.n, wl.vocab), dtype=torch.float32, device=dev)

        def step_checked(i):
            sampler.log_probs(logits[i % copies], params, n=wl.n, no_top_k=wl.no_top_k,
                              no_top_p=wl.no_top_p, gather_indices=gather,
                              token_to_request_index=req, output=full)

        lp_args = [[sampler._h, ctypes.c_void_p(lg.data_ptr()), dt_code, lg.shape[0], lg.stride(0),
                    wl.n, None if gather is None else ctypes.c_void_p(gather.data_ptr()),
                    None if req is None else ctypes.c_void_p(req.data_ptr()), prm_ref,
                    int(wl.no_top_k), int(wl.no_top_p), None, ctypes.c_void_p(full.data_ptr()),
                    stream_ptr] for lg in logits]
        ts_log_probs = lib.ts_log_probs

        def step(i):
            st = ts_log_probs(*lp_args[i % copies])
            if st != tsa.TS_OK:
                raise RuntimeError(f"ts_log_probs failed with status {st}")

    if args.call == "raw_log_probs":
        step_checked(0)                    # the ids to read: one sample of the workload
        torch.cuda.synchronize()
        tok = ids.clone()
        raw = torch.empty(wl.n, dtype=torch.float32, device=dev)

        def step_checked(i):
            sampler.raw_log_probs_at(logits[i % copies], tok, n=wl.n, gather_indices=gather,
                                     output=raw)

        raw_args = [[sampler._h, ctypes.c_void_p(lg.data_ptr()), dt_code, lg.shape[0], lg.stride(0),
                     wl.n, None if gather is None else ctypes.c_void_p(gather.data_ptr()),
                     ctypes.c_void_p(tok.data_ptr()), ctypes.c_void_p(raw.data_ptr()), stream_ptr]
                    for lg in logits]
        ts_raw = lib.ts_raw_log_probs_at

        def step(i):
            st = ts_raw(*raw_args[i % copies])
            if st != tsa.TS_OK:
                raise RuntimeError(f"ts_raw_log_probs_at failed with status {st}")

    verify = None
    if args.call == "verify_chain":
        if wl.token_to_request_index is None:
            print("--call verify_chain needs the speculative workload (--workload spec_mix)",
                  file=sys.stderr)
            sys.exit(2)
        verify = verify_inputs(wl, sampler, logits[0], params, gather, req, dev)
        vb, vn, cand, tgt = verify["bs"], verify["n"], verify["cand"], verify["tgt"]
        pred = torch.empty(vb * vn, dtype=torch.int32, device=dev)
        aidx = torch.empty(vb * vn, dtype=torch.int32, device=dev)
        alen = torch.empty(vb, dtype=torch.int32, device=dev)

        def step_checked(i):
            tsa.verify_chain(cand.view(vb, vn), tgt, predicts=pred, accept_index=aidx.view(vb, vn),
                             accept_length=alen)

        v_args = [vb, vn, ctypes.c_void_p(cand.data_ptr()), ctypes.c_void_p(tgt.data_ptr()),
                  ctypes.c_void_p(pred.data_ptr()), ctypes.c_void_p(aidx.data_ptr()),
                  ctypes.c_void_p(alen.data_ptr()), stream_ptr]
        ts_verify = lib.ts_verify_chain

        def step(i):
            st = ts_verify(*v_args)
            if st != tsa.TS_OK:
                raise RuntimeError(f"ts_verify_chain failed with status {st}")

        nbytes = vb * (16 * vn + 4)

    if args.copy_probe_mb:
        a = torch.empty(args.copy_probe_mb << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()

    for i in range(args.warmup):
        (step_checked if i < 2 else step)(i)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)       # the stream ts_sample launches on
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = ev0.elapsed_time(ev1) / args.steps

    rows = wl.n if verify is None else verify["bs"] * verify["n"]
    rows_per_s = rows * args.steps / wall
    gbps = (logits_bytes(wl) if verify is None else 0) * args.steps / wall / 1e9
    achieved = nbytes / (kernel_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": rows_per_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "logits_read_gbps": gbps,
        "pct_hbm_peak": 100.0 * gbps / HBM_PEAK_GBPS,
        "config": {"workload": f"{args.workload}: {DESCRIPTIONS[args.workload]}",
                   "rows": rows, "vocab": wl.vocab, "logits_dtype": str(wl.logits.dtype).split(".")[-1],
                   "route": ["none", "top-k", "top-p", "joint"][tsa.select_route(wl.no_top_k, wl.no_top_p)],
                   "call": args.call,
                   "input_copies": copies, "logits_bytes_per_step": logits_bytes(wl),
                   "algorithmic_bytes_per_step": nbytes},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(args.workload) if args.call == "sample" else None,
                     "kernel_ms_per_launch": kernel_ms},
    }
    if verify is not None:
        out["config"]["verify"] = {"requests": verify["bs"], "rows_per_request": verify["n"],
                                   "mean_accepted_drafts": float(alen.float().mean().item())}
        out["roofline"]["bound"] = "launch"
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = (verify_cpu_baseline(verify, args.cpu_budget) if verify is not None
                               else cpu_baseline(wl, args.cpu_budget, args.call))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
