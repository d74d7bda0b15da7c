"""Throughput of one sampling step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--call sample|log_probs] [--gpus 1]

A step is one ts_sample call over the whole batch (every row: filters, noise,
draw and the fused log-prob), on synthetic logits already resident in HBM.
The default workload is 256 rows x 128256 bf16 logits with per-row top-k and
top-p (joint route).  Inputs rotate over enough copies to exceed the 256 MB
Infinity Cache, so each step reads its logits from HBM.

Prints one JSON line: rows/s (value), logits-read GB/s, % of the 8 TB/s HBM
peak, the roofline record of the sampling kernel (HIP events on the launch
stream) with the measured read ceiling of its launch shape, the CPU oracle's
rate over a process pool, and the parity of the last timed step's output
against that oracle (every row; near ties counted).
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
    "joint_128k_shifted": "joint_128k with row r's logits shifted by U[-16,0] before rounding to bf16",
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


def cpu_baseline_and_parity(wl, budget_s: float, call: str, gpu_out, step_offset: int,
                            token_ids=None):
    """The fp64 oracle over a pool of host processes (oracle.parallel), on the
    rows of the last timed step.  Its first pass computes every row of that
    step and is compared with the GPU's output of that step (the parity
    record); further passes over all rows at other step offsets run until
    about ``budget_s`` seconds of CPU work are done, and the rate over every
    pass is the baseline."""
    import oracle
    from oracle.parallel import Pool, host_cores
    from tests import parity
    x = wl.logits_f64()
    params = wl.params_numpy()
    gather = None if wl.gather_indices is None else wl.gather_indices.numpy()
    req = None if wl.token_to_request_index is None else wl.token_to_request_index.numpy()
    kw = dict(gather_indices=gather, token_to_request_index=req, no_top_k=wl.no_top_k,
              no_top_p=wl.no_top_p)
    with Pool() as pool:
        pool.warm()
        workers = pool.workers

        def one_pass(off):
            if call == "sample":
                return pool.run("sample", x, wl.n, params, step_offset=off, light=True, **kw)
            if call == "raw_log_probs":
                return oracle.raw_log_probs_at(x, wl.n, token_ids, gather_indices=gather)
            return pool.run("log_probs", x, wl.n, params, **kw)

        t0 = time.perf_counter()
        first = one_pass(step_offset)
        passes = 1
        while (time.perf_counter() - t0) * workers < budget_s and passes < 64:
            one_pass(step_offset + passes)
            passes += 1
        dt = time.perf_counter() - t0
        if call == "sample":
            res = first
            rep = parity.compare_samples(gpu_out[0], gpu_out[1], res)
        elif call == "raw_log_probs":
            got, want = gpu_out, first
            ok = (np.array_equal(np.isnan(got), np.isnan(want))
                  and np.array_equal(np.isneginf(got), np.isneginf(want)))
            fin = np.isfinite(want)
            ok = ok and float(np.max(np.abs(got[fin] - want[fin]), initial=0.0)) <= parity.LP_ATOL
            rep = parity.Report(rows=wl.n, mismatches=[] if ok else ["raw log-probs differ"])
        else:
            res = pool.run("sample", x, wl.n, params, step_offset=step_offset, light=True, **kw)
            rep = parity.compare_log_probs(gpu_out, first, res)
    how = "one process" if call == "raw_log_probs" else f"{workers} worker processes"
    base = {"value": wl.n * passes / dt, "unit": "rows/s",
            "cores": 1 if call == "raw_log_probs" else workers, "host_cores": host_cores(),
            "kind": "oracle",
            "sample": f"{passes} pass(es) over all {wl.n} rows of the same workload (the first at "
                      f"the last timed step's offset), fp64 numpy, {how} ({dt:.1f} s)"}
    par = {"step_offset": step_offset, "rows": rep.rows, "flagged": rep.flagged,
           "took_alternative": rep.diverged_flagged, "mismatches": len(rep.mismatches)}
    if rep.mismatches:
        par["first_mismatches"] = rep.mismatches[:3]
    return base, par


def read_ceiling(wl, logits, steps: int, warmup: int):
    """The read-ceiling probe: the same logits bytes read with the sampling
    kernel's launch shape (1024 threads per row, 16-byte loads), timed with
    HIP events over the same rotating copies.  None when a row does not fit
    that shape (more than 16 loads per thread)."""
    from token_sampling_scaled_amd import probes
    row_bytes = wl.vocab * wl.logits.element_size()
    nvec = -(-row_bytes // 16)
    if row_bytes % 16 or nvec > 16 * 1024:
        return None
    nv = 1
    while nv * 1024 < nvec:
        nv *= 2
    dev = logits[0].device
    out = torch.empty(wl.n, dtype=torch.int32, device=dev)
    plib = probes.library()
    args = [probes.read_rows_args(lg, wl.n, row_bytes, nv, out) for lg in logits]
    for i in range(warmup):
        plib.tsp_read_rows(*args[i % len(args)])
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        st = plib.tsp_read_rows(*args[(warmup + i) % len(args)])
        if st != 0:
            raise RuntimeError(f"tsp_read_rows failed with status {st}")
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"kernel_ms_per_launch": ms, "gbps": wl.n * row_bytes / (ms * 1e-3) / 1e9,
            "shape": f"{wl.n} workgroups x 1024 threads x {nv} 16-byte loads"}


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


def mask_cpu_baseline(originals, mask_words, gpu_masked, budget_s: float):
    """The oracle's vocabulary mask (python loops, one process) over rows of the
    same buffer until about ``budget_s`` seconds (at most 2 s: it is slow per
    entry), compared bit for bit with the GPU's masked rows."""
    import oracle
    x = originals.double().numpy()
    got = gpu_masked.double().numpy()
    t0 = time.perf_counter()
    rows = 0
    mismatches = 0
    while rows < x.shape[0] and (rows == 0 or time.perf_counter() - t0 < min(budget_s, 2.0)):
        want = oracle.apply_vocab_mask(x[rows:rows + 1], mask_words[rows:rows + 1])
        mismatches += int(not np.array_equal(want[0], got[rows]))
        rows += 1
    dt = time.perf_counter() - t0
    base = {"value": rows / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"the first {rows} rows of the buffer, python loops over entries, one "
                      f"process ({dt:.2f} s)"}
    return base, {"rows": rows, "mismatches": mismatches}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="joint_128k", choices=sorted(synth.WORKLOAD_IDS))
    ap.add_argument("--copies", type=int, default=0, help="input copies to rotate (0: auto)")
    ap.add_argument("--call", default="sample",
                    choices=("sample", "log_probs", "raw_log_probs", "verify_chain", "vocab_mask"),
                    help="time ts_sample (default), ts_log_probs with full [n, V] rows, "
                         "ts_raw_log_probs_at at the sampled ids, or ts_verify_chain over the "
                         "decode requests of the speculative workload (spec_mix), or "
                         "ts_apply_vocab_mask in place over the whole logits buffer with a seeded "
                         "mask allowing each entry with probability 1/2")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="CPU-seconds of oracle work for the baseline (over all its workers)")
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

    mask = None
    if args.call == "vocab_mask":
        # one mask row per buffer row, each bit set with probability 1/2; masking
        # is idempotent, so the rotating copies can be masked again every step
        nb = logits[0].shape[0]
        mrng = np.random.default_rng(9)
        mask_words = mrng.integers(0, 2**32, size=(nb, (wl.vocab + 31) // 32), dtype=np.int64)
        mask = torch.from_numpy(mask_words.astype(np.uint32).view(np.int32)).to(dev)
        originals = logits[0].cpu()

        def step_checked(i):
            tsa.apply_vocab_mask(logits[i % copies], mask)

        m_args = [[wl.vocab, ctypes.c_void_p(lg.data_ptr()), dt_code, lg.shape[0], lg.stride(0),
                   ctypes.c_void_p(mask.data_ptr()), mask.stride(0), None, stream_ptr]
                  for lg in logits]
        ts_mask = lib.ts_apply_vocab_mask

        def step(i):
            st = ts_mask(*m_args[i % copies])
            if st != tsa.TS_OK:
                raise RuntimeError(f"ts_apply_vocab_mask failed with status {st}")

        # every 16-byte vector holds allowed and masked entries: each is read and written
        nbytes = 2 * nb * wl.vocab * wl.logits.element_size() + mask.numel() * 4

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

    last_offset = args.warmup + args.steps - 1
    ceiling = None
    if verify is None and args.call == "sample":
        ceiling = read_ceiling(wl, logits, args.steps, min(args.warmup, 5))

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
    if ceiling is not None:
        out["roofline"]["read_ceiling"] = ceiling
        out["roofline"]["pct_of_read_ceiling"] = 100.0 * ceiling["kernel_ms_per_launch"] / kernel_ms
    if verify is not None:
        out["config"]["verify"] = {"requests": verify["bs"], "rows_per_request": verify["n"],
                                   "mean_accepted_drafts": float(alen.float().mean().item())}
        out["roofline"]["bound"] = "launch"
    if mask is not None:
        out["config"]["rows"] = int(logits[0].shape[0])
        out["value"] = logits[0].shape[0] * args.steps / wall
    if not args.no_cpu_baseline:
        if mask is not None:
            out["cpu_baseline"], out["parity"] = mask_cpu_baseline(
                originals, mask_words, logits[0].cpu(), args.cpu_budget)
        elif verify is not None:
            out["cpu_baseline"] = verify_cpu_baseline(verify, args.cpu_budget)
        else:
            if args.call == "sample":
                gpu_out = (ids.cpu().numpy(), lps.cpu().numpy())
            elif args.call == "raw_log_probs":
                gpu_out = raw.cpu().numpy()
            else:
                gpu_out = full.cpu().numpy()
            out["cpu_baseline"], out["parity"] = cpu_baseline_and_parity(
                wl, args.cpu_budget, args.call, gpu_out, last_offset,
                token_ids=tok.cpu().numpy() if args.call == "raw_log_probs" else None)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
