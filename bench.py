"""Throughput of the DFlash 2 path selector on one MI355X.

One step = the whole selector over one batch of draft blocks, inputs already
resident in HBM: top-16 of every position, the gate and candidate projections,
every adjacent pair scored and the walk, as one dsel_select_path call.  Prints
one JSON line (one GPU).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all|c1|c2|c3|c4]

By default every graded workload is measured in one run (c2, c3, c4; the
headline line is c4, the largest, with per-workload records for all three),
plus the latency shape c1 in a record of its own.
Workloads (synthetic, seeded; see synth.CONFIGS): c1 one block of 16 (latency
shape), c2 64 blocks of 16, c3 128 blocks of 8 with the sampled walk, c4 256
blocks of 16 with fp32 logits and both walks.
"""
import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft blocks/s through selector + achieved HBM GB/s & MFMA % of peak"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
K = 16
GRADED = ("c2", "c3", "c4")
HEADLINE = "c4"
LATENCY = "c1"  # one block of 16: measured too (its own record), never the headline
# HBM byte counters against a plain 1 GiB device copy (--calibrate-copy): per
# copied GiB FETCH_SIZE reads 0.5 GiB and WRITE_SIZE 1 GiB, so the counters'
# KiB are multiplied by these factors to give bytes moved.
FETCH_FACTOR = 2.0
WRITE_FACTOR = 1.0
# kernels whose traffic is recorded, and the sources each is built from
TRAFFIC_KERNELS = {
    "topk16": ("topk16_kernel", ["common.h", "topk16.h"]),
    "project_pairs": ("project_pair_kernel", ["common.h", "project.h", "pairwalk.h", "fused.h"]),
    "verify_stats": ("verify_stats_kernel", ["common.h", "verify.h"]),
}
STAGES = ("gate", "topk", "project", "pair_walk")


def walk_modes(cfg):
    return {"greedy": [0], "sampled": [1], "both": [0, 1]}[cfg.walk]


def describe(cfg):
    walk = {"greedy": "greedy walk", "sampled": "sampled walk (T=1)", "both": "greedy and sampled walks"}[cfg.walk]
    return (f"{cfg.name}: {cfg.batch} blocks x {cfg.block} positions, vocab {cfg.vocab}, "
            f"d {cfg.d}, r {cfg.r}, {cfg.logits_dtype} logits, {walk}")


def dtype_of(cfg):
    """The arithmetic the step computes in: the logits' type for the top-16
    (compares), bf16 x bf16 -> fp32 MFMA for the projections, fp32 pairs."""
    return "bf16" if cfg.logits_dtype == "bf16" else "f32+bf16"


def algorithmic(cfg):
    """Bytes / FLOP every stage must move / do once per step."""
    es = 2 if cfg.logits_dtype == "bf16" else 4
    rows = cfg.batch * cfg.block
    topk_bytes = rows * cfg.vocab * es + rows * K * 8
    a_rows = cfg.batch * K * (cfg.block - 1)  # candidates that are someone's predecessor
    b_rows = cfg.batch * cfg.block * K        # candidates that need B
    cand_flop = 2.0 * cfg.d * cfg.r * (a_rows + b_rows)
    gate_flop = 2.0 * cfg.d * cfg.r * (rows + cfg.batch)  # gate rows + verified tokens
    gather_bytes = rows * K * cfg.d * 2                   # the gathered E rows, bf16
    pair_flop = 2.0 * cfg.r * K * K * (rows - cfg.batch) + 2.0 * cfg.r * K * cfg.batch
    return dict(topk_bytes=topk_bytes, cand_flop=cand_flop, gate_flop=gate_flop, gather_bytes=gather_bytes,
                pair_flop=pair_flop)


def kernel_source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "draft_selection_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload, kernel="topk16"):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when
    there are none or the kernel source changed since they were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != kernel_source_hash(t.get("sources", [])):
        return None
    return float(t["fetch_bytes"]) + float(t["write_bytes"])


def _counter_per_dispatch(run_dir, match):
    """Mean Counter_Value over the dispatches whose kernel name contains `match`
    in a rocprofv3 --pmc CSV directory (one counter per run)."""
    import csv
    import glob

    vals = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if match in row["Kernel_Name"]:
                    key = (path, row["Dispatch_Id"])
                    vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
    if not vals:
        raise SystemExit(f"no dispatch of {match} in {run_dir}")
    return sum(vals.values()) / len(vals), len(vals)


def record_traffic(workload, fetch_dir, write_dir, command):
    """Write profiles/<kernel>_<workload>_traffic.json from a FETCH_SIZE run and
    a WRITE_SIZE run of this script (KiB per dispatch, scaled by the copy
    calibration), stamped with a hash of the kernel's sources."""
    for kernel, (match, sources) in TRAFFIC_KERNELS.items():
        try:
            f_kib, nf = _counter_per_dispatch(fetch_dir, match)
            w_kib, nw = _counter_per_dispatch(write_dir, match)
        except SystemExit:  # not dispatched in these runs
            continue
        rec = {"kernel": match, "workload": workload, "command": command,
               "fetch_kib_per_dispatch": round(f_kib, 1), "write_kib_per_dispatch": round(w_kib, 1),
               "dispatches": [nf, nw], "fetch_factor": FETCH_FACTOR, "write_factor": WRITE_FACTOR,
               "fetch_bytes": round(f_kib * 1024 * FETCH_FACTOR),
               "write_bytes": round(w_kib * 1024 * WRITE_FACTOR),
               "sources": sources, "source_hash": kernel_source_hash(sources)}
        out = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
        with open(out, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(out, rec["fetch_bytes"], rec["write_bytes"])


def _counters_by_dispatch(run_dir, match):
    """{dispatch: {counter: value}} over the dispatches of kernels whose name
    contains `match` in a rocprofv3 --pmc CSV directory."""
    import csv
    import glob

    out = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if match in row["Kernel_Name"]:
                    d = out.setdefault((path, row["Dispatch_Id"]), {})
                    d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
                    d["ns"] = float(row["End_Timestamp"]) - float(row["Start_Timestamp"])
    if not out:
        raise SystemExit(f"no dispatch of {match} in {run_dir}")
    return list(out.values())


XCDS = 8        # MI355X: GRBM_GUI_ACTIVE comes summed over its 8 XCDs
SIMDS = 1024    # 256 CUs x 4 SIMDs


def record_mfma(workload, run_dir, command):
    """Write profiles/project_pairs_<workload>_mfma.json from one rocprofv3
    --pmc run of SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES and
    GRBM_GUI_ACTIVE: executed bf16 MFMA FLOP per dispatch (MOPS x 512) and the
    matrix cores' busy fraction (busy cycles summed over SIMDs / (active cycles
    x SIMDs), rocprofv3's MfmaUtil)."""
    match, sources = TRAFFIC_KERNELS["project_pairs"]
    ds_ = _counters_by_dispatch(run_dir, match)
    n = len(ds_)
    mops = sum(d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for d in ds_) / n
    busy = sum(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in ds_) / n
    act = sum(d["GRBM_GUI_ACTIVE"] for d in ds_) / n / XCDS
    ns = sum(d["ns"] for d in ds_) / n
    rec = {"kernel": match, "workload": workload, "command": command, "dispatches": n,
           "mfma_flop_per_dispatch": mops * 512, "mfma_busy_cycles": busy, "active_cycles_per_xcd": act,
           "clock_ghz": round(act / ns, 3), "mfma_util": round(busy / (act * SIMDS), 4),
           "sources": sources, "source_hash": kernel_source_hash(sources)}
    out = os.path.join(ROOT, "profiles", f"project_pairs_{workload}_mfma.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(out, rec["mfma_util"], rec["clock_ghz"], rec["mfma_flop_per_dispatch"])


def mfma_from_profile(workload):
    """The committed counter record of the fused candidate projection, or None
    when there is none or its sources changed since."""
    path = os.path.join(ROOT, "profiles", f"project_pairs_{workload}_mfma.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != kernel_source_hash(t.get("sources", [])):
        return None
    return {"mfma_util": t["mfma_util"], "clock_ghz": t["clock_ghz"],
            "mfma_flop_per_dispatch": t["mfma_flop_per_dispatch"]}


def calibrate_copy():
    """Three plain device copies of 1 GiB: the reference dispatch for the HBM
    byte counters."""
    import torch

    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print("copied 3 x 1 GiB", flush=True)


def _cpu_model():
    """The host CPU's model name as lscpu reports it (else /proc/cpuinfo)."""
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _omp_threads(n=None):
    """The OpenMP team size of the oracle's runtime (libgomp, shared by the
    process), set to `n` if given; returns the previous maximum, or None if
    libgomp is not there."""
    import ctypes

    try:
        gomp = ctypes.CDLL("libgomp.so.1")
    except OSError:
        return None
    prev = gomp.omp_get_max_threads()
    if n is not None:
        gomp.omp_set_num_threads(int(n))
    return prev


def cpu_baseline(cfg, inp, run_s=3.0, runs=3, single_core=False):
    """The oracle as it stands on the host cores: the whole selector (top-16,
    fp64 projections, scores, walk) over a bounded sample of the workload's
    blocks, sized so that one run takes about `run_s` seconds, timed stage by
    stage inside the C library on the monotonic clock; the median of `runs`
    runs.  With `single_core`, one more run on a single OpenMP thread."""
    import oracle
    import synth

    oracle.build(force=False)
    mode = walk_modes(cfg)[0]
    sub1 = synth.sub_blocks(inp, np.arange(1))
    oracle.time_selector(sub1, mode, cfg.temperature)  # warm the pages and the thread team
    _, sec1, _ = oracle.time_selector(sub1, mode, cfg.temperature)
    n = int(max(1, min(cfg.batch, run_s / max(sum(sec1.values()), 1e-6))))
    sub = synth.sub_blocks(inp, np.arange(n))
    results = []
    for _ in range(runs):
        _, sec, threads = oracle.time_selector(sub, mode, cfg.temperature)
        results.append((sum(sec.values()), sec))
    results.sort(key=lambda x: x[0])
    total, sec = results[len(results) // 2]
    single = None
    if single_core:
        prev = _omp_threads(1)
        if prev is not None:
            try:
                n1 = int(max(1, min(cfg.batch, run_s / max(sum(sec1.values()) * threads, 1e-6))))
                _, s1, _ = oracle.time_selector(synth.sub_blocks(inp, np.arange(n1)), mode, cfg.temperature)
                single = {"value": round(n1 / sum(s1.values()), 3), "unit": "blocks/s", "blocks": n1,
                          "s": round(sum(s1.values()), 2), "cores": 1}
            finally:
                _omp_threads(prev)
    return {"value": round(n / total, 3), "unit": "blocks/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {cfg.batch} blocks of {cfg.name}, whole selector (top-16, fp64 projections, "
                      f"scores, {['greedy', 'sampled'][mode]} walk); median of {runs} runs "
                      f"({', '.join(f'{r[0]:.2f}' for r in sorted(results, key=lambda x: x[0]))} s)",
            "ms_per_block": {k: round(v * 1e3 / n, 3) for k, v in sec.items()},
            "single_core": single, "nproc": os.cpu_count(), "cpu_model": _cpu_model(),
            "build": "gcc -O2 -fopenmp, no fast-math; clock_gettime(CLOCK_MONOTONIC) around each stage in C"}


def time_verify(args, cfg, mode, lib, P, dt, cand_id, wres, stream, cache=None):
    """Verification of the drafted blocks (the step after the walk) against
    synthetic target logits [batch, block + 1, vocab]: HIP-event time per call
    and the HBM rate of its one pass over the target logits.  `cache` (a dict)
    keeps the device target logits for a second walk mode."""
    import torch

    import synth

    B, L, V = cfg.batch, cfg.block, cfg.vocab
    dev = cand_id.device
    cache = {} if cache is None else cache
    if "tl" not in cache:
        tl = synth.make_target_logits(cfg)
        ua, ur = synth.make_verify_uniforms(cfg)
        if tl.dtype == np.uint16:
            cache["tl"] = torch.from_numpy(tl.view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            cache["tl"] = torch.from_numpy(tl).to(dev)
        del tl
        cache["ua"], cache["ur"] = torch.from_numpy(ua).to(dev), torch.from_numpy(ur).to(dev)
    d_tl, d_ua, d_ur = cache["tl"], cache["ua"], cache["ur"]
    n_acc = torch.empty(B, dtype=torch.int32, device=dev)
    out_tok = torch.empty((B, L + 1), dtype=torch.int32, device=dev)
    wsb = lib.dsel_verify_workspace_bytes(B, L, V)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    q = wres.get("q")
    import ctypes as C
    sp = C.c_void_p(stream.cuda_stream)

    def call():
        st = lib.dsel_verify(P(d_tl), dt, B, L, None, V, V, P(cand_id), P(wres["path_slot"]),
                             P(q) if mode == 1 else None, mode, C.c_float(cfg.temperature),
                             P(d_ua) if mode == 1 else None, P(d_ur) if mode == 1 else None,
                             P(n_acc), P(out_tok), P(ws), wsb, sp)
        if st:
            raise RuntimeError(f"dsel_verify status {st}")

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    k = min(args.steps, 50)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(k):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / k
    nbytes = B * (L + 1) * V * (2 if cfg.logits_dtype == "bf16" else 4)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"mode": "sampled" if mode == 1 else "greedy", "us_per_call": round(us, 2),
            "target_logits_bytes": nbytes, "GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
            "mean_accepted": round(float(n_acc.float().mean()), 3),
            "data": "synthetic target logits: draft logits + N(0,1) noise, fresh row after the block"}


def time_gather(args, cfg, E, cand_id, stream):
    """The candidate GEMM's gather alone (dsel_gather_probe: the same LDS-DMA
    addressing, no MFMA) on the step's candidates: its HBM rate over the
    algorithmic bytes, every gathered row once."""
    import torch

    import draft_selection_amd as ds

    out = torch.empty(max(ds.lib().dsel_gather_probe_words(cfg.batch, cfg.block, cfg.d), 1), dtype=torch.int32,
                      device=E.device)
    for _ in range(3):
        ds.gather_probe(E, cand_id, out=out, stream=stream)
    torch.cuda.synchronize()
    k = min(args.steps, 50)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(k):
        ds.gather_probe(E, cand_id, out=out, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / k
    nbytes = algorithmic(cfg)["gather_bytes"]
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us_per_call": round(us, 2), "gathered_bytes": nbytes, "GB/s": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "what": "E[cand_id] rows into LDS through the candidate GEMM's LDS-DMA addressing, no MFMA"}


def time_conv(args, cfg, stream):
    """The dynamic two-tap convolution unit at the workload's drafter shape
    (x [batch, block, d]): HIP-event time per call, its HBM rate over the
    algorithmic bytes and the MFMA rate of its correction GEMM."""
    import ctypes as C

    import torch

    import draft_selection_amd as ds
    import synth

    c = synth.make_conv(cfg)
    dev = torch.device("cuda", torch.cuda.current_device())

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    x, xp, base, W = bf(c["x"]), bf(c["x_prev"]), bf(c["base"]), bf(c["W_c"])
    B, L, d = cfg.batch, cfg.block, cfg.d
    y = torch.empty_like(x)
    lib = ds.lib()
    wsb = lib.dsel_dyn_conv_workspace_bytes(B, L, d)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    P = ds._ptr
    sp = C.c_void_p(stream.cuda_stream)

    def call():
        st = lib.dsel_dyn_conv(P(x), P(xp), P(base), P(W), B, L, None, d, P(y), P(ws), wsb, sp)
        if st:
            raise RuntimeError(f"dsel_dyn_conv status {st}")

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    k = min(args.steps, 50)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(k):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / k
    M, N = B * L, 2 * (d // 16)
    nbytes = 2 * M * d * 2 + N * d * 2 + B * d * 2 + 2 * d * 2  # x, y, W_c, x_prev, base
    flop = 2 * M * N * d
    gbs = nbytes / (us * 1e-6) / 1e9
    tfs = flop / (us * 1e-6) / 1e12
    return {"us_per_call": round(us, 2), "bytes": nbytes, "GB/s": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "flop": flop, "TFLOP/s": round(tfs, 2),
            "mfma_frac": round(tfs / BF16_PEAK_TFLOPS, 4),
            "shape": f"x [{B}, {L}, {d}], W_c [{N}, {d}]",
            "data": "synthetic: x, x_prev ~ N(0,1); base tap 0 ~ 1 + N(0,0.01), tap 1 ~ N(0,0.01); W_c ~ N(0,(0.1/sqrt d)^2)"}


def time_lmhead(args, cfg, E, stream):
    """The LM head with the fused top-16 at the workload's shape (rows = batch x
    block hidden states against E, tied embeddings): HIP-event time per call
    and its MFMA rate; beside it the unfused route (torch's GEMM writing bf16
    logits, then select_topk), timed the same way."""
    import ctypes as C

    import torch
    import torch.nn.functional as F

    import draft_selection_amd as ds
    import synth

    dev = E.device
    R, V, dd = cfg.batch * cfg.block, cfg.vocab, cfg.d
    h = torch.from_numpy(synth.make_h(cfg).reshape(R, dd).view(np.int16)).to(dev).view(torch.bfloat16)
    lib = ds.lib()
    P = ds._ptr
    sp = C.c_void_p(stream.cuda_stream)
    cid = torch.empty((R, 16), dtype=torch.int32, device=dev)
    cu = torch.empty((R, 16), dtype=torch.float32, device=dev)
    wsb = lib.dsel_lmhead_topk_workspace_bytes(R, V)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)

    def fused():
        st = lib.dsel_lmhead_topk(P(h), P(E), R, V, dd, P(cid), P(cu), P(ws), wsb, sp)
        if st:
            raise RuntimeError(f"dsel_lmhead_topk status {st}")

    def unfused():
        with torch.cuda.stream(stream):
            z = F.linear(h, E)  # [R, V] bf16 logits in HBM
            ds.select_topk(z.view(1, R, V), stream=stream)

    def timed(fn, k):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(k):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / k

    k = 10
    us = timed(fused, k)
    us_unfused = timed(unfused, k)
    flop = 2.0 * R * V * dd
    tfs = flop / (us * 1e-6) / 1e12
    return {"us_per_call": round(us, 1), "flop": flop, "TFLOP/s": round(tfs, 1),
            "mfma_frac": round(tfs / BF16_PEAK_TFLOPS, 4), "logit_bytes_not_written": R * V * 2,
            "unfused_us": round(us_unfused, 1), "unfused": "torch F.linear (bf16 logits to HBM) + dsel_select_topk",
            "shape": f"h [{R}, {dd}] x E [{V}, {dd}]^T", "data": "synthetic h ~ N(0,1), E ~ N(0,0.02) (tied embeddings)"}


def stage_means(evs):
    """Mean microseconds between consecutive stage events over the steps."""
    out = {n: round(float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) * 1e3, 2)
           for i, n in enumerate(STAGES)}
    out["step"] = round(float(np.mean([e[0].elapsed_time(e[len(STAGES)]) for e in evs])) * 1e3, 2)
    return out


def stage_pcts(evs):
    """p10 / p50 / p90 microseconds of every stage and of the step."""
    out = {}
    for i, n in enumerate(STAGES):
        v = np.array([e[i].elapsed_time(e[i + 1]) for e in evs]) * 1e3
        out[n] = [round(float(x), 2) for x in np.percentile(v, (10, 50, 90))]
    v = np.array([e[0].elapsed_time(e[len(STAGES)]) for e in evs]) * 1e3
    out["step"] = [round(float(x), 2) for x in np.percentile(v, (10, 50, 90))]
    return out


def fused_route(ds, B, L, r):
    """Does dsel_select_path take the fused route for this shape (the rule of
    include/dsel.h: blocks of at most 16 positions and at least 128 workgroups)?"""
    nb = 16 // L if L <= 16 else 0
    return nb > 0 and -(-B // nb) * ds.pair_groups(r) >= 128


def graph_time(torch, fn, steps, warmup):
    """ms per call of `fn(stream)` captured once as a HIP graph, replayed `steps`
    times (after `warmup` replays) between two synchronisations."""
    stream = torch.cuda.current_stream()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        fn(cap)
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(torch.cuda.current_stream())
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    del g
    return ms


def bench_workload(args, name, ds, torch):
    """Every measurement of one workload; returns its record."""
    import ctypes as C

    import synth

    cfg = synth.CONFIGS[name]
    lib = ds.lib()
    P = ds._ptr
    dev = torch.device("cuda:0")
    print(f"[bench] {describe(cfg)}: generating inputs", file=sys.stderr, flush=True)
    t0 = time.time()
    inp = synth.make(cfg)
    d = synth.to_device(inp, dev)
    gen_s = time.time() - t0
    stream = torch.cuda.current_stream()
    B, L, V, r = cfg.batch, cfg.block, cfg.vocab, cfg.r
    dt = ds.BF16 if cfg.logits_dtype == "bf16" else ds.F32
    modes = walk_modes(cfg)
    fused = fused_route(ds, B, L, r)
    nq = ds.pair_groups(r)

    # outputs and workspaces allocated once, outside the timed regions
    cand_id = torch.empty((B, L, K), dtype=torch.int32, device=dev)
    cand_u = torch.empty((B, L, K), dtype=torch.float32, device=dev)
    xwsb = lib.dsel_select_path_workspace_bytes(B, L, V, dt, cfg.d, r)
    xws = torch.empty(max(xwsb, 256), dtype=torch.uint8, device=dev)
    walks = {m: ds._walk_args(cand_id, m, cfg.temperature, d["uniforms"], m == 1, True) for m in modes}

    def path_args(lens):
        return ds.PathArgs(d["logits"].data_ptr(), dt, V, V, d["E"].data_ptr(), cfg.d, d["W_A"].data_ptr(),
                           d["W_B"].data_ptr(), d["W_H"].data_ptr(), r, d["h"].data_ptr(), d["verified"].data_ptr(),
                           B, L, None if lens is None else lens.data_ptr(), cand_id.data_ptr(), cand_u.data_ptr(),
                           None, None, None, None)

    pargs = {False: path_args(None)}

    def step(strm, mode, lens=None):
        key = lens is not None
        if key not in pargs:
            pargs[key] = path_args(lens)
        st = lib.dsel_select_path(C.byref(pargs[key]), C.byref(walks[mode][0]), P(xws), xwsb,
                                  C.c_void_p(strm.cuda_stream))
        if st:
            raise RuntimeError(f"dsel_select_path status {st}")

    # stage-by-stage route (eager, HIP events between the stages): the same
    # kernels as the one call, its gate reduction as a launch of its own
    A_full = torch.empty((B, L, K, r), dtype=torch.float32, device=dev)  # gate's A(verified) rows
    G = torch.empty((B, L, r), dtype=torch.float32, device=dev)
    pwsb = ds.project_workspace_bytes(B, L, cfg.d, r)
    pws = torch.empty(max(pwsb, 16), dtype=torch.uint8, device=dev)
    twsb = ds.topk_workspace_bytes(B * L, V, d["logits"].dtype)
    tws = torch.empty(max(twsb, 16), dtype=torch.uint8, device=dev)
    if fused:
        part = torch.empty((B, L, nq, K, K), dtype=torch.float32, device=dev)
    else:
        B_cur = torch.empty_like(A_full)
        S = torch.empty((B, L, K, K), dtype=torch.float32, device=dev)

    def stages(strm, ev, mode, lens=None):
        sp = C.c_void_p(strm.cuda_stream)
        LN = P(lens) if lens is not None else None
        ev[0].record(strm)
        s0 = lib.dsel_project_gate(P(d["E"]), V, cfg.d, P(d["W_A"]), P(d["W_H"]), r, P(d["h"]), P(d["verified"]),
                                   B, L, LN, P(A_full), P(G), P(pws), pwsb, sp)
        ev[1].record(strm)
        s1 = lib.dsel_select_topk(P(d["logits"]), dt, B, L, LN, V, V, P(cand_id), P(cand_u), P(tws), twsb, sp)
        ev[2].record(strm)
        if fused:
            s2 = lib.dsel_project_pairs(P(d["E"]), V, cfg.d, P(d["W_A"]), P(d["W_B"]), r, P(cand_id), P(G),
                                        P(A_full), L * K * r, B, L, LN, P(part), None, None, sp)
            ev[3].record(strm)
            s3 = lib.dsel_walk_pairs(P(cand_u), P(part), B, L, LN, nq, None, C.byref(walks[mode][0]), sp)
        else:
            s2 = lib.dsel_project_cand(P(d["E"]), V, cfg.d, P(d["W_A"]), P(d["W_B"]), r, P(cand_id), B, L, LN,
                                       P(A_full), P(B_cur), P(pws), pwsb, sp)
            ev[3].record(strm)
            s3 = lib.dsel_score_pairs(P(cand_u), P(A_full), P(B_cur), P(G), B, L, LN, r, P(S),
                                      C.byref(walks[mode][0]), sp)
        ev[4].record(strm)
        if s0 or s1 or s2 or s3:
            raise RuntimeError(f"dsel status {s0} {s1} {s2} {s3}")

    def new_events(n):
        return [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)] for _ in range(n)]

    res_walks = {}
    for m in modes:
        for _ in range(args.warmup):
            step(stream, m)
        torch.cuda.synchronize()
        if args.separate:
            scratch = new_events(1)[0]
            ms = graph_time(torch, lambda s, m=m: stages(s, scratch, m), args.steps, args.warmup)
        else:
            ms = graph_time(torch, lambda s, m=m: step(s, m), args.steps, args.warmup)
        res_walks[["greedy", "sampled"][m]] = {"ms_per_step": round(ms, 5), "blocks/s": round(B / (ms * 1e-3), 1),
                                               "us_per_block": round(ms * 1e3 / B, 4)}
    assert ds.device_error() == 0
    mode = modes[0]

    # eager stage timing (warm), then cold: a 1 GiB write before every step
    # evicts L2 and the Infinity Cache (the events exclude that write)
    evs = new_events(args.steps)
    t0 = time.perf_counter()
    for i in range(args.steps):
        stages(stream, evs[i], mode)
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - t0
    cold = cold_pct = None
    if not args.no_cold:
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        cevs = new_events(args.steps)
        for i in range(args.steps):
            flush.fill_(float(i))
            stages(stream, cevs[i], mode)
        torch.cuda.synchronize()
        del flush
        cold, cold_pct = stage_means(cevs), stage_pcts(cevs)
    warm = stage_means(evs)

    # a ragged batch of the same shape (each block 5, 8 or 16 positions); a
    # batch of a few blocks has no mix to speak of
    ragged = None
    if not args.no_ragged and L > 1 and B >= 8:
        lens_np = synth.make_block_len(cfg)
        lens = torch.from_numpy(lens_np).to(dev)
        revs = new_events(min(args.steps, 50))
        for e in revs:
            stages(stream, e, mode, lens)
        torch.cuda.synchronize()
        ms_r = graph_time(torch, lambda s: step(s, mode, lens), args.steps, args.warmup)
        assert ds.device_error() == 0
        pos = int(lens_np.sum())
        ms_u = res_walks[["greedy", "sampled"][mode]]["ms_per_step"]
        ragged = {"lengths": "each block %s positions, drawn uniformly" % " / ".join(map(str, sorted(set(lens_np.tolist())))),
                  "positions": pos, "padded_positions": B * L, "ms_per_step": round(ms_r, 5),
                  "blocks/s": round(B / (ms_r * 1e-3), 1), "positions/s": round(pos / (ms_r * 1e-3), 1),
                  "uniform_positions/s": round(B * L / (ms_u * 1e-3), 1),
                  "positions_rate_vs_uniform": round((pos / ms_r) / (B * L / ms_u), 4),
                  "stages_us": stage_means(revs)}

    # the legs after the step: verification of the drafted blocks, the
    # convolution unit, the gather alone, the LM head with its top-16
    verify = None
    if not args.no_verify:
        verify, vcache = {}, {}
        for m in modes:
            step(stream, m)
            verify[["greedy", "sampled"][m]] = time_verify(args, cfg, m, lib, P, dt, cand_id, walks[m][1], stream,
                                                           vcache)
        del vcache
    conv = None if args.no_conv or cfg.d % 512 else time_conv(args, cfg, stream)
    gather = time_gather(args, cfg, d["E"], cand_id, stream)
    lmhead = time_lmhead(args, cfg, d["E"], stream) if (args.lmhead or name in ("c2", "c4")) and not args.no_lmhead \
        else None

    alg = algorithmic(cfg)
    st_topk, st_proj = warm["topk"], warm["project"]
    topk_gbs = alg["topk_bytes"] / (st_topk * 1e-6) / 1e9
    proj_tfs = alg["cand_flop"] / (st_proj * 1e-6) / 1e12
    kproj = "project_pairs" if fused else "project_cand"
    if st_topk >= st_proj:
        roof = {"kernel": "topk16", "bound": "hbm", "achieved": round(topk_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(topk_gbs / HBM_PEAK_GBS, 4), "traffic": traffic_from_profile(name, "topk16"),
                "per_launch": f"{alg['topk_bytes']} algorithmic bytes (every logit once, 16 keys out per row) / "
                              f"{st_topk} us (HIP events)"}
    else:
        roof = {"kernel": kproj, "bound": "mfma", "achieved": round(proj_tfs, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(proj_tfs / BF16_PEAK_TFLOPS, 4),
                "traffic": traffic_from_profile(name, "project_pairs") if fused else None,
                "per_launch": f"{alg['cand_flop']:.4g} algorithmic projection FLOP (2 d r per needed A or B row) / "
                              f"{st_proj} us (HIP events)"}
    prim = res_walks[["greedy", "sampled"][mode]]
    rec = {
        "workload": describe(cfg),
        "route": {ds.ROUTE_FUSED: "fused (dsel_project_pairs + dsel_walk_pairs kernels)",
                  ds.ROUTE_SMALL: "small-batch (three launches: top-16 beside the gate GEMM, candidate GEMM "
                                  "with the list merge, pair tables and walk)",
                  ds.ROUTE_SEPARATE: "separate kernels"}[ds.select_path_route(B, L, V, d["logits"].dtype, cfg.d, r)],
        "value": prim["blocks/s"], "unit": "blocks/s", "ms_per_step": prim["ms_per_step"],
        "us_per_block": prim["us_per_block"], "walks": res_walks, "dtype": dtype_of(cfg),
        "config": {"workload": describe(cfg), "batch": B, "block": L, "vocab": V, "d": cfg.d, "r": r,
                   "logits": cfg.logits_dtype, "walk": cfg.walk},
        "ms_per_step_eager": round(wall_eager * 1e3 / args.steps, 5),
        "stages_us": warm, "stages_us_p10_p50_p90": stage_pcts(evs),
        "stages_us_cold": cold, "stages_us_cold_p10_p50_p90": cold_pct,
        "select_topk_hbm": {"GB/s": round(topk_gbs, 1), "frac": round(topk_gbs / HBM_PEAK_GBS, 4)},
        "project_mfma": {"kernel": kproj, "TFLOP/s": round(proj_tfs, 2), "frac": round(proj_tfs / BF16_PEAK_TFLOPS, 4),
                         "counters": mfma_from_profile(name) if fused else None},
        "project_gather": {"GB/s": round(alg["gather_bytes"] / (st_proj * 1e-6) / 1e9, 1),
                           "frac": round(alg["gather_bytes"] / (st_proj * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "gather_probe": gather, "roofline": roof, "verify": verify, "dyn_conv": conv, "lmhead_topk": lmhead,
        "ragged": ragged, "input_generation_s": round(gen_s, 1),
    }
    del d, xws, A_full, G, pws, tws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print(f"[bench] {name}: timing the oracle on the host", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(cfg, inp, single_core=(name == "c2"))
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="all", choices=["all", "c1", "c2", "c3", "c4"],
                    help="all (default): c2, c3 and c4 in one run, headline c4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true", help="skip the pass that evicts the caches before every step")
    ap.add_argument("--no-verify", action="store_true", help="skip timing dsel_verify after the walk")
    ap.add_argument("--no-conv", action="store_true", help="skip timing the convolution unit (dsel_dyn_conv)")
    ap.add_argument("--no-ragged", action="store_true", help="skip the ragged batch (per-block lengths)")
    ap.add_argument("--lmhead", action="store_true", help="time the LM head with its top-16 at every workload "
                                                          "(by default at c2 and c4)")
    ap.add_argument("--no-lmhead", action="store_true", help="skip the LM head leg")
    ap.add_argument("--separate", action="store_true",
                    help="time the graph of the stage-by-stage calls instead of one dsel_select_path call")
    ap.add_argument("--record-mfma", nargs=2, metavar=("RUN_DIR", "COMMAND"),
                    help="write profiles/project_pairs_<workload>_mfma.json from a rocprofv3 --pmc run")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--record-traffic", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "COMMAND"),
                    help="write profiles/*_traffic.json for --workload from two rocprofv3 --pmc runs")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args.workload, *args.record_traffic)
        return
    if args.record_mfma:
        record_mfma(args.workload, *args.record_mfma)
        return
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only (the selector shards by draft block with no exchange, "
              "so one GPU's share is the whole measurement); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import draft_selection_amd as ds

    names = (LATENCY,) + GRADED if args.workload == "all" else (args.workload,)
    head = HEADLINE if args.workload == "all" else args.workload
    recs = {}
    for n in names:
        recs[n] = bench_workload(args, n, ds, torch)
        print(f"[bench] {n}: {recs[n]['value']} blocks/s, {recs[n]['ms_per_step']} ms/step", file=sys.stderr,
              flush=True)
    h = recs[head]
    out = {
        "metric": METRIC, "value": h["value"], "unit": "blocks/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": h["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": h["dtype"], "data": "synthetic",
        "config": h["config"], "us_per_block": h["us_per_block"],
        "timing": "value: one dsel_select_path call per step, captured once as a HIP graph and replayed K times "
                  "(first walk mode of the workload); stages_us: the same kernels called stage by stage, eager, "
                  "HIP events on the launch stream; stages_us_cold: after a 1 GiB cache-evicting write",
        "step_call": "stage-by-stage calls" if args.separate else "dsel_select_path",
        "roofline": h["roofline"],
        "cpu_baseline": h.get("cpu_baseline"),
        "headline": head,
        "workloads": recs,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
