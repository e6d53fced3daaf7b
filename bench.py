"""Throughput of the DFlash 2 path selector on one MI355X.

One step = the whole selector over one batch of draft blocks, inputs already
resident in HBM: select_topk -> project -> score_pairs with the fused walk.
Prints one JSON line (rank 0, one GPU).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2]

Workloads (synthetic, seeded; see synth.CONFIGS): c1 one block of 16 (latency
shape), c2 64 blocks of 16 (the default: batched throughput), c3 128 blocks of 8
with the sampled walk, c4 256 blocks of 16 with fp32 logits.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft blocks/s through selector + achieved HBM GB/s & MFMA % of peak"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
K = 16
# HBM byte counters against a plain 1 GiB device copy (--calibrate-copy): per
# copied GiB FETCH_SIZE reads 0.5 GiB and WRITE_SIZE 1 GiB, so the counters'
# KiB are multiplied by these factors to give bytes moved.
FETCH_FACTOR = 2.0
WRITE_FACTOR = 1.0
# kernels whose traffic is recorded, and the sources each is built from
TRAFFIC_KERNELS = {
    "topk16": ("topk16_kernel", ["common.h", "topk16.h"]),
    "project_cand": ("project_cand_kernel", ["common.h", "project.h"]),
    "verify_stats": ("verify_stats_kernel", ["common.h", "verify.h"]),
}


def describe(cfg):
    walk = {"greedy": "greedy walk", "sampled": "sampled walk (T=1)", "both": "greedy walk"}[cfg.walk]
    return (f"{cfg.name}: {cfg.batch} blocks x {cfg.block} positions, vocab {cfg.vocab}, "
            f"d {cfg.d}, r {cfg.r}, {cfg.logits_dtype} logits, {walk}")


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
    return dict(topk_bytes=topk_bytes, cand_flop=cand_flop, gate_flop=gate_flop, gather_bytes=gather_bytes)


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
        f_kib, nf = _counter_per_dispatch(fetch_dir, match)
        w_kib, nw = _counter_per_dispatch(write_dir, match)
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
    """Write profiles/project_cand_<workload>_mfma.json from one rocprofv3
    --pmc run of SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES and
    GRBM_GUI_ACTIVE: executed bf16 MFMA FLOP per dispatch (MOPS x 512) and the
    matrix cores' busy fraction (busy cycles summed over SIMDs / (active cycles
    x SIMDs), rocprofv3's MfmaUtil)."""
    match, sources = TRAFFIC_KERNELS["project_cand"]
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
    out = os.path.join(ROOT, "profiles", f"project_cand_{workload}_mfma.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(out, rec["mfma_util"], rec["clock_ghz"], rec["mfma_flop_per_dispatch"])


def mfma_from_profile(workload):
    """The committed counter record of the candidate GEMM, or None when there
    is none or its sources changed since."""
    path = os.path.join(ROOT, "profiles", f"project_cand_{workload}_mfma.json")
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
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_stages(oracle, sub, mode, T, acc):
    """One oracle pass over `sub`, stage by stage, adding seconds to `acc`."""
    t0 = time.perf_counter()
    cand_id, cand_u = oracle.select_topk(sub["logits"])
    t1 = time.perf_counter()
    A, Bm, G = oracle.project(sub["E"], sub["W_A"], sub["W_B"], sub["W_H"], sub["h"], cand_id, sub["verified"])
    t2 = time.perf_counter()
    S = oracle.score_pairs(cand_u, A, Bm, G)
    t3 = time.perf_counter()
    oracle.walk(S, cand_id, mode, sub.get("uniforms"), T)
    t4 = time.perf_counter()
    for k, dt in zip(("select_topk", "project", "score_pairs", "walk"), (t1 - t0, t2 - t1, t3 - t2, t4 - t3)):
        acc[k] = acc.get(k, 0.0) + dt
    return t4 - t0


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


def cpu_baseline(cfg, inp, budget_s=15.0, single_core_s=3.0):
    """The oracle as it stands, on the host cores, over as many blocks as fit in
    about `budget_s` seconds (at least one), stage by stage; for the smaller
    workloads also a few blocks on one core."""
    import oracle
    import synth

    oracle.build(force=False)
    mode = 1 if cfg.walk == "sampled" else 0
    done, t_total, stages = 0, 0.0, {}
    chunk = 1
    while done < cfg.batch and t_total < budget_s:
        n = min(chunk, cfg.batch - done)
        sub = synth.sub_blocks(inp, np.arange(done, done + n))
        t_total += _oracle_stages(oracle, sub, mode, cfg.temperature, stages)
        done += n
        chunk = min(2 * chunk, 16)
    prev = _omp_threads(1) if cfg.d <= 2560 else None
    single = None
    if prev is not None:
        try:
            n1, t1 = 0, 0.0
            while n1 < cfg.batch and t1 < single_core_s:
                t1 += _oracle_stages(oracle, synth.sub_blocks(inp, np.arange(n1, n1 + 1)), mode, cfg.temperature, {})
                n1 += 1
            single = {"value": n1 / t1, "unit": "blocks/s", "blocks": n1, "s": round(t1, 2)}
        finally:
            _omp_threads(prev)
    cores = _omp_threads() or int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": done / t_total, "unit": "blocks/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {cfg.batch} blocks of {cfg.name}, whole selector "
                      f"(top-16, fp64 projections, scores, walk), {t_total:.1f} s",
            "ms_per_block": {k: round(v * 1e3 / done, 3) for k, v in stages.items()},
            "single_core": single, "nproc": os.cpu_count(), "cpu_model": _cpu_model(),
            "build": "gcc -O2 -fopenmp, no fast-math; perf_counter around each stage call"}


def time_verify(args, cfg, mode, lib, P, dt, cand_id, wres, stream):
    """Verification of the drafted blocks (the step after the walk) against
    synthetic target logits [batch, block + 1, vocab]: HIP-event time per call
    and the HBM rate of its one pass over the target logits."""
    import torch

    import synth

    B, L, V = cfg.batch, cfg.block, cfg.vocab
    tl = synth.make_target_logits(cfg)
    ua, ur = synth.make_verify_uniforms(cfg)
    dev = cand_id.device
    if tl.dtype == np.uint16:
        d_tl = torch.from_numpy(tl.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        d_tl = torch.from_numpy(tl).to(dev)
    del tl
    d_ua, d_ur = torch.from_numpy(ua).to(dev), torch.from_numpy(ur).to(dev)
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


def stage_pcts(evs):
    """p10 / p50 / p90 microseconds of every stage and of the step."""
    names = ("project_gate", "select_topk", "project_cand", "score_pairs_walk")
    out = {}
    for i, n in enumerate(names):
        v = np.array([e[i].elapsed_time(e[i + 1]) for e in evs]) * 1e3
        out[n] = [round(float(x), 2) for x in np.percentile(v, (10, 50, 90))]
    v = np.array([e[0].elapsed_time(e[4]) for e in evs]) * 1e3
    out["step"] = [round(float(x), 2) for x in np.percentile(v, (10, 50, 90))]
    return out


def stage_means(evs):
    """Mean microseconds between consecutive stage events over the steps."""
    names = ("project_gate", "select_topk", "project_cand", "score_pairs_walk")
    out = {n: round(float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) * 1e3, 2)
           for i, n in enumerate(names)}
    out["step"] = round(float(np.mean([e[0].elapsed_time(e[4]) for e in evs])) * 1e3, 2)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2", choices=["c1", "c2", "c3", "c4"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gate", default="serial", choices=["serial", "side", "overlap"],
                    help="run the gate GEMM before the top-16 (serial), beside it on a second stream "
                         "(side: split along d, with its reduce; overlap: one workgroup per tile)")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the pass that evicts the caches before every step")
    ap.add_argument("--no-verify", action="store_true",
                    help="skip timing the verification of the drafted blocks (dsel_verify)")
    ap.add_argument("--no-conv", action="store_true",
                    help="skip timing the dynamic two-tap convolution unit (dsel_dyn_conv)")
    ap.add_argument("--separate", action="store_true",
                    help="time the graph of separate calls instead of one dsel_select_path call")
    ap.add_argument("--no-ragged", action="store_true",
                    help="skip timing the same step on a ragged batch (per-block lengths)")
    ap.add_argument("--lmhead", action="store_true",
                    help="also time the LM head with the fused top-16 (dsel_lmhead_topk) and the unfused route")
    ap.add_argument("--record-mfma", nargs=2, metavar=("RUN_DIR", "COMMAND"),
                    help="write profiles/project_cand_<workload>_mfma.json from a rocprofv3 --pmc run")
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
    import synth

    cfg = synth.CONFIGS[args.workload]
    mode = 1 if cfg.walk == "sampled" else 0
    print(f"[bench] generating {describe(cfg)}", file=sys.stderr, flush=True)
    inp = synth.make(cfg)
    dev = torch.device("cuda:0")
    d = synth.to_device(inp, dev)
    stream = torch.cuda.current_stream()

    # outputs and workspace allocated once, outside the timed region
    B, L, V = cfg.batch, cfg.block, cfg.vocab
    cand_id = torch.empty((B, L, K), dtype=torch.int32, device=dev)
    cand_u = torch.empty((B, L, K), dtype=torch.float32, device=dev)
    A_prev = torch.empty((B, L, K, cfg.r), dtype=torch.float32, device=dev)
    B_cur = torch.empty_like(A_prev)
    G = torch.empty((B, L, cfg.r), dtype=torch.float32, device=dev)
    wsb = ds.topk_workspace_bytes(B * L, V, d["logits"].dtype)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    pwsb = ds.project_workspace_bytes(B, L, cfg.d, cfg.r)
    pws = torch.empty(max(pwsb, 1), dtype=torch.uint8, device=dev)
    S = torch.empty((B, L, K, K), dtype=torch.float32, device=dev)
    # the sampled walk also returns its step distributions q: verification needs them
    wargs, wres = ds._walk_args(cand_id, mode, cfg.temperature, d["uniforms"], mode == 1, True)

    import ctypes as C
    lib = ds.lib()
    P = ds._ptr
    dt = ds.BF16 if cfg.logits_dtype == "bf16" else ds.F32

    side = ds.side_stream(dev)
    ss = C.c_void_p(side.cuda_stream)
    fork = [torch.cuda.Event() for _ in range(2)]

    # the whole step as one dsel_select_path call (the gate's split-K
    # reduction rides in the top-16 launch); the eager stage timing below uses
    # the separate calls, which give the same bits
    fused = args.gate == "serial" and not args.separate
    xwsb = lib.dsel_select_path_workspace_bytes(B, L, V, dt, cfg.d, cfg.r)
    xws = torch.empty(max(xwsb, 16), dtype=torch.uint8, device=dev)

    def path_args(lens):
        return ds.PathArgs(d["logits"].data_ptr(), dt, V, V, d["E"].data_ptr(), cfg.d, d["W_A"].data_ptr(),
                           d["W_B"].data_ptr(), d["W_H"].data_ptr(), cfg.r, d["h"].data_ptr(),
                           d["verified"].data_ptr(), B, L, None if lens is None else lens.data_ptr(),
                           cand_id.data_ptr(), cand_u.data_ptr(), A_prev.data_ptr(), B_cur.data_ptr(),
                           G.data_ptr(), S.data_ptr())

    pargs = {}

    def step(strm, ev=None, lens=None):
        # the gate GEMM needs no candidates: either it runs first, or on a side
        # stream beside the top-16 (the side stream first waits for the
        # previous step).  `lens`: per-block lengths of a ragged batch.
        sp = C.c_void_p(strm.cuda_stream)
        if fused and ev is None:
            key = lens is not None
            if key not in pargs:
                pargs[key] = path_args(lens)
            st = lib.dsel_select_path(C.byref(pargs[key]), C.byref(wargs), P(xws), xwsb, sp)
            if st:
                raise RuntimeError(f"dsel_select_path status {st}")
            return
        LN = P(lens) if lens is not None else None
        if ev is not None:
            ev[0].record(strm)
        par = args.gate in ("side", "overlap")
        if par:
            fork[0].record(strm)
            side.wait_event(fork[0])
        if args.gate == "side":
            s0 = lib.dsel_project_gate(P(d["E"]), V, cfg.d, P(d["W_A"]), P(d["W_H"]), cfg.r, P(d["h"]),
                                       P(d["verified"]), B, L, LN, P(A_prev), P(G), P(pws), pwsb, ss)
        elif args.gate == "overlap":
            s0 = lib.dsel_project_gate_overlap(P(d["E"]), V, cfg.d, P(d["W_A"]), P(d["W_H"]), cfg.r, P(d["h"]),
                                               P(d["verified"]), B, L, LN, P(A_prev), P(G), ss)
        else:
            s0 = lib.dsel_project_gate(P(d["E"]), V, cfg.d, P(d["W_A"]), P(d["W_H"]), cfg.r, P(d["h"]),
                                       P(d["verified"]), B, L, LN, P(A_prev), P(G), P(pws), pwsb, sp)
        if par:
            fork[1].record(side)
        if ev is not None:
            ev[1].record(strm)
        s1 = lib.dsel_select_topk(P(d["logits"]), dt, B, L, LN, V, V, P(cand_id), P(cand_u), P(ws), wsb, sp)
        if ev is not None:
            ev[2].record(strm)
        if par:
            strm.wait_event(fork[1])
        s2 = lib.dsel_project_cand(P(d["E"]), V, cfg.d, P(d["W_A"]), P(d["W_B"]), cfg.r, P(cand_id),
                                   B, L, LN, P(A_prev), P(B_cur), P(pws), pwsb, sp)
        if ev is not None:
            ev[3].record(strm)
        s3 = lib.dsel_score_pairs(P(cand_u), P(A_prev), P(B_cur), P(G), B, L, LN, cfg.r, P(S),
                                  C.byref(wargs), sp)
        if ev is not None:
            ev[4].record(strm)
        if s0 or s1 or s2 or s3:
            raise RuntimeError(f"dsel status {s0} {s1} {s2} {s3}")

    for _ in range(args.warmup):
        step(stream)
    torch.cuda.synchronize()

    # (1) eager timed region: K steps with HIP events around every stage on the
    # stream the kernels run on (per-kernel durations for the roofline)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(stream, evs[i])
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - t0

    # (2) the step captured once as a HIP graph (launch overhead removed),
    # replayed K times: the throughput figure
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        step(cap)
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step(torch.cuda.current_stream())
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert ds.device_error() == 0

    # (3) cold caches: before every step a 1 GiB write evicts L2 and the
    # Infinity Cache; the stage events exclude that write
    cold = cold_pct = None
    if not args.no_cold:
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        cevs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
        for i in range(args.steps):
            flush.fill_(float(i))
            step(stream, cevs[i])
        torch.cuda.synchronize()
        del flush
        cold = stage_means(cevs)
        cold_pct = stage_pcts(cevs)

    # (4) a ragged batch: the same step with each block at its own length
    # (the 5 / 8 / 16 mix), one HIP graph replayed K times
    ragged = None
    if not args.no_ragged and L > 1:
        lens_np = synth.make_block_len(cfg)
        lens = torch.from_numpy(lens_np).to(dev)
        revs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
        for i in range(args.steps):
            step(stream, revs[i], lens=lens)
        torch.cuda.synchronize()
        rgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(rgraph):
            step(torch.cuda.current_stream(), lens=lens)
        for _ in range(args.warmup):
            rgraph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            rgraph.replay()
        torch.cuda.synchronize()
        ms_r = (time.perf_counter() - t0) * 1e3 / args.steps
        assert ds.device_error() == 0
        pos = int(lens_np.sum())
        ragged = {"lengths": "each block %s positions, drawn uniformly"
                             % " / ".join(map(str, sorted(set(lens_np.tolist())))),
                  "positions": pos, "padded_positions": B * L,
                  "ms_per_step": round(ms_r, 5), "blocks/s": round(B / (ms_r * 1e-3), 1),
                  "positions/s": round(pos / (ms_r * 1e-3), 1),
                  "uniform_positions/s": round(B * L / (wall / args.steps), 1),
                  "stages_us": stage_means(revs)}
        del rgraph

    verify = None if args.no_verify else time_verify(args, cfg, mode, lib, P, dt, cand_id, wres, stream)
    conv = None if args.no_conv or cfg.d % 512 else time_conv(args, cfg, stream)
    gather = time_gather(args, cfg, d["E"], cand_id, stream)
    lmhead = time_lmhead(args, cfg, d["E"], stream) if args.lmhead else None

    ms_step = wall * 1e3 / args.steps
    warm = stage_means(evs)
    st_topk, st_proj, st_pair = warm["select_topk"], warm["project_cand"], warm["score_pairs_walk"]
    alg = algorithmic(cfg)
    topk_gbs = alg["topk_bytes"] / (st_topk * 1e-6) / 1e9
    proj_tfs = alg["cand_flop"] / (st_proj * 1e-6) / 1e12

    if st_topk >= st_proj:
        roof = {"kernel": "topk16", "bound": "hbm", "achieved": round(topk_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(topk_gbs / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profile(cfg.name, "topk16")}
    else:
        roof = {"kernel": "project_cand", "bound": "mfma", "achieved": round(proj_tfs, 2),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(proj_tfs / BF16_PEAK_TFLOPS, 4),
                "traffic": traffic_from_profile(cfg.name, "project_cand")}

    out = {
        "metric": METRIC,
        "value": round(B / (ms_step * 1e-3), 1),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": describe(cfg), "batch": B, "block": L, "vocab": V, "d": cfg.d,
                   "r": cfg.r, "logits": cfg.logits_dtype, "walk": "sampled" if mode else "greedy"},
        "us_per_block": round(ms_step * 1e3 / B, 4),
        "ms_per_step_eager": round(wall_eager * 1e3 / args.steps, 5),
        "timing": "value: the step (step_call) as one HIP graph replayed K times; stages: eager separate calls with "
                  "HIP events on the launch stream (stages_us_cold: after a 1 GiB cache-evicting write)",
        "stages_us": warm,
        "stages_us_cold": cold,
        "stages_us_p10_p50_p90": stage_pcts(evs),
        "stages_us_cold_p10_p50_p90": cold_pct,
        "select_topk_hbm": {"GB/s": round(topk_gbs, 1), "frac": round(topk_gbs / HBM_PEAK_GBS, 4)},
        "project_cand_mfma": {"TFLOP/s": round(proj_tfs, 2), "frac": round(proj_tfs / BF16_PEAK_TFLOPS, 4),
                              "counters": mfma_from_profile(cfg.name)},
        "project_cand_gather": {"GB/s": round(alg["gather_bytes"] / (st_proj * 1e-6) / 1e9, 1),
                                "frac": round(alg["gather_bytes"] / (st_proj * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "gather_probe": gather,
        "project_gate": args.gate,
        "step_call": "dsel_select_path" if fused else "separate calls",
        "roofline": roof,
        "verify": verify,
        "dyn_conv": conv,
        "lmhead_topk": lmhead,
        "ragged": ragged,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
