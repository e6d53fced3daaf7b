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


def describe(cfg):
    walk = {"greedy": "greedy walk", "sampled": "sampled walk (T=1)", "both": "greedy walk"}[cfg.walk]
    return (f"{cfg.name}: {cfg.batch} blocks x {cfg.block} positions, vocab {cfg.vocab}, "
            f"d {cfg.d}, r {cfg.r}, {cfg.logits_dtype} logits, {walk}")


def algorithmic(cfg):
    """Bytes / FLOP every stage must move / do once per step."""
    es = 2 if cfg.logits_dtype == "bf16" else 4
    rows = cfg.batch * cfg.block
    topk_bytes = rows * cfg.vocab * es + rows * K * 8
    a_rows = cfg.batch * (K * (cfg.block - 1) + 1)   # predecessors that need A
    b_rows = cfg.batch * cfg.block * K               # candidates that need B
    proj_flop = 2.0 * cfg.d * cfg.r * (a_rows + b_rows + rows)
    return dict(topk_bytes=topk_bytes, proj_flop=proj_flop)


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


def cpu_baseline(cfg, inp, budget_s=15.0):
    """The oracle as it stands, on the host cores, over as many blocks as fit in
    about `budget_s` seconds (at least one)."""
    import oracle
    import synth

    oracle.build(force=False)
    mode = 1 if cfg.walk == "sampled" else 0
    done, t_total = 0, 0.0
    chunk = 1
    while done < cfg.batch and t_total < budget_s:
        n = min(chunk, cfg.batch - done)
        sub = synth.sub_blocks(inp, np.arange(done, done + n))
        t0 = time.perf_counter()
        oracle.run(sub, mode, cfg.temperature)
        t_total += time.perf_counter() - t0
        done += n
        chunk = min(2 * chunk, 16)
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": done / t_total, "unit": "blocks/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {cfg.batch} blocks of {cfg.name}, whole selector "
                      f"(top-16, fp64 projections, scores, walk), {t_total:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2", choices=["c1", "c2", "c3", "c4"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the selector is block-parallel and this build runs on "
              "a single MI355X; run it with --gpus 1", file=sys.stderr)
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
    wargs, wres = ds._walk_args(cand_id, mode, cfg.temperature, d["uniforms"], False, True)

    import ctypes as C
    lib = ds.lib()
    sp = C.c_void_p(stream.cuda_stream)
    P = ds._ptr
    dt = ds.BF16 if cfg.logits_dtype == "bf16" else ds.F32

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        s1 = lib.dsel_select_topk(P(d["logits"]), dt, B, L, V, V, P(cand_id), P(cand_u), P(ws), wsb, sp)
        if ev is not None:
            ev[1].record(stream)
        s2 = lib.dsel_project(P(d["E"]), V, cfg.d, P(d["W_A"]), P(d["W_B"]), P(d["W_H"]), cfg.r,
                              P(d["h"]), P(cand_id), P(d["verified"]), B, L, P(A_prev), P(B_cur),
                              P(G), sp)
        if ev is not None:
            ev[2].record(stream)
        s3 = lib.dsel_score_pairs(P(cand_u), P(A_prev), P(B_cur), P(G), B, L, cfg.r, None,
                                  C.byref(wargs), sp)
        if ev is not None:
            ev[3].record(stream)
        if s1 or s2 or s3:
            raise RuntimeError(f"dsel status {s1} {s2} {s3}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps, per-stage HIP events on the launch stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert ds.device_error() == 0

    ms_step = wall * 1e3 / args.steps
    st_topk = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e3   # us
    st_proj = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) * 1e3
    st_pair = float(np.mean([e[2].elapsed_time(e[3]) for e in evs])) * 1e3
    alg = algorithmic(cfg)
    topk_gbs = alg["topk_bytes"] / (st_topk * 1e-6) / 1e9
    proj_tfs = alg["proj_flop"] / (st_proj * 1e-6) / 1e12

    traffic = traffic_from_profile(cfg.name)
    if st_topk >= st_proj:
        roof = {"kernel": "topk16", "bound": "hbm", "achieved": round(topk_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(topk_gbs / HBM_PEAK_GBS, 4),
                "traffic": traffic}
    else:
        roof = {"kernel": "project", "bound": "mfma", "achieved": round(proj_tfs, 2),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(proj_tfs / BF16_PEAK_TFLOPS, 4), "traffic": None}

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
        "stages_us": {"select_topk": round(st_topk, 2), "project": round(st_proj, 2),
                      "score_pairs_walk": round(st_pair, 2)},
        "select_topk_hbm": {"GB/s": round(topk_gbs, 1), "frac": round(topk_gbs / HBM_PEAK_GBS, 4)},
        "project_mfma": {"TFLOP/s": round(proj_tfs, 2), "frac": round(proj_tfs / BF16_PEAK_TFLOPS, 4)},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
