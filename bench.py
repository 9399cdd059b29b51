#!/usr/bin/env python3
"""Benchmark of the small-batch decode step on one MI355X.

``python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]``

A step is one ``mk_decode_step``: one persistent kernel launch that runs the
whole decode pass (all layers, attention over the paged K/V, lm_head and the
sampler) for the batch. The sampled tokens are fed back as the next step's
inputs and the sequence lengths advance on the device, so the timed loop has
no host synchronisation. Inputs are seeded and synthetic (weights ~N(0, 0.02),
prefilled K/V ~N(0, 1)) and already resident in HBM when timing starts.

Prints ONE JSON line: tokens/s of the whole job, ms per step, the roofline of
the decode kernel (algorithmic HBM bytes per launch / mean launch time, from
HIP events on the launch stream) and the fp64 CPU oracle's rate on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X published HBM3E bandwidth
PAGE = 16
KERNEL_SOURCES = ["decode_persistent_step_amd/csrc/mk_kernel.hip", "decode_persistent_step_amd/csrc/mk_device.h",
                  "decode_persistent_step_amd/csrc/mk_params.h", "decode_persistent_step_amd/csrc/mk_api.cpp"]


# ----------------------------------------------------------------- bench math
def ideal_tokens_per_s(bandwidth_Bps: float, bytes_per_token: float) -> float:
    """Bandwidth-bound ceiling: every active byte crosses HBM once per token."""
    return bandwidth_Bps / bytes_per_token


def budget_us(tokens_per_s: float) -> float:
    return 1e6 / tokens_per_s


def overhead_fraction(tokens_per_s: float, layers: int, us_per_layer: float) -> float:
    return layers * us_per_layer / budget_us(tokens_per_s)


def launch_cap(us_per_token: float) -> float:
    return 1e6 / us_per_token


def mbu(tokens_per_s: float, bytes_per_token: float, bandwidth_Bps: float) -> float:
    return tokens_per_s * bytes_per_token / bandwidth_Bps


def generation_time_s(tokens: float, tokens_per_s: float) -> float:
    return tokens / tokens_per_s


def arithmetic_intensity(flops: float, bytes_: float) -> float:
    return flops / bytes_


def weight_bytes_per_step(shape, batch: int) -> int:
    """bf16 weight bytes one step streams: every projection, the gains, lm_head
    and the batch's embedding rows. For an MoE model: the router and the
    attention projections; the selected experts are counted separately
    (expert_bytes), since which experts a step reads depends on its routing."""
    L, d = shape.n_layers, shape.d_model
    per_layer = (shape.n_q_heads + 2 * shape.n_kv_heads) * shape.head_dim * d \
        + d * shape.n_q_heads * shape.head_dim + 2 * d
    per_layer += shape.n_experts * d if shape.moe else 3 * shape.ffn_dim * d
    return 2 * (L * per_layer + shape.vocab * d + d + batch * d)


def expert_bytes(shape) -> int:
    """bf16 bytes of one expert's gate, up and down matrices (MoE)."""
    return 2 * 3 * shape.expert_ffn_dim * shape.d_model


def kv_bytes_per_step(shape, positions) -> int:
    """K/V bytes one step moves for requests decoding at ``positions``: per
    layer the cached keys and values in the window (positions lo..p-1) are read
    and the new token's key and value (position p) are written."""
    hd = shape.n_kv_heads * shape.head_dim
    tot = 0
    for p in positions:
        for w in shape.windows():
            lo = max(0, p - w + 1) if w > 0 else 0
            tot += (p - lo) * hd * 2 * 2  # read
            tot += hd * 2 * 2             # written
    return tot


def algorithmic_bytes(shape, positions) -> int:
    return weight_bytes_per_step(shape, len(positions)) + kv_bytes_per_step(shape, positions)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# --------------------------------------------------------------------- setup
def setup(wl, steps_total: int, seed: int = 0):
    import torch
    import workload
    from decode_persistent_step_amd import Decoder, session
    shape = wl.shape
    ctx = wl.contexts(seed)
    B = len(ctx)
    w = workload.gen_weights(shape, seed=seed)
    need = [workload.pages_needed(c, steps_total) for c in ctx]
    mpps = max(need)
    n_pages = sum(need)
    dec = Decoder(shape, session.upload_weights(w), n_pages, mpps, B)
    pages = dec.kv_alloc(n_pages)
    rows = workload.page_assignment(pages, need, seed=seed, shuffle=wl.shuffle_pages)
    for b, c in enumerate(ctx):
        for l in range(shape.n_layers):
            session.prefill_kv(dec, l, rows[b], workload.gen_kv(shape, b, l, 0, c, seed=seed),
                               workload.gen_kv(shape, b, l, 1, c, seed=seed))
    pt = session.page_table_tensor(rows, mpps)
    torch.cuda.synchronize()
    return dec, w, ctx, rows, pt, mpps, n_pages


def run_gpu(wl, steps: int, warmup: int, seed: int = 0, cooperative: bool = True):
    import torch
    import workload
    dec, w, ctx, rows, pt, mpps, n_pages = setup(wl, steps + warmup, seed)
    dec.set_cooperative(cooperative)
    B = len(ctx)
    dev = "cuda"
    seq = torch.tensor(ctx, dtype=torch.int32, device=dev)
    toks = [torch.tensor(wl.initial_tokens(seed), dtype=torch.int32, device=dev),
            torch.empty(B, dtype=torch.int32, device=dev)]
    temps = torch.tensor(wl.temperatures(), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    cur = 0
    for s in range(warmup):
        dec.decode_step(seq, pt, toks[cur], temps, seed=seed, step=s, tokens_out=toks[1 - cur])
        seq.add_(1)
        cur = 1 - cur
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    pos0 = [c + warmup for c in ctx]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record(stream)
        dec.decode_step(seq, pt, toks[cur], temps, seed=seed, step=warmup + s, tokens_out=toks[1 - cur])
        ev[s][1].record(stream)
        seq.add_(1)
        cur = 1 - cur
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    experts = dec.moe_experts_used() if wl.shape.moe else 0  # warmup + timed steps
    rc, where = dec.last_error()
    if rc != 0:
        raise RuntimeError(f"device error {rc} at {where}")
    launch_ms = np.array([a.elapsed_time(b) for a, b in ev])
    step_bytes = np.array([algorithmic_bytes(wl.shape, [p + s for p in pos0]) for s in range(steps)], dtype=np.float64)
    if wl.shape.moe:
        # the selected experts' bytes, spread evenly over the steps (the counter
        # covers warmup and timed steps alike)
        step_bytes += experts * expert_bytes(wl.shape) / (steps + warmup)
    info = dec.launch_info()
    dec.close()
    return {"B": B, "wall_s": wall, "launch_ms": launch_ms, "step_bytes": step_bytes, "weights": w,
            "ctx": ctx, "info": info}


def cpu_baseline(wl, weights, target_s: float = 15.0, seed: int = 0):
    """The fp64 oracle as it stands, on the host cores, over a bounded number of
    steps of the same workload (its own pool, prefilled identically)."""
    import oracle
    import workload
    shape = wl.shape
    ctx = wl.contexts(seed)
    B = len(ctx)
    need = [workload.pages_needed(c, 64) for c in ctx]
    mpps = max(need)
    orc = oracle.OracleModel(shape, weights, sum(need), mpps)
    rows = workload.page_assignment(list(range(sum(need))), need, seed=seed, shuffle=wl.shuffle_pages)
    for b, c in enumerate(ctx):
        for l in range(shape.n_layers):
            orc.prefill_from(rows[b], l, workload.gen_kv(shape, b, l, 0, c, seed=seed),
                             workload.gen_kv(shape, b, l, 1, c, seed=seed))
    pt = np.full((B, mpps), -1, dtype=np.int32)
    for b, r in enumerate(rows):
        pt[b, :len(r)] = r
    seq = list(ctx)
    toks = wl.initial_tokens(seed)
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        out, _ = orc.decode_step(seq, pt, toks, wl.temperatures(), seed=seed, step=len(times))
        times.append(time.perf_counter() - t0)
        toks = [int(t) for t in out]
        seq = [p + 1 for p in seq]
        if time.perf_counter() - t_start >= target_s or len(times) >= 60:
            break
    med = float(np.median(times))
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": B / med, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(times)} decode steps of {wl.key} (batch {B}) from position {ctx}, "
                      f"median {med * 1e3:.1f} ms/step, fp64, OpenMP over rows/heads"}


def traffic_from_profiles(wl_key: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they
    were taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{wl_key}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("kernel_hash") != kernel_hash():
        return None
    return t.get("bytes_per_launch")


def _counter_mean(csv_path: str, name_part: str, counter: str, last: int = 0):
    """Median per-dispatch value (KiB) of one rocprofv3 counter over the dispatches of
    kernels whose name contains name_part (only the last ``last`` of them if > 0)."""
    import csv
    vals = []
    with open(csv_path) as fh:
        for r in csv.DictReader(fh):
            if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter:
                vals.append(float(r["Counter_Value"]))
    if last:
        vals = vals[-last:]
    if not vals:
        raise ValueError(f"no {counter} rows for {name_part} in {csv_path}")
    return float(np.median(vals)), len(vals)


def ingest_counters(wl_key: str, dec_fetch: str, dec_write: str, cal_fetch: str, cal_write: str,
                    copy_bytes: int, commands: str) -> dict:
    """Turn four rocprofv3 --pmc CSVs (FETCH_SIZE and WRITE_SIZE of the decode
    kernel and of the known-size copy) into HBM bytes per decode launch, and
    write profiles/traffic_<wl>.json plus a text summary beside it."""
    f_dec, nf = _counter_mean(dec_fetch, "mk_decode_kernel", "FETCH_SIZE")
    w_dec, nw = _counter_mean(dec_write, "mk_decode_kernel", "WRITE_SIZE")
    # the copy runs three times after torch's fill of its source: the last three dispatches
    f_cal, _ = _counter_mean(cal_fetch, "elementwise", "FETCH_SIZE", 3)
    w_cal, _ = _counter_mean(cal_write, "elementwise", "WRITE_SIZE", 3)
    kf = copy_bytes / (f_cal * 1024.0)
    kw = copy_bytes / (w_cal * 1024.0)
    fetch_b = f_dec * 1024.0 * kf
    write_b = w_dec * 1024.0 * kw
    out = {"workload": wl_key, "kernel": "mk_decode_kernel", "kernel_hash": kernel_hash(),
           "fetch_kib_per_dispatch": f_dec, "write_kib_per_dispatch": w_dec, "dispatches": [nf, nw],
           "copy_bytes": copy_bytes, "copy_fetch_kib": f_cal, "copy_write_kib": w_cal,
           "fetch_scale": round(kf, 4), "write_scale": round(kw, 4),
           "fetch_bytes_per_launch": int(fetch_b), "write_bytes_per_launch": int(write_b),
           "bytes_per_launch": int(fetch_b + write_b), "commands": commands}
    with open(os.path.join(ROOT, "profiles", f"traffic_{wl_key}.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    return out


def calibrate_copy(mib: int) -> int:
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n * 4}), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="dense2b_b1")
    ap.add_argument("--also", default="dense2b_b8,moe30b_b8",
                    help="comma-separated workloads reported beside (empty: none)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain fp32 copy kernel (out = in * 1) over MIB MiB, three times: "
                         "the known-size reference for rocprofv3's FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--ingest-counters", default="", metavar="DIR",
                    help="host only: read DIR/pmc_{dec,cal}_{FETCH,WRITE}_SIZE/run_counter_collection.csv "
                         "and write profiles/traffic_<workload>.json")
    ap.add_argument("--ingest-copy-mib", type=int, default=1024)
    ap.add_argument("--plain-launch", action="store_true",
                    help="ordinary (non-cooperative) kernel launch, for rocprofv3's kernel trace")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        return 2
    if args.calibrate_copy:
        return calibrate_copy(args.calibrate_copy)
    if args.ingest_counters:
        d = args.ingest_counters
        cmds = open(os.path.join(d, "commands.txt")).read() if os.path.exists(os.path.join(d, "commands.txt")) else ""
        t = ingest_counters(args.workload, *(os.path.join(d, f"pmc_{k}_{c}", "run_counter_collection.csv")
                                             for k, c in (("dec", "FETCH_SIZE"), ("dec", "WRITE_SIZE"),
                                                          ("cal", "FETCH_SIZE"), ("cal", "WRITE_SIZE"))),
                            copy_bytes=args.ingest_copy_mib << 20, commands=cmds)
        print(json.dumps(t))
        return 0
    import workload
    wl = workload.WORKLOADS[args.workload]
    r = run_gpu(wl, args.steps, args.warmup, cooperative=not args.plain_launch)
    B = r["B"]
    total_ms = r["wall_s"] * 1e3
    tps = B * args.steps / r["wall_s"]
    launch_ms = r["launch_ms"]
    achieved = float(np.sum(r["step_bytes"]) / (np.sum(launch_ms) * 1e-3) / 1e9)
    out = {
        "metric": "decode tokens/s and achieved HBM GB/s (MBU) per step at batch 1 and 8",
        "value": round(tps, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 weights/KV, fp32 activations",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.key}: ~2B dense decoder (L={wl.shape.n_layers}, d={wl.shape.d_model}, "
                        f"{wl.shape.n_q_heads}/{wl.shape.n_kv_heads} heads x {wl.shape.head_dim}, "
                        f"FFN {wl.shape.ffn_dim}, vocab {wl.shape.vocab}), batch {B}, "
                        f"context {r['ctx']}, 16-token shuffled pages, {wl.sampling} sampling",
            "batch": B, "context": r["ctx"], "page_size": PAGE,
            "launch": r["info"],
        },
        "latency_us": {"median": round(float(np.median(launch_ms)) * 1e3, 2),
                       "p10": round(float(np.percentile(launch_ms, 10)) * 1e3, 2),
                       "p90": round(float(np.percentile(launch_ms, 90)) * 1e3, 2)},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic_from_profiles(wl.key),
            "kernel": "mk_decode_kernel",
            "algorithmic_bytes_per_launch": int(np.mean(r["step_bytes"])),
            "mean_launch_us": round(float(np.mean(launch_ms)) * 1e3, 2),
        },
    }
    for i, key in enumerate(k for k in args.also.split(",") if k):
        wl2 = workload.WORKLOADS[key]
        r2 = run_gpu(wl2, max(16, args.steps // 4), args.warmup, cooperative=not args.plain_launch)
        ach2 = float(np.sum(r2["step_bytes"]) / (np.sum(r2["launch_ms"]) * 1e-3) / 1e9)
        rec = {"workload": wl2.key, "batch": r2["B"], "context": r2["ctx"],
               "tokens_per_s": round(r2["B"] * len(r2["launch_ms"]) / r2["wall_s"], 2),
               "ms_per_step": round(r2["wall_s"] * 1e3 / len(r2["launch_ms"]), 4),
               "achieved_GBps": round(ach2, 1), "frac": round(ach2 / HBM_PEAK_GBPS, 4),
               "algorithmic_bytes_per_launch": int(np.mean(r2["step_bytes"]))}
        out["also" if i == 0 else f"also_{wl2.key}"] = rec
        del r2
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, r["weights"], args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
