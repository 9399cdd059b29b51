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
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PAGE = 16
KERNEL_SOURCES = ["decode_persistent_step_amd/csrc/mk_kernel.hip", "decode_persistent_step_amd/csrc/mk_device.h",
                  "decode_persistent_step_amd/csrc/mk_params.h", "decode_persistent_step_amd/csrc/mk_api.cpp"]
PREFILL_SOURCES = ["decode_persistent_step_amd/csrc/mk_prefill.hip", "decode_persistent_step_amd/csrc/mk_prefill.h",
                   "decode_persistent_step_amd/csrc/mk_device.h", "decode_persistent_step_amd/csrc/mk_api.cpp"]


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
    if getattr(shape, "weight_format", "bf16") == "fp8":
        # FP8: one byte per weight of every linear map plus a 4-byte scale per
        # output row; norm gains and the embedding rows stay bf16
        qkv_rows = (shape.n_q_heads + 2 * shape.n_kv_heads) * shape.head_dim
        lin = qkv_rows * d + d * shape.n_q_heads * shape.head_dim + 3 * shape.ffn_dim * d
        rows = qkv_rows + d + 2 * shape.ffn_dim + d
        return L * (lin + 4 * rows + 2 * 2 * d) + shape.vocab * d + 4 * shape.vocab + 2 * d + 2 * batch * d
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


def kernel_hash(sources=None) -> str:
    h = hashlib.sha256()
    for f in sources or KERNEL_SOURCES:
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


def prefill_flops(shape, pos0: int, n: int) -> dict:
    """Algorithmic flops of prefilling n prompt tokens from position pos0: the
    linear maps of every layer for every token (2 flops per weight), causal
    attention (QK^T and PV, 2 x 2 x head_dim flops per query head and visible
    position, the sliding window applied), and lm_head for the last position."""
    d, Hq, Hkv, dh, F, V = (shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                            shape.ffn_dim, shape.vocab)
    lin = 2 * (d * (Hq + 2 * Hkv) * dh + Hq * dh * d + d * 2 * F + F * d)
    p = np.arange(pos0, pos0 + n, dtype=np.float64)
    att = 0.0
    for w in shape.windows():
        span = p + 1 if w <= 0 else np.minimum(p + 1, w)
        att += float(np.sum(4.0 * Hq * dh * span))
    return {"linear": float(shape.n_layers) * n * lin, "attention": att, "lm_head": 2.0 * d * V,
            "total": float(shape.n_layers) * n * lin + att + 2.0 * d * V}


def run_prefill_gpu(shape, n: int, reps: int, warmup: int = 1, seed: int = 0):
    """Times `reps` prefills of an n-token prompt from position 0 into one
    request's shuffled pages (the same pages each time), with HIP events on the
    decoder's stream."""
    import torch
    import workload
    from decode_persistent_step_amd import Decoder, session
    w = workload.gen_weights(shape, seed=seed)
    need = workload.pages_needed(n, 1)
    dec = Decoder(shape, session.upload_weights(w), need, need, 1)
    pages = [int(p) for p in workload.shuffle_i32(np.asarray(dec.kv_alloc(need)), seed)]
    pt = torch.tensor(pages, dtype=torch.int32, device="cuda")
    prompt = torch.tensor([workload.draw_mod(seed, 100 + i, shape.vocab) for i in range(n)],
                          dtype=torch.int32, device="cuda")
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        dec.prefill(prompt, 0, pt, token_out=tok)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        dec.prefill(prompt, 0, pt, token_out=tok)
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    rc, where = dec.last_error()
    if rc != 0:
        raise RuntimeError(f"device error {rc} at {where}")
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    dec.close()
    fl = prefill_flops(shape, 0, n)
    tflops = fl["total"] / (float(np.mean(ms)) * 1e-3) / 1e12
    return {"workload": f"prefill of a {n}-token prompt into 16-token shuffled pages, {shape.name} "
                        f"(L={shape.n_layers}, d={shape.d_model}, {shape.weight_format} "
                        f"weights), chunks of 1024",
            "prompt_tokens": n, "reps": reps,
            "tokens_per_s": round(n * reps / wall, 1),
            "ms_per_prefill": round(float(np.mean(ms)), 3),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "algorithmic_flops": fl,
                         "note": "whole prefill (every kernel of it) over the model's flops; the GEMMs issue "
                                 "two bf16 products per weight (activation hi and lo halves)"},
            "kernel_hash": kernel_hash(PREFILL_SOURCES)}


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
                    copy_bytes: int, commands: str, alg_bytes: int = 0) -> dict:
    """Turn four rocprofv3 --pmc CSVs (FETCH_SIZE and WRITE_SIZE of the decode
    kernel and of the known-size copy) into HBM bytes per decode launch, and
    write profiles/traffic_<wl>.json plus a markdown summary beside it
    (against alg_bytes, the algorithmic bytes per launch, when given)."""
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
    md = [f"# mk_decode_kernel - {wl_key} - HBM traffic from rocprofv3 counters", "",
          "Commands (from the repository root; each counter in a run of its own):", "", "```", commands.strip(), "```", "",
          "| quantity | value |", "|---|---|",
          f"| FETCH_SIZE per decode dispatch (median of {nf}) | {f_dec:.1f} KiB |",
          f"| WRITE_SIZE per decode dispatch (median of {nw}) | {w_dec:.1f} KiB |",
          f"| copy kernel, {copy_bytes} B read and written: FETCH_SIZE | {f_cal:.1f} KiB |",
          f"| same copy: WRITE_SIZE | {w_cal:.1f} KiB |",
          f"| scale FETCH_SIZE -> bytes (copy bytes / counter bytes) | {kf:.4g} |",
          f"| scale WRITE_SIZE -> bytes | {kw:.4g} |",
          f"| HBM bytes read per decode launch | {int(fetch_b):,} |",
          f"| HBM bytes written per decode launch | {int(write_b):,} |",
          f"| total (bench.py roofline.traffic) | {int(fetch_b + write_b):,} |"]
    if alg_bytes:
        md += ["", f"Algorithmic bytes per launch of the same workload (bench.py's accounting): {alg_bytes:,}; "
                   f"measured traffic is {100.0 * ((fetch_b + write_b) / alg_bytes - 1.0):+.1f}% from it."]
    md += [f"Valid for kernel sources hash {kernel_hash()} (bench.py drops the figure when the sources change)."]
    with open(os.path.join(ROOT, "profiles", f"traffic_{wl_key}.md"), "w") as fh:
        fh.write("\n".join(md) + "\n")
    return out


STAGES = {False: ["QKV", "ATT", "O", "GU", "DN"], True: ["QKV", "ATT", "O", "RT", "GU (experts)", "DN (experts)"]}


def stage_summary(traces, shape, wl_key: str, steps_meta: str, command: str) -> str:
    """Per-stage timeline of the decode kernel from mk_set_trace buffers (100 MHz
    stamps, [workgroups][S * L + 1][8] per step): for each stage kind, the
    median over layers, steps and workgroups (and the worst workgroup) of the
    time from the stage's start to the next stage's start, split into streaming
    (inputs in LDS to the stage's end barrier), epilogue and publish, waiting for
    the next stage's producers, and loading its inputs; plus when compute wave 0
    had its operand in LDS. Times in microseconds."""
    spl = 6 if shape.moe else 5
    L = shape.n_layers
    names = STAGES[shape.moe] + ["LM"]
    rows = {k: {f: [] for f in ("total", "total_max", "stream", "epi", "wait", "inputs", "operand")} for k in names}
    for tr in traces:
        tr = tr.astype(np.int64)
        S = spl * L + 1
        for sid in range(S):
            kind = names[-1] if sid == S - 1 else names[sid % spl]
            start = tr[:, sid, 0]
            b_out = tr[:, sid, 5]
            att = kind == "ATT"
            epi_end = tr[:, sid, 6] if att else tr[:, sid, 2]
            r = rows[kind]
            if sid + 1 < S:
                tot = (tr[:, sid + 1, 0] - start) / 100.0
                r["total"].append(np.median(tot))
                r["total_max"].append(np.max(tot))
                r["wait"].append(np.median((tr[:, sid, 3] - epi_end) / 100.0))
                r["inputs"].append(np.median((tr[:, sid, 4] - tr[:, sid, 3]) / 100.0))
            r["stream"].append(np.median((b_out - start) / 100.0))
            r["epi"].append(np.median((epi_end - b_out) / 100.0))
            if not att:
                r["operand"].append(np.median(((tr[:, sid, 6] >> 16) & 0xFFFF) / 100.0))
    step_us = [float(np.median((tr[:, -1, 0] - tr[:, 0, 0]) / 100.0)) for tr in traces]
    out = [f"# mk_decode_kernel - {wl_key} - per-stage timeline", "",
           f"Kernel sources hash {kernel_hash()}. {steps_meta}", "",
           "Command (from the repository root):", "", "```", command, "```", "",
           "Each workgroup stamps its own timeline (`mk_set_trace`, 100 MHz clock). Per stage kind, over layers,",
           "steps and workgroups: median (and worst workgroup, median over layers) of the stage's span from its",
           "start (inputs in LDS, B_in) to the next stage's start, split into: streaming to the end barrier (B_out);",
           "epilogue and publish of the stage's outputs (attention: the cross-workgroup segment merge); wait for",
           "the next stage's producers (flags; 0 where the next inputs are tagged words polled directly); loading",
           "the next inputs into LDS (attention's q and new K/V). 'operand in LDS' is when compute wave 0 had",
           "this stage's GEMV operand, counted from the stage's start. Times in microseconds.", "",
           "| stage | span (median) | span (worst WG) | streaming | epilogue + publish | wait producers | "
           "load next inputs | operand in LDS |", "|---|---|---|---|---|---|---|---|"]
    fmt = lambda v: f"{np.mean(v):.2f}" if len(v) else "-"
    for k in names:
        r = rows[k]
        out.append(f"| {k} | {fmt(r['total'])} | {fmt(r['total_max'])} | {fmt(r['stream'])} | {fmt(r['epi'])} | "
                   f"{fmt(r['wait'])} | {fmt(r['inputs'])} | {fmt(r['operand'])} |")
    per_layer = sum(np.mean(rows[k]["total"]) for k in names[:-1])
    out += ["", f"Per layer (sum of the stage spans): {per_layer:.2f} us; first stage start to last stage start, "
                f"median over workgroups: {np.median(step_us):.1f} us per step."]
    return "\n".join(out) + "\n"


def run_stage_trace(wl, steps: int, warmup: int, seed: int = 0) -> str:
    import torch
    dec, w, ctx, rows, pt, mpps, n_pages = setup(wl, steps + warmup, seed)
    del w
    info = dec.launch_info()
    S = (6 if wl.shape.moe else 5) * wl.shape.n_layers + 1
    buf = torch.zeros((info["workgroups"], S, 8), dtype=torch.int64, device="cuda")
    B = len(ctx)
    seq = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    toks = [torch.tensor(wl.initial_tokens(seed), dtype=torch.int32, device="cuda"),
            torch.empty(B, dtype=torch.int32, device="cuda")]
    temps = torch.tensor(wl.temperatures(), dtype=torch.float32, device="cuda")
    dec.set_trace(buf)
    traces, cur = [], 0
    for s in range(steps + warmup):
        dec.decode_step(seq, pt, toks[cur], temps, seed=seed, step=s, tokens_out=toks[1 - cur])
        seq.add_(1)
        cur = 1 - cur
        if s >= warmup:
            torch.cuda.synchronize()
            traces.append(buf.cpu().numpy().copy())
            print(f"[stage-trace] {wl.key} step {s} traced", flush=True)
    dec.set_trace(None)
    rc, where = dec.last_error()
    if rc != 0:
        raise RuntimeError(f"device error {rc} at {where}")
    dec.close()
    meta = f"{wl.key}, batch {B}, contexts {ctx}, {steps} traced steps after {warmup} untraced."
    cmd = f"python3 bench.py --workload {wl.key} --stage-trace {steps} --warmup {warmup}"
    text = stage_summary(traces, wl.shape, wl.key, meta, cmd)
    path = os.path.join(ROOT, "profiles", f"stages_{wl.key}.md")
    with open(path, "w") as fh:
        fh.write(text)
    return path


def summarize_kernel_trace(csv_path: str, bench_log: str, command: str) -> str:
    """Per-workload summary of the decode kernel's dispatches in a rocprofv3
    kernel trace (kernel_trace.csv) of one default bench.py run, whose JSON line
    (in bench_log) gives the workload order, the dispatches of each (warmup and
    timed steps) and its algorithmic bytes per launch. Writes
    profiles/mk_decode_kernel_bench_workloads.md."""
    import csv
    line = [l for l in open(bench_log) if l.startswith("{") and '"metric"' in l][-1]
    out = json.loads(line)
    runs = [(out["config"]["workload"].split(":")[0], out["warmup"] + out["steps"],
             out["roofline"]["algorithmic_bytes_per_launch"])]
    for k, v in out.items():
        if k == "also" or (k.startswith("also_") and k != "also_prefill"):
            runs.append((v["workload"], out["warmup"] + max(16, out["steps"] // 4), v["algorithmic_bytes_per_launch"]))
    rows = [r for r in csv.DictReader(open(csv_path)) if "mk_decode_kernel" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    need = sum(n for _, n, _ in runs)
    if len(rows) != need:
        raise RuntimeError(f"{len(rows)} decode dispatches in the trace, {need} expected from the bench line")
    lines = [
        "# mk_decode_kernel - the decode workloads of bench.py - rocprofv3 kernel-trace summary", "",
        f"Kernel sources hash {kernel_hash()}. Command (from any directory; REPO is the repository root; the",
        "ordinary launch is used because rocprofv3's tracer has crashed at exit after cooperative launches;",
        "the kernel and its work are the same):", "", "```", command, "```", "",
        "Per-dispatch durations split by workload in the bench's order (warmup and timed steps); algorithmic",
        "bytes per launch from the same run's bench line (weights once, K/V of every attended position, the",
        "K/V written; MoE: the selected experts' bytes); frac = bytes / mean duration / 8 TB/s.", "",
        "| workload | kernel | dispatches | mean us | min us | max us | algorithmic bytes | GB/s | frac |",
        "|---|---|---|---|---|---|---|---|---|"]
    i = 0
    for key, n, nbytes in runs:
        sel = rows[i:i + n]
        i += n
        dur = np.array([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in sel])
        names = sorted({r["Kernel_Name"].split("(")[0].replace("mk::", "").replace("void ", "") for r in sel})
        gbps = nbytes / (dur.mean() * 1e-6) / 1e9
        lines.append(f"| {key} | `{'`, `'.join(names)}` | {n} | {dur.mean():.1f} | {dur.min():.1f} | {dur.max():.1f} | "
                     f"{nbytes:,} | {gbps:.0f} | {gbps / HBM_PEAK_GBPS:.3f} |")
    path = os.path.join(ROOT, "profiles", "mk_decode_kernel_bench_workloads.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return path


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
    ap.add_argument("--also", default="dense2b_b8,swa2b_b4,moe30b_b8,dense2b_b1_fp8",
                    help="comma-separated workloads reported beside (empty: none)")
    ap.add_argument("--prefill-tokens", type=int, default=8192,
                    help="also time paged prefill of a prompt this long on the dense ~2B model (0: skip)")
    ap.add_argument("--prefill-only", action="store_true", help="only the prefill leg (no decode lines)")
    ap.add_argument("--prefill-weights", choices=["bf16", "fp8"], default="bf16",
                    help="weight format of the prefill leg's ~2B model (FP8: E4M3 tiles decoded to bf16 "
                         "for the matrix cores)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain fp32 copy kernel (out = in * 1) over MIB MiB, three times: "
                         "the known-size reference for rocprofv3's FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--ingest-counters", default="", metavar="DIR",
                    help="host only: read DIR/pmc_{dec,cal}_{FETCH,WRITE}_SIZE/run_counter_collection.csv "
                         "and write profiles/traffic_<workload>.json")
    ap.add_argument("--ingest-copy-mib", type=int, default=1024)
    ap.add_argument("--summarize-kernel-trace", nargs=2, metavar=("CSV", "BENCH_LOG"), default=None,
                    help="host only: summarize a rocprofv3 kernel trace of one default bench.py run (its "
                         "kernel_trace.csv and the run's output) into profiles/mk_decode_kernel_bench_workloads.md")
    ap.add_argument("--trace-command", default="", help="the profiling command, quoted in the summary")
    ap.add_argument("--ingest-alg-bytes", type=int, default=0,
                    help="algorithmic bytes per launch of the workload, for the summary's comparison")
    ap.add_argument("--plain-launch", action="store_true",
                    help="ordinary (non-cooperative) kernel launch, for rocprofv3's kernel trace")
    ap.add_argument("--stage-trace", type=int, default=0, metavar="STEPS",
                    help="only trace STEPS steps of --workload per stage (mk_set_trace) and write "
                         "profiles/stages_<workload>.md")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        return 2
    if args.calibrate_copy:
        return calibrate_copy(args.calibrate_copy)
    if args.summarize_kernel_trace:
        print(summarize_kernel_trace(*args.summarize_kernel_trace, args.trace_command))
        return 0
    if args.ingest_counters:
        d = args.ingest_counters
        cmds = open(os.path.join(d, "commands.txt")).read() if os.path.exists(os.path.join(d, "commands.txt")) else ""
        t = ingest_counters(args.workload, *(os.path.join(d, f"pmc_{k}_{c}", "run_counter_collection.csv")
                                             for k, c in (("dec", "FETCH_SIZE"), ("dec", "WRITE_SIZE"),
                                                          ("cal", "FETCH_SIZE"), ("cal", "WRITE_SIZE"))),
                            copy_bytes=args.ingest_copy_mib << 20, commands=cmds, alg_bytes=args.ingest_alg_bytes)
        print(json.dumps(t))
        return 0
    import workload
    wl = workload.WORKLOADS[args.workload]
    if args.stage_trace:
        print(json.dumps({"stage_trace": run_stage_trace(wl, args.stage_trace, args.warmup)}), flush=True)
        return 0
    if args.prefill_only:
        shape = workload.DENSE2B_FP8 if args.prefill_weights == "fp8" else workload.DENSE2B
        print(json.dumps({"prefill": run_prefill_gpu(shape, args.prefill_tokens, max(1, args.steps))}), flush=True)
        return 0
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
        "dtype": "bf16 weights and K/V; fp32 activations entering every GEMV and attention product as "
                 "hi/lo bf16 pairs (~16 significant bits); fp32 accumulation",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.key}: ~2B dense decoder{' (FP8 E4M3 weights)' if wl.shape.weight_format == 'fp8' else ''} "
                        f"(L={wl.shape.n_layers}, d={wl.shape.d_model}, "
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
               "algorithmic_bytes_per_launch": int(np.mean(r2["step_bytes"])),
               "traffic": traffic_from_profiles(wl2.key)}
        out["also" if i == 0 else f"also_{wl2.key}"] = rec
        del r2
    if args.prefill_tokens > 0:
        out["also_prefill"] = run_prefill_gpu(workload.DENSE2B_FP8 if args.prefill_weights == "fp8" else
                                              workload.DENSE2B, args.prefill_tokens, 5)
    # the pages' own figures for this path (another GPU: context, not the target)
    out["pages_context"] = {
        "speedup_vs_vllm_decode_only_batch1_8k": 1.58,
        "fraction_of_theoretical_ceiling": 0.62,
        "hardware": "1x NVIDIA H100, BF16, batch 1, 8K context (Cohere Megakernel page, table 'Rakamlar')",
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, r["weights"], args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
