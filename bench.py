#!/usr/bin/env python3
"""Benchmark of RIPE self-speculative verification on one MI355X.

One step = the verify pass of one draft block per sequence through every
loop of every recurrent layer (for r in 1..R: for each layer: one
ripe_verify_attn call over that layer's cache at depth r), followed by a
ripe_commit of the accepted rows into every layer.  Inputs are synthetic and
seeded, shaped like the workloads in workloads/synth.py; caches are filled
through ripe_commit before timing, so they are resident in HBM when the
timed region starts.

Printed: one JSON line with the whole-step KV-read bandwidth (value), the
verified draft tokens per second, the roofline of the verify kernel
(algorithmic bytes per call / average call duration measured with HIP
events on the launch stream), and the float64 oracle timed on host cores on
a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="c3", choices=["c2", "c3", "c4", "c5-full", "c5-ripe",
                                                       "c5-deepest"])
    ap.add_argument("--layout", default=None, help="override the workload's layout")
    ap.add_argument("--split-len", type=int, default=0)
    ap.add_argument("--layers", type=int, default=None, help="recurrent layers (default: workload's)")
    ap.add_argument("--depths", default="all", help="'all' or comma list of depths per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--json-out", default=None)
    return ap.parse_args()


# ---------------------------------------------------------------------------
# workload geometry
# ---------------------------------------------------------------------------
def geometry(name: str, layout_override=None):
    from workloads import make_case
    if name.startswith("c5"):
        layout = name.split("-")[1]
        case = make_case("c5", layout=layout)
    else:
        case = make_case(name)
        layout = case.layout
    if layout_override:
        layout = layout_override
    return case, layout


def kv_read_bytes(layout, R, W, seq_len, groups, Hkv, D, elem):
    """Algorithmic K+V bytes one verify call reads: every distinct
    (position, plane) pair the call's groups need, plus the groups' own rows."""
    P_pos = 2 * Hkv * D * elem
    by_seq = {}
    for g in groups:
        by_seq.setdefault(g[0], set()).add(g[1])
    total = 0
    for b, depths in by_seq.items():
        T = int(seq_len[b])
        if layout == "deepest":
            U = T
        elif layout == "full":
            U = T * len(depths)
        else:
            Wb = min(W, T)
            low = [r for r in depths if r < R]
            U = (T - Wb) + Wb * len(low) + (Wb if len(low) < len(depths) else 0)
        total += U * P_pos
    total += sum(g[3] for g in groups) * P_pos
    return total


def io_bytes(groups, Hq, D, elem):
    rows = sum(g[3] for g in groups)
    return rows * Hq * D * 2 * elem + rows * Hq * 4


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle on a bounded sample
# ---------------------------------------------------------------------------
def cpu_baseline(case, layout, budget_s):
    from oracle import ripe_oracle as ro
    cores = len(os.sched_getaffinity(0))
    threads = cores
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        if info:
            threads = max(int(i.get("num_threads", 1)) for i in info)
    except Exception:
        pass
    seqs = list(range(min(case.B, 4)))
    c = ro.LogicalCache(layout, case.dtype, case.R, case.W, case.B, case.t_max, case.Hkv, case.D)
    for b in seqs:
        ro.fill_prefix(c, b, int(case.seq_len[b]), case.planes.values)
    elem = 2 if case.dtype == "bf16" else 4
    done_bytes = 0
    calls = 0
    t0 = time.perf_counter()
    depths = [1, case.R // 2, case.R]
    while True:
        for r in depths:
            groups = [(b, r, case.blocks[b][0], case.blocks[b][1]) for b in seqs]
            ro.verify(c, groups, case.q, case.kv_new, case.scale, case.Hq)
            done_bytes += kv_read_bytes(layout, case.R, case.W, case.seq_len, groups, case.Hkv,
                                        case.D, elem)
            calls += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done_bytes / dt / 1e9, "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{calls} float64 verify calls (one layer, depths {depths}) over sequences "
                      f"{seqs} of the {case.name} workload, {layout} layout, {dt:.1f} s wall; "
                      f"host has {cores} cores"}


# ---------------------------------------------------------------------------
# GPU run
# ---------------------------------------------------------------------------
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the verify path shards by sequence or KV head with no exchange; see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import self_speculative_verify_ripe_amd as rp
    from workloads import device_kv_rows

    case, layout = geometry(args.workload, args.layout)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dt = torch.bfloat16 if case.dtype == "bf16" else torch.float32
    elem = 2 if case.dtype == "bf16" else 4
    L = args.layers or case.L_r
    R, W, B, Hkv, Hq, D, k = case.R, case.W, case.B, case.Hkv, case.Hq, case.D, case.blocks[0][1]
    growth = (args.steps + args.warmup) * k
    t_max = int(-(-(int(case.seq_len.max()) + growth + k) // 32) * 32)
    depths = list(range(1, R + 1)) if args.depths == "all" else [int(x) for x in args.depths.split(",")]
    if case.fixed_groups is not None:
        base_groups = [(g.seq, g.depth, g.row_start, g.n_rows) for g in case.fixed_groups]
        group_sets = [base_groups]
    else:
        group_sets = [[(b, r, case.blocks[b][0], case.blocks[b][1]) for b in range(B)]
                      for r in depths]
    packed_sets = [rp.pack_groups(gs) for gs in group_sets]
    n_rows = case.n_rows
    desc = rp.make_desc(layout, case.dtype, R, W, B, t_max, Hkv, D, Hq, max_rows=n_rows,
                        max_groups=2 * B, split_len=args.split_len)
    cache_bytes = rp.ripe_layout_bytes(desc)
    ws_bytes = rp.ripe_layout_bytes(desc, rp.RIPE_BYTES_WORKSPACE)
    stream = torch.cuda.current_stream()

    # -- fill every layer's cache through the commit path ------------------
    t_fill = time.perf_counter()
    caches = []
    for layer in range(L):
        cache = torch.empty(cache_bytes, dtype=torch.uint8, device=dev)
        sl = np.zeros(B, dtype=np.int32)
        for b in range(B):
            T = int(case.seq_len[b])
            if T == 0:
                continue
            need = None
            if layout == "deepest":
                need = [R]
            elif layout == "ripe":
                need = None  # plane R for all rows, planes < R for the last W rows
            rows = device_kv_rows(1000003 * (layer + 1) + b, R, T, Hkv, D, 0.81, dev, dt, planes=need)
            na = np.zeros(B, dtype=np.int32)
            na[b] = T
            rp.ripe_commit(desc, cache, sl, na, np.zeros(B, dtype=np.int32), rows, T)
            del rows
        caches.append(cache)
    seq_len0 = case.seq_len.astype(np.int32).copy()
    torch.cuda.synchronize()
    t_fill = time.perf_counter() - t_fill
    print(f"[bench] filled {L} x {cache_bytes/2**30:.2f} GiB caches in {t_fill:.1f}s", flush=True)

    gen = torch.Generator(device=dev)
    gen.manual_seed(20261203)
    q = (torch.randn((n_rows, Hq, D), generator=gen, device=dev) / D ** 0.5).to(dt)
    kv_new = torch.randn((2, R, n_rows, Hkv, D), generator=gen, device=dev).to(dt)
    out = torch.empty((n_rows, Hq, D), dtype=dt, device=dev)
    lse = torch.empty((n_rows, Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    n_accept = case.n_accept.astype(np.int32)
    src_row = case.src_row.astype(np.int32)

    seq_len = seq_len0.copy()
    n_calls = len(group_sets) * L

    def step_bytes(sl):
        """Per-call algorithmic bytes (KV read; all incl. q/out/lse) for the
        current committed lengths."""
        kv = [kv_read_bytes(layout, R, W, sl, gs, Hkv, D, elem) for gs in group_sets]
        io = [io_bytes(gs, Hq, D, elem) for gs in group_sets]
        return kv, io

    def one_step(events, ev0):
        nonlocal seq_len
        i = ev0
        for gi in range(len(group_sets)):
            gs = packed_sets[gi]
            for layer in range(L):
                if events is not None:
                    events[i][0].record(stream)
                rp.ripe_verify_attn(desc, caches[layer], seq_len, gs, n_rows, 1.0, q, kv_new, out,
                                    lse, None, ws, ws_bytes, stream)
                if events is not None:
                    events[i][1].record(stream)
                i += 1
        sl = seq_len
        for layer in range(L):
            sl = seq_len.copy()
            rp.ripe_commit(desc, caches[layer], sl, n_accept, src_row, kv_new, n_rows, stream)
        seq_len = sl

    for _ in range(args.warmup):
        one_step(None, 0)
    torch.cuda.synchronize()
    # byte counts of every timed call, computed before timing starts
    per_step = []
    sl = seq_len.copy()
    for _ in range(args.steps):
        kv, io = step_bytes(sl)
        per_step.append((kv, io))
        sl = sl + n_accept
    total_kv = sum(sum(kv) * L for kv, _ in per_step)
    call_bytes = np.array([kv[gi] + io[gi] for kv, io in per_step for gi in range(len(group_sets))
                           for _ in range(L)], dtype=np.float64)
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n_calls * args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    wall0 = time.perf_counter()
    for k in range(args.steps):
        one_step(events, k * n_calls)
    host_s = time.perf_counter() - wall0
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    elapsed = t0.elapsed_time(t1) / 1e3
    call_s = np.array([a.elapsed_time(b) / 1e3 for a, b in events])
    calls_per_step = len(group_sets) * L
    rows_per_step = sum(g[3] for g in group_sets[0])
    verified_tok_s = rows_per_step * args.steps / elapsed if case.fixed_groups is None else \
        rows_per_step * args.steps / (elapsed * R / len(depths))
    avg_call = float(call_s.mean())
    achieved = float(call_bytes.mean()) / avg_call / 1e9
    result = {
        "metric": "verify-attn KV read GB/s (% of HBM peak) and verified draft tokens/s, 1 GPU",
        "value": round(total_kv / elapsed / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic (seeded; caches filled through ripe_commit)",
        "config": {"workload": f"{case.name} {layout}: B={B}, T~U[{int(case.seq_len.min())},"
                               f"{int(case.seq_len.max())}], R={R}, layers={L}, Hq/Hkv={Hq}/{Hkv}, "
                               f"D={D}, k={k}, W={W}, depths/step={len(depths)}",
                   "calls_per_step": calls_per_step, "split_len": args.split_len or "default"},
        "hbm_frac": round(total_kv / elapsed / 1e9 / HBM_PEAK_GBS, 4),
        "verified_tokens_per_s": round(verified_tok_s, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "ripe_verify_attn call (verify_partial + verify_merge)",
                     "avg_call_us": round(avg_call * 1e6, 2),
                     "alg_bytes_per_call": int(call_bytes.mean())},
        "wall_s": round(wall, 3),
        "host_enqueue_us_per_call": round(host_s / (n_calls * args.steps) * 1e6, 1),
        "gpu_us_per_call": round(elapsed / (n_calls * args.steps) * 1e6, 2),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case, layout, args.cpu_seconds)
    line = json.dumps(result)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
