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
(algorithmic bytes per call / average call duration: the time between HIP
events on the launch stream that bracket each step's verify calls, divided by
the number of calls), and the float64 oracle timed on host cores on a bounded
sample.  Unless --no-extra: the other workloads' figures, one step's verify
calls captured into a HIP graph and replayed (graph_replay), the accept
call at the c4 shape (accept), and the per-position substitution error on c2
with its tail statistics under both plane-decay directions (side_stats).
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
LLC_BYTES = 256 << 20  # MI355X last-level (Infinity) cache
ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="c3", choices=["c1", "c2", "c3", "c4", "c5-full", "c5-ripe",
                                                       "c5-deepest"])
    ap.add_argument("--layout", default=None, help="override the workload's layout")
    ap.add_argument("--split-len", type=int, default=0)
    ap.add_argument("--page-len", type=int, default=0,
                    help="paged cache with pages of this many positions, in a seeded random pool order")
    ap.add_argument("--layers", type=int, default=None, help="recurrent layers (default: workload's)")
    ap.add_argument("--depths", default="workload",
                    help="'workload' (the workload's depths), 'all' or a comma list")
    ap.add_argument("--no-extra", action="store_true",
                    help="measure only --workload (skip the other workloads' figures)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run a plain device copy of MIB MiB before the timed region")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--side-stats-only", action="store_true",
                    help="run only the side-statistics leg and print its JSON")
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
def _to_storage(x, dtype):
    """float64 values (exact in ``dtype``) -> the storage words a cache holds."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    return x32 if dtype == "f32" else (x32.view(np.uint32) >> 16).astype(np.uint16)


def _from_storage(w, dtype):
    """storage words -> float64 (exact)."""
    if dtype == "f32":
        return w.astype(np.float64)
    return (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def cpu_baseline(case, layout, budget_s):
    """The float64 oracle timed on the host cores on a bounded sample: verify
    calls of one recurrent layer over the first four sequences at depths
    1, R/2 and R.  Each call starts from the cache's storage words (bf16 or
    fp32), converts the planes it reads to float64 and runs the oracle, so
    the conversion is inside the timed loop.  Timed with the BLAS pool as it
    is, then with one thread; tokens/s is extrapolated from the per-call time
    to the whole batch and to L_r * R calls per verified draft block."""
    from oracle import ripe_oracle as ro
    cores = len(os.sched_getaffinity(0))
    threads = cores
    limits = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        info = threadpool_info()
        if info:
            threads = max(int(i.get("num_threads", 1)) for i in info)
        limits = threadpool_limits
    except Exception:
        pass
    seqs = list(range(min(case.B, 4)))
    R, W = case.R, case.W
    depths = [1, R // 2, R]
    # storage words of every (sequence, plane) the sampled calls read
    store = {}
    for b in seqs:
        T = int(case.seq_len[b])
        for p in sorted(set(depths) | {R}):
            if layout == "deepest" and p != R:
                continue
            j0 = max(0, T - W) if (layout == "ripe" and p < R) else 0
            store[(b, p)] = (j0, _to_storage(case.planes.values(0, b, p, j0, T), case.dtype),
                             _to_storage(case.planes.values(1, b, p, j0, T), case.dtype))
    elem = 2 if case.dtype == "bf16" else 4

    def one_call(r):
        c = ro.LogicalCache(layout, case.dtype, R, W, case.B, case.t_max, case.Hkv, case.D)
        for b in seqs:
            c.seq_len[b] = int(case.seq_len[b])
            for p in ({r, R} if layout != "deepest" else {R}):
                j0, kw, vw = store[(b, p)]
                if layout == "full" and p != r:
                    continue
                if kw.shape[0]:
                    c.put_range(b, p, j0, _from_storage(kw, case.dtype), _from_storage(vw, case.dtype))
        groups = [(b, r, case.blocks[b][0], case.blocks[b][1]) for b in seqs]
        ro.verify(c, groups, case.q, case.kv_new, case.scale, case.Hq)
        return kv_read_bytes(layout, R, W, case.seq_len, groups, case.Hkv, case.D, elem)

    def timed(seconds):
        done, calls = 0, 0
        t0 = time.perf_counter()
        while True:
            for r in depths:
                done += one_call(r)
                calls += 1
            if time.perf_counter() - t0 >= seconds:
                break
        return done, calls, time.perf_counter() - t0

    done, calls, dt = timed(budget_s / 2)
    one = None
    if limits is not None:
        with limits(limits=1):
            d1, c1, t1 = timed(budget_s / 2)
        one = {"value": round(d1 / t1 / 1e9, 4), "unit": "GB/s", "cores": 1, "calls": c1,
               "wall_s": round(t1, 1)}
    # per-call time over the whole batch (bytes scale), then a full verification pass
    groups_all = [(b, depths[-1], case.blocks[b][0], case.blocks[b][1]) for b in range(case.B)]
    batch_bytes = kv_read_bytes(layout, R, W, case.seq_len, groups_all, case.Hkv, case.D, elem)
    t_call = batch_bytes / (done / dt)
    rows = sum(case.blocks[b][1] for b in range(case.B))
    tokens = rows / (case.L_r * R * t_call)
    return {"value": done / dt / 1e9, "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "one_thread": one,
            "verified_tokens_per_s": round(tokens, 4),
            "tokens_extrapolated": f"per-call time scaled from the sample's bytes to the whole batch "
                                   f"({batch_bytes / 1e6:.1f} MB per call), times L_r * R = {case.L_r * R} calls",
            "sample": f"{calls} float64 verify calls (one layer, depths {depths}) over sequences "
                      f"{seqs} of the {case.name} workload, {layout} layout, each converting its "
                      f"planes from {case.dtype} storage inside the timed loop, {dt:.1f} s wall; "
                      f"host has {cores} cores"}


# ---------------------------------------------------------------------------
# GPU run
# ---------------------------------------------------------------------------
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "verify_attn_c3_ripe_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "self_speculative_verify_ripe_amd", "csrc", f)
                  for f in ("verify.hip", "plan.h", "api.hip")]


def kernel_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counted_traffic(workload: str):
    """HBM bytes per verify call from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known size),
    or None when there is none for this workload or the kernel sources have
    changed since it was taken."""
    try:
        kv = dict(line.split(":", 1) for line in open(TRAFFIC_FILE) if ":" in line
                  and not line.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("workload") != workload or kv.get("kernel_source_sha256_16") != kernel_source_digest():
        return None
    return int(float(kv["hbm_bytes_per_call"]))


def run_workload(name, layout_override, steps, warmup, split_len, layers, depths_arg,
                 copy_calibration_mib=0, graph=False, page_len=0, floor=False):
    import torch
    import self_speculative_verify_ripe_amd as rp
    from workloads import device_kv_rows

    case, layout = geometry(name, layout_override)
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if case.dtype == "bf16" else torch.float32
    elem = 2 if case.dtype == "bf16" else 4
    L = layers or case.L_r
    R, W, B, Hkv, Hq, D = case.R, case.W, case.B, case.Hkv, case.Hq, case.D
    k = case.blocks[0][1]
    growth = (steps + warmup) * int(case.n_accept.max())
    t_max = int(-(-(int(case.seq_len.max()) + growth + case.n_rows) // 32) * 32)
    table, n_pages = None, 0
    if page_len:
        # every block of every sequence gets its own page, placed in a seeded
        # random order over the pool
        t_max = -(-t_max // page_len) * page_len
        nb = t_max // page_len
        n_pages = B * nb
        table = np.random.default_rng(7).permutation(n_pages).astype(np.int32).reshape(B, nb)
    if depths_arg == "all":
        depths = list(range(1, R + 1))
    elif depths_arg in (None, "workload"):
        depths = list(case.depths)
    else:
        depths = [int(x) for x in depths_arg.split(",")]
    if case.fixed_groups is not None:
        group_sets = [[(g.seq, g.depth, g.row_start, g.n_rows) for g in case.fixed_groups]]
    else:
        group_sets = [[(b, r, case.blocks[b][0], case.blocks[b][1]) for b in range(B)]
                      for r in depths]
    packed_sets = [rp.pack_groups(gs) for gs in group_sets]
    n_rows = case.n_rows
    desc = rp.make_desc(layout, case.dtype, R, W, B, t_max, Hkv, D, Hq, max_rows=n_rows,
                        max_groups=2 * B, split_len=split_len, page_len=page_len, n_pages=n_pages)
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
            need = [R] if layout == "deepest" else None
            rows = device_kv_rows(1000003 * (layer + 1) + b, R, T, Hkv, D, case.planes.decay, dev, dt,
                                  planes=need)
            na = np.zeros(B, dtype=np.int32)
            na[b] = T
            rp.ripe_commit(desc, cache, sl, na, np.zeros(B, dtype=np.int32), rows, T, block_table=table)
            del rows
        caches.append(cache)
    seq_len0 = case.seq_len.astype(np.int32).copy()
    torch.cuda.synchronize()
    t_fill = time.perf_counter() - t_fill
    print(f"[bench] {name} {layout}: filled {L} x {cache_bytes/2**30:.2f} GiB caches in "
          f"{t_fill:.1f}s", flush=True)

    gen = torch.Generator(device=dev)
    gen.manual_seed(20261203)
    q = (torch.randn((n_rows, Hq, D), generator=gen, device=dev) / D ** 0.5).to(dt)
    kv_new = torch.randn((2, R, n_rows, Hkv, D), generator=gen, device=dev).to(dt)
    out = torch.empty((n_rows, Hq, D), dtype=dt, device=dev)
    lse = torch.empty((n_rows, Hq), dtype=torch.float32, device=dev)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    n_accept = case.n_accept.astype(np.int32)
    src_row = case.src_row.astype(np.int32)

    seq_len = seq_len0.copy()
    n_calls = len(group_sets) * L

    def step_bytes(sl):
        kv = [kv_read_bytes(layout, R, W, sl, gs, Hkv, D, elem) for gs in group_sets]
        io = [io_bytes(gs, Hq, D, elem) for gs in group_sets]
        return kv, io

    def one_step(events):
        # One event pair brackets the step's verify calls: an event around
        # every call would add its own few microseconds to each call.
        nonlocal seq_len
        if events is not None:
            events[0].record(stream)
        for gi in range(len(group_sets)):
            gs = packed_sets[gi]
            for layer in range(L):
                rp.ripe_verify_attn(desc, caches[layer], seq_len, gs, n_rows, 1.0, q, kv_new, out,
                                    lse, None, ws, ws_bytes, stream, block_table=table)
        if events is not None:
            events[1].record(stream)
        sl = seq_len
        for layer in range(L):
            sl = seq_len.copy()
            rp.ripe_commit(desc, caches[layer], sl, n_accept, src_row, kv_new, n_rows, stream, block_table=table)
        seq_len = sl

    # Python's cyclic garbage collector can pause the host for tens of
    # milliseconds at an arbitrary call, leaving the GPU idle: collect once
    # here and keep it off while the steps run.
    gc.collect()
    gc.disable()
    for _ in range(warmup):
        one_step(None)
    if copy_calibration_mib:
        # A plain device copy of known size, outside the timed region: the
        # reference that scales the FETCH_SIZE / WRITE_SIZE counters.
        n = (copy_calibration_mib << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)  # reads and writes exactly MIB MiB
        del src, dst
    torch.cuda.synchronize()
    per_step = []
    sl = seq_len.copy()
    for _ in range(steps):
        kv, io = step_bytes(sl)
        per_step.append((kv, io))
        sl = sl + n_accept
    total_kv = sum(sum(kv) * L for kv, _ in per_step)
    # distinct K/V bytes one step reads over all its calls and layers: under
    # the 256 MB last-level cache the calls are served from it, not from HBM
    union = {}
    for gs in group_sets:
        for g in gs:
            union.setdefault((g[0], g[1]), g)
    step_set = kv_read_bytes(layout, R, W, seq_len, list(union.values()), Hkv, D, elem) * L
    call_bytes = np.array([kv[gi] + io[gi] for kv, io in per_step for gi in range(len(group_sets))
                           for _ in range(L)], dtype=np.float64)
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    wall0 = time.perf_counter()
    for st in range(steps):
        one_step(events[st])
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    # Host cost of a call: a few calls in the timed loop's order, enqueued
    # right after a sync while the launch queue has room.  (Timing the loop
    # above would measure the GPU's pace: once the runtime's queue of kernel
    # arguments is full, each launch waits for the GPU.)
    n_probe = min(8, n_calls)
    h0 = time.perf_counter()
    for i in range(n_probe):
        gi, layer = divmod(i, L)
        rp.ripe_verify_attn(desc, caches[layer], seq_len, packed_sets[gi], n_rows, 1.0, q, kv_new, out,
                            lse, None, ws, ws_bytes, stream, block_table=table)
    host_s = time.perf_counter() - h0
    torch.cuda.synchronize()
    gc.enable()
    elapsed = t0.elapsed_time(t1) / 1e3
    verify_s = np.array([a.elapsed_time(b) / 1e3 for a, b in events])
    rows_per_step = sum(g[3] for g in group_sets[0])
    avg_call = float(verify_s.sum()) / (n_calls * steps)
    # A draft block is verified once it has passed all R loops of every
    # recurrent layer.  A step covering fewer depths (c2: r in {4, 32}; c4:
    # one mixed-depth call per layer) is extrapolated to all R loops with its
    # mean call time; the commit time is measured.
    covers_all = case.fixed_groups is None and len(depths) == R
    commit_s = max(0.0, elapsed / steps - float(verify_s.sum()) / steps)
    pass_s = elapsed / steps if covers_all else avg_call * L * R + commit_s
    achieved = float(call_bytes.mean()) / avg_call / 1e9
    res = {
        "value": total_kv / elapsed / 1e9,
        "elapsed": elapsed,
        "ms_per_step": elapsed / steps * 1e3,
        "verified_tokens_per_s": rows_per_step / pass_s,
        "tokens_extrapolated": not covers_all,
        "achieved": achieved,
        "avg_call_us": avg_call * 1e6,
        "alg_bytes_per_call": int(call_bytes.mean()),
        "calls_per_step": n_calls,
        "wall": wall,
        "host_us_per_call": host_s / n_probe * 1e6,
        "gpu_us_per_call": elapsed / (n_calls * steps) * 1e6,
        "describe": f"{case.name} {layout}: B={B}, T~U[{int(case.seq_len.min())},"
                    f"{int(case.seq_len.max())}], R={R}, layers={L}, Hq/Hkv={Hq}/{Hkv}, D={D}, "
                    f"k={k}, W={W}, depths/step={len(depths) if case.fixed_groups is None else 'mixed'}"
                    + (f", paged: {page_len}-position pages in random pool order" if page_len else ""),
        "case": case,
        "layout": layout,
        "dtype": case.dtype,
        "step_working_set_bytes": int(step_set),
        "cache_resident": bool(step_set < LLC_BYTES),
    }
    if floor and layout == "ripe" and case.dtype == "bf16" and D == 128 and not page_len:
        res["read_floor"] = read_floor(caches, cache_bytes, seq_len, W, B, Hkv, t_max, split_len,
                                       res["avg_call_us"])
    if graph:
        res["graph"] = graph_replay(one_step_verify_calls=lambda st: [
            rp.ripe_verify_attn(desc, caches[layer], seq_len, packed_sets[gi], n_rows, 1.0, q, kv_new, out,
                                lse, None, ws, ws_bytes, st, block_table=table)
            for gi in range(len(group_sets)) for layer in range(L)], n_calls=n_calls, steps=steps)
    del caches, q, kv_new, out, lse, ws
    torch.cuda.empty_cache()
    return res


def default_split(B, Hkv, t_max):
    """The library's default split length for a descriptor (its rule, restated)."""
    if B * Hkv >= 448:
        return 8192
    work = B * Hkv * t_max
    s = max(1024, -(-work // 1024))
    s = min(s, max(256, -(-work // 448)))
    s = -(-s // 32) * 32
    return min(max(s, 256), 8192)


def floor_pieces(seq_len, W, B, Hkv, S, n_xcd=8, cus_per_xcd=32):
    """The deep-plane pieces of one RIPE verify call below depth R in the
    planner's grid order: each sequence's [0, T - W) cut into near-equal
    pieces of at most S positions (multiples of 32 but the last), the last
    one extended by the W window positions (the ring's bytes, read here from
    the deep plane); the pieces of one (sequence, KV head) on one XCD, the
    units spread over the XCDs by their steps, largest first, and each XCD's
    pieces paired largest with smallest on its compute units.  Rows of
    (b, h, c0, len); len 0 marks an empty grid slot."""
    units = []
    for b in range(B):
        T = int(seq_len[b])
        Wb = min(W, T)
        deep = T - Wb
        cuts = []
        if deep > 0:
            n = -(-deep // S)
            pl = -(-(-(-deep // n)) // 32) * 32
            cuts = [[c0, min(pl, deep - c0)] for c0 in range(0, deep, pl)]
        if cuts:
            cuts[-1][1] += Wb
        elif T > 0:
            cuts = [[0, T]]
        for h in range(Hkv):
            units.append([(b, h, c0, ln) for c0, ln in cuts])
    steps = lambda it: -(-it[3] // 32)
    cost = [sum(steps(i) for i in u) for u in units]
    load, per_xcd = [0] * n_xcd, [[] for _ in range(n_xcd)]
    for u in sorted(range(len(units)), key=lambda u: -cost[u]):
        x = min(range(n_xcd), key=lambda k: load[k])
        load[x] += cost[u]
        per_xcd[x] += units[u]
    rows = max(len(v) for v in per_xcd)
    grid = [(0, 0, 0, 0)] * (rows * n_xcd)
    for x in range(n_xcd):
        v = sorted(per_xcd[x], key=lambda it: -steps(it))
        nx = len(v)
        if cus_per_xcd < nx <= 2 * cus_per_xcd:
            P, Sx = nx - cus_per_xcd, 2 * cus_per_xcd - nx
            for k in range(P):
                grid[x + n_xcd * k] = v[Sx + k]
                grid[x + n_xcd * (cus_per_xcd + k)] = v[nx - 1 - k]
            for k in range(Sx):
                grid[x + n_xcd * (P + k)] = v[k]
        else:
            for k in range(nx):
                grid[x + n_xcd * k] = v[k]
    return np.array(grid, dtype=np.int32)


def read_floor(caches, cache_bytes, seq_len, W, B, Hkv, t_max, split_len, call_us, reps=40):
    """Roofline context: the same byte ranges as one verify call (the deep
    plane's pieces and window bytes, in the same grid order, two 4-wavefront
    work-groups per compute unit) read by a kernel that only reads them
    (measure/read_floor.hip), back to back over the layers' caches."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "self_speculative_verify_ripe_amd", "measure", "libripe_readfloor.so"))
    lib.ripe_read_floor.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 5 + [ctypes.c_void_p] * 2
    lib.ripe_read_floor.restype = ctypes.c_int
    S = split_len or default_split(B, Hkv, t_max)
    grid = floor_pieces(seq_len, W, B, Hkv, S)
    live = grid[:, 3] > 0
    assert np.all(grid[live, 0] < B) and np.all(grid[live, 1] < Hkv) and np.all(grid[:, 2] >= 0) \
        and np.all(grid[:, 2] + grid[:, 3] <= t_max), "read-floor pieces outside the cache"
    items = torch.from_numpy(grid).cuda()
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    lds = 68608  # the bf16 D = 128 verify kernel's LDS per work-group
    def launch(i):
        base = caches[i % len(caches)].data_ptr()
        rc = lib.ripe_read_floor(base, base + cache_bytes // 2, items.data_ptr(), len(grid), Hkv, t_max, 128,
                                 lds, sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"ripe_read_floor failed ({rc})")
    for i in range(2 * len(caches)):
        launch(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        launch(i)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    nbytes = int(grid[:, 3].astype(np.int64).sum()) * 2 * 128 * 2  # K and V rows, bf16
    return {"what": "a read-only kernel over the call's deep-plane pieces (window bytes read from the deep plane) "
                    "in the planner's grid order, with the verify kernel's load pattern, cache policy, "
                    "work-group shape and LDS footprint; back-to-back launches over the layers' caches",
            "pieces": int(live.sum()), "split_len": S, "bytes": nbytes, "us": round(us, 2),
            "GB/s": round(nbytes / us / 1e3, 1), "frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
            "verify_call_over_floor": round(call_us / us, 3)}


def library_read(nbytes: int, reps: int = 40, buffers: int = 4):
    """Context for the roofline: one library reduction (torch.sum with fp32
    accumulation) streaming a contiguous bf16 buffer of `nbytes` -- one verify
    call's algorithmic bytes -- rotating over `buffers` buffers so that
    consecutive launches do not hit the last-level cache: the rate at which a
    general-purpose library kernel reads the same bytes in one launch.  It is
    a reference point, not a bound, and not part of the verify path."""
    import torch
    n = nbytes // 2
    bufs = [torch.ones(n, dtype=torch.bfloat16, device="cuda") for _ in range(buffers)]
    for i in range(2 * buffers):
        bufs[i % buffers].sum(dtype=torch.float32)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        bufs[i % buffers].sum(dtype=torch.float32)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del bufs
    torch.cuda.empty_cache()
    return {"op": "torch.sum(dtype=float32) over a contiguous bf16 buffer of the call's algorithmic bytes, "
                  f"{buffers} buffers in rotation, {reps} launches",
            "bytes": int(n * 2), "us": round(us, 2), "GB/s": round(n * 2 / us / 1e3, 1),
            "frac": round(n * 2 / us / 1e3 / HBM_PEAK_GBS, 4)}


def graph_replay(one_step_verify_calls, n_calls, steps):
    """One step's verify calls (fixed lengths) captured into a HIP graph
    (torch.cuda.CUDAGraph) and replayed: mean call time from HIP events, and
    the host time per replay."""
    import torch
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        one_step_verify_calls(st)  # warm the library's plan cache on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        one_step_verify_calls(st)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    h0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    host = time.perf_counter() - h0
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3
    return {"avg_call_us": round(t / (steps * n_calls) * 1e6, 2),
            "host_us_per_replay": round(host / steps * 1e6, 1), "calls_per_replay": n_calls}


def run_accept(calls: int = 50, warmup: int = 5, B: int = 16, k: int = 4, V: int = 65536,
               temperature: float = 0.8):
    """ripe_accept at the c4 shape (16 sequences, k = 4 draft rows per chain,
    a fallback for about 40% of them) over a 64K vocabulary: mean call time
    with HIP events on the launch stream, and the logit bytes the row
    statistics kernel reads (every target and draft row that a decision may
    need: both chains' rows for sequences with a fallback, the primary's
    otherwise)."""
    import torch
    import self_speculative_verify_ripe_amd as rp
    from workloads import accept_inputs
    dev = torch.device("cuda:0")
    inp = accept_inputs(20261203, B, k, V, temperature)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    args = [t(inp.target), t(inp.draft), t(inp.tokens), t(inp.has_fallback), t(inp.rand.view(np.int32))]
    outs = [torch.empty(B, dtype=torch.int32, device=dev) for _ in range(3)]
    d = rp.make_accept_desc(B, k, V, temperature)
    ws = torch.empty(max(256, rp.ripe_accept_workspace_bytes(d)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        rp.ripe_accept(d, *args, *outs, ws, None, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(calls):
        rp.ripe_accept(d, *args, *outs, ws, None, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / calls
    n_fb = int(inp.has_fallback.astype(bool).sum())
    rows = B * (2 * k + 1) + n_fb * (2 * k)  # primary k+1 target + k draft; fallback k target + k draft
    nbytes = rows * V * 4
    return {"workload": f"c4 shape: B={B}, k={k}, V={V}, temperature {temperature}, {n_fb} fallbacks",
            "avg_call_us": round(us, 2), "logit_bytes_per_call": nbytes,
            "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "n_accept_histogram": np.bincount(outs[0].cpu().numpy(), minlength=k + 1).tolist()}


def run_side_stats(reps: int = 20, warmup: int = 3, depths=(4, 16, 28)):
    """Side statistics on c2 (one sequence, T = 1024, R = 32, Hq = Hkv = 40,
    D = 128, bf16, k = 8 rows, 1% of the positions with 8x plane noise), under
    both directions of the plane decay.  Per depth r: ripe_position_error on
    the FULL cache (mean call time with HIP events on the launch stream, its
    algorithmic bytes: the verify pass's K/V of plane r, then K/V of planes r
    and R per (position, KV head), plus queries, outputs and error rows), the
    tail statistics of its error row, and the exact squared output errors of
    the DEEPEST and RIPE caches against the FULL fp32 output, beside the
    squared error of rounding that output to bf16."""
    import torch
    import self_speculative_verify_ripe_amd as rp
    from workloads import make_case
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    res, nbytes, describe = {}, 0, ""
    for conv in ("workload", "pages"):
        case = make_case("c2", layout="full", convention=conv)
        T, R, H, D, Hq = int(case.seq_len[0]), case.R, case.Hkv, case.D, case.Hq
        describe = (f"c2 FULL/DEEPEST/RIPE: B=1, T={T}, R={R}, Hq/Hkv={Hq}/{H}, D={D}, bf16, k={case.n_rows}, "
                    f"W={case.W}, {len(case.planes.tail[0])} tail positions with 8x plane noise")
        rows = torch.zeros((2, R, T, H, D), dtype=torch.bfloat16, device=dev)
        for p in sorted(set(depths) | {R}):
            for kind in (0, 1):
                v = case.planes.values(kind, 0, p, 0, T).astype(np.float32)
                rows[kind, p - 1] = torch.from_numpy(v).to(dev).to(torch.bfloat16)
        caches = {}
        for lay in ("full", "deepest", "ripe"):
            d = rp.make_desc(lay, "bf16", R, case.W, 1, case.t_max, H, D, Hq, max_rows=case.n_rows,
                             max_groups=1)
            c = torch.zeros(rp.ripe_layout_bytes(d), dtype=torch.uint8, device=dev)
            rp.ripe_commit(d, c, np.zeros(1, np.int32), np.array([T], np.int32), np.zeros(1, np.int32), rows, T)
            caches[lay] = (d, c, rp.new_workspace(d, dev))
        del rows
        q = torch.from_numpy(case.q.astype(np.float32)).to(dev).to(torch.bfloat16)
        kv = torch.from_numpy(case.kv_new.astype(np.float32)).to(dev).to(torch.bfloat16)
        dF, cF, _ = caches["full"]
        err = torch.zeros((1, case.t_max), dtype=torch.float32, device=dev)
        cond = torch.zeros_like(err)
        o32 = torch.zeros((case.n_rows, Hq, D), dtype=torch.float32, device=dev)
        lse = torch.zeros((case.n_rows, Hq), dtype=torch.float32, device=dev)
        ws = torch.zeros(rp.ripe_layout_bytes(dF, rp.RIPE_BYTES_POSERR_WORKSPACE), dtype=torch.uint8, device=dev)
        per_depth = {}
        for r in depths:
            groups = case.groups_at(r)
            g4 = [(g.seq, g.depth, g.row_start, g.n_rows) for g in groups]
            nbytes = (kv_read_bytes("full", R, case.W, case.seq_len, g4, H, D, 2)        # verify pass
                      + case.n_rows * Hq * D * (2 + 4) + case.n_rows * Hq * 4
                      + 4 * T * H * D * 2                                                 # planes r, R
                      + case.n_rows * Hq * (D * (2 + 4) + 4) + 2 * case.t_max * 4)

            def call():
                rp.ripe_position_error(dF, cF, case.seq_len, groups, case.n_rows, case.scale, q, kv, err, cond,
                                       o32, lse, ws, None, stream)
            for _ in range(warmup):
                call()
            torch.cuda.synchronize()
            e0, e1 = ev(), ev()
            e0.record(stream)
            for _ in range(reps):
                call()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            stats = torch.empty((1, rp.RIPE_TAIL_STATS), dtype=torch.float64, device=dev)
            rp.ripe_position_error_tail(err, [T], case.W, stats, cond=cond, stream=stream)
            torch.cuda.synchronize()
            st = {k: (None if v != v else v) for k, v in zip(rp.TAIL_FIELDS, stats[0].cpu().tolist())}
            for k in ("tail_positions", "ill_conditioned", "positions"):
                st[k] = None if st[k] is None else int(st[k])
            exact = {}
            for lay in ("deepest", "ripe"):
                d, c, wsv = caches[lay]
                ob = torch.zeros((case.n_rows, Hq, D), dtype=torch.bfloat16, device=dev)
                rp.ripe_verify_attn(d, c, case.seq_len, groups, case.n_rows, case.scale, q, kv, ob, None, None,
                                    wsv, None, stream)
                torch.cuda.synchronize()
                exact[lay] = float(((ob.float() - o32) ** 2).sum())
            floor = float(((o32.to(torch.bfloat16).float() - o32) ** 2).sum())
            rnd = lambda x: None if x is None else (round(x, 6) if isinstance(x, float) else x)
            per_depth[f"r={r}"] = {
                "call_us": round(us, 2), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                **{k: rnd(v) for k, v in st.items() if k not in ("positions", "total")},
                "first_order_sq_err": st["total"],
                "deepest_sq_err": exact["deepest"], "ripe_sq_err": exact["ripe"],
                "bf16_rounding_sq_err": floor}
        res[conv] = per_depth
        del caches, ws
        torch.cuda.empty_cache()
    return {"workload": describe, "alg_bytes_per_call": nbytes, "by_convention": res}


EXTRA_WORKLOADS = [("c1", "ripe"), ("c1", "full"), ("c1", "deepest"),
                   ("c2", "ripe"), ("c2", "full"), ("c2", "deepest"), ("c4", None),
                   ("c5-ripe", None), ("c5-full", None), ("c5-deepest", None)]
# 279 KB per c1 call is 35 ns at the 8 TB/s peak: any launch dominates it
NOTES = {"c1": "launch-bound, correctness-only (279 KB per call, 35 ns at 8 TB/s)"}
# the headline workload again over a paged cache (pages of 256 and 1024 positions)
PAGED_WORKLOADS = [("c3", 256), ("c3", 1024)]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the verify path shards by sequence or KV head with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    if args.side_stats_only:
        print(json.dumps({"side_stats": run_side_stats()}), flush=True)
        return
    r = run_workload(args.workload, args.layout, args.steps, args.warmup, args.split_len,
                     args.layers, args.depths, args.copy_calibration, graph=not args.no_extra,
                     page_len=args.page_len, floor=not args.no_extra)
    workload_key = f"{args.workload}-{r['layout']}" if not args.workload.startswith("c5") \
        else args.workload
    traffic = counted_traffic(workload_key) if args.split_len == 0 and args.layers is None \
        and args.depths in (None, "workload") and args.page_len == 0 else None
    result = {
        "metric": "verify-attn KV read GB/s (% of HBM peak) and verified draft tokens/s, 1 GPU",
        "value": round(r["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": r["dtype"],
        "data": "synthetic (seeded; caches filled through ripe_commit)",
        "config": {"workload": r["describe"], "calls_per_step": r["calls_per_step"],
                   "split_len": args.split_len or "default"},
        "hbm_frac": round(r["value"] / HBM_PEAK_GBS, 4),
        "verified_tokens_per_s": round(r["verified_tokens_per_s"], 1),
        "verified_tokens_extrapolated_to_R_loops": r["tokens_extrapolated"],
        "roofline": {"bound": "hbm", "achieved": round(r["achieved"], 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(r["achieved"] / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "ripe_verify_attn call = verify_attn_kernel (units merged in the kernel; verify_merge_kernel follows only launches whose units have more than 8 split items)",
                     "avg_call_us": round(r["avg_call_us"], 2),
                     "alg_bytes_per_call": r["alg_bytes_per_call"]},
        "wall_s": round(r["wall"], 3),
        "host_us_per_call": round(r["host_us_per_call"], 1),
        "gpu_us_per_call": round(r["gpu_us_per_call"], 2),
        "cache_resident": r["cache_resident"],
        "step_working_set_MB": round(r["step_working_set_bytes"] / 1e6, 1),
    }
    if "graph" in r:
        result["graph_replay"] = r["graph"]
    if not args.no_extra:
        lr = library_read(r["alg_bytes_per_call"])
        lr["verify_call_over_library_read"] = round(r["avg_call_us"] / lr["us"], 3)
        result["roofline"]["library_read"] = lr
    if "read_floor" in r:
        result["roofline"]["read_floor"] = r["read_floor"]
    if not args.no_extra:
        extra = {}
        for name, lay in EXTRA_WORKLOADS:
            if name == args.workload and (lay is None or lay == r["layout"]):
                continue
            e = run_workload(name, lay, max(2, min(args.steps, 3)), 1, 0, None, None,
                             graph=name in ("c1", "c2"))
            row = {
                "GB/s": round(e["value"], 1), "hbm_frac": round(e["value"] / HBM_PEAK_GBS, 4),
                "call_GB/s": round(e["achieved"], 1), "avg_call_us": round(e["avg_call_us"], 2),
                "verified_tokens_per_s": round(e["verified_tokens_per_s"], 1),
                "tokens_extrapolated": e["tokens_extrapolated"],
                "ms_per_step": round(e["ms_per_step"], 3), "calls_per_step": e["calls_per_step"],
                "host_us_per_call": round(e["host_us_per_call"], 1),
                "cache_resident": e["cache_resident"],
                "step_working_set_MB": round(e["step_working_set_bytes"] / 1e6, 1),
                "workload": e["describe"]}
            if e["cache_resident"]:
                row["residency"] = ("one step's calls read under 256 MB over all layers: served from the "
                                    "last-level cache, not HBM (cache-warm figure)")
            if name in NOTES:
                row["note"] = NOTES[name]
            if "graph" in e:
                row["graph_replay"] = e["graph"]
            extra[f"{name}-{e['layout']}" if not name.startswith("c5") else name] = row
        for name, P in PAGED_WORKLOADS:
            e = run_workload(name, None, max(2, min(args.steps, 3)), 1, 0, None, None, page_len=P)
            extra[f"{name}-{e['layout']}-paged{P}"] = {
                "GB/s": round(e["value"], 1), "hbm_frac": round(e["value"] / HBM_PEAK_GBS, 4),
                "call_GB/s": round(e["achieved"], 1), "avg_call_us": round(e["avg_call_us"], 2),
                "ms_per_step": round(e["ms_per_step"], 3), "workload": e["describe"]}
        result["by_workload"] = extra
    if not args.no_extra:
        result["accept"] = run_accept()
        result["side_stats"] = run_side_stats()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(r["case"], r["layout"], args.cpu_seconds)
    line = json.dumps(result)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
