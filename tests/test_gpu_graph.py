"""Drafting calls (k = 1) and HIP-graph capture of the verify sweep.

* Drafting at depth r_d < R is the verify call with one-row groups (RIPE
  abstract: draft with a few loops); checked against the oracle.
* A sweep of verify calls over (depth, recurrent layer), the same sweep
  over a paged cache, and an accept call, captured into one HIP graph
  (torch.cuda.CUDAGraph) and replayed several times with eager work and
  synchronisations between the replays: every
  replay must reproduce the eager results bit for bit.  The library makes no
  allocation, memset or host synchronisation inside a call, so its launches
  can be captured; the captured calls keep the sequence lengths and groups
  they were captured with (commits, which advance lengths on the host, stay
  outside the graph).
"""
import numpy as np
import pytest
import torch

import self_speculative_verify_ripe_amd as rp
from oracle import layout as olay
from oracle import ripe_oracle as ro
from workloads import Group, accept_inputs, make_case

from gpu_util import DEV, Device, check, gpu_verify, make_desc, oracle_cache, upload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("layout", ["full", "deepest", "ripe"])
def test_drafting_one_row_groups(layout):
    case = make_case("c3", B=5, T_range=(40, 300), R=8, k=1, Hkv=2, Hq=8)
    oc = oracle_cache(case, layout)
    cache = upload(olay.encode(oc))
    desc = make_desc(case, layout)
    dev = Device(case)
    for r_d in (1, 3):
        groups = case.groups_at(r_d)
        assert all(g.n_rows == 1 for g in groups)
        gpu = gpu_verify(desc, cache, case, dev, groups)
        ref = ro.verify(oc, groups, case.q, case.kv_new, case.scale, case.Hq)
        check(case, groups, gpu, ref, tag=f"draft r_d={r_d} {layout}")


def sweep_setup():
    case = make_case("c3", B=3, T_range=(100, 700), R=4, Hkv=2, Hq=8)
    # two recurrent layers' caches: the case's prefix, and the same prefix with
    # the planes scaled (different values, same lengths)
    oc = oracle_cache(case, "ripe")
    raw = olay.encode(oc)
    layers = [upload(raw)]
    second = torch.from_numpy(raw.view(np.int16).copy()).to(DEV).view(torch.bfloat16) * 0.5
    layers.append(second.view(torch.uint8).contiguous())
    desc = make_desc(case, "ripe", split_len=64)
    dev = Device(case)
    packed = [rp.pack_groups(case.groups_at(r)) for r in range(1, case.R + 1)]
    n_calls = len(packed) * len(layers)
    outs = [torch.zeros((case.n_rows, case.Hq, case.D), dtype=torch.bfloat16, device=DEV) for _ in range(n_calls)]
    lses = [torch.zeros((case.n_rows, case.Hq), dtype=torch.float32, device=DEV) for _ in range(n_calls)]
    ws = rp.new_workspace(desc, DEV)
    return case, layers, desc, dev, packed, outs, lses, ws


def run_sweep(case, layers, desc, dev, packed, outs, lses, ws, stream):
    i = 0
    for gs in packed:
        for cache in layers:
            rp.ripe_verify_attn(desc, cache, case.seq_len, gs, case.n_rows, case.scale, dev.q, dev.kv_new,
                                outs[i], lses[i], None, ws, None, stream)
            i += 1


def test_verify_sweep_graph_replays_match_eager():
    case, layers, desc, dev, packed, outs, lses, ws = sweep_setup()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        run_sweep(case, layers, desc, dev, packed, outs, lses, ws, stream)
    torch.cuda.synchronize()
    eager = [(o.clone(), l.clone()) for o, l in zip(outs, lses)]
    assert all(torch.isfinite(o.float()).all() for o, _ in eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        run_sweep(case, layers, desc, dev, packed, outs, lses, ws, stream)
    torch.cuda.synchronize()
    for rep in range(3):
        for o, l in zip(outs, lses):  # cleared outside the graph, by a kernel
            o.zero_()
            l.zero_()
        # unrelated eager work on the same workspace between replays
        other = torch.zeros_like(outs[0])
        rp.ripe_verify_attn(desc, layers[0], case.seq_len, packed[0], case.n_rows, 0.5, dev.q, dev.kv_new,
                            other, None, None, ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, ((o, l), (eo, el)) in enumerate(zip(zip(outs, lses), eager)):
            assert torch.equal(o, eo) and torch.equal(l, el), f"replay {rep}, call {i}"


@pytest.mark.parametrize("P", [32, 128])
def test_paged_sweep_graph_replays_match_eager(P):
    """The paged verify call under capture.  With a split length of 64,
    32-position pages take the step-by-step page reads and 128-position pages
    the pieces cut at page boundaries; the block table travels in the
    captured kernel arguments."""
    case = make_case("c3", B=3, T_range=(100, 700), R=4, Hkv=2, Hq=8, t_max=768)
    oc = oracle_cache(case, "ripe")
    nb = case.t_max // P
    N = case.B * nb + 2
    table = np.random.default_rng(P).permutation(N)[:case.B * nb].reshape(case.B, nb).astype(np.int32)
    cache = upload(olay.encode_paged(oc, table, P, N))
    desc = rp.make_desc("ripe", case.dtype, case.R, case.W, case.B, case.t_max, case.Hkv, case.D, case.Hq,
                        max_rows=case.n_rows, max_groups=case.B, split_len=64, page_len=P, n_pages=N)
    dev = Device(case)
    packed = [rp.pack_groups(case.groups_at(r)) for r in range(1, case.R + 1)]
    outs = [torch.zeros((case.n_rows, case.Hq, case.D), dtype=torch.bfloat16, device=DEV) for _ in packed]
    lses = [torch.zeros((case.n_rows, case.Hq), dtype=torch.float32, device=DEV) for _ in packed]
    ws = rp.new_workspace(desc, DEV)
    stream = torch.cuda.Stream()

    def sweep():
        for gs, o, l in zip(packed, outs, lses):
            rp.ripe_verify_attn(desc, cache, case.seq_len, gs, case.n_rows, case.scale, dev.q, dev.kv_new, o, l,
                                None, ws, None, stream, block_table=table)

    print(f"[case] paged graph P={P}", flush=True)
    with torch.cuda.stream(stream):
        sweep()
    torch.cuda.synchronize()
    eager = [(o.clone(), l.clone()) for o, l in zip(outs, lses)]
    # the eager calls themselves agree with the oracle
    r = case.R
    ref = ro.verify(oc, case.groups_at(r), case.q, case.kv_new, case.scale, case.Hq)
    check(case, case.groups_at(r), (eager[r - 1][0], eager[r - 1][1], None), ref, tag=f"paged graph P={P}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        sweep()
    torch.cuda.synchronize()
    for rep in range(3):
        for o, l in zip(outs, lses):  # cleared outside the graph, by a kernel
            o.zero_()
            l.zero_()
        other = torch.zeros_like(outs[0])  # eager work on the same workspace between replays
        rp.ripe_verify_attn(desc, cache, case.seq_len, packed[0], case.n_rows, 0.5, dev.q, dev.kv_new, other,
                            None, None, ws, block_table=table)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, ((o, l), (eo, el)) in enumerate(zip(zip(outs, lses), eager)):
            assert torch.equal(o, eo) and torch.equal(l, el), f"P={P} replay {rep}, call {i}"


def test_accept_graph_replays_match_eager():
    inp = accept_inputs(91, 12, 4, 3000, 0.8, fallback_frac=0.5)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    args = [t(inp.target), t(inp.draft), t(inp.tokens), t(inp.has_fallback), t(inp.rand.view(np.int32))]
    d = rp.make_accept_desc(12, 4, 3000, 0.8)
    outs = [torch.zeros(12, dtype=torch.int32, device=DEV) for _ in range(3)]
    ws = torch.zeros(rp.ripe_accept_workspace_bytes(d), dtype=torch.uint8, device=DEV)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        rp.ripe_accept(d, *args, *outs, ws, None, stream)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        rp.ripe_accept(d, *args, *outs, ws, None, stream)
    for rep in range(3):
        for o in outs:
            o.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {rep}"
