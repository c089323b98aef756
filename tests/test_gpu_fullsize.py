"""Parity at the full sizes of the benchmark workloads, in the launch
configuration bench.py times (the whole batch in one call, default split
length).  The GPU cache is filled through ripe_commit from seeded device
rows; a sample of sequences is checked against the oracle built from the
same rows (outputs within tolerance, plane_sel and committed bytes exact)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import self_speculative_verify_ripe_amd as rp
from oracle import layout as olay
from oracle import ripe_oracle as ro
from workloads import device_kv_rows, make_case

from gpu_util import DEV, LSE_TOL, OUT_TOL, TORCH_DT, Device, rows_of

pytestmark = pytest.mark.gpu

SEED = 4242


def bench_desc(case, layout, t_max):
    return rp.make_desc(layout, case.dtype, case.R, case.W, case.B, t_max, case.Hkv, case.D, case.Hq,
                        max_rows=case.n_rows, max_groups=2 * case.B)


def fill(case, layout, desc, t_max, sample, planes=None):
    """A device cache holding every sequence's committed prefix (through
    ripe_commit), and an oracle cache holding the sampled sequences with the
    same values.  ``planes`` restricts the planes the oracle keeps (FULL)."""
    R, B, W = case.R, case.B, case.W
    dt = TORCH_DT[case.dtype]
    cache = torch.empty(rp.ripe_layout_bytes(desc), dtype=torch.uint8, device=DEV)
    oc = ro.LogicalCache(layout, case.dtype, R, W, B, t_max, case.Hkv, case.D)
    sl = np.zeros(B, dtype=np.int32)
    for b in range(B):
        T = int(case.seq_len[b])
        if T == 0:
            continue
        rows = device_kv_rows(SEED * 1000 + b, R, T, case.Hkv, case.D, case.planes.decay, DEV, dt,
                              planes=[R] if layout == "deepest" else None)
        na = np.zeros(B, dtype=np.int32)
        na[b] = T
        rp.ripe_commit(desc, cache, sl, na, np.zeros(B, dtype=np.int32), rows, T)
        if b in sample:
            oc.seq_len[b] = T
            for p in oc.planes_held():
                if planes is not None and p not in planes:
                    continue
                j0 = max(0, T - W) if (layout == "ripe" and p < R) else 0
                k = rows[0, p - 1, j0:T].float().cpu().numpy().astype(np.float64)
                v = rows[1, p - 1, j0:T].float().cpu().numpy().astype(np.float64)
                oc.put_range(b, p, j0, k, v)
        del rows
    torch.cuda.synchronize()
    assert np.array_equal(sl, case.seq_len.astype(np.int32))
    return cache, oc


def run_and_check(case, desc, cache, oc, groups, sample, seq_len, tag):
    """One call over every group; the sampled sequences' groups against the oracle."""
    dev = Device(case)
    n_rows = case.n_rows
    out = torch.full((n_rows, case.Hq, case.D), float("nan"), dtype=TORCH_DT[case.dtype], device=DEV)
    lse = torch.full((n_rows, case.Hq), float("nan"), dtype=torch.float32, device=DEV)
    ps = torch.full((len(groups), desc.t_max), -1, dtype=torch.int8, device=DEV)
    ws = rp.new_workspace(desc, DEV)
    print(f"[case] {tag}: {len(groups)} groups, sampled sequences {sorted(sample)}", flush=True)
    rp.ripe_verify_attn(desc, cache, seq_len, groups, n_rows, case.scale, dev.q, dev.kv_new, out, lse,
                        ps, ws)
    torch.cuda.synchronize()
    picked = [(gi, g) for gi, g in enumerate(groups) if g.seq in sample]
    sub = [g for _, g in picked]
    ref_out, ref_lse, ref_sels = ro.verify(oc, sub, case.q, case.kv_new, case.scale, case.Hq)
    rows = rows_of(sub)
    o = out.float().cpu().numpy()[rows]
    err = float(np.max(np.abs(o - ref_out[rows])))
    lerr = float(np.max(np.abs(lse.cpu().numpy()[rows] - ref_lse[rows])))
    assert np.all(np.isfinite(o)), tag
    assert err <= OUT_TOL[case.dtype], f"{tag}: out max abs err {err}"
    assert lerr <= LSE_TOL, f"{tag}: lse max abs err {lerr}"
    p = ps.cpu().numpy()
    for k, (gi, g) in enumerate(picked):
        T = int(seq_len[g.seq])
        assert np.array_equal(p[gi, :T], ref_sels[k]), f"{tag}: plane_sel of group {gi}"
        assert np.all(p[gi, T:] == -1), f"{tag}: plane_sel past T"
    print(f"[case] {tag}: out err {err:.2e} lse err {lerr:.2e}", flush=True)
    return out, lse


def t_max_of(case, growth=0):
    return int(-(-(int(case.seq_len.max()) + growth + case.n_rows) // 32) * 32)


def test_c3_full_size_sampled():
    case = make_case("c3")
    t_max = t_max_of(case)
    desc = bench_desc(case, "ripe", t_max)
    sample = {0, 3, 10, 15}  # includes the shortest and the longest prefixes
    cache, oc = fill(case, "ripe", desc, t_max, sample)
    sl = case.seq_len.astype(np.int32)
    for r in (1, 17, 32):
        out, lse = run_and_check(case, desc, cache, oc, case.groups_at(r), sample, sl, f"c3 r={r}")
    # block independence at full size: one sequence alone, same descriptor, bit-exact
    dev = Device(case)
    g = case.groups_at(32, [10])
    o1 = torch.full_like(out, float("nan"))
    l1 = torch.full_like(lse, float("nan"))
    rp.ripe_verify_attn(desc, cache, sl, g, case.n_rows, case.scale, dev.q, dev.kv_new, o1, l1, None,
                        rp.new_workspace(desc, DEV))
    torch.cuda.synchronize()
    rows = torch.from_numpy(rows_of(g)).to(DEV)
    assert torch.equal(o1[rows], out[rows]) and torch.equal(l1[rows], lse[rows])


def region_slices(layout, R, W, B, t_max, H, D, b):
    """Element ranges of sequence b in the cache byte layout (K block, then V
    block; RIPE: deep region, then ring)."""
    We = min(W, t_max) if layout == "ripe" else 0
    per = {"full": R * t_max, "deepest": t_max, "ripe": t_max}[layout]
    deep = B * H * per * D
    ring = B * (R - 1) * H * We * D if layout == "ripe" else 0
    region = deep + ring
    out = []
    for base in (0, region):
        out.append((base + b * H * per * D, base + (b + 1) * H * per * D))
        if ring:
            r0 = base + deep + b * (R - 1) * H * We * D
            out.append((r0, r0 + (R - 1) * H * We * D))
    return out


def test_c4_full_size_mixed_depths_and_commit():
    case = make_case("c4")
    t_max = t_max_of(case, growth=int(case.n_accept.max()))
    desc = bench_desc(case, "ripe", t_max)
    fb = [g.seq for g in case.fixed_groups if g.depth == 16]
    sample = {0, 5, 15} | set(fb[:2])
    cache, oc = fill(case, "ripe", desc, t_max, sample)
    groups = case.groups()
    sl = case.seq_len.astype(np.int32)
    run_and_check(case, desc, cache, oc, groups, sample, sl, "c4 before commit")
    # commit the accepted rows, on the GPU and (sampled sequences) in the oracle
    dev = Device(case)
    na = case.n_accept.astype(np.int32)
    src = case.src_row.astype(np.int32)
    sl2 = rp.ripe_commit(desc, cache, sl.copy(), na, src, dev.kv_new, case.n_rows)
    torch.cuda.synchronize()
    assert np.array_equal(sl2, sl + na)
    na_s = np.array([na[b] if b in sample else 0 for b in range(case.B)])
    ro.commit(oc, na_s, src, case.kv_new)
    # committed bytes of the sampled sequences, bit-exact (slots the oracle
    # does not hold are its NaN fill and are not compared)
    ref = olay.encode(oc).view(np.uint16)
    got = cache.cpu().numpy().view(np.uint16)
    for b in sorted(sample):
        for e0, e1 in region_slices("ripe", case.R, case.W, case.B, t_max, case.Hkv, case.D, b):
            held = ref[e0:e1] != 0x7FC0
            assert held.any()
            assert np.array_equal(got[e0:e1][held], ref[e0:e1][held]), f"commit bytes, sequence {b}"
    run_and_check(case, desc, cache, oc, groups, sample, sl2, "c4 after commit")


@pytest.mark.parametrize("layout", ["ripe", "full", "deepest"])
def test_c5_full_size_sampled(layout):
    """The fixed-memory sweep at its full sizes (FULL: B=4, T=8192; RIPE and
    DEEPEST: B=64, T~U[4096, 8192]), one call over the whole batch, sampled
    sequences at depths 1, 16 and 32 against the oracle."""
    case = make_case("c5", layout=layout)
    t_max = t_max_of(case)
    desc = bench_desc(case, layout, t_max)
    sample = {0, case.B - 1} | ({int(np.argmax(case.seq_len))} if case.B > 4 else set())
    depths = (1, 16, 32)
    cache, oc = fill(case, layout, desc, t_max, sample, planes=set(depths) if layout == "full" else None)
    sl = case.seq_len.astype(np.int32)
    for r in depths:
        run_and_check(case, desc, cache, oc, case.groups_at(r), sample, sl, f"c5 {layout} r={r}")


def test_whole_segment_rule_past_the_longest_piece():
    """At least 448 (sequence, KV head) pairs keep each segment whole up to the
    longest piece (8192 positions); longer sequences split into two pieces,
    so their units merge again (B = 56, Hkv = 8: 448 units; T in [8200,
    8600]; RIPE at depths 1 and R, DEEPEST at depth 4), sampled sequences
    against the oracle."""
    for layout, depths in (("ripe", (1, 8)), ("deepest", (4,))):
        case = make_case("c5", layout=layout, B=56, T_range=(8200, 8600), R=8, D=64)
        assert case.B * case.Hkv >= 448
        t_max = t_max_of(case)
        desc = bench_desc(case, layout, t_max)
        sample = {0, int(np.argmax(case.seq_len)), case.B - 1}
        cache, oc = fill(case, layout, desc, t_max, sample)
        sl = case.seq_len.astype(np.int32)
        for r in depths:
            run_and_check(case, desc, cache, oc, case.groups_at(r), sample, sl, f"whole-segment {layout} r={r}")
        del cache
        torch.cuda.empty_cache()
