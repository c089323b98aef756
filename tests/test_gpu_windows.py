"""RIPE windows of any width W >= 0 on the GPU, against the float64 oracle.

The ring of We = min(W, t_max) slots keeps its V in 8-slot blocks plus one
narrower block for the last We mod 8 slots (include/ripe.h).  Widths below
cover: BF16 narrow blocks of odd width, whose runs may start 2 bytes into a
dword (the kernel shifts them into place), narrow blocks whose runs start on
a dword but not on 16 bytes (We mod 8 in {2, 4, 6}; fp32 at any width), and
rings wider than a 32-position step.  Checks: outputs
within tolerance and plane_sel exact; the RIPE identities bit-exact at any W
(W >= T equals FULL); a window as long as the draft block (W = k) verifying
each block identically alone and batched; committed bytes bit-exact,
including commits longer than the window; parents in flight over such
rings."""
import numpy as np
import pytest
import torch

import self_speculative_verify_ripe_amd as rp
from oracle import layout as olay
from oracle import ripe_oracle as ro
from workloads import Group, make_case

from gpu_util import DEV, Device, check, gpu_verify, make_desc, oracle_cache, upload

pytestmark = pytest.mark.gpu

WIDTHS = [1, 3, 4, 5, 6, 12, 40, 50, 100]


def run_case(case, groups, W, split_len=0, tag=""):
    print(f"[case] {tag} W={W} {case.dtype} T={list(case.seq_len)} split={split_len}", flush=True)
    oc = oracle_cache(case, "ripe", W=W)
    cache = upload(olay.encode(oc))
    desc = make_desc(case, "ripe", W=W, split_len=split_len)
    gpu = gpu_verify(desc, cache, case, Device(case), groups)
    check(case, groups, gpu, ro.verify(oc, groups, case.q, case.kv_new, case.scale, case.Hq), tag=f"{tag} W={W}")
    return gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("W", WIDTHS)
def test_any_window_matches_oracle(dtype, W):
    # lengths below, at and above the window; depths 1, 4 and R = 5
    case = make_case("c3", B=4, T_range=(0, 160), R=5, W=W, dtype=dtype, Hkv=2, Hq=8)
    case.seq_len[:] = [0, max(1, W - 1), W + 1, 160]
    for r in (1, 4, 5):
        run_case(case, case.groups_at(r), W, tag=f"r={r}")
    run_case(case, case.groups_at(4), W, split_len=32, tag="r=4 split 32")


@pytest.mark.parametrize("W", [12, 40, 100])
def test_wide_window_equals_full_bitexact(W):
    """W >= T: every position keeps all planes, so RIPE runs FULL's pieces;
    the ring's last, narrow V block is read for the newest positions."""
    case = make_case("c3", B=3, T_range=(W - 3, W), R=6, Hkv=2, Hq=8)
    dev = Device(case)
    groups = case.groups_at(3)
    res = {}
    for name, layout in (("full", "full"), ("ripe", "ripe")):
        oc = oracle_cache(case, layout, W=W)
        desc = make_desc(case, layout, W=W, split_len=64)
        res[name] = gpu_verify(desc, upload(olay.encode(oc)), case, dev, groups)
        check(case, groups, res[name], ro.verify(oc, groups, case.q, case.kv_new, case.scale, case.Hq), tag=name)
    for a, b in zip(res["ripe"], res["full"]):
        assert torch.equal(a, b)


def test_window_of_the_draft_length_batched_equals_alone():
    """W = k = 4, the LoopSpec shape (primary and fallback branches of 4 rows
    at depths 8 and 16): each branch verified alone equals the batched call
    bit for bit."""
    case = make_case("c4", T_range=(300, 500), W=4)
    assert all(g.n_rows == 4 for g in case.fixed_groups)
    oc = oracle_cache(case, "ripe", W=4)
    cache = upload(olay.encode(oc))
    dev = Device(case)
    desc = make_desc(case, "ripe", W=4, split_len=128)
    groups = case.groups()
    out, lse, ps = gpu_verify(desc, cache, case, dev, groups)
    check(case, groups, (out, lse, ps), ro.verify(oc, groups, case.q, case.kv_new, case.scale, case.Hq),
          tag="W=k=4 batched")
    for gi, g in enumerate(groups):
        o1, l1, p1 = gpu_verify(desc, cache, case, dev, [g])
        rows = slice(g.row_start, g.row_start + g.n_rows)
        assert torch.equal(out[rows], o1[rows]) and torch.equal(lse[rows], l1[rows]), f"group {gi}"
        assert torch.equal(ps[gi], p1[0])


@pytest.mark.parametrize("W", [3, 5, 6, 64])
def test_two_depths_per_sequence_any_window(W):
    """Each sequence's rows split into two groups at different depths in one
    call -- the launches that stream their K rows non-temporally -- with
    rings of odd width (whose V is also read with a shift) and even width,
    against the oracle; every group alone equals the batched call bit for
    bit."""
    case = make_case("c3", B=4, T_range=(3, 150), R=6, k=8, Hkv=2, Hq=8, W=W)
    groups = []
    for b in range(case.B):
        s, n = case.blocks[b]
        groups += [Group(b, (1, 2, 3, 5)[b], s, n // 2), Group(b, 4 + b % 2, s + n // 2, n - n // 2)]
    print(f"[case] two depths W={W} T={list(case.seq_len)}", flush=True)
    oc = oracle_cache(case, "ripe", W=W)
    cache = upload(olay.encode(oc))
    dev = Device(case)
    desc = make_desc(case, "ripe", W=W, split_len=32)
    out, lse, ps = gpu_verify(desc, cache, case, dev, groups)
    check(case, groups, (out, lse, ps), ro.verify(oc, groups, case.q, case.kv_new, case.scale, case.Hq),
          tag=f"two depths W={W}")
    for gi, g in enumerate(groups):
        o1, l1, _ = gpu_verify(desc, cache, case, dev, [g])
        rows = slice(g.row_start, g.row_start + g.n_rows)
        assert torch.equal(out[rows], o1[rows]) and torch.equal(lse[rows], l1[rows]), f"group {gi}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("W", [3, 12, 40, 100])
def test_commit_any_window_bytes(dtype, W):
    """Commits of 0..k rows (some longer than the window) land bit-exactly
    where the oracle's encoder puts them; verification afterwards matches."""
    case = make_case("c3", B=4, T_range=(50, 200), R=4, W=W, dtype=dtype, Hkv=2, Hq=4, k=12)
    case.n_accept[:] = [0, 2, 7, 12]
    case.src_row[:] = [s for s, _ in case.blocks]
    oc = oracle_cache(case, "ripe", W=W)
    cache = upload(olay.encode(oc))
    dev = Device(case)
    desc = make_desc(case, "ripe", W=W)
    print(f"[case] commit W={W} {dtype}", flush=True)
    sl = rp.ripe_commit(desc, cache, case.seq_len.astype(np.int32).copy(), case.n_accept, case.src_row,
                        dev.kv_new, case.n_rows)
    torch.cuda.synchronize()
    ro.commit(oc, case.n_accept, case.src_row, case.kv_new)
    assert np.array_equal(cache.cpu().numpy(), olay.encode(oc)), "cache bytes differ after commit"
    groups = case.groups_at(2)
    gpu = gpu_verify(desc, cache, case, dev, groups, seq_len=sl)
    check(case, groups, gpu, ro.verify(oc, groups, case.q, case.kv_new, case.scale, case.Hq), seq_len=sl,
          tag=f"after commit W={W}")


@pytest.mark.parametrize("W,kp", [(12, 5), (40, 7), (5, 9), (100, 3)])
def test_inflight_parent_any_window(W, kp):
    """A parent block in flight moves the window: the oldest ring slots, some
    in the narrow last block, are hidden."""
    case = make_case("c3", B=4, T_range=(2, 150), R=6, k=kp + 5, Hkv=2, Hq=8, W=W)
    groups = []
    for b in range(case.B):
        s, n = case.blocks[b]
        groups.append(Group(b, (1, 3, 6, 2)[b], s + kp, n - kp, parent_row_start=s, parent_rows=kp))
    print(f"[case] inflight W={W} kp={kp} T={list(case.seq_len)}", flush=True)
    oc = oracle_cache(case, "ripe", W=W)
    cache = upload(olay.encode(oc))
    desc = make_desc(case, "ripe", W=W, split_len=32)
    gpu = gpu_verify(desc, cache, case, Device(case), groups)
    check(case, groups, gpu, ro.verify(oc, groups, case.q, case.kv_new, case.scale, case.Hq), tag=f"inflight W={W}")
