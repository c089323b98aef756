"""GPU parity of ripe_verify_attn_inflight: groups verified while their parent
block is still in flight (LoopSpec summary: the next position is computed
before the current one is confirmed).

* against the float64 oracle, every layout, windows that cover the parent,
  cut it, or are empty, prefixes shorter and longer than the window (ring
  slots hidden once the parent's commit would push them out of the window);
* siblings at two depths sharing one parent (the primary and fallback
  branches of LoopSpec);
* the defining property on the GPU: equal, within the fp32 tolerance, to
  committing the parent with ripe_commit and verifying afterwards;
* the RIPE identities, bit for bit: a window covering prefix and parent
  equals the full cache, W = 0 equals the deepest plane alone.
"""
import numpy as np
import pytest
import torch

import self_speculative_verify_ripe_amd as rp
from oracle import layout as olay
from oracle import ripe_oracle as ro
from workloads import Group, make_case

from gpu_util import DEV, Device, check, gpu_verify, make_desc, oracle_cache, rows_of, upload

pytestmark = pytest.mark.gpu


def with_parents(case, kp, depth_of=lambda b: 2):
    """Split each sequence's block of kp + k rows into an in-flight parent
    (its first kp rows) and the child group that follows it."""
    groups = []
    for b in range(case.B):
        s, n = case.blocks[b]
        groups.append(Group(b, depth_of(b), s + kp, n - kp, parent_row_start=s, parent_rows=kp))
    return groups


def run(case, layout, groups, W=None, split_len=0, tag=""):
    print(f"[case] {tag} {layout} W={W if W is not None else case.W} T={list(case.seq_len)}", flush=True)
    oc = oracle_cache(case, layout, W=W)
    cache = upload(olay.encode(oc))
    desc = make_desc(case, layout, W=W, split_len=split_len)
    gpu = gpu_verify(desc, cache, case, Device(case), groups)
    ref = ro.verify(oc, groups, case.q, case.kv_new, case.scale, case.Hq)
    check(case, groups, gpu, ref, tag=f"{tag} {layout}")
    return gpu


@pytest.mark.parametrize("layout", ["full", "deepest", "ripe"])
@pytest.mark.parametrize("W,kp,T_range", [
    (8, 3, (20, 90)),     # window cut by the parent: ring slots hidden, wrapping
    (16, 16, (5, 40)),    # parent as long as the window
    (24, 30, (3, 70)),    # parent longer than the window: some parent rows at plane R
    (64, 5, (2, 50)),     # window covers prefix and parent
    (0, 4, (10, 60)),     # no window
    (8, 4, (0, 6)),       # empty and short prefixes: the parent is most of what is read
])
def test_inflight_matches_oracle(layout, W, kp, T_range):
    case = make_case("c3", B=4, T_range=T_range, R=6, k=kp + 5, Hkv=2, Hq=8, W=W)
    groups = with_parents(case, kp, depth_of=lambda b: (1, 3, 6, 2)[b])  # depth R = 6 included
    run(case, layout, groups, split_len=32, tag=f"kp={kp}")
    run(case, layout, groups, tag=f"kp={kp} default split")


def test_inflight_siblings_share_parent_fp32():
    case = make_case("c1", k=12)  # fp32, R=4, W=8, T=128, one sequence
    s, _ = case.blocks[0]
    kp = 4
    groups = [Group(0, 2, s + kp, 4, s, kp), Group(0, 4, s + kp + 4, 4, s, kp)]
    for layout in ("full", "deepest", "ripe"):
        run(case, layout, groups, tag="siblings")


def test_inflight_equals_commit_then_verify_fp32():
    case = make_case("c1", k=10, T_range=(100, 100))  # t_max leaves room for the parent's commit
    s, _ = case.blocks[0]
    kp = 6
    child = [Group(0, 3, s + kp, 4, s, kp)]
    for layout in ("full", "deepest", "ripe"):
        oc = oracle_cache(case, layout)
        cache = upload(olay.encode(oc))
        desc = make_desc(case, layout)
        dev = Device(case)
        out1, lse1, _ = gpu_verify(desc, cache, case, dev, child, with_ps=False)
        sl = case.seq_len.astype(np.int32).copy()
        rp.ripe_commit(desc, cache, sl, np.array([kp], np.int32), np.array([s], np.int32), dev.kv_new,
                       case.n_rows)
        out2, lse2, _ = gpu_verify(desc, cache, case, dev, [Group(0, 3, s + kp, 4)], seq_len=sl, with_ps=False)
        rows = slice(s + kp, s + kp + 4)
        assert torch.allclose(out1[rows], out2[rows], atol=1e-5, rtol=0), layout
        assert torch.allclose(lse1[rows], lse2[rows], atol=1e-5, rtol=0), layout


@pytest.mark.parametrize("kp", [3, 9])
def test_inflight_ripe_identities_bitexact(kp):
    case = make_case("c3", B=3, T_range=(20, 60), R=4, k=kp + 4, Hkv=2, Hq=4, t_max=96)
    groups = with_parents(case, kp, depth_of=lambda b: 1 + b)
    res = {}
    for layout, W in (("full", 0), ("deepest", 0), ("ripe", 96), ("ripe", 0)):
        res[(layout, W)] = run(case, layout, groups, W=W, tag="identity")
    rows = torch.from_numpy(rows_of(groups)).to(DEV)  # the parents' rows are not outputs
    for a, b in ((("ripe", 96), ("full", 0)), (("ripe", 0), ("deepest", 0))):
        for x, y in zip(res[a][:2], res[b][:2]):
            assert torch.equal(x[rows], y[rows]), (a, b)
