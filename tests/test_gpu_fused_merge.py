"""The split-K merge done inside the verify kernel by the last work item of
each (sequence, KV head, column chunk) unit, through the L2 of the XCD that
all the unit's items run on.  Checks: the arrival counters are zero after
every call; calls of different inputs alternating on one workspace each
match the oracle (a partial left over from another call, or read from a
stale cache line, would show); units of more than 255 items, which use the
separate merge kernel instead, match the oracle too; the paths agree with
each other through the oracle."""
import numpy as np
import pytest
import torch

import self_speculative_verify_ripe_amd as rp
from self_speculative_verify_ripe_amd import binding
from oracle import layout as olay
from oracle import ripe_oracle as ro
from workloads import make_case

from gpu_util import DEV, Device, check, gpu_verify, make_desc, oracle_cache, upload

pytestmark = pytest.mark.gpu


def counters_zero(ws):
    torch.cuda.synchronize()
    head = ws[256:binding.RIPE_WORKSPACE_ZERO_BYTES]
    return bool((head == 0).all())


def test_counters_left_zero_and_alternating_calls():
    # one descriptor (same t_max) for both caches, so one workspace serves both
    cases = [make_case("c3", B=6, T_range=(200, 900), R=6, t_max=928, seed_offset=s) for s in (11, 12)]
    ocs = [oracle_cache(c, "ripe") for c in cases]
    caches = [upload(olay.encode(o)) for o in ocs]
    devs = [Device(c) for c in cases]
    desc = make_desc(cases[0], "ripe", split_len=128)
    ws = rp.new_workspace(desc, DEV)
    for rnd in range(3):
        for i, (c, o, ca, dv) in enumerate(zip(cases, ocs, caches, devs)):
            r = (3, 6, 1)[rnd]
            groups = c.groups_at(r)
            print(f"[case] alternating round {rnd} case {i} r={r}", flush=True)
            gpu = gpu_verify(desc, ca, c, dv, groups, ws=ws)
            check(c, groups, gpu, ro.verify(o, groups, c.q, c.kv_new, c.scale, c.Hq), tag=f"round {rnd} case {i}")
            assert counters_zero(ws), "arrival counters not reset"


@pytest.mark.parametrize("layout", ["full", "ripe"])
def test_units_of_more_than_255_items(layout):
    """Pieces of 32 positions over 9000-position prefixes: 282 items per
    unit, beyond the fused merge's 255, so the launch keeps the separate
    merge kernel; shorter pieces' results (fused) agree through the oracle."""
    case = make_case("c3", B=2, T_range=(8990, 9000), R=3, Hkv=1, Hq=2, D=64, t_max=9024)
    oc = oracle_cache(case, layout, planes={2, 3} if layout == "full" else None)
    cache = upload(olay.encode(oc))
    dev = Device(case)
    groups = case.groups_at(2)
    ref = ro.verify(oc, groups, case.q, case.kv_new, case.scale, case.Hq)
    for split in (32, 64):
        desc = make_desc(case, layout, split_len=split)
        ws = rp.new_workspace(desc, DEV)
        print(f"[case] {layout} split {split}", flush=True)
        gpu = gpu_verify(desc, cache, case, dev, groups, ws=ws)
        check(case, groups, gpu, ref, tag=f"{layout} split {split}")
        assert counters_zero(ws)
