"""Seeded random sweep of verify configurations against the float64 oracle.

Each case draws, from its own seed: layout, dtype, head dim, KV heads and
GQA ratio, R, window, batch, prefix lengths (empty ones included), split
length, an unpaged or paged cache (random page placement), one to three
sibling groups per sequence at random depths, and for some cases a parent
block in flight.  Every case is compared with the oracle by the same check
as the hand-written parity tests (plane_sel bit-exact, outputs within the
dtype tolerance, LSE within 1e-3).
"""
import numpy as np
import pytest
import torch

import self_speculative_verify_ripe_amd as rp
from oracle import layout as olay
from oracle import ripe_oracle as ro
from workloads import Group, make_case

from gpu_util import DEV, TORCH_DT, Device, check, oracle_cache, upload

pytestmark = pytest.mark.gpu

T_MAX = 384


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    c = dict(
        layout=["full", "deepest", "ripe"][rng.integers(3)],
        dtype=["f32", "bf16"][rng.integers(2)],
        D=int(rng.choice([64, 128])),
        Hkv=int(rng.integers(1, 4)),
        G=int(rng.choice([1, 2, 4, 5])),
        R=int(rng.choice([1, 3, 6])),
        W=int(rng.choice([0, 3, 8, 12, 16, 24, 32, 40, 64, 100, 160])),
        B=int(rng.integers(1, 7)),
        k=int(rng.integers(2, 13)),
        split_len=int(rng.choice([0, 32, 64, 96])),
        P=int(rng.choice([0, 0, 32, 64, 128])),
        parent=bool(rng.random() < 0.3),
    )
    c["T_hi"] = int(rng.integers(1, T_MAX - 2 * c["k"]))
    return c, rng


@pytest.mark.parametrize("seed", range(30))
def test_random_config(seed):
    c, rng = draw(seed)
    print(f"[case] seed={seed} {c}", flush=True)
    case = make_case("c3", layout=c["layout"], B=c["B"], T_range=(0, c["T_hi"]), R=c["R"], k=c["k"], W=c["W"],
                     Hkv=c["Hkv"], Hq=c["Hkv"] * c["G"], D=c["D"], dtype=c["dtype"], t_max=T_MAX,
                     seed_offset=seed)
    if c["B"] > 1:
        case.seq_len[0] = 0  # one empty prefix
    # groups: per sequence an optional parent block (its first kp rows), then
    # one to three sibling groups at random depths over the remaining rows
    groups = []
    for b, (s, n) in enumerate(case.blocks):
        kp = int(rng.integers(1, n)) if c["parent"] and n > 1 else 0
        rows = n - kp
        n_g = int(rng.integers(1, min(3, rows) + 1))
        cuts = np.sort(rng.choice(np.arange(1, rows), size=n_g - 1, replace=False)) if n_g > 1 else []
        bounds = [0, *[int(x) for x in cuts], rows]
        for i in range(n_g):
            groups.append(Group(b, int(rng.integers(1, c["R"] + 1)), s + kp + bounds[i], bounds[i + 1] - bounds[i],
                                s if kp else 0, kp))
    oc = oracle_cache(case, c["layout"])
    dev = Device(case)
    P = c["P"]
    if P:
        nb = T_MAX // P
        N = case.B * nb + 2
        table = rng.permutation(N)[:case.B * nb].reshape(case.B, nb).astype(np.int32)
        cache = upload(olay.encode_paged(oc, table, P, N))
    else:
        table, N = None, 0
        cache = upload(olay.encode(oc))
    desc = rp.make_desc(c["layout"], c["dtype"], c["R"], c["W"], case.B, T_MAX, c["Hkv"], c["D"], case.Hq,
                        max_rows=case.n_rows, max_groups=len(groups), split_len=c["split_len"], page_len=P,
                        n_pages=N)
    out = torch.full((case.n_rows, case.Hq, case.D), float("nan"), dtype=TORCH_DT[case.dtype], device=DEV)
    lse = torch.full((case.n_rows, case.Hq), float("nan"), dtype=torch.float32, device=DEV)
    ps = torch.full((len(groups), T_MAX), -1, dtype=torch.int8, device=DEV)
    rp.ripe_verify_attn(desc, cache, case.seq_len, groups, case.n_rows, case.scale, dev.q, dev.kv_new, out, lse,
                        ps, rp.new_workspace(desc, DEV), block_table=table)
    torch.cuda.synchronize()
    ref = ro.verify(oc, groups, case.q, case.kv_new, case.scale, case.Hq)
    check(case, groups, (out, lse, ps), ref, tag=f"seed {seed}")
