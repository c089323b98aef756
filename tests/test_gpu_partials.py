"""Split partials of 16-bit caches: each work item stores O / L in fp16,
scaled per column by a power of two that keeps it below 2^15.  With V
values far beyond fp16's range (every V value, cached and draft, times
2^20, which is exact in bf16 and float64) the outputs stay finite and match
the oracle within the standard bf16 tolerance scaled by the same 2^20; the
LSE, which does not depend on V, is unchanged.  Both merge paths run: units
of at most 8 items merge in the verify kernel, longer ones in the merge
kernel."""
import numpy as np
import pytest
import torch

from oracle import layout as olay
from oracle import ripe_oracle as ro
from workloads import make_case

from gpu_util import DEV, LSE_TOL, OUT_TOL, Device, gpu_verify, make_desc, rows_of, to_dev, upload

pytestmark = pytest.mark.gpu

SCALE = 2.0 ** 20


def scaled_cache(case, layout):
    c = ro.LogicalCache(layout, case.dtype, case.R, case.W, case.B, case.t_max, case.Hkv, case.D)
    for b in range(case.B):
        T = int(case.seq_len[b])
        c.seq_len[b] = T
        for p in c.planes_held():
            j0 = max(0, T - case.W) if (c.layout == ro.RIPE and p < case.R) else 0
            if T > j0:
                c.put_range(b, p, j0, case.planes.values(0, b, p, j0, T),
                            case.planes.values(1, b, p, j0, T) * SCALE)
    return c


@pytest.mark.parametrize("layout", ["ripe", "full"])
@pytest.mark.parametrize("split_len", [32, 128])
def test_values_beyond_fp16_range(layout, split_len):
    case = make_case("c3", layout=layout, B=4, T_range=(150, 300), R=6, Hkv=2, Hq=8, k=6)
    kv = case.kv_new.copy()
    kv[1] *= SCALE
    oc = scaled_cache(case, layout)
    cache = upload(olay.encode(oc))
    dev = Device(case)
    dev.kv_new = to_dev(kv, case.dtype)
    desc = make_desc(case, layout, split_len=split_len)
    print(f"[case] V x 2^20 {layout} split_len={split_len} T={list(case.seq_len)}", flush=True)
    for r in (1, 4, 6):
        groups = case.groups_at(r)
        out, lse, _ = gpu_verify(desc, cache, case, dev, groups)
        ref_out, ref_lse, _ = ro.verify(oc, groups, case.q, kv, case.scale, case.Hq)
        rows = rows_of(groups)
        o = out.float().cpu().numpy()[rows]
        assert np.all(np.isfinite(o)), f"r={r}: non-finite output"
        assert np.abs(o).max() > 65504, "the outputs must reach past fp16's range"
        err = float(np.max(np.abs(o - ref_out[rows])))
        assert err <= OUT_TOL["bf16"] * SCALE, f"r={r}: out err {err} (scaled tolerance {OUT_TOL['bf16'] * SCALE})"
        lerr = float(np.max(np.abs(lse.cpu().numpy()[rows] - ref_lse[rows])))
        assert lerr <= LSE_TOL, f"r={r}: lse err {lerr}"
