"""Helpers shared by the GPU parity tests: build oracle caches from seeded
workloads, move them to the device in the ABI byte layout (via the oracle's
own encoder), call the library through its C ABI and compare."""
from __future__ import annotations

import numpy as np
import torch

import self_speculative_verify_ripe_amd as rp
from oracle import layout as olay
from oracle import ripe_oracle as ro

DEV = "cuda"
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}
OUT_TOL = {"f32": 1e-5, "bf16": 2e-2}
LSE_TOL = 1e-3


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """float64 values that are exact in ``dtype`` -> device tensor."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(TORCH_DT[dtype]).to(DEV)


def oracle_cache(case, layout, W=None, planes=None, seqs=None) -> ro.LogicalCache:
    """Logical cache holding the case's committed prefixes.  ``planes``
    restricts which planes are stored for FULL (others stay NaN in bytes);
    ``seqs`` restricts which sequences are filled."""
    W = case.W if W is None else W
    c = ro.LogicalCache(layout, case.dtype, case.R, W, case.B, case.t_max, case.Hkv, case.D)
    for b in (range(case.B) if seqs is None else seqs):
        T = int(case.seq_len[b])
        c.seq_len[b] = T
        for p in c.planes_held():
            if planes is not None and p not in planes:
                continue
            j0 = max(0, T - W) if (c.layout == ro.RIPE and p < case.R) else 0
            if T > j0:
                c.put_range(b, p, j0, case.planes.values(0, b, p, j0, T),
                            case.planes.values(1, b, p, j0, T))
    return c


def upload(buf: np.ndarray) -> torch.Tensor:
    t = torch.empty(buf.size, dtype=torch.uint8, device=DEV)
    t.copy_(torch.from_numpy(buf))
    return t


def make_desc(case, layout, W=None, split_len=0, max_rows=None, max_groups=None):
    return rp.make_desc(layout, case.dtype, case.R, case.W if W is None else W, case.B, case.t_max,
                        case.Hkv, case.D, case.Hq,
                        max_rows=case.n_rows if max_rows is None else max_rows,
                        max_groups=(2 * case.B + 8) if max_groups is None else max_groups,
                        split_len=split_len)


class Device:
    """Device copies of a case's per-call inputs."""

    def __init__(self, case):
        self.case = case
        self.q = to_dev(case.q, case.dtype)
        self.kv_new = to_dev(case.kv_new, case.dtype)


def gpu_verify(desc, cache_dev, case, dev: Device, groups, seq_len=None, with_ps=True,
               with_lse=True, ws=None):
    n_rows = case.n_rows
    out = torch.full((n_rows, case.Hq, case.D), float("nan"), dtype=TORCH_DT[case.dtype],
                     device=DEV)
    lse = torch.full((n_rows, case.Hq), float("nan"), dtype=torch.float32, device=DEV) \
        if with_lse else None
    ps = torch.full((max(len(groups), 1), case.t_max), -1, dtype=torch.int8, device=DEV) \
        if with_ps else None
    if ws is None:
        ws = rp.new_workspace(desc, DEV)
    sl = case.seq_len if seq_len is None else seq_len
    rp.ripe_verify_attn(desc, cache_dev, sl, groups, n_rows, case.scale, dev.q, dev.kv_new, out,
                        lse, ps, ws)
    torch.cuda.synchronize()
    return out, lse, ps


def rows_of(groups):
    idx = []
    for g in groups:
        idx.extend(range(g.row_start, g.row_start + g.n_rows))
    return np.array(idx, dtype=np.int64)


def check(case, groups, gpu, ref, seq_len=None, tag=""):
    """Compare GPU (out, lse, plane_sel) with the oracle's on the groups'
    rows: plane_sel bit-exact, out within the dtype tolerance, lse within
    1e-3.  Returns the max abs errors."""
    out, lse, ps = gpu
    ref_out, ref_lse, ref_sels = ref
    rows = rows_of(groups)
    o = out.float().cpu().numpy()[rows]
    err = float(np.max(np.abs(o - ref_out[rows]))) if rows.size else 0.0
    assert np.all(np.isfinite(o)), f"{tag}: non-finite output"
    assert err <= OUT_TOL[case.dtype], f"{tag}: out max abs err {err}"
    lerr = 0.0
    if lse is not None:
        l = lse.cpu().numpy()[rows]
        lerr = float(np.max(np.abs(l - ref_lse[rows])))
        assert lerr <= LSE_TOL, f"{tag}: lse max abs err {lerr}"
    if ps is not None:
        sl = case.seq_len if seq_len is None else seq_len
        p = ps.cpu().numpy()
        for gi, g in enumerate(groups):
            T = int(sl[g.seq])
            assert np.array_equal(p[gi, :T], ref_sels[gi]), f"{tag}: plane_sel group {gi}"
            assert np.all(p[gi, T:] == -1), f"{tag}: plane_sel written past T"
    return err, lerr
