"""GPU parity of ripe_position_error (per-position plane-substitution error of
a FULL cache) against the float64 oracle (oracle/side_stats.py).

Tolerances, per position j:

    |gpu - oracle| <= (rtol + 2 kappa_j eps) * oracle + 1e-6 * max_j,

kappa_j = max over the group's rows and heads of a / (1 - a + c) (a, c the
position's softmax weights at planes r and R, from the oracle in float64).
The kernel computes the single-term update in fp32 from direct differences,
so its own rounding is ~1e-6 relative; what dominates is the FULL output O and
LSE it starts from, whose errors reach e_j amplified by kappa_j (twice: e is a
square).  kappa_j <= 1 unless position j holds more than half of some row's
attention at plane r; then e_j is ill-conditioned and the fp32 value is an
estimate (the header says so, and cond reports kappa).  eps: fp32 caches
1e-5 (O within ~1e-6); bf16 caches 1e-3 (the verify pass rounds the
probabilities to bf16 for the MFMA, relative 2^-9 per term, moving O by
~1e-4).  rtol: 1e-4 (fp32), 1e-2 (bf16).  The fp32 outputs themselves are
checked at 1e-5 (fp32 caches) and, for bf16 caches, at 2^-8 max|v| over the
values the groups read: the verify pass normalises by the unrounded
probability sum, so rounding each probability to bf16 (2^-9 relative) moves
O by at most 2^-9 max|v|, and the 1% tail positions carry |v| up to ~25.
The LSE is checked at 1e-3, cond against kappa at 1e-3 + 4e-5 kappa
relative.
"""
import numpy as np
import pytest
import torch

import self_speculative_verify_ripe_amd as rp
from oracle import layout as olay
from oracle import ripe_oracle as ro
from oracle import side_stats as ss
from workloads import Group, make_case

from gpu_util import DEV, Device, make_desc, oracle_cache, upload

pytestmark = pytest.mark.gpu

E_RTOL = {"f32": 1e-4, "bf16": 1e-2}
E_EPS = {"f32": 1e-5, "bf16": 1e-3}
O_TOL = {"f32": 1e-5, "bf16": 2.0 ** -8}  # bf16: times max |v| read
LSE_TOL = 1e-3


def oracle_kappa(oc, groups, case):
    """kappa_j per group from the oracle's float64 FULL outputs."""
    G = case.Hq // case.Hkv
    _, lse, _ = ro.verify(oc, groups, case.q, case.kv_new, case.scale, case.Hq)
    res = []
    for g in groups:
        T = int(case.seq_len[g.seq])
        Kr, _ = oc.get(g.seq, g.depth, 0, T)
        KR, _ = oc.get(g.seq, case.R, 0, T)
        k = np.zeros(T)
        for h in range(case.Hq):
            Q = case.q[g.row_start:g.row_start + g.n_rows, h]
            L = lse[g.row_start:g.row_start + g.n_rows, h][:, None]
            a = np.exp(case.scale * (Q @ Kr[:, h // G].T) - L)
            c = np.exp(case.scale * (Q @ KR[:, h // G].T) - L)
            k = np.maximum(k, (a / (1.0 - a + c)).max(axis=0))
        res.append(k)
    return res


def run(case, groups, tag="", check_out=True, definition=False):
    """ripe_position_error against the oracle: its rank-one form, or with
    ``definition`` the definition itself (one attention per substituted
    position; small inputs only)."""
    print(f"[case] {tag} {case.dtype} T={list(case.seq_len)[:6]} groups={len(groups)}", flush=True)
    planes = {g.depth for g in groups} | {case.R}
    oc = oracle_cache(case, "full", planes=planes)
    cache = upload(olay.encode(oc))
    desc = make_desc(case, "full", max_groups=len(groups))
    dev = Device(case)
    ng = len(groups)
    err = torch.full((ng, case.t_max), float("nan"), dtype=torch.float32, device=DEV)
    cond = torch.full((ng, case.t_max), float("nan"), dtype=torch.float32, device=DEV)
    out = torch.full((case.n_rows, case.Hq, case.D), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((case.n_rows, case.Hq), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.zeros(rp.ripe_layout_bytes(desc, rp.RIPE_BYTES_POSERR_WORKSPACE), dtype=torch.uint8, device=DEV)
    rp.ripe_position_error(desc, cache, case.seq_len, groups, case.n_rows, case.scale, dev.q, dev.kv_new,
                           err, cond, out, lse, ws)
    torch.cuda.synchronize()
    e = err.cpu().numpy().astype(np.float64)
    kg = cond.cpu().numpy().astype(np.float64)
    form = ss.position_error if definition else ss.position_error_rank1
    ref = form(oc, groups, case.q, case.kv_new, case.scale, case.Hq)
    kap = oracle_kappa(oc, groups, case)
    n_ill = n_pos = 0
    for gi, (g, want, kj) in enumerate(zip(groups, ref, kap)):
        T = int(case.seq_len[g.seq])
        assert np.all(e[gi, T:] == 0.0) and np.all(kg[gi, T:] == 0.0), f"{tag} group {gi}: entries past T"
        got = e[gi, :T]
        assert np.all(np.isfinite(got)) and np.all(got >= 0.0)
        assert np.all(np.abs(kg[gi, :T] - kj) <= (1e-3 + 4e-5 * kj) * kj + 1e-6), f"{tag} group {gi}: cond"
        n_ill += int((kj > 1.0).sum())
        n_pos += T
        top = want.max(initial=0.0)
        bad = np.abs(got - want) > (E_RTOL[case.dtype] + 2 * kj * E_EPS[case.dtype]) * want + 1e-6 * top
        assert not bad.any(), (f"{tag} group {gi} (depth {g.depth}): {bad.sum()} positions, e.g. j="
                               f"{np.nonzero(bad)[0][:5]} gpu {got[bad][:3]} oracle {want[bad][:3]}")
        if g.depth == case.R:
            assert np.all(got == 0.0)
    print(f"[case] {tag}: {n_ill} of {n_pos} positions ill-conditioned", flush=True)
    assert n_ill <= max(2, 0.02 * n_pos), f"{tag}: {n_ill} positions with kappa > 1"
    if check_out:
        o_ref, l_ref, _ = ro.verify(oc, groups, case.q, case.kv_new, case.scale, case.Hq)
        rows = np.concatenate([np.arange(g.row_start, g.row_start + g.n_rows) for g in groups])
        o = out.cpu().numpy()[rows]
        ls = lse.cpu().numpy()[rows]
        vmax = 1.0
        if case.dtype == "bf16":
            for g in groups:
                T = int(case.seq_len[g.seq])
                vmax = max(vmax, np.abs(oc.get(g.seq, g.depth, 0, T)[1]).max(initial=0.0),
                           np.abs(case.kv_new[1, g.depth - 1, g.row_start:g.row_start + g.n_rows]).max())
        assert np.abs(o - o_ref[rows]).max() <= O_TOL[case.dtype] * vmax, tag
        assert np.abs(ls - l_ref[rows]).max() <= LSE_TOL, tag
    return e, ref, kap


def test_against_the_definition_fp32():
    """The definition (one full attention per substituted position), not the
    rank-one identity the kernel evaluates: c1's shape, groups at three
    depths."""
    case = make_case("c1", layout="full", k=12)  # fp32, R=4, Hkv=Hq=4, D=64, T=128
    groups = [Group(0, 1, 0, 4), Group(0, 2, 4, 5), Group(0, 4, 9, 3)]
    run(case, groups, tag="c1 definition", definition=True)


@pytest.mark.parametrize("convention", ["workload", "pages"])
def test_against_the_definition_c2_shape(convention):
    """The definition on c2's structure (bf16, R=32, 1% tail positions with 8x
    plane noise, k=8), reduced to T=200 and 4 heads, at depths 4 and 28."""
    case = make_case("c2", layout="full", T_range=(200, 200), Hkv=4, Hq=4, convention=convention)
    for r in (4, 28):
        _, _, kap = run(case, case.groups_at(r), tag=f"c2 definition {convention} r={r}", definition=True)
        assert set(np.nonzero(kap[0] > 1.0)[0]) <= set(case.planes.tail[0].tolist())


def test_fp32_groups_at_several_depths():
    case = make_case("c1", layout="full", k=12)  # fp32, R=4, Hkv=Hq=4, D=64, T=128
    groups = [Group(0, 1, 0, 4), Group(0, 3, 4, 5), Group(0, 4, 9, 3)]
    run(case, groups, tag="c1 depths 1/3/4")


@pytest.mark.parametrize("convention", ["workload", "pages"])
@pytest.mark.parametrize("r", [4, 28, 32])
def test_c2_tail_shape(convention, r):
    """c2's structure (1% of positions with 8x plane noise) on 4 heads."""
    case = make_case("c2", layout="full", T_range=(333, 333), Hkv=4, Hq=4, convention=convention)
    _, _, kap = run(case, case.groups_at(r), tag=f"c2 {convention} r={r}")
    # only the 1% tail positions can hold most of a row's attention
    assert set(np.nonzero(kap[0] > 1.0)[0]) <= set(case.planes.tail[0].tolist())


def test_gqa_ragged_lengths_and_column_chunks():
    # G = 4 query heads per KV head, k = 5 rows: 20 columns (two chunks of 16);
    # lengths not multiples of 32, one empty prefix
    case = make_case("c3", layout="full", B=4, T_range=(3, 150), R=6, Hkv=2, Hq=8, k=5)
    case.seq_len[1] = 0
    run(case, case.groups_at(2), tag="gqa r=2")
    run(case, case.groups_at(5), tag="gqa r=5")


def test_more_groups_than_one_launch():
    # 140 groups: two depths per sequence on disjoint rows, 128 groups per launch
    case = make_case("c3", layout="full", B=70, T_range=(1, 40), R=3, Hkv=1, Hq=2, k=4, D=64)
    groups = []
    for b in range(case.B):
        s, _ = case.blocks[b]
        groups += [Group(b, 1, s, 2), Group(b, 2, s + 2, 2)]
    run(case, groups, tag="140 groups", check_out=False)


def test_full_size_c2():
    """The workload the side statistics are reported on: T = 1024, R = 32,
    40 heads, D = 128, k = 8, both conventions, depth 4."""
    for convention in ("workload", "pages"):
        case = make_case("c2", layout="full", convention=convention)
        e, ref, kap = run(case, case.groups_at(4), tag=f"c2 full size {convention}")
        assert set(np.nonzero(kap[0] > 1.0)[0]) <= set(case.planes.tail[0].tolist())
        T = int(case.seq_len[0])
        n = T // 100
        # the reported statistic, the share of the top 1% positions, agrees
        top_g = np.argsort(-e[0, :T], kind="stable")[:n]
        top_o = np.argsort(-ref[0], kind="stable")[:n]
        share = lambda x, idx: x[idx].sum() / x.sum()
        assert abs(share(e[0, :T], top_g) - share(ref[0], top_o)) < 1e-3


def check_tail(stats, err, cond, T, W, frac):
    """ripe_position_error_tail's rows against the oracle's tail_statistics
    on the same float32 rows: counts and the in-window fraction exact, sums
    and shares within 1e-12 relative (double sums in another order)."""
    got = stats.cpu().numpy()
    for i, t in enumerate(T):
        ref = ss.tail_statistics(err[i], int(t), W, cond=None if cond is None else cond[i], tail_frac=frac)
        row = dict(zip(rp.TAIL_FIELDS, got[i]))
        assert row["tail_positions"] == ref["tail_positions"] and row["positions"] == t, i
        assert np.isclose(row["total"], float(np.asarray(err[i][:t], np.float64).sum()), rtol=1e-12, atol=0), i
        for k in ("tail_share", "window_share", "tail_in_window", "ill_conditioned", "ill_conditioned_share"):
            want = ref[k]
            if want is None:
                assert np.isnan(row[k]), (i, k, row[k])
            elif k in ("tail_in_window", "ill_conditioned"):
                assert row[k] == want, (i, k, row[k], want)
            else:
                assert abs(row[k] - want) <= 1e-12 * abs(want) + 1e-300, (i, k, row[k], want)


@pytest.mark.parametrize("with_cond", [False, True])
def test_tail_statistics_kernel_edge_rows(with_cond):
    """Rows with many equal values (the tail ends inside a run of ties, some
    of them in the window), -0.0 entries, all zeros, T = 0 and 1, a row of
    70,000 positions, padding past T that must be ignored, and more rows
    than one launch holds."""
    rng = np.random.default_rng(20261204)
    stride = 70016
    T = [0, 1, 2, 7, 100, 333, 1024, 5000, 70000, 64, 64, 257] + list(rng.integers(0, 400, size=600))
    rows = len(T)
    err = np.full((rows, stride), 1e30, dtype=np.float32)  # padding: larger than anything inside T
    for i, t in enumerate(T):
        kind = i % 4
        if kind == 0:
            v = rng.integers(0, 5, size=t).astype(np.float32)           # ties everywhere
        elif kind == 1:
            v = rng.exponential(1.0, size=t).astype(np.float32) ** 4  # heavy tail
        elif kind == 2:
            v = np.zeros(t, dtype=np.float32)
            v[::7] = -0.0
        else:
            v = np.full(t, 3.0, dtype=np.float32)
            v[: t // 3] = 5.0                                          # the largest values first
        err[i, :t] = v
    cond = (rng.random((rows, stride)) * 2.0).astype(np.float32) if with_cond else None
    dev_err = torch.from_numpy(err).to(DEV)
    dev_cond = torch.from_numpy(cond).to(DEV) if with_cond else None
    for W, frac in ((64, 0.01), (0, 0.3), (100000, 1.0), (5, 0.05)):
        print(f"[case] tail rows={rows} W={W} frac={frac} cond={with_cond}", flush=True)
        stats = torch.full((rows, rp.RIPE_TAIL_STATS), -1.0, dtype=torch.float64, device=DEV)
        rp.ripe_position_error_tail(dev_err, T, W, stats, cond=dev_cond, tail_frac=frac)
        torch.cuda.synchronize()
        check_tail(stats, err, cond, T, W, frac)


def test_tail_statistics_kernel_on_position_error_rows():
    """The tail figures of ripe_position_error's own rows (c2's structure,
    4 heads, both conventions) equal the oracle's on the same rows."""
    for convention in ("workload", "pages"):
        case = make_case("c2", layout="full", T_range=(333, 333), Hkv=4, Hq=4, convention=convention)
        groups = case.groups_at(4)
        planes = {4, case.R}
        oc = oracle_cache(case, "full", planes=planes)
        desc = make_desc(case, "full", max_groups=len(groups))
        dev = Device(case)
        err = torch.zeros((len(groups), case.t_max), dtype=torch.float32, device=DEV)
        cond = torch.zeros_like(err)
        ws = torch.zeros(rp.ripe_layout_bytes(desc, rp.RIPE_BYTES_POSERR_WORKSPACE), dtype=torch.uint8, device=DEV)
        rp.ripe_position_error(desc, upload(olay.encode(oc)), case.seq_len, groups, case.n_rows, case.scale,
                               dev.q, dev.kv_new, err, cond, None, None, ws)
        T = [int(case.seq_len[g.seq]) for g in groups]
        stats = torch.zeros((len(groups), rp.RIPE_TAIL_STATS), dtype=torch.float64, device=DEV)
        rp.ripe_position_error_tail(err, T, case.W, stats, cond=cond)
        torch.cuda.synchronize()
        check_tail(stats, err.cpu().numpy(), cond.cpu().numpy(), T, case.W, 0.01)
