"""GPU parity of paged caches (ripe_verify_attn_paged, ripe_commit_paged).

* verify through a random block table against the float64 oracle, every
  layout, pages of 32, 64 and 256 positions, ragged lengths, spare pages
  left NaN (a wrong page address shows up as NaN);
* with pages shorter than the split length (256 positions for these
  shapes), paging changes only where a step is read from: for every such
  page size and placement the results equal the unpaged call's bit for bit
  (the same pieces in the same order); pages of 256 positions and more are
  cut at page boundaries and checked against the oracle;
* commit through the table: the cache bytes equal the oracle's commit
  encoded by the oracle's paged encoder, rows crossing page boundaries and
  RIPE windows shorter than the rows committed included;
* two LoopSpec branches forked from one prefix: shared prefix pages,
  private last page and ring each, different rows committed to each, then
  verified -- against the oracle, byte for byte and in the outputs;
* a parent block in flight over a paged cache.
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


def paged_cache(case, layout, P, seed=0, spare=3, W=None, oc=None):
    oc = oracle_cache(case, layout, W=W) if oc is None else oc
    nb = case.t_max // P
    N = case.B * nb + spare
    rng = np.random.default_rng(seed)
    table = rng.permutation(N)[:case.B * nb].reshape(case.B, nb).astype(np.int32)
    desc = rp.make_desc(layout, case.dtype, case.R, case.W if W is None else W, case.B, case.t_max, case.Hkv,
                        case.D, case.Hq, max_rows=case.n_rows, max_groups=2 * case.B + 8, page_len=P, n_pages=N)
    return oc, desc, table, N


def verify_paged(desc, cache, table, case, dev, groups, seq_len=None, parents=None):
    out = torch.full((case.n_rows, case.Hq, case.D), float("nan"), dtype=TORCH_DT[case.dtype], device=DEV)
    lse = torch.full((case.n_rows, case.Hq), float("nan"), dtype=torch.float32, device=DEV)
    ps = torch.full((max(len(groups), 1), case.t_max), -1, dtype=torch.int8, device=DEV)
    ws = rp.new_workspace(desc, DEV)
    rp.ripe_verify_attn(desc, cache, case.seq_len if seq_len is None else seq_len, groups, case.n_rows,
                        case.scale, dev.q, dev.kv_new, out, lse, ps, ws, parents=parents, block_table=table)
    torch.cuda.synchronize()
    return out, lse, ps


@pytest.mark.parametrize("layout", ["full", "deepest", "ripe"])
@pytest.mark.parametrize("P", [32, 64, 256])
def test_paged_verify_matches_oracle(layout, P):
    case = make_case("c3", B=5, T_range=(1, 480), R=6, Hkv=2, Hq=8, k=5, t_max=512)
    print(f"[case] paged verify {layout} P={P} T={list(case.seq_len)}", flush=True)
    oc, desc, table, N = paged_cache(case, layout, P, seed=P)
    cache = upload(olay.encode_paged(oc, table, P, N))
    dev = Device(case)
    for r in (2, 6):
        groups = case.groups_at(r)
        gpu = verify_paged(desc, cache, table, case, dev, groups)
        ref = ro.verify(oc, groups, case.q, case.kv_new, case.scale, case.Hq)
        check(case, groups, gpu, ref, tag=f"paged {layout} P={P} r={r}")


@pytest.mark.parametrize("layout", ["full", "deepest", "ripe"])
def test_paged_equals_unpaged_bitexact(layout):
    case = make_case("c3", B=4, T_range=(100, 500), R=4, Hkv=2, Hq=8, t_max=512)
    print(f"[case] paged == unpaged {layout}", flush=True)
    dev = Device(case)
    oc = oracle_cache(case, layout)
    res = {}
    for r in (2, 4):
        groups = case.groups_at(r)
        d0 = rp.make_desc(layout, case.dtype, case.R, case.W, case.B, case.t_max, case.Hkv, case.D, case.Hq,
                          max_rows=case.n_rows, max_groups=2 * case.B + 8)
        out = torch.full((case.n_rows, case.Hq, case.D), float("nan"), dtype=TORCH_DT[case.dtype], device=DEV)
        lse = torch.full((case.n_rows, case.Hq), float("nan"), dtype=torch.float32, device=DEV)
        rp.ripe_verify_attn(d0, upload(olay.encode(oc)), case.seq_len, groups, case.n_rows, case.scale, dev.q,
                            dev.kv_new, out, lse, None, rp.new_workspace(d0, DEV))
        torch.cuda.synchronize()
        for P, seed in ((32, 1), (64, 2), (64, 3), (128, 4)):
            _, desc, table, N = paged_cache(case, layout, P, seed=seed, oc=oc)
            po, pl, _ = verify_paged(desc, upload(olay.encode_paged(oc, table, P, N)), table, case, dev, groups)
            assert torch.equal(po, out) and torch.equal(pl, lse), (layout, r, P, seed)


@pytest.mark.parametrize("layout", ["full", "deepest", "ripe"])
@pytest.mark.parametrize("P", [32, 64])
def test_paged_commit_bytes(layout, P):
    case = make_case("c3", B=4, T_range=(20, 200), R=4, Hkv=2, Hq=8, k=40, t_max=320, W=16)
    print(f"[case] paged commit {layout} P={P}", flush=True)
    oc, desc, table, N = paged_cache(case, layout, P, seed=7)
    cache = upload(olay.encode_paged(oc, table, P, N))
    dev = Device(case)
    n_accept = np.array([0, 7, 33, 40], np.int32)    # none, within a page, across pages, more than W
    src = np.array([b * 40 for b in range(4)], np.int32)
    sl = case.seq_len.astype(np.int32).copy()
    rp.ripe_commit(desc, cache, sl, n_accept, src, dev.kv_new, case.n_rows, block_table=table)
    torch.cuda.synchronize()
    ro.commit(oc, n_accept, src, case.kv_new)
    assert np.array_equal(sl, oc.seq_len)
    want = olay.encode_paged(oc, table, P, N)
    got = cache.cpu().numpy()
    # bytes the oracle holds must match exactly (slots it does not hold are NaN there)
    w = want.view(np.uint32 if case.dtype == "f32" else np.uint16)
    g = got.view(w.dtype)
    nan = 0x7FC00000 if case.dtype == "f32" else 0x7FC0
    held = w != nan
    assert np.array_equal(g[held], w[held])
    back = olay.decode_paged(got, layout, case.dtype, case.R, case.W, case.B, case.t_max, case.Hkv, case.D, sl,
                             table, P, N)
    assert back.same_contents(oc)


def test_branches_share_prefix_pages():
    """Sequences 0 and 1 are two branches forked from one 100-position
    prefix: pages of blocks 0..2 (positions 0..95) shared, block 3 copied to
    a private page each; each branch commits its own rows (primary and
    fallback of LoopSpec), then both are verified."""
    P, T0 = 32, 100
    case = make_case("c3", B=2, T_range=(T0, T0), R=4, Hkv=2, Hq=8, k=8, t_max=256, W=16)
    own = case.planes.values
    case.planes.values = lambda kind, b, p, j0, j1: own(kind, 0, p, j0, j1)  # one prefix for both branches
    print("[case] branches", flush=True)
    oc = oracle_cache(case, "ripe")
    table = np.array([[0, 1, 2, 3, 6, 7, 8, 9], [0, 1, 2, 4, 10, 11, 12, 13]], np.int32)  # block 3: pages 3 / 4
    N = 14
    desc = rp.make_desc("ripe", case.dtype, case.R, case.W, 2, case.t_max, case.Hkv, case.D, case.Hq,
                        max_rows=case.n_rows, max_groups=12, page_len=P, n_pages=N)
    cache = upload(olay.encode_paged(oc, table, P, N))
    dev = Device(case)
    # branch 0 keeps 5 rows of its block, branch 1 keeps 8 of its own
    n_accept = np.array([5, 8], np.int32)
    src = np.array([0, 8], np.int32)
    sl = case.seq_len.astype(np.int32).copy()
    rp.ripe_commit(desc, cache, sl, n_accept, src, dev.kv_new, case.n_rows, block_table=table)
    ro.commit(oc, n_accept, src, case.kv_new)
    torch.cuda.synchronize()
    assert list(sl) == [T0 + 5, T0 + 8]
    w = olay.encode_paged(oc, table, P, N).view(np.uint16)
    g = cache.cpu().numpy().view(np.uint16)
    held = w != 0x7FC0
    assert np.array_equal(g[held], w[held])
    for r in (1, 4):
        groups = [Group(0, r, 0, 8), Group(1, r, 8, 8)]
        gpu = verify_paged(desc, cache, table, case, dev, groups, seq_len=sl)
        ref = ro.verify(oc, groups, case.q, case.kv_new, case.scale, case.Hq)
        check(case, groups, gpu, ref, seq_len=sl, tag=f"branches r={r}")


def test_paged_inflight_parent():
    case = make_case("c3", B=3, T_range=(30, 200), R=5, Hkv=2, Hq=8, k=9, t_max=256, W=16)
    print("[case] paged in-flight", flush=True)
    oc, desc, table, N = paged_cache(case, "ripe", 32, seed=3)
    cache = upload(olay.encode_paged(oc, table, 32, N))
    dev = Device(case)
    kp = 4
    groups = [Group(b, 2 + b, s + kp, n - kp, s, kp) for b, (s, n) in enumerate(case.blocks)]
    gpu = verify_paged(desc, cache, table, case, dev, groups, parents=rp.pack_parents(groups))
    ref = ro.verify(oc, groups, case.q, case.kv_new, case.scale, case.Hq)
    check(case, groups, gpu, ref, tag="paged in-flight")
