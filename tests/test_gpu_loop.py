"""A few decoding steps through every entry point together, against the
oracle after each step.

Per step, for every sequence of a paged RIPE cache: a primary draft block at
depth r1 and, for some sequences, a fallback block at depth r2 (LoopSpec
branches) are verified in one call; accept / rollback runs on synthetic
logits; commit_args turns its result into n_accept / src_row; the kept rows
are committed through the block table.  The oracle takes the same steps
(ro.verify, oa.accept, ro.commit) on its logical cache: the verify outputs,
the accept decisions and, after every commit, the cache bytes must agree.
"""
import numpy as np
import pytest
import torch

import self_speculative_verify_ripe_amd as rp
from oracle import accept as oa
from oracle import layout as olay
from oracle import ripe_oracle as ro
from workloads import Group, accept_inputs, make_case, round_to

from gpu_util import DEV, TORCH_DT, check, oracle_cache, upload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("P", [32, 128])
def test_decoding_steps(P):
    k, steps, V = 4, 3, 700
    case = make_case("c3", B=4, T_range=(40, 120), R=4, Hkv=2, Hq=4, D=64, k=2 * k, W=16, t_max=256)
    B, R = case.B, case.R
    r1, r2 = 2, 3
    oc = oracle_cache(case, "ripe")
    nb = case.t_max // P
    N = B * nb + 1
    table = np.random.default_rng(P).permutation(N)[:B * nb].reshape(B, nb).astype(np.int32)
    desc = rp.make_desc("ripe", case.dtype, R, case.W, B, case.t_max, case.Hkv, case.D, case.Hq,
                        max_rows=2 * B * k, max_groups=2 * B, page_len=P, n_pages=N)
    cache = upload(olay.encode_paged(oc, table, P, N))
    ws = rp.new_workspace(desc, DEV)
    sl = case.seq_len.astype(np.int32).copy()
    rng = np.random.default_rng(11 + P)
    n_rows = 2 * B * k
    primary = np.arange(B) * 2 * k
    fallback = primary + k
    kept = fallback_kept = rollbacks = 0
    for step in range(steps):
        print(f"[case] P={P} step {step} T={list(sl)}", flush=True)
        # this step's draft rows and queries (rows of sequence b: primary
        # b*2k .. b*2k+k-1, fallback the next k)
        q = round_to(rng.standard_normal((n_rows, case.Hq, case.D)) / np.sqrt(case.D), case.dtype)
        kv = round_to(rng.standard_normal((2, R, n_rows, case.Hkv, case.D)), case.dtype)
        has_fb = rng.random(B) < 0.5
        groups = []
        for b in range(B):
            groups.append(Group(b, r1, int(primary[b]), k))
            if has_fb[b]:
                groups.append(Group(b, r2, int(fallback[b]), k))
        qd = torch.from_numpy(q.astype(np.float32)).to(TORCH_DT[case.dtype]).to(DEV)
        kvd = torch.from_numpy(kv.astype(np.float32)).to(TORCH_DT[case.dtype]).to(DEV)
        out = torch.full((n_rows, case.Hq, case.D), float("nan"), dtype=TORCH_DT[case.dtype], device=DEV)
        lse = torch.full((n_rows, case.Hq), float("nan"), dtype=torch.float32, device=DEV)
        ps = torch.full((len(groups), case.t_max), -1, dtype=torch.int8, device=DEV)
        rp.ripe_verify_attn(desc, cache, sl, groups, n_rows, case.scale, qd, kvd, out, lse, ps, ws,
                            block_table=table)
        torch.cuda.synchronize()
        ref = ro.verify(oc, groups, q, kv, case.scale, case.Hq)
        check(case, groups, (out, lse, ps), ref, seq_len=sl, tag=f"P={P} step {step}")
        # accept / rollback on synthetic logits
        # noisy drafts: rejections, fallbacks and full rollbacks all occur
        inp = accept_inputs(100 * P + step, B, k, V, 0.8, fallback_frac=0.0, draft_noise=1.5)
        inp.has_fallback[:] = has_fb
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
        na_d, br_d, nx_d = (torch.empty(B, dtype=torch.int32, device=DEV) for _ in range(3))
        rp.ripe_accept(rp.make_accept_desc(B, k, V, 0.8), t(inp.target), t(inp.draft), t(inp.tokens),
                       t(inp.has_fallback), t(inp.rand.view(np.int32)), na_d, br_d, nx_d)
        torch.cuda.synchronize()
        aref = oa.accept(inp.target, inp.draft, inp.tokens, inp.has_fallback, inp.rand, 0.8)
        assert np.all(aref.margin >= 1e-9)
        n_acc, branch = na_d.cpu().numpy(), br_d.cpu().numpy()
        assert np.array_equal(n_acc, aref.n_accept) and np.array_equal(branch, aref.branch)
        assert np.array_equal(nx_d.cpu().numpy(), aref.next_token)
        # commit the kept rows through the block table; the oracle likewise
        na, src = rp.commit_args(n_acc, branch, primary, fallback)
        kept += int(na.sum())
        fallback_kept += int(((branch == 1) & (na > 0)).sum())
        rollbacks += int((na == 0).sum())
        sl_before = sl.copy()
        rp.ripe_commit(desc, cache, sl, na, src, kvd, n_rows, block_table=table)
        torch.cuda.synchronize()
        ro.commit(oc, na, src, kv)
        assert np.array_equal(sl, sl_before + na) and np.array_equal(sl, oc.seq_len)
        want = olay.encode_paged(oc, table, P, N).view(np.uint16)
        got = cache.cpu().numpy().view(np.uint16)
        held = want != 0x7FC0
        assert np.array_equal(got[held], want[held]), f"P={P} step {step}: cache bytes"
    # the steps went through every outcome
    assert kept > 0 and fallback_kept > 0 and rollbacks > 0, (kept, fallback_kept, rollbacks)
