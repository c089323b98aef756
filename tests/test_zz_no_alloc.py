"""ripe_verify_attn_noalloc (split partials in the library's static device
scratch, no workspace argument) against ripe_verify_attn with a caller
workspace, both called through the C ABI: two calls in a row, the second
on a smaller input, so the second runs over the first call's leftover
partials.  The two entry points share their plan and kernels, so out, lse
and plane_sel must be bit-identical; the first call's outputs are also
checked against the float64 oracle (the tolerance bar of the other parity
tests)."""
import ctypes

import numpy as np
import pytest
import torch

import self_speculative_verify_ripe_amd as rp
from self_speculative_verify_ripe_amd import binding
from oracle import layout as olay
from oracle import ripe_oracle as ro
from workloads import make_case

from gpu_util import DEV, TORCH_DT, Device, check, make_desc, oracle_cache, upload

pytestmark = pytest.mark.gpu

I32P = ctypes.POINTER(ctypes.c_int32)


def outputs(case, n_groups):
    out = torch.full((case.n_rows, case.Hq, case.D), float("nan"), dtype=TORCH_DT[case.dtype], device=DEV)
    lse = torch.full((case.n_rows, case.Hq), float("nan"), dtype=torch.float32, device=DEV)
    ps = torch.full((n_groups, case.t_max), -1, dtype=torch.int8, device=DEV)
    return out, lse, ps


def call_both(case, desc, cache, groups, seq_len):
    """The same call through both entry points; returns both results."""
    dev = Device(case)
    sl = np.ascontiguousarray(seq_len, dtype=np.int32)
    garr = rp.pack_groups(groups)
    gptr = garr.ctypes.data_as(ctypes.POINTER(binding.ripe_group_t))
    stream = torch.cuda.current_stream().cuda_stream
    a = outputs(case, len(groups))
    st = binding.lib.ripe_verify_attn_noalloc(ctypes.byref(desc), cache.data_ptr(), sl.ctypes.data_as(I32P), gptr,
                                              len(garr), case.n_rows, case.scale, dev.q.data_ptr(),
                                              dev.kv_new.data_ptr(), a[0].data_ptr(), a[1].data_ptr(),
                                              a[2].data_ptr(), stream)
    assert st == 0, rp.STATUS.get(st, st)
    torch.cuda.synchronize()
    b = outputs(case, len(groups))
    # a workspace whose counters start at zero (as required) and whose
    # partial area holds garbage
    ws = torch.full((rp.ripe_layout_bytes(desc, rp.RIPE_BYTES_WORKSPACE),), 0xFF, dtype=torch.uint8, device=DEV)
    ws[:binding.RIPE_WORKSPACE_ZERO_BYTES] = 0
    st = binding.lib.ripe_verify_attn(ctypes.byref(desc), cache.data_ptr(), sl.ctypes.data_as(I32P), gptr, len(garr),
                                      case.n_rows, case.scale, dev.q.data_ptr(), dev.kv_new.data_ptr(),
                                      b[0].data_ptr(), b[1].data_ptr(), b[2].data_ptr(), ws.data_ptr(), ws.numel(),
                                      stream)
    assert st == 0, rp.STATUS.get(st, st)
    torch.cuda.synchronize()
    return a, b


def same(a, b, tag):
    for x, y, name in zip(a, b, ("out", "lse", "plane_sel")):
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.int8 else x,
                           y.view(torch.uint8) if y.dtype != torch.int8 else y), f"{tag}: {name} differs"


def test_noalloc_matches_workspace_call_twice_shrinking():
    # call 1: 12 sequences of up to 2000 positions, GQA 32/8, D = 128, bf16
    big = make_case("c3", B=12, T_range=(700, 2000), R=8, seed_offset=71)
    desc = make_desc(big, "ripe")
    oc = oracle_cache(big, "ripe")
    cache = upload(olay.encode(oc))
    groups = big.groups_at(3)
    print(f"[case] no-alloc call 1: B={big.B} T={list(big.seq_len)} r=3", flush=True)
    a, b = call_both(big, desc, cache, groups, big.seq_len)
    same(a, b, "call 1")
    check(big, groups, a, ro.verify(oc, groups, big.q, big.kv_new, big.scale, big.Hq), tag="call 1 vs oracle")
    # call 2, smaller: 3 sequences of the same cache, a different depth, fewer rows
    small = make_case("c3", B=3, T_range=(40, 300), R=8, seed_offset=72)
    desc2 = make_desc(small, "ripe")
    oc2 = oracle_cache(small, "ripe")
    cache2 = upload(olay.encode(oc2))
    groups2 = small.groups_at(8)
    print(f"[case] no-alloc call 2: B={small.B} T={list(small.seq_len)} r=8", flush=True)
    a2, b2 = call_both(small, desc2, cache2, groups2, small.seq_len)
    same(a2, b2, "call 2")
    check(small, groups2, a2, ro.verify(oc2, groups2, small.q, small.kv_new, small.scale, small.Hq),
          tag="call 2 vs oracle")


def test_noalloc_fp32_and_rejections():
    case = make_case("c1", layout="full")
    desc = make_desc(case, "full")
    oc = oracle_cache(case, "full")
    cache = upload(olay.encode(oc))
    groups = case.groups_at(2)
    print(f"[case] no-alloc fp32 c1 r=2", flush=True)
    a, b = call_both(case, desc, cache, groups, case.seq_len)
    same(a, b, "c1 fp32")
    # invalid calls are refused before any launch, as for ripe_verify_attn
    dev = Device(case)
    out, lse, ps = outputs(case, len(groups))
    bad = [(g.seq, case.R + 1, g.row_start, g.n_rows) for g in groups]
    with pytest.raises(rp.RipeError) as e:
        rp.ripe_verify_attn_noalloc(desc, cache, case.seq_len, bad, case.n_rows, case.scale, dev.q, dev.kv_new,
                                    out, lse, ps)
    assert e.value.status == -2
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
