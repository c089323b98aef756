"""C-ABI tests that need no GPU: the library loads, exports every symbol the
header declares, sizes caches by the closed-form memory model, and rejects
invalid arguments on the host before any HIP call (no compute call is made
here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import self_speculative_verify_ripe_amd as rp
from self_speculative_verify_ripe_amd import binding
from oracle import layout as oracle_layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ripe.h")

FAKE = 1 << 20  # a 256-byte aligned non-null address; never dereferenced on error paths


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ripe_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert names == ["ripe_accept", "ripe_accept_workspace_bytes", "ripe_commit", "ripe_commit_paged",
                     "ripe_layout_bytes", "ripe_position_error", "ripe_position_error_tail", "ripe_verify_attn",
                     "ripe_verify_attn_inflight",
                     "ripe_verify_attn_noalloc", "ripe_verify_attn_paged"]
    lib = ctypes.CDLL(binding.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_struct_sizes_match_header():
    assert ctypes.sizeof(rp.ripe_desc_t) == 14 * 4
    assert ctypes.sizeof(rp.ripe_group_t) == 16
    assert ctypes.sizeof(rp.ripe_accept_desc_t) == 16


@pytest.mark.parametrize("layout", ["full", "deepest", "ripe"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("W", [0, 1, 3, 4, 5, 8, 12, 16, 24, 32, 40, 64, 96, 100, 4096, 100000])
def test_cache_bytes_closed_form(layout, dtype, W):
    R, B, T, H, D = 32, 3, 1024, 8, 128
    d = rp.make_desc(layout, dtype, R, W, B, T, H, D, 32)
    got = rp.ripe_layout_bytes(d)
    assert got == oracle_layout.layout_bytes(layout, dtype, R, W, B, T, H, D)
    E = 4 if dtype == "f32" else 2
    per_seq = {"full": R * T, "deepest": T, "ripe": T + min(W, T) * (R - 1)}[layout]
    assert got == 2 * B * H * D * E * per_seq


def test_memory_identities():
    R, B, T, H, D = 32, 2, 1024, 8, 128
    full = rp.ripe_layout_bytes(rp.make_desc("full", "bf16", R, 64, B, T, H, D, 32))
    deep = rp.ripe_layout_bytes(rp.make_desc("deepest", "bf16", R, 64, B, T, H, D, 32))
    assert rp.ripe_layout_bytes(rp.make_desc("ripe", "bf16", R, 0, B, T, H, D, 32)) == deep
    assert rp.ripe_layout_bytes(rp.make_desc("ripe", "bf16", R, T, B, T, H, D, 32)) == full
    ripe = rp.ripe_layout_bytes(rp.make_desc("ripe", "bf16", R, 64, B, T, H, D, 32))
    assert ripe * 32768 == full * 3008  # T + W(R-1) over R*T at T=1024, W=64, R=32


def test_workspace_bound_positive():
    d = rp.make_desc("ripe", "bf16", 32, 64, 16, 4128, 8, 128, 32, max_rows=128, max_groups=16)
    assert rp.ripe_layout_bytes(d, rp.RIPE_BYTES_WORKSPACE) > 0


@pytest.mark.parametrize("field,value,status", [
    ("layout", 3, -1), ("dtype", 7, -1), ("R", 0, -1), ("W", -1, -1), ("batch", 0, -1),
    ("t_max", 0, -1), ("n_kv_heads", 0, -1), ("n_q_heads", 12, -1), ("head_dim", 96, -4),
    ("t_max", 100, -4), ("R", 200, -4), ("split_len", 48, -4),
    ("split_len", -32, -1),
])
def test_bad_descriptor(field, value, status):
    d = rp.make_desc("ripe", "bf16", 32, 64, 2, 1024, 8, 128, 32)
    setattr(d, field, value)
    assert binding.lib.ripe_layout_bytes(ctypes.byref(d), 0) == status


def test_limits_of_the_plan_records():
    """Values the plan narrows to 16 bits, and pieces whose byte extents feed
    32-bit buffer resources, are refused rather than wrapped."""
    d = rp.make_desc("ripe", "bf16", 4, 64, 2, 1024, 65536, 64, 65536)
    assert binding.lib.ripe_layout_bytes(ctypes.byref(d), 0) == -4
    d = rp.make_desc("ripe", "bf16", 4, 64, 2, 1024, 65535, 64, 65535)
    assert binding.lib.ripe_layout_bytes(ctypes.byref(d), 0) > 0
    d = rp.make_desc("ripe", "bf16", 4, 64, 2, 16384, 8, 128, 32, split_len=8192 + 32)
    assert binding.lib.ripe_layout_bytes(ctypes.byref(d), 0) == -4
    d.split_len = 8192
    assert binding.lib.ripe_layout_bytes(ctypes.byref(d), 0) > 0


def test_inflight_ring_wider_than_16_bits():
    # a ring of 70016 slots: fine without a parent, refused with one in flight
    d = rp.make_desc("ripe", "bf16", 2, 70016, 1, 70016, 1, 64, 1, max_rows=8, max_groups=1)
    sl = np.array([100], np.int32)
    garr = rp.pack_groups([(0, 1, 4, 4)])
    par = np.array([[0, 4]], np.int32)
    I32P = ctypes.POINTER(ctypes.c_int32)
    st = binding.lib.ripe_verify_attn_inflight(
        ctypes.byref(d), FAKE, sl.ctypes.data_as(I32P), garr.ctypes.data_as(ctypes.POINTER(rp.ripe_group_t)),
        par.ctypes.data_as(I32P), 1, 8, 1.0, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 40, None)
    assert st == -4


def test_bad_kind():
    d = rp.make_desc("ripe", "bf16", 32, 64, 2, 1024, 8, 128, 32)
    assert binding.lib.ripe_layout_bytes(ctypes.byref(d), 9) == -1
    assert binding.lib.ripe_layout_bytes(None, 0) == -1


def call_verify(desc, seq_len, groups, n_rows=16, scale=1.0, cache=FAKE, q=FAKE, kv=FAKE,
                out=FAKE, lse=None, ps=None, ws=FAKE, ws_bytes=1 << 40):
    sl = np.ascontiguousarray(np.asarray(seq_len, dtype=np.int32))
    garr, ng, _keep = binding._groups(groups if len(groups) else np.zeros((0, 4), np.int32))
    return binding.lib.ripe_verify_attn(
        ctypes.byref(desc), cache, sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), garr, ng,
        n_rows, scale, q, kv, out, lse, ps, ws, ws_bytes, None)


def desc2():
    return rp.make_desc("ripe", "bf16", 4, 8, 2, 64, 2, 64, 4, max_rows=16, max_groups=4)


@pytest.mark.parametrize("case,status", [
    (dict(seq_len=[10, 65]), -2),                       # T > t_max
    (dict(seq_len=[-1, 3]), -2),
    (dict(groups=[(2, 1, 0, 4)]), -2),                  # sequence out of range
    (dict(groups=[(0, 0, 0, 4)]), -2),                  # depth 0
    (dict(groups=[(0, 5, 0, 4)]), -2),                  # depth > R
    (dict(groups=[(0, 1, 14, 4)]), -2),                 # rows past n_rows
    (dict(groups=[(0, 1, 0, 0)]), -1),                  # empty group
    (dict(groups=[(0, 1, 0, 4), (1, 1, 3, 4)]), -1),    # overlapping rows
    (dict(scale=float("nan")), -1),
    (dict(scale=float("inf")), -1),
    (dict(q=0), -1), (dict(cache=0), -1), (dict(out=0), -1), (dict(kv=0), -1),
    (dict(q=FAKE + 2), -1),                             # misaligned
    (dict(ws=FAKE + 16), -1),                           # workspace not 256-aligned
    (dict(ws_bytes=16), -5),                            # workspace too small
    (dict(ws=0, ws_bytes=0), -5),
    (dict(n_rows=0), -1),
])
def test_verify_rejects(case, status):
    args = dict(seq_len=[10, 20], groups=[(0, 1, 0, 4), (1, 2, 4, 4)])
    args.update(case)
    assert call_verify(desc2(), **args) == status


def test_verify_no_groups_is_noop():
    assert call_verify(desc2(), [10, 20], []) == 0


def test_verify_too_many_columns():
    d = rp.make_desc("ripe", "bf16", 4, 8, 1, 64, 1, 64, 64, max_rows=2048, max_groups=4)
    assert call_verify(d, [10], [(0, 1, 0, 1100)], n_rows=2048) == -4  # 1100 * 64 columns


def call_commit(desc, seq_len, n_accept, src_row, n_rows=8, cache=FAKE, kv=FAKE):
    sl = np.ascontiguousarray(np.asarray(seq_len, dtype=np.int32))
    na = np.ascontiguousarray(np.asarray(n_accept, dtype=np.int32))
    sr = np.ascontiguousarray(np.asarray(src_row, dtype=np.int32))
    st = binding.lib.ripe_commit(ctypes.byref(desc), cache,
                                 sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                 na.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                 sr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), kv, n_rows, None)
    return st, sl


@pytest.mark.parametrize("args,status", [
    (([60, 0], [5, 0], [0, 0]), -3),     # capacity
    (([0, 0], [-1, 0], [0, 0]), -1),     # negative count
    (([0, 0], [4, 0], [6, 0]), -2),      # source rows past n_rows
    (([0, 0], [2, 0], [-1, 0]), -2),
    (([65, 0], [0, 0], [0, 0]), -2),     # committed length past t_max
])
def test_commit_rejects_and_leaves_seq_len(args, status):
    st, sl = call_commit(desc2(), *args)
    assert st == status
    assert sl.tolist() == list(args[0])


def test_commit_nothing_accepted_is_noop():
    st, sl = call_commit(desc2(), [7, 9], [0, 0], [3, 3], cache=0, kv=0)
    assert st == 0 and sl.tolist() == [7, 9]


def test_commit_null_buffers():
    st, sl = call_commit(desc2(), [7, 9], [1, 0], [0, 0], cache=0)
    assert st == -1 and sl.tolist() == [7, 9]


# ---------------------------------------------------------------------------
# ripe_accept: descriptor and argument checks (no HIP call on these paths)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("batch,k,vocab,temp,status", [
    (-1, 4, 100, 1.0, rp.binding.RipeError), (2, 0, 100, 1.0, None), (2, 65, 100, 1.0, None),
    (2, 4, 0, 1.0, None), (2, 4, (1 << 24) + 1, 1.0, None), (2, 4, 100, -0.5, None),
    (2, 4, 100, float("nan"), None), (2, 4, 100, float("inf"), None)])
def test_accept_bad_descriptor(batch, k, vocab, temp, status):
    d = rp.make_accept_desc(batch, k, vocab, temp)
    with pytest.raises(rp.RipeError) as e:
        rp.ripe_accept_workspace_bytes(d)
    expect = -4 if (k > 64 or vocab > (1 << 24)) else -1
    assert e.value.status == expect


def test_accept_workspace_bytes():
    wb = lambda B, k, V: rp.ripe_accept_workspace_bytes(rp.make_accept_desc(B, k, V, 0.8))
    assert wb(0, 1, 7) == 0
    base = wb(16, 4, 65536)
    assert base > 0 and base % 256 == 0
    # at least the row statistics (4k + 2 rows of 16 bytes per sequence) and one
    # double per 64-index tile per sequence
    assert base >= 16 * 18 * 16 + 16 * (65536 // 64) * 8
    assert wb(32, 4, 65536) > base and wb(16, 8, 65536) > base and wb(16, 4, 1 << 20) > base


def call_accept(d, **over):
    args = dict(target=FAKE, draft=FAKE, tokens=FAKE, fb=FAKE, rand=FAKE, n=FAKE, br=FAKE, nx=FAKE,
                ws=FAKE, ws_bytes=1 << 20)
    args.update(over)
    return binding.lib.ripe_accept(ctypes.byref(d), args["target"], args["draft"], args["tokens"], args["fb"],
                                   args["rand"], args["n"], args["br"], args["nx"], args["ws"],
                                   args["ws_bytes"], None)


@pytest.mark.parametrize("over,status", [
    ({"target": None}, -1), ({"tokens": None}, -1), ({"fb": None}, -1), ({"n": None}, -1),
    ({"br": None}, -1), ({"nx": None}, -1), ({"draft": None}, -1), ({"rand": None}, -1),
    ({"target": FAKE + 4}, -1), ({"nx": FAKE + 8}, -1), ({"ws": None}, -5), ({"ws_bytes": 100}, -5),
    ({"ws": FAKE + 16}, -1)])
def test_accept_rejects(over, status):
    assert call_accept(rp.make_accept_desc(2, 4, 100, 0.7), **over) == status


def test_accept_greedy_needs_no_draft_or_rand_but_checks_the_rest():
    d = rp.make_accept_desc(2, 4, 100, 0.0)
    assert call_accept(d, target=None, draft=None, rand=None) == -1


def test_accept_empty_batch_is_noop():
    assert call_accept(rp.make_accept_desc(0, 4, 100, 0.7), target=None, ws=None, ws_bytes=0) == 0


def test_commit_args_from_accept_result():
    n, src = rp.commit_args([0, 3, 2], [0, 0, 1], [10, 20, 30], [14, 24, 34])
    assert list(n) == [0, 3, 2] and list(src) == [0, 20, 34]


# ---------------------------------------------------------------------------
# ripe_verify_attn_inflight: parent-block checks (no HIP call on these paths)
# ---------------------------------------------------------------------------
def call_inflight(groups, parents, seq_len=(10, 20), n_rows=16, ws_bytes=1 << 40):
    sl = np.ascontiguousarray(np.asarray(seq_len, dtype=np.int32))
    garr, ng, _keep = binding._groups(groups)
    par = None if parents is None else np.ascontiguousarray(np.asarray(parents, dtype=np.int32).reshape(-1, 2))
    return binding.lib.ripe_verify_attn_inflight(
        ctypes.byref(desc2()), FAKE, sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), garr,
        None if par is None else par.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ng, n_rows, 1.0,
        FAKE, FAKE, FAKE, None, None, FAKE, ws_bytes, None)


@pytest.mark.parametrize("groups,parents,status", [
    ([(0, 1, 4, 4)], None, -1),                               # parents missing
    ([(0, 1, 4, 4)], [(0, -1)], -1),                          # negative parent length
    ([(0, 1, 4, 4)], [(-1, 2)], -2),                          # parent row before 0
    ([(0, 1, 4, 4)], [(14, 4)], -2),                          # parent rows past n_rows
    ([(0, 1, 4, 4), (0, 2, 8, 4)], [(0, 4), (0, 3)], -4),     # siblings with different parents
    ([(0, 1, 4, 4), (0, 2, 8, 4)], [(0, 4), (1, 4)], -4),
    ([(0, 1, 4, 4), (0, 2, 8, 4)], [(0, 4), (0, 0)], -4),     # one sibling without the parent
])
def test_inflight_rejects(groups, parents, status):
    assert call_inflight(groups, parents) == status


def test_inflight_no_groups_is_noop():
    assert call_inflight(np.zeros((0, 4), np.int32), None) == 0


# ---------------------------------------------------------------------------
# ripe_position_error: host checks (no HIP call on these paths)
# ---------------------------------------------------------------------------
def desc_full(**kw):
    args = dict(max_rows=16, max_groups=4)
    args.update(kw)
    return rp.make_desc("full", "bf16", 4, 0, 2, 64, 2, 64, 4, **args)


def call_poserr(desc=None, seq_len=(10, 20), groups=((0, 1, 0, 4), (1, 2, 4, 4)), n_rows=16, err=FAKE,
                cond=None, out=None, lse=None, ws=FAKE, ws_bytes=1 << 40, q=FAKE):
    desc = desc_full() if desc is None else desc
    sl = np.ascontiguousarray(np.asarray(seq_len, dtype=np.int32))
    garr, ng, _keep = binding._groups(list(groups) if len(groups) else np.zeros((0, 4), np.int32))
    return binding.lib.ripe_position_error(
        ctypes.byref(desc), FAKE, sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), garr, ng, n_rows, 1.0,
        q, FAKE, err, cond, out, lse, ws, ws_bytes, None)


def test_position_error_workspace_bound():
    d = desc_full()
    verify = rp.ripe_layout_bytes(d, rp.RIPE_BYTES_WORKSPACE)
    pe = rp.ripe_layout_bytes(d, rp.RIPE_BYTES_POSERR_WORKSPACE)
    a = lambda x: (x + 255) // 256 * 256
    # fp32 outputs + LSE of max_rows rows, per-KV-head sums and condition
    # numbers of max_groups groups
    assert pe == verify + a(16 * 4 * 64 * 4) + a(16 * 4 * 4) + 2 * a(4 * 2 * 64 * 4)


@pytest.mark.parametrize("case,status", [
    (dict(desc=rp.make_desc("ripe", "bf16", 4, 8, 2, 64, 2, 64, 4, max_rows=16, max_groups=4)), -4),
    (dict(desc=rp.make_desc("deepest", "bf16", 4, 0, 2, 64, 2, 64, 4, max_rows=16, max_groups=4)), -4),
    (dict(err=0), -1),
    (dict(err=FAKE + 2), -1),
    (dict(cond=FAKE + 2), -1),
    (dict(out=FAKE + 4), -1),
    (dict(lse=FAKE + 2), -1),
    (dict(ws=0, ws_bytes=0), -5),
    (dict(ws=FAKE + 16), -1),
    (dict(ws_bytes=1024), -5),           # smaller than the fp32 outputs alone
    (dict(seq_len=(10, 65)), -2),        # checked by the verify pass before any launch
    (dict(groups=((0, 5, 0, 4),)), -2),
    (dict(groups=((0, 1, 0, 4), (1, 2, 2, 4))), -1),
    (dict(q=0), -1),
    (dict(n_rows=0), -1),
])
def test_position_error_rejects(case, status):
    assert call_poserr(**case) == status


def test_position_error_no_groups_is_noop():
    assert call_poserr(groups=()) == 0


def call_tail(err=None, cond=None, T=(10, 20), n_rows=None, stride=64, window=8, frac=0.01, stats=None):
    t = np.asarray(T, dtype=np.int32)
    return binding.lib.ripe_position_error_tail(
        FAKE if err is None else err, cond, t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        len(t) if n_rows is None else n_rows, stride, window, frac, FAKE if stats is None else stats, None)


@pytest.mark.parametrize("case,status", [
    (dict(n_rows=-1), -1),
    (dict(stride=-1), -1),
    (dict(window=-1), -1),
    (dict(frac=0.0), -1),
    (dict(frac=1.5), -1),
    (dict(frac=float("nan")), -1),
    (dict(err=0), -1),
    (dict(err=FAKE + 2), -1),
    (dict(cond=FAKE + 2), -1),
    (dict(stats=0), -1),
    (dict(stats=FAKE + 4), -1),          # doubles: 8-byte aligned
    (dict(T=(10, 65)), -2),              # longer than the row stride
    (dict(T=(10, -1)), -2),
])
def test_position_error_tail_rejects(case, status):
    assert call_tail(**case) == status


def test_position_error_tail_no_rows_is_noop():
    assert call_tail(T=(), n_rows=0) == 0


# ---------------------------------------------------------------------------
# paged caches: descriptor, size, host checks (no HIP call on these paths)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("layout", ["full", "deepest", "ripe"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("P,N", [(32, 5), (64, 40), (1024, 3)])
def test_paged_cache_bytes_closed_form(layout, dtype, P, N):
    d = rp.make_desc(layout, dtype, 32, 64, 4, 1024, 8, 128, 32, page_len=P, n_pages=N)
    want = oracle_layout.paged_layout_elements(layout, 32, 64, 4, 1024, 8, 128, P, N) * (4 if dtype == "f32" else 2)
    assert rp.ripe_layout_bytes(d) == want


@pytest.mark.parametrize("P,N,status", [(48, 4, -4), (128, 4, -4), (-32, 4, -1), (32, 0, -1), (32, -1, -1)])
def test_paged_bad_descriptor(P, N, status):
    d = rp.make_desc("ripe", "bf16", 4, 8, 2, 192, 2, 64, 4, page_len=P, n_pages=N)
    assert binding.lib.ripe_layout_bytes(ctypes.byref(d), 0) == status


def paged_desc():
    return rp.make_desc("ripe", "bf16", 4, 8, 2, 64, 2, 64, 4, max_rows=16, max_groups=4, page_len=32, n_pages=4)


def call_verify_paged(desc, table, seq_len=(10, 40), groups=((0, 1, 0, 4), (1, 2, 4, 4))):
    sl = np.ascontiguousarray(np.asarray(seq_len, dtype=np.int32))
    garr, ng, _keep = binding._groups(list(groups))
    I32P = ctypes.POINTER(ctypes.c_int32)
    tab = None if table is None else np.ascontiguousarray(np.asarray(table, dtype=np.int32))
    return binding.lib.ripe_verify_attn_paged(
        ctypes.byref(desc), FAKE, None if tab is None else tab.ctypes.data_as(I32P), sl.ctypes.data_as(I32P),
        garr, None, ng, 16, 1.0, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 40, None)


@pytest.mark.parametrize("table,seq_len,status", [
    (None, (10, 40), -1),                       # table missing
    ([[0, -1], [1, 4]], (10, 40), -2),          # page 4 of 4 read by sequence 1 (positions 32..39)
    ([[-1, 9], [1, 2]], (10, 40), -2),          # sequence 0's first block unmapped
])
def test_paged_verify_rejects(table, seq_len, status):
    assert call_verify_paged(paged_desc(), table, seq_len) == status


def test_paged_entry_points_need_matching_descriptor():
    assert call_verify_paged(desc2(), [[0, 1], [2, 3]]) == -1           # unpaged descriptor
    assert call_verify(paged_desc(), [10, 20], [(0, 1, 0, 4)]) == -1      # paged descriptor, no table
    d = rp.make_desc("full", "bf16", 4, 0, 2, 64, 2, 64, 4, max_rows=16, max_groups=4, page_len=32, n_pages=4)
    assert call_poserr(desc=d) == -4


def call_commit_paged(table, seq_len=(10, 40), n_accept=(4, 4), src_row=(0, 4)):
    I32P = ctypes.POINTER(ctypes.c_int32)
    sl = np.ascontiguousarray(np.asarray(seq_len, dtype=np.int32))
    na = np.ascontiguousarray(np.asarray(n_accept, dtype=np.int32))
    sr = np.ascontiguousarray(np.asarray(src_row, dtype=np.int32))
    tab = np.ascontiguousarray(np.asarray(table, dtype=np.int32))
    st = binding.lib.ripe_commit_paged(ctypes.byref(paged_desc()), FAKE, tab.ctypes.data_as(I32P),
                                       sl.ctypes.data_as(I32P), na.ctypes.data_as(I32P), sr.ctypes.data_as(I32P),
                                       FAKE, 16, None)
    return st, sl


@pytest.mark.parametrize("table,seq_len,n_accept,status", [
    ([[0, 1], [2, 9]], (10, 40), (4, 4), -2),       # sequence 1 writes block 1: page 9 of 4
    ([[0, 1], [0, 3]], (10, 8), (4, 4), -1),        # both write page 0, slots 10..13 and 8..11
    # sequence 0 writes positions 30..33 (page 0 slots 30, 31; page 1 slots 0, 1),
    # sequence 1 positions 32..35 (its block 1: page 1 slots 0..3)
    ([[0, 1], [2, 1]], (30, 32), (4, 4), -1),
])
def test_paged_commit_rejects(table, seq_len, n_accept, status):
    st, sl = call_commit_paged(table, seq_len, n_accept)
    assert st == status
    assert list(sl) == list(seq_len)  # untouched on error


def test_paged_page_list_capacity():
    # one sequence of 69632 positions in 32-position pages: its prefix pieces
    # need 2176 page entries, more than one launch holds
    t_max, P = 69632, 32
    d = rp.make_desc("deepest", "bf16", 2, 0, 1, t_max, 1, 64, 1, max_rows=4, max_groups=1, page_len=P,
                     n_pages=t_max // P)
    table = np.arange(t_max // P, dtype=np.int32)
    I32P = ctypes.POINTER(ctypes.c_int32)
    sl = np.array([t_max - 4], np.int32)
    garr, ng, _keep = binding._groups([(0, 2, 0, 4)])
    st = binding.lib.ripe_verify_attn_paged(ctypes.byref(d), FAKE, table.ctypes.data_as(I32P),
                                            sl.ctypes.data_as(I32P), garr, None, ng, 4, 1.0, FAKE, FAKE, FAKE,
                                            None, None, FAKE, 1 << 40, None)
    assert st == -4
