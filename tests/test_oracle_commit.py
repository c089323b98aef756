"""Pins of the oracle's commit and of its byte-layout encoder.

Commit follows the RIPE abstract (the window of recent positions keeps full
depth, older positions keep only the deepest plane) and the LoopSpec summary
(rejected continuations are dropped: a commit of zero rows changes nothing).
The encoder follows the byte layout the C ABI declares; its offsets are
checked against the layout statement element by element.
"""
import numpy as np
import pytest

from oracle import layout as lay
from oracle import ripe_oracle as ro
from workloads import PlaneModel, make_case

LAYOUTS = ("full", "deepest", "ripe")


def prefix_rows(planes, b, j0, n, R):
    """The plane values of positions [j0, j0+n) arranged as draft rows
    [2, R, n, Hkv, D] (row i carries every depth of position j0+i)."""
    out = np.stack([np.stack([planes.values(kind, b, p, j0, j0 + n) for p in range(1, R + 1)])
                    for kind in (0, 1)])
    return out


def fresh(layout, W, B=2, R=4, t_max=96, Hkv=2, D=8, dtype="f32"):
    return ro.LogicalCache(layout, dtype, R, W, B, t_max, Hkv, D)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("W", [0, 3, 8, 32, 96])
def test_row_by_row_commit_equals_direct_fill(layout, W):
    planes = PlaneModel(7, 4, 2, 8, 0.88, "f32")
    lengths = [37, 70]
    a = fresh(layout, W)
    b = fresh(layout, W)
    for s, T in enumerate(lengths):
        ro.fill_prefix(a, s, T, planes.values)
        rows = prefix_rows(planes, s, 0, T, 4)
        for j in range(T):
            n = np.zeros(2, dtype=int)
            n[s] = 1
            src = np.zeros(2, dtype=int)
            src[s] = j
            ro.commit(b, n, src, rows)
    assert a.same_contents(b)
    assert np.array_equal(lay.encode(a), lay.encode(b))


@pytest.mark.parametrize("layout", LAYOUTS)
def test_commit_split_equals_commit_whole(layout):
    planes = PlaneModel(8, 4, 2, 8, 0.88, "f32")
    base = fresh(layout, 8)
    for s in range(2):
        ro.fill_prefix(base, s, 20 + 9 * s, planes.values)
    rng = np.random.default_rng(0)
    rows = rng.standard_normal((2, 4, 30, 2, 8)).astype(np.float32).astype(np.float64)
    one = base.copy()
    ro.commit(one, [13, 7], [0, 10], rows)
    two = base.copy()
    ro.commit(two, [5, 3], [0, 10], rows)
    ro.commit(two, [8, 4], [5, 13], rows)
    assert one.same_contents(two)
    assert np.array_equal(lay.encode(one), lay.encode(two))


@pytest.mark.parametrize("layout", LAYOUTS)
def test_commit_zero_rows_is_identity(layout):
    planes = PlaneModel(9, 4, 2, 8, 0.88, "f32")
    c = fresh(layout, 8)
    ro.fill_prefix(c, 0, 33, planes.values)
    before = c.copy()
    ro.commit(c, [0, 0], [5, 7], np.zeros((2, 4, 10, 2, 8)))
    assert c.same_contents(before)


def test_ripe_window_after_commit():
    """After any commit, RIPE holds planes 1..R-1 exactly at the last W
    committed positions and plane R at every committed position."""
    planes = PlaneModel(10, 5, 1, 4, 0.88, "f32")
    W = 6
    c = fresh("ripe", W, B=1, R=5, Hkv=1, D=4)
    ro.fill_prefix(c, 0, 4, planes.values)
    rng = np.random.default_rng(3)
    rows = rng.standard_normal((2, 5, 40, 1, 4))
    T = 4
    for n in (0, 1, 3, 9, 2, 7):
        ro.commit(c, [n], [0], rows)
        T += n
        assert c.held_positions(0, 5) == list(range(T))
        for p in range(1, 5):
            assert c.held_positions(0, p) == list(range(max(0, T - W), T))


def test_commit_more_rows_than_window():
    c = fresh("ripe", 4, B=1, R=3, Hkv=1, D=2)
    rows = np.arange(2 * 3 * 10 * 2, dtype=np.float64).reshape(2, 3, 10, 1, 2)
    ro.commit(c, [10], [0], rows)
    assert c.held_positions(0, 1) == [6, 7, 8, 9]
    k, v = c.get(0, 1, 6, 10)
    assert np.array_equal(k[:, 0], rows[0, 0, 6:10, 0])


def test_commit_capacity():
    c = fresh("full", 0, B=1, R=2, t_max=8, Hkv=1, D=2)
    with pytest.raises(ValueError):
        ro.commit(c, [9], [0], np.zeros((2, 2, 9, 1, 2)))


def test_verify_after_commit_equals_verify_on_filled_cache():
    case = make_case("c4", B=3, T_range=(40, 60), R=12, Hkv=2, Hq=4, D=8)
    grown = ro.LogicalCache("ripe", case.dtype, case.R, case.W, case.B, case.t_max, case.Hkv,
                            case.D)
    for b in range(case.B):
        ro.fill_prefix(grown, b, int(case.seq_len[b]), case.planes.values)
    ro.commit(grown, case.n_accept, case.src_row, case.kv_new)
    direct = ro.LogicalCache("ripe", case.dtype, case.R, case.W, case.B, case.t_max, case.Hkv,
                             case.D)
    for b in range(case.B):
        T = int(case.seq_len[b])
        n, s = int(case.n_accept[b]), int(case.src_row[b])

        def values(kind, bb, p, j0, j1, T=T, n=n, s=s):
            pre = case.planes.values(kind, bb, p, j0, min(j1, T))
            new = case.kv_new[kind, p - 1, s + max(j0, T) - T:s + j1 - T]
            return np.concatenate([pre, new]) if j1 > T else pre

        ro.fill_prefix(direct, b, T + n, values)
    assert grown.same_contents(direct)
    groups = [ro._group_fields(g) for g in case.groups()]
    a = ro.verify(grown, groups, case.q, case.kv_new, 1.0, case.Hq)
    d = ro.verify(direct, groups, case.q, case.kv_new, 1.0, case.Hq)
    assert np.array_equal(a[0], d[0]) and np.array_equal(a[1], d[1])


# ---------------------------------------------------------------------------
# encoder
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("W", [0, 1, 3, 4, 5, 8, 12, 16, 40, 64, 70, 96, 500])
def test_encode_size_and_round_trip(layout, dtype, W):
    R, B, t_max, Hkv, D = 3, 2, 96, 2, 8
    planes = PlaneModel(11, R, Hkv, D, 0.88, dtype)
    c = ro.LogicalCache(layout, dtype, R, W, B, t_max, Hkv, D)
    lengths = [0, 71]
    for b, T in enumerate(lengths):
        ro.fill_prefix(c, b, T, planes.values)
    buf = lay.encode(c)
    E = 4 if dtype == "f32" else 2
    We = min(W, t_max)
    per_seq = {"full": R * t_max, "deepest": t_max, "ripe": t_max + We * (R - 1)}[layout]
    assert buf.size == 2 * B * Hkv * D * per_seq * E
    back = lay.decode(buf, layout, dtype, R, W, B, t_max, Hkv, D, lengths)
    assert back.same_contents(c)


@pytest.mark.parametrize("We,slot,d,want", [
    # D = 4, so a full block [D][8] holds 32 elements.  Windows that are
    # multiples of 8: full blocks only (slot s: block s // 8, then d * 8 + s % 8)
    (32, 5, 2, 2 * 8 + 5), (64, 37, 1, 4 * 32 + 1 * 8 + 5), (8, 3, 3, 3 * 8 + 3),
    (40, 35, 2, 4 * 32 + 2 * 8 + 3), (40, 31, 3, 3 * 32 + 3 * 8 + 7),
    # windows below 8: one block [D][We]
    (1, 0, 2, 2), (5, 4, 1, 1 * 5 + 4), (3, 2, 3, 3 * 3 + 2),
    # 8-slot blocks, then a narrower block [D][We mod 8] for the last slots
    (12, 7, 3, 3 * 8 + 7), (12, 10, 3, 8 * 4 + 3 * 4 + 2), (100, 70, 1, 8 * 32 + 1 * 8 + 6),
    (100, 99, 3, 96 * 4 + 3 * 4 + 3), (70, 64, 0, 64 * 4), (70, 69, 3, 64 * 4 + 3 * 6 + 5),
])
def test_ring_v_offsets_hand_computed(We, slot, d, want):
    """The ring's V offsets written out by hand for the block rule the
    layout statement gives (blocks of 8 slots, then the remaining slots as
    one narrower block)."""
    assert lay.ring_v_offset(slot, d, We, 4) == want
    offs = lay.ring_v_offsets(We, 4)
    assert sorted(offs.ravel().tolist()) == list(range(We * 4))  # a permutation of the ring


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("W", [12, 40, 100])
def test_encoder_ring_offsets_any_window(dtype, W):
    """A single ring element of a window that is not a multiple of 8 lands
    where the block rule puts it, in K and V."""
    R, B, T, H, D = 3, 2, 128, 2, 4
    c = ro.LogicalCache("ripe", dtype, R, W, B, T, H, D)
    b, h, d, p, j = 1, 1, 3, 2, 117
    k = np.zeros((H, D)); v = np.zeros((H, D))
    k[h, d], v[h, d] = 7.0, 9.0
    c.put(b, p, j, k, v)
    buf = lay.encode(c)
    n_k = lay.layout_elements("ripe", R, W, B, T, H, D) // 2
    deep = B * H * T * D
    slot = j % W
    head = ((b * (R - 1) + (p - 1)) * H + h) * W * D
    assert _elem(buf, dtype, deep + head + slot * D + d) == 7.0
    assert _elem(buf, dtype, n_k + deep + head + lay.ring_v_offset(slot, d, W, D)) == 9.0


def _elem(buf, dtype, index):
    if dtype == "f32":
        return float(buf.view(np.float32)[index])
    return float((np.uint32(buf.view(np.uint16)[index]) << np.uint32(16)).view(np.float32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_encoder_offsets_match_layout_statement(dtype):
    """Single elements land at the offsets the layout statement gives."""
    R, B, T, H, D, W = 3, 2, 64, 2, 4, 16
    for layout in LAYOUTS:
        c = ro.LogicalCache(layout, dtype, R, W, B, T, H, D)
        b, h, d, j = 1, 1, 2, 45
        marks = {}
        for p in c.planes_held():
            if layout == "ripe" and p < R and not (T - W <= j):
                continue
            k = np.zeros((H, D))
            v = np.zeros((H, D))
            k[h, d] = 10.0 + p
            v[h, d] = 20.0 + p
            c.put(b, p, j, k, v)
            marks[p] = (10.0 + p, 20.0 + p)
        c.seq_len[:] = [0, 50]
        buf = lay.encode(c)
        n_k = lay.layout_elements(layout, R, W, B, T, H, D) // 2
        for p, (kv, vv) in marks.items():
            if layout == "full":
                ko = (((b * R + (p - 1)) * H + h) * T + j) * D + d
                vo = n_k + ((((b * R + (p - 1)) * H + h) * (T // 8) + j // 8) * D + d) * 8 + j % 8
            elif layout == "deepest" or p == R:
                ko = ((b * H + h) * T + j) * D + d
                vo = n_k + (((b * H + h) * (T // 8) + j // 8) * D + d) * 8 + j % 8
            else:
                deep = B * H * T * D
                We, BW = W, min(8, W)
                slot = j % We
                ko = deep + (((b * (R - 1) + (p - 1)) * H + h) * We + slot) * D + d
                vo = n_k + deep + ((((b * (R - 1) + (p - 1)) * H + h) * (We // BW) + slot // BW)
                                   * D + d) * BW + slot % BW
            assert _elem(buf, dtype, ko) == kv, (layout, p)
            assert _elem(buf, dtype, vo) == vv, (layout, p)
