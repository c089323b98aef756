"""Pins of the oracle's paged byte layout (oracle/layout.py: encode_paged,
decode_paged).

* one page per sequence (P = t_max) on page b: the bytes equal the unpaged
  encoding's, whose layout is pinned separately;
* round trip through any block table, pages shared or not;
* a block lands where the table says: page table[b][k] holds exactly the
  unpaged encoding's block k of sequence b, and untouched pages stay NaN;
* two sequences may share pages where their contents agree; conflicting
  contents raise;
* sizes: the element count matches the closed form N*P*planes + B*We*(R-1).
"""
import numpy as np
import pytest

from oracle import layout as olay
from oracle import ripe_oracle as ro
from workloads import round_to

R, HKV, D = 3, 2, 8


def cache(layout, dtype, B, T, W=8, t_max=128, seed=0, same_prefix=False):
    rng = np.random.default_rng(seed)
    planes = rng.standard_normal((2, B, R, t_max, HKV, D))
    if same_prefix:
        planes[:, 1:] = planes[:, :1]
    planes = round_to(planes, dtype)  # values exact in dtype
    c = ro.LogicalCache(layout, dtype, R, W, B, t_max, HKV, D)
    for b in range(B):
        ro.fill_prefix(c, b, T[b], lambda kind, bb, p, j0, j1: planes[kind, bb, p - 1, j0:j1])
    return c


@pytest.mark.parametrize("layout", ["full", "deepest", "ripe"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_page_per_sequence_equals_unpaged(layout, dtype):
    c = cache(layout, dtype, 3, [0, 70, 128])
    paged = olay.encode_paged(c, np.arange(3).reshape(3, 1), 128, 3)
    assert np.array_equal(paged, olay.encode(c))


@pytest.mark.parametrize("layout", ["full", "deepest", "ripe"])
@pytest.mark.parametrize("P", [32, 64])
def test_round_trip_and_block_placement(layout, P):
    T = [5, 97, 128, 40]
    c = cache(layout, "f32", 4, T, seed=P)
    nb = 128 // P
    rng = np.random.default_rng(P + 1)
    N = 4 * nb + 3                      # spare pages stay untouched
    table = rng.permutation(N)[:4 * nb].reshape(4, nb)
    buf = olay.encode_paged(c, table, P, N)
    assert buf.size == olay.paged_layout_elements(layout, R, 8, 4, 128, HKV, D, P, N) * 4
    back = olay.decode_paged(buf, layout, "f32", R, 8, 4, 128, HKV, D, c.seq_len, table, P, N)
    assert back.same_contents(c)
    # placement: page table[b][k] holds block k of sequence b of the unpaged bytes
    flat = olay.encode(c).view(np.uint32)
    u = olay._region_views(flat, layout, R, 8, 4, 128, HKV, D)
    pv = olay._pool_views(buf.view(np.uint32), layout, R, 8, 4, 128, HKV, D, P, N)
    full = layout == "full"
    for b in range(4):
        for k in range(nb):
            for pi in range(R if full else 1):
                ku = u[("K", "main")][b, pi] if full else u[("K", "main")][b]
                vu = u[("V", "main")][b, pi] if full else u[("V", "main")][b]
                assert np.array_equal(pv[("K", "pool")][table[b, k], pi], ku[:, k * P:(k + 1) * P])
                assert np.array_equal(pv[("V", "pool")][table[b, k], pi], vu[:, k * P // 8:(k + 1) * P // 8])
    unused = np.setdiff1d(np.arange(N), table.ravel())
    assert np.all(pv[("K", "pool")][unused] == 0x7FC00000)


def test_shared_pages():
    # two branches forked from one 70-position prefix: blocks 0 and 1 (positions
    # 0..63) shared, block 2 private to each
    c = cache("ripe", "bf16", 2, [70, 70], same_prefix=True)
    table = np.array([[0, 1, 2, 5], [0, 1, 3, 6]])
    buf = olay.encode_paged(c, table, 32, 8)
    back = olay.decode_paged(buf, "ripe", "bf16", R, 8, 2, 128, HKV, D, c.seq_len, table, 32, 8)
    assert back.same_contents(c)
    other = cache("ripe", "bf16", 2, [70, 70], seed=9)  # different prefixes
    with pytest.raises(ValueError):
        olay.encode_paged(other, table, 32, 8)
