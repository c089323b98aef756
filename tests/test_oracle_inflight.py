"""Pins of the oracle's in-flight parent blocks (a group verified while the
block before it is not yet committed; LoopSpec summary: the next position's
computation starts before the current one is confirmed).

* the defining property: verifying with the parent in flight equals
  committing the parent first (the oracle's commit, pinned separately) and
  verifying after it -- for every layout, window, parent length and prefix
  length, bit for bit;
* brute force with explicit loops over the positions a row sees;
* the RIPE identities: a window covering the prefix and the parent equals
  the full cache, W = 0 equals the deepest plane alone;
* a group's result does not depend on the other groups of the call;
* a planted mistake (the window anchored at the committed length, ignoring
  the parent) fails the first pin.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import ripe_oracle as ro
from workloads import Group

R, HKV, HQ, D = 4, 2, 4, 8


def make_cache(layout, W, T, seed, B=1, t_max=64):
    """T: one length for every sequence, or a list of lengths."""
    rng = np.random.default_rng(seed)
    planes = rng.standard_normal((2, B, R, t_max, HKV, D))
    c = ro.LogicalCache(layout, "f32", R, W, B, t_max, HKV, D)
    Ts = [T] * B if np.isscalar(T) else list(T)
    for b in range(B):
        ro.fill_prefix(c, b, Ts[b], lambda kind, bb, p, j0, j1: planes[kind, bb, p - 1, j0:j1])
    return c


def inputs(seed, n_rows):
    rng = np.random.default_rng(seed + 1)
    return rng.standard_normal((n_rows, HQ, D)), rng.standard_normal((2, R, n_rows, HKV, D))


CASES = list(itertools.product(["full", "deepest", "ripe"], [0, 3, 8, 64], [1, 3, 6, 12], [0, 2, 5, 20]))


@pytest.mark.parametrize("layout,W,kp,T", CASES)
def test_inflight_equals_commit_then_verify(layout, W, kp, T):
    k, r = 3, 2
    c = make_cache(layout, W, T, seed=T * 131 + kp * 7 + W)
    q, kv = inputs(T + kp, kp + k)
    child = Group(0, r, kp, k, parent_row_start=0, parent_rows=kp)
    out, lse, sels = ro.verify(c, [child], q, kv, 0.7, HQ)
    after = c.copy()
    ro.commit(after, [kp], [0], kv)
    out2, lse2, sels2 = ro.verify(after, [Group(0, r, kp, k)], q, kv, 0.7, HQ)
    rows = slice(kp, kp + k)
    assert np.array_equal(out[rows], out2[rows]) and np.array_equal(lse[rows], lse2[rows])
    assert np.array_equal(sels[0], sels2[0][:T])


def brute(layout, W, T, kp, r, cache, q, kv, child_rows, parent_start, scale):
    """Explicit loops: row i of the child sees positions 0..T-1 (plane by the
    window of the last W positions of T + kp), the parent rows, and child rows
    0..i."""
    out = np.zeros((len(child_rows), HQ, D))
    lse = np.zeros((len(child_rows), HQ))
    G = HQ // HKV
    Tp = T + kp
    for ii, row in enumerate(child_rows):
        for h in range(HQ):
            hk = h // G
            keys, vals = [], []
            for j in range(Tp):
                if layout == "full":
                    d = r
                elif layout == "deepest":
                    d = R
                else:
                    d = r if j >= Tp - W else R
                if j < T:
                    K, V = cache.get(0, d, j, j + 1)
                    keys.append(K[0, hk]); vals.append(V[0, hk])
                else:
                    keys.append(kv[0, d - 1, parent_start + j - T, hk]); vals.append(kv[1, d - 1, parent_start + j - T, hk])
            for i2 in range(ii + 1):
                keys.append(kv[0, r - 1, child_rows[i2], hk]); vals.append(kv[1, r - 1, child_rows[i2], hk])
            sc = [scale * float(np.dot(q[row, h], kk)) for kk in keys]
            wts = [math.exp(x) for x in sc]
            tot = sum(wts)
            out[ii, h] = sum(w * v for w, v in zip(wts, vals)) / tot
            lse[ii, h] = math.log(tot)
    return out, lse


@pytest.mark.parametrize("layout", ["full", "deepest", "ripe"])
@pytest.mark.parametrize("W,kp,T", [(3, 2, 6), (8, 5, 4), (2, 6, 9), (0, 3, 5)])
def test_inflight_brute_force(layout, W, kp, T):
    k, r = 2, 3
    c = make_cache(layout, W, T, seed=99 + T + kp)
    q, kv = inputs(5 + kp, kp + k + 2)
    ps = 2  # parent rows after two unrelated rows
    child = Group(0, r, ps + kp, k, parent_row_start=ps, parent_rows=kp)
    out, lse, _ = ro.verify(c, [child], q, kv, 0.5, HQ)
    rows = list(range(ps + kp, ps + kp + k))
    bo, bl = brute(layout, W, T, kp, r, c, q, kv, rows, ps, 0.5)
    assert np.allclose(out[rows], bo, atol=1e-12) and np.allclose(lse[rows], bl, atol=1e-12)


@pytest.mark.parametrize("kp,T", [(2, 7), (5, 3), (9, 12)])
def test_inflight_ripe_identities(kp, T):
    k = 3
    q, kv = inputs(kp * 10 + T, kp + 2 * k)
    groups = [Group(0, 2, kp, k, 0, kp), Group(0, 4, kp + k, k, 0, kp)]  # siblings at depths 2 and R
    res = {}
    for layout, W in (("full", 0), ("deepest", 0), ("ripe", T + kp), ("ripe", 0)):
        c = make_cache(layout, W, T, seed=5)
        res[(layout, W)] = ro.verify(c, groups, q, kv, 0.6, HQ)
    for a, b in ((("ripe", T + kp), ("full", 0)), (("ripe", 0), ("deepest", 0))):
        assert np.array_equal(res[a][0][kp:], res[b][0][kp:]) and np.array_equal(res[a][1][kp:], res[b][1][kp:])


def test_inflight_group_independent_of_batch():
    B, W, kp, k = 3, 6, 4, 3
    c = make_cache("ripe", W, [10, 4, 0], seed=7, B=B)
    q, kv = inputs(77, B * (kp + k))
    groups = [Group(b, 2 + b % 2, b * (kp + k) + kp, k, b * (kp + k), kp) for b in range(B)]
    out, lse, _ = ro.verify(c, groups, q, kv, 0.8, HQ)
    for g in groups:
        o1, l1, _ = ro.verify(c, [g], q, kv, 0.8, HQ)
        rows = slice(g.row_start, g.row_start + g.n_rows)
        assert np.array_equal(o1[rows], out[rows]) and np.array_equal(l1[rows], lse[rows])


def test_mutation_window_anchored_at_committed_length_fails(monkeypatch):
    real = ro.plane_select
    monkeypatch.setattr(ro, "plane_select", lambda layout, R_, W, T, r, parent_rows=0: real(layout, R_, W, T, r))
    with pytest.raises(AssertionError):
        test_inflight_equals_commit_then_verify("ripe", 8, 3, 20)
