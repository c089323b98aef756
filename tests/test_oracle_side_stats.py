"""Pins of the per-position substitution error (oracle/side_stats.py).

* the definition (one attention per substituted position) and the rank-one
  form agree to rounding over head groupings, several groups, depths and
  prefix lengths (including 0 and 1);
* depth r = R substitutes a plane by itself: the error is exactly zero;
* closed form, derived by hand: with q = 0 every visible key has the same
  weight, so row i (which sees T + i + 1 keys) changes by
  (v_R[j] - v_r[j]) / (T + i + 1) when position j is substituted;
* tie to the verify oracle: when planes r and R differ at one position j0
  only, the DEEPEST output is exactly the FULL output with j0 substituted, so
  e_j0 equals the squared distance of the two verify outputs and every other
  e_j is zero;
* planted mistakes (the weights' difference with the wrong sign, the
  substituted plane taken as plane 1, the group's own rows counted as
  prefix) fail one of the pins.
"""
import numpy as np
import pytest

from oracle import ripe_oracle as ro
from oracle import side_stats as ss
from workloads import Group


def full_cache(R, B, T, Hkv, D, seed, t_max=64, planes=None):
    """FULL cache with random planes (or planes[kind, b, p-1, j, h, d])."""
    rng = np.random.default_rng(seed)
    if planes is None:
        planes = rng.standard_normal((2, B, R, t_max, Hkv, D))
    c = ro.LogicalCache("full", "f32", R, 0, B, t_max, Hkv, D)
    Ts = [T] * B if np.isscalar(T) else list(T)
    for b in range(B):
        ro.fill_prefix(c, b, Ts[b], lambda kind, bb, p, j0, j1: planes[kind, bb, p - 1, j0:j1])
    return c, planes


def inputs(seed, n_rows, Hq, D, R, Hkv):
    rng = np.random.default_rng(seed + 7)
    return 0.5 * rng.standard_normal((n_rows, Hq, D)), rng.standard_normal((2, R, n_rows, Hkv, D))


@pytest.mark.parametrize("Hkv,Hq", [(2, 2), (2, 6), (1, 4)])
@pytest.mark.parametrize("T", [[0, 9], [1, 14], [23, 5]])
def test_definition_equals_rank1(Hkv, Hq, T):
    R, D, k = 5, 8, 3
    c, _ = full_cache(R, 2, T, Hkv, D, seed=sum(T) + Hq)
    q, kv = inputs(sum(T), 4 * k, Hq, D, R, Hkv)
    groups = [Group(0, 2, 0, k), Group(1, 4, k, k), Group(0, 1, 2 * k, 2), Group(1, 5, 3 * k, k)]
    brute = ss.position_error(c, groups, q, kv, 0.9, Hq)
    fast = ss.position_error_rank1(c, groups, q, kv, 0.9, Hq)
    for g, x, y in zip(groups, brute, fast):
        assert x.shape == (T[g.seq],) and y.shape == x.shape
        assert np.allclose(x, y, rtol=1e-10, atol=1e-14), (g, np.abs(x - y).max())
        if g.depth == R:
            assert np.all(x == 0.0) and np.all(y == 0.0)
        elif x.size:
            assert x.min() > 0.0


def test_closed_form_uniform_weights():
    R, D, Hkv, Hq, k, T = 4, 3, 1, 2, 3, 6
    c, planes = full_cache(R, 1, T, Hkv, D, seed=3)
    q = np.zeros((k, Hq, D))
    _, kv = inputs(1, k, Hq, D, R, Hkv)
    r = 2
    g = Group(0, r, 0, k)
    want = np.zeros(T)
    for j in range(T):
        dv = planes[1, 0, R - 1, j, 0] - planes[1, 0, r - 1, j, 0]
        for i in range(k):
            want[j] += Hq * float((dv ** 2).sum()) / (T + i + 1) ** 2
    for fn in (ss.position_error, ss.position_error_rank1):
        got = fn(c, [g], q, kv, 1.3, Hq)[0]
        assert np.allclose(got, want, rtol=1e-12, atol=0), fn.__name__


@pytest.mark.parametrize("j0", [0, 4, 10])
def test_single_differing_position_equals_deepest(j0):
    R, D, Hkv, Hq, k, T, r = 4, 8, 2, 4, 3, 11, 2
    rng = np.random.default_rng(j0)
    planes = np.repeat(rng.standard_normal((2, 1, 1, 64, Hkv, D)), R, axis=2)
    planes[:, 0, r - 1, j0] += 0.7 * rng.standard_normal((2, Hkv, D))  # plane r differs at j0 only
    c, _ = full_cache(R, 1, T, Hkv, D, seed=0, planes=planes)
    deep = ro.LogicalCache("deepest", "f32", R, 0, 1, 64, Hkv, D)
    ro.fill_prefix(deep, 0, T, lambda kind, bb, p, a, b_: planes[kind, bb, p - 1, a:b_])
    q, kv = inputs(5, k, Hq, D, R, Hkv)
    g = Group(0, r, 0, k)
    o_full, _, _ = ro.verify(c, [g], q, kv, 1.0, Hq)
    o_deep, _, _ = ro.verify(deep, [g], q, kv, 1.0, Hq)
    total = float(((o_deep - o_full) ** 2).sum())
    assert total > 1e-6
    for fn in (ss.position_error, ss.position_error_rank1):
        e = fn(c, [g], q, kv, 1.0, Hq)[0]
        assert np.isclose(e[j0], total, rtol=1e-10, atol=0), fn.__name__
        assert np.all(np.delete(e, j0) < 1e-25), fn.__name__


def test_rejects_non_full_cache():
    c = ro.LogicalCache("ripe", "f32", 4, 8, 1, 64, 1, 8)
    with pytest.raises(ValueError):
        ss.position_error_rank1(c, [Group(0, 1, 0, 1)], np.zeros((1, 1, 8)), np.zeros((2, 4, 1, 1, 8)), 1.0, 1)


# --- planted mistakes -------------------------------------------------------

def _rank1_wrong_sign(cache, groups, q, kv_new, scale, n_q_heads):
    """Copy of the rank-one form with the weights' difference negated."""
    G = n_q_heads // cache.Hkv
    out, lse, _ = ro.verify(cache, groups, q, kv_new, scale, n_q_heads)
    res = []
    for g in groups:
        b, r, s, k = ro._group_fields(g)
        T = int(cache.seq_len[b])
        Kr, Vr = cache.get(b, r, 0, T)
        KR, VR = cache.get(b, cache.R, 0, T)
        e = np.zeros(T)
        for h in range(n_q_heads):
            hk = h // G
            L = lse[s:s + k, h][:, None]
            a = np.exp(scale * (q[s:s + k, h] @ Kr[:, hk].T) - L)
            cc = np.exp(scale * (q[s:s + k, h] @ KR[:, hk].T) - L)
            num = a[:, :, None] * (VR[:, hk] - Vr[:, hk])[None] + (a - cc)[:, :, None] * (
                VR[None, :, hk] - out[s:s + k, h][:, None, :])
            e += ((num / (1.0 + cc - a)[:, :, None]) ** 2).sum(axis=(0, 2))
        res.append(e)
    return res


def test_mutation_wrong_sign_fails():
    with pytest.raises(AssertionError):
        orig = ss.position_error_rank1
        try:
            ss.position_error_rank1 = _rank1_wrong_sign
            test_definition_equals_rank1(2, 6, [23, 5])
        finally:
            ss.position_error_rank1 = orig


def test_mutation_plane_one_fails(monkeypatch):
    real_get = ro.LogicalCache.get

    def get_plane1_for_R(self, b, p, j0, j1):  # the "deepest" plane taken as plane 1
        return real_get(self, b, 1 if p == self.R else p, j0, j1)

    monkeypatch.setattr(ro.LogicalCache, "get", get_plane1_for_R)
    with pytest.raises(AssertionError):
        test_closed_form_uniform_weights()


def test_mutation_own_rows_in_prefix_fails(monkeypatch):
    # visibility that lets every row see all of the group's rows (no causal
    # mask) changes the row counts of the closed form
    monkeypatch.setattr(ro, "visibility", lambda T, k: np.ones((k, T + k), dtype=bool))
    with pytest.raises(AssertionError):
        test_closed_form_uniform_weights()
