"""Pins of the float64 oracle against facts fixed outside the oracle itself.

* hand-derived closed-form cases (tests/golden/closed_form_cases.json);
* brute force with explicit loops, no max subtraction, planes read straight
  from the seeded generator with the window written as "the W most recent
  positions";
* a library attention routine (torch float64 scaled_dot_product_attention)
  where the full and one-plane layouts reduce to plain causal attention;
* invariants the RIPE read rule implies: W >= T equals the full cache, W = 0
  equals the deepest plane alone, at depth R all three layouts agree, and a
  group's result does not depend on what it is batched with;
* mutation checks: plausible mistakes planted in the oracle (on the CPU) make
  at least one pin fail.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import ripe_oracle as ro
from workloads import Group, PlaneModel, make_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")
LAYOUTS = ("full", "deepest", "ripe")


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def build_golden(case, layout):
    R, W, T, Hkv, D = case["R"], case["W"], case["T"], case["Hkv"], case["D"]
    cache = ro.LogicalCache(layout, "f64", R, W, 1, T + 2, Hkv, D)

    def plane_values(kind, b, p, j0, j1):
        arr = np.array(case["planes"]["KV"[kind]][str(p)], dtype=np.float64)
        return arr[j0:j1].reshape(j1 - j0, Hkv, D)

    ro.fill_prefix(cache, 0, T, plane_values)
    k = case["group"][3]
    q = np.array(case["q"], dtype=np.float64).reshape(k, case["Hq"], D)
    kv_new = np.zeros((2, R, k, Hkv, D))
    for kind, name in enumerate("KV"):
        for p in range(1, R + 1):
            kv_new[kind, p - 1] = np.array(case["kv_new"][name][str(p)]).reshape(k, Hkv, D)
    return cache, q, kv_new


def check_golden():
    for case in golden()["cases"]:
        k, Hq, D = case["group"][3], case["Hq"], case["D"]
        for layout in LAYOUTS:
            cache, q, kv_new = build_golden(case, layout)
            out, lse, sels = ro.verify(cache, [tuple(case["group"])], q, kv_new, case["scale"], Hq)
            exp = case["expect"][layout]
            np.testing.assert_allclose(out, np.array(exp["out"]).reshape(k, Hq, D), rtol=0,
                                       atol=1e-12, err_msg=f"{case['name']} {layout}")
            np.testing.assert_allclose(lse, np.array(exp["lse"]).reshape(k, Hq), rtol=0,
                                       atol=1e-12, err_msg=f"{case['name']} {layout}")
            assert sels[0].tolist() == exp["plane_sel"], (case["name"], layout)


def tiny_planes(seed, R, Hkv, D):
    return PlaneModel(seed, R, Hkv, D, 0.88, "f32")


def brute_force_group(planes, layout, R, W, T, g, q, kv_new, scale, Hq, Hkv):
    """Explicit loops, exp without max subtraction, planes straight from the
    generator.  The RIPE window is 'the W most recent positions'."""
    b, r, s, k = g
    G = Hq // Hkv
    recent = set(list(range(T))[-W:]) if W > 0 else set()
    out = np.zeros((k, Hq, q.shape[2]))
    lse = np.zeros((k, Hq))
    for i in range(k):
        for h in range(Hq):
            hk = h // G
            terms = []  # (score, value vector)
            for j in range(T):
                if layout == "full":
                    p = r
                elif layout == "deepest":
                    p = R
                else:
                    p = r if j in recent else R
                kvec = planes.values(0, b, p, j, j + 1)[0, hk]
                vvec = planes.values(1, b, p, j, j + 1)[0, hk]
                terms.append((scale * sum(q[s + i, h, d] * kvec[d] for d in range(len(kvec))), vvec))
            for i2 in range(i + 1):
                kvec = kv_new[0, r - 1, s + i2, hk]
                vvec = kv_new[1, r - 1, s + i2, hk]
                terms.append((scale * sum(q[s + i, h, d] * kvec[d] for d in range(len(kvec))), vvec))
            wsum = sum(math.exp(sc) for sc, _ in terms)
            acc = sum(math.exp(sc) * v for sc, v in terms)
            out[i, h] = acc / wsum
            lse[i, h] = math.log(wsum)
    return out, lse


def tiny_setup(seed, layout, W, lengths, groups, R=3, Hkv=2, Hq=4, D=3, scale=0.7):
    planes = tiny_planes(seed, R, Hkv, D)
    B = len(lengths)
    t_max = max(lengths) + 8
    cache = ro.LogicalCache(layout, "f32", R, W, B, t_max, Hkv, D)
    for b, T in enumerate(lengths):
        ro.fill_prefix(cache, b, T, planes.values)
    n_rows = max(g[2] + g[3] for g in groups)
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n_rows, Hq, D))
    kv_new = rng.standard_normal((2, R, n_rows, Hkv, D))
    return planes, cache, q, kv_new, scale


TINY_GROUPS = [(0, 1, 0, 2), (1, 3, 2, 3), (1, 2, 5, 1), (2, 2, 6, 2)]
TINY_LENGTHS = [5, 0, 7]


def check_bruteforce(layout, W, seed=5):
    planes, cache, q, kv_new, scale = tiny_setup(seed, layout, W, TINY_LENGTHS, TINY_GROUPS)
    out, lse, sels = ro.verify(cache, TINY_GROUPS, q, kv_new, scale, 4)
    for g in TINY_GROUPS:
        b, r, s, k = g
        bo, bl = brute_force_group(planes, layout, 3, W, TINY_LENGTHS[b], g, q, kv_new, scale, 4, 2)
        np.testing.assert_allclose(out[s:s + k], bo, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[s:s + k], bl, rtol=1e-12, atol=1e-12)


def check_torch_sdpa(layout, seed=11):
    """FULL / DEEPEST read one plane everywhere, so one group is plain
    attention over [that plane's prefix; the block's own rows] with an offset
    causal mask."""
    R, Hkv, Hq, D, T, k, r = 4, 2, 4, 16, 37, 5, 2
    planes = PlaneModel(seed, R, Hkv, D, 0.88, "f32")
    cache = ro.LogicalCache(layout, "f32", R, 0, 1, 64, Hkv, D)
    ro.fill_prefix(cache, 0, T, planes.values)
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((k, Hq, D))
    kv_new = rng.standard_normal((2, R, k, Hkv, D))
    scale = 0.3
    out, lse, _ = ro.verify(cache, [(0, r, 0, k)], q, kv_new, scale, Hq)
    p = r if layout == "full" else R
    K = np.concatenate([planes.values(0, 0, p, 0, T), kv_new[0, r - 1]], axis=0)  # [T+k, Hkv, D]
    V = np.concatenate([planes.values(1, 0, p, 0, T), kv_new[1, r - 1]], axis=0)
    G = Hq // Hkv
    Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0)  # [Hq, T+k, D]
    Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0)
    Qt = torch.from_numpy(q).permute(1, 0, 2)  # [Hq, k, D]
    mask = torch.ones(k, T + k, dtype=torch.bool)
    mask[:, T:] = torch.tril(torch.ones(k, k, dtype=torch.bool))
    ref = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, attn_mask=mask, scale=scale)
    scores = scale * Qt @ Kt.transpose(1, 2)
    ref_lse = torch.logsumexp(scores.masked_fill(~mask, -math.inf), dim=-1)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse.T.numpy(), rtol=0, atol=1e-12)


def verify_case(case, layout, W, groups):
    cache = ro.LogicalCache(layout, case.dtype, case.R, W, case.B, case.t_max, case.Hkv, case.D)
    for b in range(case.B):
        ro.fill_prefix(cache, b, int(case.seq_len[b]), case.planes.values)
    return ro.verify(cache, groups, case.q, case.kv_new, case.scale, case.Hq)


def small_c3():
    return make_case("c3", B=3, T_range=(40, 90), R=6, Hkv=2, Hq=8, D=16, W=8)


def check_invariants():
    case = small_c3()
    T_max = int(case.seq_len.max())
    for r in (1, 3, case.R):
        groups = case.groups_at(r)
        full = verify_case(case, "full", case.W, groups)
        deep = verify_case(case, "deepest", case.W, groups)
        wide = verify_case(case, "ripe", T_max, groups)     # W >= T: the whole prefix keeps full depth
        zero = verify_case(case, "ripe", 0, groups)         # W = 0: only the deepest plane
        for a, b in ((wide, full), (zero, deep)):
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
            assert all(np.array_equal(x, y) for x, y in zip(a[2], b[2]))
        if r == case.R:
            ripe = verify_case(case, "ripe", case.W, groups)
            assert np.array_equal(ripe[0], full[0]) and np.array_equal(ripe[0], deep[0])


def check_window_count():
    for T in (0, 1, 7, 64, 100):
        for W in (0, 1, 8, 64, 200):
            for r in (1, 5):
                sel = ro.plane_select("ripe", 8, W, T, r)
                at_r = np.nonzero(sel == r)[0]
                assert len(at_r) == min(W, T)
                assert sorted(at_r.tolist()) == list(range(T))[len(range(T)) - min(W, T):]
                assert np.all(sel[sel != r] == 8)


# ---------------------------------------------------------------------------
# the pins
# ---------------------------------------------------------------------------
def test_golden_closed_forms():
    check_golden()


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("W", [0, 1, 2, 5, 9])
def test_bruteforce_tiny(layout, W):
    check_bruteforce(layout, W)


@pytest.mark.parametrize("layout", ["full", "deepest"])
def test_library_attention_special_case(layout):
    check_torch_sdpa(layout)


def test_layout_invariants():
    check_invariants()


def test_window_positions():
    check_window_count()


@pytest.mark.parametrize("W", [1, 3, 4, 5, 8, 12, 40, 100])
def test_batched_equals_alone(W):
    case = small_c3()
    groups = case.groups_at(2)
    out, lse, sels = verify_case(case, "ripe", W, groups)
    for g, sel in zip(groups, sels):
        o1, l1, s1 = verify_case(case, "ripe", W, [g])
        rows = slice(g.row_start, g.row_start + g.n_rows)
        assert np.array_equal(out[rows], o1[rows]) and np.array_equal(lse[rows], l1[rows])
        assert np.array_equal(sel, s1[0])


@pytest.mark.parametrize("W", [4, 64])
def test_mixed_depth_branches_are_siblings(W):
    """Two branches of one sequence at different depths in one call give what
    each gives alone (LoopSpec: branches at different depths, one batched
    call); W = 4 is the branches' own length k."""
    case = make_case("c4", B=3, T_range=(50, 70), R=20, Hkv=2, Hq=4, D=8)
    groups = case.groups()
    assert all(g.n_rows == 4 for g in groups)
    out, lse, _ = verify_case(case, "ripe", W, groups)
    for g in groups:
        o1, l1, _ = verify_case(case, "ripe", W, [g])
        rows = slice(g.row_start, g.row_start + g.n_rows)
        assert np.array_equal(out[rows], o1[rows]) and np.array_equal(lse[rows], l1[rows])


def test_ripe_reads_only_what_ripe_keeps():
    """The read rule and the storage rule agree: a RIPE cache never holds
    plane r < R outside the window, and verification never asks for it."""
    case = small_c3()
    cache = ro.LogicalCache("ripe", case.dtype, case.R, case.W, case.B, case.t_max, case.Hkv,
                            case.D)
    for b in range(case.B):
        ro.fill_prefix(cache, b, int(case.seq_len[b]), case.planes.values)
        T = int(case.seq_len[b])
        for p in range(1, case.R):
            assert cache.held_positions(b, p) == list(range(max(0, T - case.W), T))
    ro.verify(cache, case.groups_at(1), case.q, case.kv_new, case.scale, case.Hq)
    with pytest.raises(KeyError):
        cache.get(0, 1, 0, 1)


def test_memory_model():
    mem = golden()["memory"]
    R, W, T = mem["R"], mem["W"], mem["T"]
    ripe = ro.memory_positions("ripe", R, W, T)
    full = ro.memory_positions("full", R, W, T)
    deep = ro.memory_positions("deepest", R, W, T)
    assert (ripe, full, deep) == (mem["ripe_positions"], mem["full_positions"],
                                  mem["deepest_positions"])
    assert ripe / full == mem["ratio_recurrent_only"]
    ratio = (ripe + deep) / (full + deep)
    assert ratio == pytest.approx(mem["ratio_with_equal_single_plane_layers"], abs=1e-15)
    assert round(ratio, 3) == mem["page_value"]
    # W = 0 is one shared plane; W >= T is the full cache
    assert ro.memory_positions("ripe", R, 0, T) == deep
    assert ro.memory_positions("ripe", R, 5000, T) == full


# ---------------------------------------------------------------------------
# planted mistakes must fail a pin
# ---------------------------------------------------------------------------
def _plane_select_off_by_one(layout, R, W, T, r, parent_rows=0):
    layout = ro.layout_code(layout)
    out = np.empty(T, dtype=np.int8)
    for j in range(T):
        out[j] = r if layout == ro.FULL else (R if layout == ro.DEEPEST else
                                              (r if j > T + parent_rows - W else R))
    return out


def _attend_lse_without_max(q, keys, vals, visible, scale):
    s = np.where(visible, scale * (q @ keys.T), -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return (e @ vals) / l, np.log(l)[:, 0]


MUTANTS = {
    "window_off_by_one": ("plane_select", _plane_select_off_by_one),
    "draft_rows_from_deepest": ("draft_rows", lambda kv, r, s, k: (kv[0, -1, s:s + k],
                                                                  kv[1, -1, s:s + k])),
    "no_causal_mask": ("visibility", lambda T, k: np.ones((k, T + k), dtype=bool)),
    "gqa_modulo": ("kv_head", lambda h, G: h % 2),
    "lse_without_max": ("attend", _attend_lse_without_max),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ro, attr, fn)
    failures = 0
    for check in (check_golden, lambda: check_bruteforce("ripe", 2),
                  lambda: check_torch_sdpa("full"), check_window_count):
        try:
            check()
        except (AssertionError, KeyError, IndexError):
            failures += 1
    assert failures > 0, f"mutant {name} survived every pin"
