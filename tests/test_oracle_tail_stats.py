"""Pins of the oracle's tail figures of an error row (oracle/side_stats.py
tail_statistics): hand-worked arrays, and a brute-force check of the tail
selection (every subset of a small row)."""
import itertools

import numpy as np

from oracle.side_stats import tail_statistics


def test_hand_worked_row():
    # 200 positions: two large errors (at 10 and 190), the rest 1.0
    e = np.ones(200)
    e[10], e[190] = 99.0, 101.0
    s = tail_statistics(e, 200, 20)
    assert s["tail_positions"] == 2
    assert np.isclose(s["tail_share"], 200.0 / 398.0)
    assert s["tail_in_window"] == 0.5                 # 190 is in [180, 200), 10 is not
    assert np.isclose(s["window_share"], (19 + 101) / 398.0)
    assert s["ill_conditioned"] is None


def test_condition_counts_and_padding_ignored():
    e = np.array([4.0, 1.0, 3.0, 2.0, 77.0, 77.0])    # entries past T are ignored
    cond = np.array([0.2, 3.0, 0.5, 1.5, 9.0, 9.0])
    s = tail_statistics(e, 4, 1, cond=cond, tail_frac=0.5)
    assert s["tail_positions"] == 2 and np.isclose(s["tail_share"], 0.7)
    assert s["tail_in_window"] == 0.0                 # positions 0 and 2; the window is {3}
    assert s["ill_conditioned"] == 2 and np.isclose(s["ill_conditioned_share"], 0.3)


def test_ties_and_degenerate_rows():
    s = tail_statistics(np.full(150, 2.0), 150, 50)
    assert s["tail_positions"] == 1 and s["tail_in_window"] == 0.0   # the lowest of equal values
    z = tail_statistics(np.zeros(64), 64, 8)
    assert z["tail_share"] is None and z["window_share"] is None
    empty = tail_statistics(np.zeros(0), 0, 8)
    assert empty["tail_positions"] == 0 and empty["tail_in_window"] is None


def test_tail_is_the_best_subset_brute_force():
    """The tail of n positions carries the largest sum any n positions can,
    and among subsets with that sum it is the lexicographically lowest one
    (ties to the lower position): checked against every subset."""
    rng = np.random.default_rng(7)
    for trial in range(40):
        T = int(rng.integers(1, 9))
        e = rng.integers(0, 4, size=T).astype(np.float64)  # many ties
        frac = float(rng.choice([0.01, 0.3, 0.5, 1.0]))
        W = int(rng.integers(0, T + 1))
        n = max(1, int(np.floor(frac * T)))
        best = max(itertools.combinations(range(T), n), key=lambda c: (e[list(c)].sum(), [-j for j in c]))
        s = tail_statistics(e, T, W, tail_frac=frac)
        assert s["tail_positions"] == n
        total = e.sum()
        if total > 0:
            assert np.isclose(s["tail_share"], e[list(best)].sum() / total)
        w0 = max(0, T - W)
        assert s["tail_in_window"] == np.mean([j >= w0 for j in best])
