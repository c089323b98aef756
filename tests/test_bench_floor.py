"""Host-side checks of bench.py's read-floor pieces: they cover exactly the
positions one RIPE verify call reads from the deep plane and the window, and
sit in the grid as the planner places a call's items (a unit's pieces on grid
positions equal mod 8, one XCD)."""
import numpy as np
import pytest

import bench
from workloads import make_case


@pytest.mark.parametrize("name", ["c3", "c4"])
def test_floor_pieces_cover_each_sequence_once(name):
    case = make_case(name)
    t_max = int(-(-(int(case.seq_len.max()) + 64 + case.n_rows) // 32) * 32)
    S = bench.default_split(case.B, case.Hkv, t_max)
    grid = bench.floor_pieces(case.seq_len, case.W, case.B, case.Hkv, S)
    live = grid[grid[:, 3] > 0]
    assert np.all(live[:, 2] + live[:, 3] <= t_max)
    for b in range(case.B):
        T = int(case.seq_len[b])
        for h in range(case.Hkv):
            rows = live[(live[:, 0] == b) & (live[:, 1] == h)]
            rows = rows[np.argsort(rows[:, 2])]
            ends = rows[:, 2] + rows[:, 3]
            assert rows[0, 2] == 0 and ends[-1] == T and np.all(rows[1:, 2] == ends[:-1])
            assert np.all(rows[:-1, 3] <= S) and np.all(rows[:-1, 2] % 32 == 0)
    # every unit's pieces on one XCD (grid position mod 8)
    pos = np.nonzero(grid[:, 3] > 0)[0]
    xcd = {}
    for p in pos:
        key = (int(grid[p, 0]), int(grid[p, 1]))
        assert xcd.setdefault(key, p % 8) == p % 8


def test_default_split_matches_the_library_rule():
    # the library's rule (see csrc/api.hip split_len) at the workloads' shapes
    assert bench.default_split(16, 8, 4064) == 1024
    assert bench.default_split(1, 40, 1088) == 256
    assert bench.default_split(4, 8, 8288) == 608
    assert bench.default_split(64, 8, 8288) == 8192
