"""GPU parity at the planner's limits, against the float64 oracle: a
sequence of 60-70 thousand positions (about 100 pieces per KV head, merged
by the merge kernel), more groups than one launch carries (128), and more
work items than one launch carries (2048), which cuts a call into several
launches inside a sequence's KV heads.  Tolerances as in test_gpu_parity:
plane_sel exact, out within 2e-2 (bf16), lse within 1e-3."""
import pytest

from workloads import Group, make_case

from test_gpu_parity import run_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("layout", ["ripe", "deepest"])
def test_long_sequences(layout):
    case = make_case("c3", layout=layout, B=2, T_range=(60000, 70000), R=4, Hkv=2, Hq=8, D=64, k=8)
    run_case(case, layout, case.groups_at(2), tag="T ~ 65K")


def test_more_groups_than_one_launch():
    # 20 sequences with eight 2-row groups each (depths 1, 2, 3 in turn):
    # 160 groups in one call, so the cut is by groups, not by sequences
    case = make_case("c3", B=20, T_range=(20, 90), R=3, Hkv=2, Hq=4, D=64, k=16)
    groups = []
    for b in range(case.B):
        s, _ = case.blocks[b]
        groups += [Group(b, 1 + j % 3, s + 2 * j, 2) for j in range(8)]
    run_case(case, "ripe", groups, tag="160 groups")


@pytest.mark.parametrize("split_len", [256, 512])
def test_more_items_than_one_launch(split_len):
    # 64 sequences x 8 KV heads x 5-10 pieces: 2.5-5 thousand items
    case = make_case("c3", B=64, T_range=(2000, 2400), R=3, Hkv=8, Hq=8, D=64, k=4)
    run_case(case, "ripe", case.groups_at(2), split_len=split_len, tag=f"items, split {split_len}")
