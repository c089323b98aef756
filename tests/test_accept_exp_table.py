"""The table-driven e^x of the accept row statistics (accept.hip, exp_tab):
its constants and its accuracy, read from the kernel source and checked on
the CPU.  The constants are pinned to their definitions (ln 2 and 256 / ln 2,
computed here to 50 digits), and the algorithm (the two-step reduction, the
table of 2^(j/256), the degree-4 Taylor polynomial, the scaling by 2^n) is
replayed in float64 against a 50-digit e^x over the range the kernel uses
(x <= 0, down to the subnormals)."""
import math
import os
import re
from decimal import Decimal, getcontext

import numpy as np

SRC = os.path.join(os.path.dirname(__file__), "..", "self_speculative_verify_ripe_amd", "csrc", "accept.hip")
getcontext().prec = 50


def constants():
    s = open(SRC).read()

    def scalar(name):
        tok = re.search(r"constexpr (?:double|int) %s = ([^;]+);" % name, s).group(1).strip()
        return float.fromhex(tok) if tok.startswith("0x") else float(tok)

    return scalar("kLn2Head"), scalar("kLn2Rest"), scalar("kTableScale"), int(scalar("kExpTable"))


def test_constants_match_their_definitions():
    head, rest, scale, size = constants()
    ln2 = Decimal(2).ln()
    assert size == 256
    mant, _ = math.frexp(head)
    assert float(mant * 2 ** 32).is_integer()  # 32 significant bits: N * head / 256 is exact
    assert abs(Decimal(head) + Decimal(rest) - ln2) < Decimal("1.5e-26")  # half a unit of rest
    assert rest == float(ln2 - Decimal(head))
    assert scale == float(Decimal(size) / ln2)


def exp_tab(x, head, rest, scale, size):
    """The kernel's steps in float64 (separate multiplies and adds where the
    kernel fuses them, which only adds rounding)."""
    x = np.asarray(x, dtype=np.float64)
    table = np.exp2(np.arange(size) / size)
    nd = np.rint(np.where(np.isfinite(x), x, 0.0) * scale)
    n = nd.astype(np.int64)
    r = (x - nd * (head / size)) - nd * (rest / size)
    e = (((r * (1.0 / 24.0) + 1.0 / 6.0) * r + 0.5) * r + 1.0) * r + 1.0
    out = np.ldexp(table[n & (size - 1)] * e, n >> 8)
    return np.where(x >= -746.0, out, 0.0)


def test_accuracy_over_the_range():
    c = constants()
    rng = np.random.default_rng(12)
    xs = np.concatenate([-rng.random(20000) * 40.0, -rng.random(5000) * 708.0, -np.linspace(0, 2, 2001),
                         np.array([-1e-300, -0.00135, -0.0013538, -700.0, -708.3])])
    got = exp_tab(xs, *c)
    worst = 0.0
    for x, g in zip(xs[::5], got[::5]):
        ref = Decimal(float(x)).exp()
        worst = max(worst, float(abs(Decimal(float(g)) - ref) / ref))
    assert worst < 5e-16, worst
    assert exp_tab(np.array([0.0]), *c)[0] == 1.0  # a row's max contributes exactly 1


def test_subnormal_range_and_special_values():
    c = constants()
    xs = np.array([-710.0, -720.0, -740.0, -744.4, -745.1, -745.2, -746.5, -1000.0, -np.inf])
    got = exp_tab(xs, *c)
    ref = np.exp(xs)
    assert np.all(np.abs(got - ref) <= 2 * 5e-324), (got, ref)
    assert got[-1] == 0.0 and got[-2] == 0.0
