"""Summary of the per-position substitution error that ripe_position_error
returns (host-side reporting over the kernel's output).

The RIPE abstract (zhuanzhiai.com paper page) states two figures for one
model: 1% of positions carry most of the error of storing only the deepest
plane, and a 64-position window at full depth removes most of those tail
positions.  tail_statistics gives the same two quantities for one group's
error row; on synthetic inputs they describe the inputs, not the model.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np


def tail_statistics(err, T: int, W: int, cond=None, tail_frac: float = 0.01) -> Dict[str, Optional[float]]:
    """err, cond: one group's rows of ripe_position_error's outputs (host
    arrays, at least T entries); T: its prefix length; W: a RIPE window.

    * tail_positions: floor(tail_frac * T), at least 1 (0 if T = 0);
    * tail_share: the share of sum_j e_j carried by the tail_positions
      largest e_j (ties to the lower position);
    * tail_in_window: the fraction of those positions that fall in the last W
      positions, where RIPE keeps every plane;
    * window_share: the share of sum_j e_j carried by the last W positions
      (the first-order share of the DEEPEST error a RIPE window removes);
    * ill_conditioned: positions with cond > 1 (their e_j is an fp32
      estimate; None without cond) and ill_conditioned_share their share of
      sum_j e_j.
    Shares are None when sum_j e_j is 0."""
    e = np.asarray(err, dtype=np.float64)[:T]
    n_tail = 0 if T == 0 else max(1, int(math.floor(tail_frac * T)))
    top = np.argsort(-e, kind="stable")[:n_tail]
    total = float(e.sum())
    w0 = max(0, T - W)
    share = (lambda x: float(x) / total) if total > 0 else (lambda x: None)
    res = {
        "positions": int(T),
        "tail_positions": n_tail,
        "tail_share": share(e[top].sum()),
        "tail_in_window": float(np.mean(top >= w0)) if n_tail else None,
        "window_share": share(e[w0:].sum()),
        "ill_conditioned": None,
        "ill_conditioned_share": None,
    }
    if cond is not None:
        ill = np.asarray(cond, dtype=np.float64)[:T] > 1.0
        res["ill_conditioned"] = int(ill.sum())
        res["ill_conditioned_share"] = share(e[ill].sum())
    return res
