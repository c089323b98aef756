"""Per-position plane-substitution error -- TEST INFRASTRUCTURE ONLY.

A plain float64 NumPy statement of the side statistic the GPU harness
computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the library never does,
and this module imports nothing from the library.

Source: RIPE abstract (zhuanzhiai.com paper page, abstract paragraph).
Whether the deepest plane alone is enough depends on how close the late
planes already are to it; on one of the two models a small set of positions
(1%) carries most of the error of storing only the deepest plane, and keeping
every plane for a short window of the newest positions removes most of those
tail positions.

Reading (the pages name the error without defining it): the error that
storing plane R instead of plane r at prefix position j introduces into the
depth-r verification output of a group is

    e_j = sum over the group's rows i and query heads h of
          || O^(j)[i, h] - O[i, h] ||^2,

where O is the output over the FULL cache (every prefix position read at
plane r, the group's own rows at depth r) and O^(j) the same output with
position j alone read at plane R.  The group's own rows are never
substituted.  ``position_error`` is that definition written out (one
attention per substituted position); ``position_error_rank1`` is the same
quantity from the softmax identity for a single changed term, in float64,
fast enough for full-size inputs.  The two are pinned against each other
and against closed forms in tests/test_oracle_side_stats.py.

``tail_statistics`` reads the abstract's two tail figures off one group's
error row (reading: the tail is the floor(1% T) largest e_j, ties to the
lower position; its share of sum_j e_j, and the fraction of its positions in
the last W), written out with a stable sort; it is pinned by hand-worked
rows in tests/test_oracle_tail_stats.py.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional

import numpy as np

from . import ripe_oracle as ro


def _check_full(cache: ro.LogicalCache) -> None:
    if cache.layout != ro.FULL:
        raise ValueError("the substitution error is defined on a FULL cache (every plane held)")


def position_error(cache: ro.LogicalCache, groups: Iterable, q: np.ndarray, kv_new: np.ndarray,
                   scale: float, n_q_heads: int) -> List[np.ndarray]:
    """e [T_b] per group, by definition: for every prefix position j, the
    attention recomputed with position j read at plane R instead of plane r.
    Cost O(T^2) per (group, head): small inputs only."""
    _check_full(cache)
    n_rows, Hq, D = q.shape
    G = n_q_heads // cache.Hkv
    R = cache.R
    res = []
    for g in groups:
        b, r, s, k = ro._group_fields(g)
        T = int(cache.seq_len[b])
        Kr, Vr = cache.get(b, r, 0, T)
        KR, VR = cache.get(b, R, 0, T)
        Kn, Vn = ro.draft_rows(kv_new, r, s, k)
        vis = ro.visibility(T, k)
        e = np.zeros(T)
        for h in range(Hq):
            hk = ro.kv_head(h, G)
            keys = np.concatenate([Kr[:, hk], Kn[:, hk]], axis=0)
            vals = np.concatenate([Vr[:, hk], Vn[:, hk]], axis=0)
            base, _ = ro.attend(q[s:s + k, h], keys, vals, vis, scale)
            for j in range(T):
                ks, vs = keys.copy(), vals.copy()
                ks[j], vs[j] = KR[j, hk], VR[j, hk]
                sub, _ = ro.attend(q[s:s + k, h], ks, vs, vis, scale)
                e[j] += float(((sub - base) ** 2).sum())
        res.append(e)
    return res


def position_error_rank1(cache: ro.LogicalCache, groups: Iterable, q: np.ndarray, kv_new: np.ndarray,
                         scale: float, n_q_heads: int) -> List[np.ndarray]:
    """e [T_b] per group from the single-term softmax identity.  With
    a = exp(scale q.k_r[j] - lse) and c = exp(scale q.k_R[j] - lse) (lse of the
    FULL output), replacing the term of position j gives

        O^(j) = (O - a v_r[j] + c v_R[j]) / (1 - a + c),

    so O^(j) - O = (a (v_R - v_r) + (c - a)(v_R - O)) / (1 + c - a)."""
    _check_full(cache)
    G = n_q_heads // cache.Hkv
    R = cache.R
    groups = list(groups)
    out, lse, _ = ro.verify(cache, groups, q, kv_new, scale, n_q_heads)
    res = []
    for g in groups:
        b, r, s, k = ro._group_fields(g)
        T = int(cache.seq_len[b])
        Kr, Vr = cache.get(b, r, 0, T)
        KR, VR = cache.get(b, R, 0, T)
        e = np.zeros(T)
        for h in range(n_q_heads):
            hk = ro.kv_head(h, G)
            Q = q[s:s + k, h]                      # [k, D]
            O = out[s:s + k, h]                    # [k, D]
            L = lse[s:s + k, h][:, None]           # [k, 1]
            a = np.exp(scale * (Q @ Kr[:, hk].T) - L)   # [k, T]
            c = np.exp(scale * (Q @ KR[:, hk].T) - L)
            dv = VR[:, hk] - Vr[:, hk]             # [T, D]
            # delta[i, j, :] = (a dv[j] + (c - a)(v_R[j] - O[i])) / (1 + c - a)
            num = a[:, :, None] * dv[None] + (c - a)[:, :, None] * (VR[None, :, hk] - O[:, None, :])
            delta = num / (1.0 + c - a)[:, :, None]
            e += (delta ** 2).sum(axis=(0, 2))
        res.append(e)
    return res


def tail_statistics(err, T: int, W: int, cond=None, tail_frac: float = 0.01) -> Dict[str, Optional[float]]:
    """One group's row: err (and cond) host arrays of at least T entries, T
    its prefix length, W a RIPE window.

    * tail_positions: floor(tail_frac * T), at least 1 (0 when T = 0);
    * tail_share: the share of sum_j e_j carried by the tail_positions
      largest e_j (among equal values the lower positions first);
    * tail_in_window: the fraction of those positions among the last W;
    * window_share: the share of sum_j e_j carried by the last W positions;
    * ill_conditioned: positions with cond > 1, and ill_conditioned_share
      their share of sum_j e_j (None without cond).
    Shares are None when sum_j e_j is 0, tail_in_window when there is no
    tail position."""
    e = np.asarray(err, dtype=np.float64)[:T]
    n_tail = 0 if T == 0 else max(1, int(math.floor(tail_frac * T)))
    order = np.argsort(-e, kind="stable")  # largest first; equal values keep position order
    top = order[:n_tail]
    total = float(e.sum())
    w0 = max(0, T - W)

    def share(x):
        return float(x) / total if total > 0 else None

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
