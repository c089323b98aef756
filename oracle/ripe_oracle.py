"""RIPE verify / commit oracle -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 NumPy statement of what the RIPE hot path computes.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the library never does, and this module imports
nothing from the library.

Sources (the pages are cited by page and passage):

* RIPE abstract (zhuanzhiai.com paper page, abstract paragraph):
  - opening sentence: the looped model repeats its recurrent block R times for
    every token, so each recurrent layer caches R K/V planes; drafting uses
    few loops and verification uses all R, so it reads every plane;
  - sentence on the deepest plane: one plane (the last) can serve every depth;
  - sentence introducing RIPE: only the last plane is kept for old positions,
    while the most recent W positions keep all R planes;
  - sentence on the 64-position window: when W is no shorter than the draft
    block, a block's verification result cannot depend on the other blocks
    of its batch.
* LoopSpec summary (rit.work blog, "pipelined looped transformers"): branches
  at different recurrent depths are processed in one batched call; a rejected
  branch is dropped and decoding rolls back to the confirmed prefix.

Readings taken where the pages are silent:

* depth r is 1-based, plane R is the deepest;
* the window is anchored at the committed length T: prefix position j is read
  from plane r iff j >= T - W (else from plane R), the same for every row of a
  draft block;
* a block's own (draft) keys and values are those of depth r, and row i of a
  block sees the block's rows 0..i;
* GQA: query head h reads KV head h // (Hq / Hkv);
* a group never sees the rows of another group (branches are siblings);
* log-sum-exp is natural-log and includes the running maximum.

Parity status: every function here is pinned by tests/test_oracle_pins.py and
tests/test_oracle_commit.py (brute force, a library attention routine, the
layout invariants, closed-form fixtures in tests/golden/).
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Sequence, Tuple

import numpy as np

FULL, DEEPEST, RIPE = 0, 1, 2
LAYOUT_CODES = {"full": FULL, "deepest": DEEPEST, "ripe": RIPE}


def layout_code(layout) -> int:
    return LAYOUT_CODES[layout] if isinstance(layout, str) else int(layout)


def _group_fields(g) -> Tuple[int, int, int, int]:
    if isinstance(g, tuple):
        return tuple(int(x) for x in g[:4])  # type: ignore[return-value]
    return int(g.seq), int(g.depth), int(g.row_start), int(g.n_rows)


def _parent_fields(g) -> Tuple[int, int]:
    """(row_start, n_rows) of a group's in-flight parent block; (0, 0) if none."""
    if isinstance(g, tuple):
        return (int(g[4]), int(g[5])) if len(g) >= 6 else (0, 0)
    return int(getattr(g, "parent_row_start", 0)), int(getattr(g, "parent_rows", 0))


# ---------------------------------------------------------------------------
# plane selection (RIPE abstract: full cache reads plane r; one shared plane
# reads plane R; RIPE keeps the deepest plane except a recent window)
# ---------------------------------------------------------------------------
def plane_select(layout, R: int, W: int, T: int, r: int, parent_rows: int = 0) -> np.ndarray:
    """Plane (1..R) that a query issued at depth r reads for each committed
    prefix position j in [0, T).  With a parent block of ``parent_rows`` rows
    still in flight, the prefix is read as it will be once the parent is
    committed: the window is the last W positions of T + parent_rows."""
    layout = layout_code(layout)
    if not 1 <= r <= R:
        raise ValueError("depth out of range")
    out = np.empty(T, dtype=np.int8)
    for j in range(T):
        if layout == FULL:
            out[j] = r
        elif layout == DEEPEST:
            out[j] = R
        else:
            out[j] = r if j >= T + parent_rows - W else R
    return out


# ---------------------------------------------------------------------------
# logical cache: for each sequence and plane, which positions are held
# ---------------------------------------------------------------------------
class LogicalCache:
    """The positions and planes a layout keeps, without any byte layout.

    * FULL holds planes 1..R at every committed position;
    * DEEPEST holds plane R at every committed position;
    * RIPE holds plane R at every committed position and planes 1..R-1 at the
      last W committed positions.

    Values are kept in float64 and must already be exactly representable in
    the cache dtype.  Reading a (plane, position) that the layout does not
    hold raises KeyError.
    """

    def __init__(self, layout, dtype: str, R: int, W: int, B: int, t_max: int, Hkv: int, D: int):
        self.layout = layout_code(layout)
        self.dtype, self.R, self.W, self.B = dtype, R, W, B
        self.t_max, self.Hkv, self.D = t_max, Hkv, D
        self.seq_len = np.zeros(B, dtype=np.int64)
        # dense planes: (b, p) -> (K [t_max,H,D], V [t_max,H,D], held mask [t_max])
        self._dense: Dict[Tuple[int, int], Tuple[np.ndarray, np.ndarray, np.ndarray]] = {}
        # sparse planes (RIPE planes below R): (b, p) -> {j: (K [H,D], V [H,D])}
        self._sparse: Dict[Tuple[int, int], Dict[int, Tuple[np.ndarray, np.ndarray]]] = {}

    # -- which planes live where ------------------------------------------
    def planes_held(self) -> List[int]:
        if self.layout == FULL:
            return list(range(1, self.R + 1))
        if self.layout == DEEPEST:
            return [self.R]
        return list(range(1, self.R + 1)) if self.W > 0 else [self.R]

    def _is_sparse(self, p: int) -> bool:
        return self.layout == RIPE and p < self.R

    def _dense_plane(self, b: int, p: int):
        key = (b, p)
        if key not in self._dense:
            shape = (self.t_max, self.Hkv, self.D)
            self._dense[key] = (np.full(shape, np.nan), np.full(shape, np.nan),
                                np.zeros(self.t_max, dtype=bool))
        return self._dense[key]

    def put(self, b: int, p: int, j: int, k: np.ndarray, v: np.ndarray) -> None:
        if p not in self.planes_held():
            raise KeyError(f"layout does not hold plane {p}")
        if not 0 <= j < self.t_max:
            raise IndexError(j)
        if self._is_sparse(p):
            self._sparse.setdefault((b, p), {})[j] = (np.array(k, dtype=np.float64),
                                                     np.array(v, dtype=np.float64))
        else:
            K, V, held = self._dense_plane(b, p)
            K[j], V[j], held[j] = k, v, True

    def put_range(self, b: int, p: int, j0: int, k: np.ndarray, v: np.ndarray) -> None:
        n = k.shape[0]
        if self._is_sparse(p):
            for i in range(n):
                self.put(b, p, j0 + i, k[i], v[i])
        else:
            if p not in self.planes_held():
                raise KeyError(p)
            K, V, held = self._dense_plane(b, p)
            K[j0:j0 + n], V[j0:j0 + n], held[j0:j0 + n] = k, v, True

    def drop(self, b: int, p: int, j: int) -> None:
        if self._is_sparse(p):
            self._sparse.get((b, p), {}).pop(j, None)
        elif (b, p) in self._dense:
            K, V, held = self._dense[(b, p)]
            K[j], V[j], held[j] = np.nan, np.nan, False

    def holds(self, b: int, p: int, j: int) -> bool:
        if self._is_sparse(p):
            return j in self._sparse.get((b, p), {})
        if (b, p) not in self._dense:
            return False
        return bool(self._dense[(b, p)][2][j])

    def get(self, b: int, p: int, j0: int, j1: int) -> Tuple[np.ndarray, np.ndarray]:
        """K, V of plane p at positions [j0, j1): arrays [j1-j0, Hkv, D]."""
        n = j1 - j0
        if n <= 0:
            z = np.zeros((0, self.Hkv, self.D))
            return z, z.copy()
        if self._is_sparse(p):
            store = self._sparse.get((b, p), {})
            try:
                ks = [store[j][0] for j in range(j0, j1)]
                vs = [store[j][1] for j in range(j0, j1)]
            except KeyError as e:
                raise KeyError(f"plane {p} not held at position {e}") from None
            return np.stack(ks), np.stack(vs)
        if (b, p) not in self._dense:
            raise KeyError(f"plane {p} of sequence {b} not held")
        K, V, held = self._dense[(b, p)]
        if not held[j0:j1].all():
            raise KeyError(f"plane {p} not held at some position in [{j0},{j1})")
        return K[j0:j1].copy(), V[j0:j1].copy()

    def dense_plane(self, b: int, p: int) -> Tuple[np.ndarray, np.ndarray]:
        """K, V [t_max, Hkv, D] of a plane held at every position (NaN where
        no value is held)."""
        if self._is_sparse(p):
            raise KeyError("plane is windowed")
        if (b, p) not in self._dense:
            shape = (self.t_max, self.Hkv, self.D)
            return np.full(shape, np.nan), np.full(shape, np.nan)
        K, V, _ = self._dense[(b, p)]
        return K, V

    def held_positions(self, b: int, p: int) -> List[int]:
        if self._is_sparse(p):
            return sorted(self._sparse.get((b, p), {}))
        if (b, p) not in self._dense:
            return []
        return [int(j) for j in np.nonzero(self._dense[(b, p)][2])[0]]

    def copy(self) -> "LogicalCache":
        c = LogicalCache(self.layout, self.dtype, self.R, self.W, self.B, self.t_max, self.Hkv,
                         self.D)
        c.seq_len = self.seq_len.copy()
        c._dense = {k: (a.copy(), b.copy(), m.copy()) for k, (a, b, m) in self._dense.items()}
        c._sparse = {k: {j: (a.copy(), b.copy()) for j, (a, b) in d.items()}
                     for k, d in self._sparse.items()}
        return c

    def same_contents(self, other: "LogicalCache") -> bool:
        if not np.array_equal(self.seq_len, other.seq_len):
            return False
        for b in range(self.B):
            for p in self.planes_held():
                pa, pb = self.held_positions(b, p), other.held_positions(b, p)
                if pa != pb:
                    return False
                for j in pa:
                    ka, va = self.get(b, p, j, j + 1)
                    kb, vb = other.get(b, p, j, j + 1)
                    if not (np.array_equal(ka, kb) and np.array_equal(va, vb)):
                        return False
        return True


def fill_prefix(cache: LogicalCache, b: int, T: int, plane_values) -> None:
    """Set sequence b to hold a committed prefix of length T whose plane-p
    values come from ``plane_values(kind, b, p, j0, j1)`` (kind 0 = K, 1 = V).
    Only the (plane, position) pairs the layout keeps are stored."""
    if T > cache.t_max:
        raise ValueError("prefix longer than capacity")
    for p in cache.planes_held():
        if cache.layout == RIPE and p < cache.R:
            j0 = max(0, T - cache.W)
        else:
            j0 = 0
        if T > j0:
            cache.put_range(b, p, j0, plane_values(0, b, p, j0, T), plane_values(1, b, p, j0, T))
    cache.seq_len[b] = T


# ---------------------------------------------------------------------------
# commit (RIPE abstract, sentence introducing RIPE: recent positions hold every plane;
# LoopSpec summary: rejected continuations are dropped, accepted ones kept)
# ---------------------------------------------------------------------------
def commit(cache: LogicalCache, n_accept: Sequence[int], src_row: Sequence[int],
           kv_new: np.ndarray) -> None:
    """Append n_accept[b] accepted draft rows (starting at draft row
    src_row[b]) to sequence b, in place.

    kv_new is [2, R, n_rows, Hkv, D]: K and V of every draft row at every
    depth.  A new position keeps what its layout keeps; in RIPE, positions that
    fall out of the window of the last W committed positions lose planes
    1..R-1 and keep only plane R.
    """
    R = cache.R
    for b in range(cache.B):
        n = int(n_accept[b])
        if n < 0:
            raise ValueError("negative accept count")
        if n == 0:
            continue
        T = int(cache.seq_len[b])
        if T + n > cache.t_max:
            raise ValueError("capacity exceeded")
        s = int(src_row[b])
        for i in range(n):
            j = T + i
            for p in cache.planes_held():
                cache.put(b, p, j, kv_new[0, p - 1, s + i], kv_new[1, p - 1, s + i])
        T_new = T + n
        if cache.layout == RIPE:
            for p in range(1, R):
                for j in cache.held_positions(b, p):
                    if j < T_new - cache.W:
                        cache.drop(b, p, j)
        cache.seq_len[b] = T_new


# ---------------------------------------------------------------------------
# verification attention
# ---------------------------------------------------------------------------
def gather_prefix(cache: LogicalCache, b: int, r: int,
                  parent_rows: int = 0) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Keys, values [T, Hkv, D] and plane ids [T] that a depth-r query of
    sequence b reads from the committed prefix (with ``parent_rows`` rows of
    a parent block in flight, see plane_select)."""
    T = int(cache.seq_len[b])
    sel = plane_select(cache.layout, cache.R, cache.W, T, r, parent_rows)
    K = np.empty((T, cache.Hkv, cache.D))
    V = np.empty((T, cache.Hkv, cache.D))
    j = 0
    while j < T:
        p = int(sel[j])
        j1 = j
        while j1 < T and sel[j1] == p:
            j1 += 1
        K[j:j1], V[j:j1] = cache.get(b, p, j, j1)
        j = j1
    return K, V, sel


def attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, visible: np.ndarray,
           scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of queries q [n, D] over keys/vals [m, D] where
    visible[i, j] says whether query i may see key j.  Returns (out [n, D],
    lse [n]) with lse = natural-log log-sum-exp of the visible scores."""
    s = scale * (q @ keys.T)
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    out = (e @ vals) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


def draft_rows(kv_new: np.ndarray, r: int, s: int, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """K, V [k, Hkv, D] of a group's own rows: the draft rows at depth r."""
    return kv_new[0, r - 1, s:s + k], kv_new[1, r - 1, s:s + k]


def parent_block(kv_new: np.ndarray, layout, R: int, W: int, T: int, r: int, s: int,
                 k: int) -> Tuple[np.ndarray, np.ndarray]:
    """K, V [k, Hkv, D] of an in-flight parent block (draft rows s..s+k-1, to
    become positions T..T+k-1), each row at the plane it will be read from
    once committed: FULL depth r, DEEPEST depth R, RIPE depth r inside the
    window of the last W positions of T + k and depth R before it."""
    layout = layout_code(layout)
    K = np.empty((k,) + kv_new.shape[3:])
    V = np.empty((k,) + kv_new.shape[3:])
    for i in range(k):
        if layout == FULL:
            d = r
        elif layout == DEEPEST:
            d = R
        else:
            d = r if T + i >= T + k - W else R
        K[i], V[i] = kv_new[0, d - 1, s + i], kv_new[1, d - 1, s + i]
    return K, V


def visibility(T: int, k: int) -> np.ndarray:
    """[k, T + k] mask: every row sees the whole committed prefix; row i of the
    block sees the block's rows 0..i."""
    vis = np.ones((k, T + k), dtype=bool)
    vis[:, T:] = np.tril(np.ones((k, k), dtype=bool))
    return vis


def kv_head(h: int, G: int) -> int:
    """KV head read by query head h when G query heads share one KV head."""
    return h // G


def verify(cache: LogicalCache, groups: Iterable, q: np.ndarray, kv_new: np.ndarray,
           scale: float, n_q_heads: int) -> Tuple[np.ndarray, np.ndarray, List[np.ndarray]]:
    """Verification attention for every group (draft block or branch).

    q is [n_rows, Hq, D]; kv_new is [2, R, n_rows, Hkv, D].  Group g (sequence
    b, depth r, rows [s, s + k)) attends, for query head h and KV head
    h // (Hq / Hkv), over the committed prefix read per the layout's plane
    rule at depth r, then over its own rows s..s+i at depth r (row i).  A
    group with a parent block in flight (parent_rows > 0) reads the prefix and
    then every parent row as they will be read once the parent is committed
    (plane_select, parent_block), so the result equals committing the parent
    first (LoopSpec summary: the next position's computation starts before
    the current one is confirmed).

    Returns out [n_rows, Hq, D] (NaN for rows no group covers), lse
    [n_rows, Hq] and the plane ids each group read (int8 [T_b]).
    """
    n_rows, Hq, D = q.shape
    if Hq != n_q_heads or n_q_heads % cache.Hkv:
        raise ValueError("head counts")
    G = n_q_heads // cache.Hkv
    out = np.full((n_rows, Hq, D), np.nan)
    lse = np.full((n_rows, Hq), np.nan)
    sels = []
    for g in groups:
        b, r, s, k = _group_fields(g)
        ps, kp = _parent_fields(g)
        Kp, Vp, sel = gather_prefix(cache, b, r, kp)
        sels.append(sel)
        if kp:  # the in-flight parent block follows the committed prefix
            Ka, Va = parent_block(kv_new, cache.layout, cache.R, cache.W, Kp.shape[0], r, ps, kp)
            Kp, Vp = np.concatenate([Kp, Ka]), np.concatenate([Vp, Va])
        T = Kp.shape[0]
        Kn, Vn = draft_rows(kv_new, r, s, k)
        vis = visibility(T, k)
        for h in range(Hq):
            hk = kv_head(h, G)
            keys = np.concatenate([Kp[:, hk], Kn[:, hk]], axis=0)
            vals = np.concatenate([Vp[:, hk], Vn[:, hk]], axis=0)
            o, ls = attend(q[s:s + k, h], keys, vals, vis, scale)
            out[s:s + k, h] = o
            lse[s:s + k, h] = ls
    return out, lse, sels


def memory_positions(layout, R: int, W: int, T: int) -> int:
    """Position-planes one recurrent layer holds for one sequence of length T
    (RIPE abstract: memory of the full cache vs one plane vs RIPE)."""
    layout = layout_code(layout)
    if layout == FULL:
        return R * T
    if layout == DEEPEST:
        return T
    return T + min(W, T) * (R - 1)
