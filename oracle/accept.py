"""Accept / rollback oracle -- TEST INFRASTRUCTURE ONLY.

A plain float64 NumPy statement of the acceptance step that follows
verification.  Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import it; the library never does.

Sources (cited by page and passage):

* LoopSpec summary (rit.work blog, "pipelined looped transformers"):
  - section on the second branch: besides the early draft, a fallback token
    is prepared from a deeper intermediate state, drawn not from that state's
    whole distribution but from what remains of it once the first proposal is
    taken out; it is spawned only when the deeper state is less confident in
    the first token (that gate is the caller's: whether a fallback exists is
    an input here);
  - same section: the final check tries the first draft, then the fallback,
    and restarts only after both are rejected;
  - same section: with greedy decoding the check returns the token the
    original model would have chosen; with sampling, each output keeps the
    probability it has under ordinary decoding.
* RIPE abstract (zhuanzhiai.com paper page): the verify pass runs the draft
  block through all R loops, so the target distributions come from depth R.

The scheme written out (with the readings taken where the page is silent):

* Per sequence there is a primary chain of k draft tokens x_0..x_{k-1} and,
  optionally, a fallback chain y_0..y_{k-1} that replaces the primary from
  position 0 (the fallback is an alternative to the first draft, not a
  continuation).
* Target rows: softmax(target_logits[b][c][i] / tau) scores position i of
  chain c, for i = 0..k (row k is the bonus position after a fully accepted
  chain).  Position 0 of both chains follows the same committed prefix, so
  the fallback chain's row 0 is never read: position 0 always uses the
  primary's row 0.
* Draft rows: q_i = softmax(draft_logits[b][0][i] / tau) is the distribution
  x_i was drawn from.  For the fallback, draft_logits[b][1][0] holds the
  deeper state's logits d, and y_0 was drawn from the residual
  q'_0 = norm(max(0, softmax(d / tau) - q_0)); rows 1..k-1 are the
  distributions y_1.. were drawn from.
* Speculative sampling (tau > 0), with uniforms u = word * 2^-32 taken from
  the random words rand[b] (word i for primary test i, word k for the
  fallback's first test, word k + i for fallback test i >= 1, word 2k for the
  final draw):
  - token t of a row is accepted iff u * q(t) < p(t), i.e. with probability
    min(1, p(t)/q(t));
  - first rejection of the primary at position j: with no fallback, or
    j > 0, n = j tokens of the primary are kept and the next token is drawn
    from norm(max(0, p_j - q_j));
  - j = 0 with a fallback: the fallback's first token is tested against the
    residual target r = norm(max(0, p_0 - q_0)) with its own draft
    distribution q'_0; if accepted the fallback chain continues with the
    ordinary test; if rejected nothing is kept and the next token is drawn
    from norm(max(0, r - q'_0)) (restart after two rejections);
  - a fully accepted chain adds a bonus token drawn from its row k;
  - a draw from weights w takes the first index whose running sum exceeds
    u * sum(w); if rounding leaves no such index, the last index with w > 0;
    a residual with no mass (possible only through rounding) is replaced by
    the row's target distribution.
* Greedy (tau = 0): a token is accepted iff it is the row's arg max (lowest
  index on ties); the next token is the arg max of the target row where the
  kept chain stopped (for a restart: of the primary's row 0).
* A token outside [0, V) is never accepted.

Float64 throughout (the logits are float32 inputs).  Pinned by
tests/test_oracle_accept.py: exact acceptance and draw probabilities found by
bisection over the random words, the lossless property (closed form and a
Monte Carlo run of the whole function), greedy decoding of a tiny synthetic
model, and hand-worked cases in tests/golden/accept_cases.json.
"""
from __future__ import annotations

from typing import NamedTuple, Optional

import numpy as np

TWO32 = 4294967296.0


class AcceptResult(NamedTuple):
    n_accept: np.ndarray    # int32 [B]: tokens kept
    branch: np.ndarray      # int32 [B]: 0 primary, 1 fallback (0 when nothing is kept)
    next_token: np.ndarray  # int32 [B]: correction or bonus token
    margin: np.ndarray      # float64 [B]: smallest relative margin of a float decision


def uniform(word) -> float:
    """Random word -> u in [0, 1) (exact in float64)."""
    return float(int(word)) / TWO32


def softmax(logits, tau: float) -> np.ndarray:
    """softmax(z / tau) in float64: exp((z - max z) * (1 / tau)) / sum."""
    z = np.asarray(logits, dtype=np.float32).astype(np.float64)
    e = np.exp((z - z.max()) * (1.0 / float(tau)))
    return e / e.sum()


def argmax(logits) -> int:
    """Arg max, lowest index on ties."""
    return int(np.argmax(np.asarray(logits, dtype=np.float32)))


def check_token(p: np.ndarray, q: np.ndarray, t: int, u: float):
    """Accept t iff u * q(t) < p(t); returns (accepted, relative margin)."""
    if t < 0 or t >= p.size:
        return False, np.inf
    a, b = u * q[t], p[t]
    if a == 0.0 and b == 0.0:
        return False, np.inf  # exact zeros: no rounding can flip this
    return bool(a < b), abs(b - a) / max(b, a, 1e-300)


def residual(a: np.ndarray, c: np.ndarray) -> np.ndarray:
    """Weights max(0, a - c) (unnormalised)."""
    return np.maximum(a - c, 0.0)


def draw(w: np.ndarray, u: float, fallback: np.ndarray):
    """First index whose running sum exceeds u * sum(w); returns (index, relative margin)."""
    W = w.sum()
    if not W > 0.0:
        w = fallback
        W = w.sum()
    target = u * W
    c = np.cumsum(w)
    above = np.nonzero(c > target)[0]
    if above.size:
        i = int(above[0])
    else:
        i = int(np.nonzero(w > 0)[0][-1])
    # distance of the target to the nearest running-sum boundary
    gap = np.min(np.abs(c - target)) if c.size else np.inf
    return i, gap / W


def accept(target_logits, draft_logits, tokens, has_fallback, rand, temperature: float) -> AcceptResult:
    """Accept / rollback for a batch.

    target_logits [B][2][k+1][V] float32; draft_logits [B][2][k][V] float32;
    tokens [B][2][k] int; has_fallback [B] bool; rand [B][2k+1] uint32;
    temperature: > 0 speculative sampling, 0 greedy.
    """
    tl = np.asarray(target_logits, dtype=np.float32)
    dl = np.asarray(draft_logits, dtype=np.float32)
    tok = np.asarray(tokens, dtype=np.int64)
    fb = np.asarray(has_fallback).astype(bool)
    rw = np.asarray(rand, dtype=np.uint64)
    B, _, k1, V = tl.shape
    k = k1 - 1
    n_out = np.zeros(B, np.int32)
    br_out = np.zeros(B, np.int32)
    nx_out = np.zeros(B, np.int32)
    mg_out = np.full(B, np.inf)
    tau = float(np.float32(temperature))  # the temperature is a float32 parameter
    for b in range(B):
        if tau == 0.0:
            n, br, nx = _greedy(tl[b], tok[b], bool(fb[b]), k, V)
            mg = np.inf
        else:
            n, br, nx, mg = _sample(tl[b], dl[b], tok[b], bool(fb[b]), rw[b], k, tau)
        n_out[b], br_out[b], nx_out[b], mg_out[b] = n, br, nx, mg
    return AcceptResult(n_out, br_out, nx_out, mg_out)


def _greedy(tl, tok, fb, k, V):
    def ok(row, t):
        return 0 <= t < V and t == argmax(row)
    j = 0
    while j < k and ok(tl[0][j], int(tok[0][j])):
        j += 1
    if j == k:
        return k, 0, argmax(tl[0][k])
    if j > 0 or not fb:
        return j, 0, argmax(tl[0][j])
    if not ok(tl[0][0], int(tok[1][0])):  # the fallback's first token against the same row
        return 0, 0, argmax(tl[0][0])
    j = 1
    while j < k and ok(tl[1][j], int(tok[1][j])):
        j += 1
    return j, 1, argmax(tl[1][j])


def _sample(tl, dl, tok, fb, rw, k, tau):
    margin = np.inf
    p = [softmax(tl[0][i], tau) for i in range(k + 1)]
    j = 0
    while j < k:
        q = softmax(dl[0][j], tau)
        acc, m = check_token(p[j], q, int(tok[0][j]), uniform(rw[j]))
        margin = min(margin, m)
        if not acc:
            break
        j += 1
    u_last = uniform(rw[2 * k])
    if j == k:
        t, m = draw(p[k], u_last, p[k])
        return k, 0, t, min(margin, m)
    q_j = softmax(dl[0][j], tau)
    if j > 0 or not fb:
        t, m = draw(residual(p[j], q_j), u_last, p[j])
        return j, 0, t, min(margin, m)
    # the fallback's first token against the residual target
    w_r = residual(p[0], q_j)
    r = w_r / w_r.sum() if w_r.sum() > 0 else p[0]
    w_m = residual(softmax(dl[1][0], tau), q_j)
    q1 = w_m / w_m.sum() if w_m.sum() > 0 else np.zeros_like(w_m)
    y = int(tok[1][0])
    acc, m = check_token(r, q1, y, uniform(rw[k]))
    margin = min(margin, m)
    if 0 <= y < r.size:  # r(y), q'(y) come through max(0, .): how close each clamp was
        pm = softmax(dl[1][0], tau)
        for a, c in ((p[0][y], q_j[y]), (pm[y], q_j[y])):
            margin = min(margin, abs(a - c) / max(a, c, 1e-300))
    if not acc:
        t, m = draw(residual(r, q1), u_last, r)
        return 0, 0, t, min(margin, m)
    pf = [None] + [softmax(tl[1][i], tau) for i in range(1, k + 1)]
    j = 1
    while j < k:
        q = softmax(dl[1][j], tau)
        acc, m = check_token(pf[j], q, int(tok[1][j]), uniform(rw[k + j]))
        margin = min(margin, m)
        if not acc:
            break
        j += 1
    if j == k:
        t, m = draw(pf[k], u_last, pf[k])
        return k, 1, t, min(margin, m)
    q_j = softmax(dl[1][j], tau)
    t, m = draw(residual(pf[j], q_j), u_last, pf[j])
    return j, 1, t, min(margin, m)
