"""Pins of the accept / rollback oracle against facts fixed outside it.

* hand-worked cases (tests/golden/accept_cases.json);
* exact acceptance and draw probabilities: the decisions are monotone in the
  random word, so bisection over the 2^32 words measures them exactly;
* the lossless property of speculative sampling, as a closed form over the
  oracle's own residuals and as a Monte Carlo run of the whole function;
* greedy verification reproduces the greedy decode of a tiny synthetic model;
* mutation checks: plausible mistakes planted in the oracle make a pin fail.
"""
import json
import os

import numpy as np
import pytest

from oracle import accept as oa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "accept_cases.json")
TWO32 = 1 << 32


def words(us):
    return np.array([int(u * TWO32) for u in us], dtype=np.uint32)


def run_case(c):
    logit = lambda a: np.log(np.asarray(a, dtype=np.float64)).astype(np.float32)
    tl = logit(c["target"])[None]
    dl = logit(c["draft"])[None]
    tok = np.asarray(c["tokens"], dtype=np.int32)[None]
    fb = np.array([c["has_fallback"]])
    rw = words(c["uniforms"])[None]
    return oa.accept(tl, dl, tok, fb, rw, c["temperature"])


@pytest.mark.parametrize("name", [c["name"] for c in json.load(open(GOLDEN))["cases"]])
def test_golden_cases(name):
    c = next(c for c in json.load(open(GOLDEN))["cases"] if c["name"] == name)
    r = run_case(c)
    assert [int(r.n_accept[0]), int(r.branch[0]), int(r.next_token[0])] == c["expect"], c["note"]
    assert r.margin[0] > 1e-3  # every hand-worked decision has a wide margin


# ---------------------------------------------------------------------------
# exact probabilities by bisection over the random word
# ---------------------------------------------------------------------------
def accepted_words(p, q, t):
    """Number of random words whose uniform accepts t (acceptance is monotone)."""
    lo, hi = 0, TWO32  # invariant: word lo - 1 accepts (or lo = 0), word hi rejects (or hi = 2^32)
    if oa.check_token(p, q, t, oa.uniform(TWO32 - 1))[0]:
        return TWO32
    while lo < hi:
        mid = (lo + hi) // 2
        if oa.check_token(p, q, t, oa.uniform(mid))[0]:
            lo = mid + 1
        else:
            hi = mid
    return lo


@pytest.mark.parametrize("seed", range(6))
def test_acceptance_probability_is_min_one_ratio(seed):
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.ones(7))
    q = rng.dirichlet(np.ones(7))
    for t in range(7):
        n = accepted_words(p, q, t)
        assert abs(n / TWO32 - min(1.0, p[t] / q[t])) <= 2.0 / TWO32


def first_word_at_least(w, index):
    """Smallest word whose draw returns an index >= `index` (draws are monotone in u)."""
    lo, hi = 0, TWO32
    while lo < hi:
        mid = (lo + hi) // 2
        if oa.draw(w, oa.uniform(mid), w)[0] >= index:
            hi = mid
        else:
            lo = mid + 1
    return lo


@pytest.mark.parametrize("seed", range(4))
def test_draw_probabilities_are_the_weights(seed):
    rng = np.random.default_rng(100 + seed)
    w = rng.random(6)
    w[rng.integers(0, 6)] = 0.0  # an index with no weight is never drawn
    bounds = [first_word_at_least(w, i) for i in range(6)] + [TWO32]
    for i in range(6):
        assert abs((bounds[i + 1] - bounds[i]) / TWO32 - w[i] / w.sum()) <= 2.0 / TWO32


# ---------------------------------------------------------------------------
# lossless: the first kept token is distributed as the target row 0
# ---------------------------------------------------------------------------
def first_token_law(p0, q0, m):
    """P(first token = t) for one position with a fallback, from the acceptance
    probabilities min(1, ratio) and the oracle's residual weights."""
    V = p0.size
    w_r = oa.residual(p0, q0)
    r = w_r / w_r.sum()
    w_m = oa.residual(m, q0)
    q1 = w_m / w_m.sum()
    w_f = oa.residual(r, q1)
    F = w_f / w_f.sum() if w_f.sum() > 0 else r
    law = np.zeros(V)
    for x in range(V):
        a = min(1.0, p0[x] / q0[x])
        law[x] += q0[x] * a
        for y in range(V):
            if q1[y] == 0:
                continue
            bp = min(1.0, r[y] / q1[y])
            law[y] += q0[x] * (1 - a) * q1[y] * bp
            law += q0[x] * (1 - a) * q1[y] * (1 - bp) * F
    return law


@pytest.mark.parametrize("seed", range(8))
def test_lossless_closed_form(seed):
    rng = np.random.default_rng(200 + seed)
    V = 5
    p0, q0, m = (oa.softmax(rng.normal(size=V).astype(np.float32), 0.8) for _ in range(3))
    law = first_token_law(p0, q0, m)
    assert np.allclose(law, p0, atol=1e-12, rtol=0)


def caller_draws(rng, tl, dl, tau, k):
    """Draft tokens as a caller draws them: x_i ~ q_i, y_0 ~ residual of the
    deeper state after q_0, y_i ~ the fallback's rows."""
    V = tl.shape[-1]
    x = [rng.choice(V, p=oa.softmax(dl[0][i], tau)) for i in range(k)]
    w = oa.residual(oa.softmax(dl[1][0], tau), oa.softmax(dl[0][0], tau))
    y = [rng.choice(V, p=w / w.sum())] + [rng.choice(V, p=oa.softmax(dl[1][i], tau)) for i in range(1, k)]
    return np.array([x, y], dtype=np.int32)


def test_lossless_monte_carlo():
    """The whole function: over many independent draws, the first kept token
    follows softmax(target row 0) (each frequency within 5 standard errors)."""
    rng = np.random.default_rng(7)
    V, k, tau, N = 5, 2, 0.8, 40000
    tl = rng.normal(size=(2, k + 1, V)).astype(np.float32)
    dl = rng.normal(size=(2, k, V)).astype(np.float32)
    dl[1][0] = tl[0][0] + rng.normal(scale=0.3, size=V).astype(np.float32)  # a deeper, closer state
    toks = np.stack([caller_draws(rng, tl, dl, tau, k) for _ in range(N)])
    rw = rng.integers(0, TWO32, size=(N, 2 * k + 1), dtype=np.uint64).astype(np.uint32)
    r = oa.accept(np.broadcast_to(tl, (N,) + tl.shape), np.broadcast_to(dl, (N,) + dl.shape), toks,
                  np.ones(N, bool), rw, tau)
    first = np.where(r.n_accept > 0, toks[np.arange(N), r.branch, 0], r.next_token)
    p0 = oa.softmax(tl[0][0], tau)
    counts = np.bincount(first, minlength=V)
    z = (counts - N * p0) / np.sqrt(N * p0 * (1 - p0))
    assert np.all(np.abs(z) < 5.0), (counts / N, p0)
    # both branches and the restart all occur in this setting
    assert (r.branch == 1).any() and ((r.n_accept == 0)).any() and (r.n_accept == k).any()


# ---------------------------------------------------------------------------
# greedy: the kept tokens and the next token are the model's greedy decode
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(10))
def test_greedy_reproduces_greedy_decode(seed):
    rng = np.random.default_rng(300 + seed)
    V, k = 6, 4
    table = rng.normal(size=(V, V)).astype(np.float32)  # logits of the next token given the previous
    c = int(rng.integers(V))
    g = []
    prev = c
    for _ in range(k + 1):
        prev = int(np.argmax(table[prev]))
        g.append(prev)
    B = 32
    tok = np.zeros((B, 2, k), np.int32)
    tl = np.zeros((B, 2, k + 1, V), np.float32)
    fb = rng.random(B) < 0.6
    for b in range(B):
        for ch in range(2):
            agree = int(rng.integers(0, k + 1))  # chain agrees with the greedy decode for this many tokens
            for i in range(k):
                tok[b, ch, i] = g[i] if i < agree else (g[i] + 1 + int(rng.integers(V - 1))) % V
            parents = [c] + list(tok[b, ch])
            for i in range(k + 1):
                tl[b, ch, i] = table[parents[i]]
    dl = np.zeros((B, 2, k, V), np.float32)
    r = oa.accept(tl, dl, tok, fb, np.zeros((B, 2 * k + 1), np.uint32), 0.0)
    for b in range(B):
        agree_p = next((i for i in range(k) if tok[b, 0, i] != g[i]), k)
        agree_f = next((i for i in range(k) if tok[b, 1, i] != g[i]), k)
        use_f = agree_p == 0 and fb[b] and agree_f > 0
        n, ch = (agree_f, 1) if use_f else (agree_p, 0)
        assert (int(r.n_accept[b]), int(r.branch[b])) == (n, ch)
        emitted = list(tok[b, ch, :n]) + [int(r.next_token[b])]
        assert emitted == g[:n + 1]


# ---------------------------------------------------------------------------
# mutation checks: planted mistakes fail a pin (CPU only)
# ---------------------------------------------------------------------------
def test_mutation_swapped_ratio_fails(monkeypatch):
    monkeypatch.setattr(oa, "check_token", lambda p, q, t, u: (bool(u * p[t] < q[t]), 1.0))
    with pytest.raises(AssertionError):
        test_acceptance_probability_is_min_one_ratio(0)


def test_mutation_residual_without_subtraction_fails(monkeypatch):
    monkeypatch.setattr(oa, "residual", lambda a, c: np.maximum(a, 0.0))
    with pytest.raises(AssertionError):
        test_lossless_closed_form(0)


def test_mutation_greedy_next_from_wrong_row_fails(monkeypatch):
    real = oa._greedy

    def wrong(tl, tok, fb, k, V):
        n, br, nx = real(tl, tok, fb, k, V)
        return n, br, oa.argmax(tl[br][0])  # always row 0
    monkeypatch.setattr(oa, "_greedy", wrong)
    with pytest.raises(AssertionError):
        for s in range(10):
            test_greedy_reproduces_greedy_decode(s)
