"""GPU parity of ripe_accept against the float64 oracle (oracle/accept.py).

The outputs are integers decided by floating-point comparisons.  Both sides
decide in double; they can differ only when a decision falls within rounding
of its threshold, which the oracle reports as a relative margin.  Sequences
whose margin is below 1e-9 are not compared (none are expected: each case
asserts how many there were), every other output must match exactly.
"""
import numpy as np
import pytest
import torch

import self_speculative_verify_ripe_amd as rp
from oracle import accept as oa
from workloads import accept_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
MARGIN = 1e-9


def gpu_accept(inp, temperature, ws=None):
    B, _, k1, V = inp.target.shape
    d = rp.make_accept_desc(B, k1 - 1, V, temperature)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    n = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    br = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    nx = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    rp.ripe_accept(d, t(inp.target), t(inp.draft), t(inp.tokens), t(inp.has_fallback),
                   t(inp.rand.view(np.int32)), n, br, nx, ws)
    torch.cuda.synchronize()
    return n.cpu().numpy(), br.cpu().numpy(), nx.cpu().numpy()


def compare(inp, temperature, tag, max_ambiguous=0):
    ref = oa.accept(inp.target, inp.draft, inp.tokens, inp.has_fallback, inp.rand, temperature)
    n, br, nx = gpu_accept(inp, temperature)
    sure = ref.margin >= MARGIN
    assert int((~sure).sum()) <= max_ambiguous, f"{tag}: {int((~sure).sum())} near-threshold decisions"
    for name, got, want in (("n_accept", n, ref.n_accept), ("branch", br, ref.branch),
                            ("next_token", nx, ref.next_token)):
        bad = np.nonzero(sure & (got != want))[0]
        assert bad.size == 0, f"{tag}: {name} differs at sequences {bad[:8]}: {got[bad[:8]]} vs {want[bad[:8]]}"
    # the ambiguous ones are still valid outputs
    V = inp.target.shape[-1]
    k = inp.tokens.shape[-1]
    assert np.all((n >= 0) & (n <= k) & (br >= 0) & (br <= 1) & (nx >= 0) & (nx < V))
    return ref


@pytest.mark.parametrize("temperature", [0.0, 0.7, 1.0])
@pytest.mark.parametrize("k,V", [(1, 5), (4, 1000), (4, 1003), (8, 4096)])
def test_accept_matches_oracle(temperature, k, V):
    inp = accept_inputs(9000 + k * 7 + V, 96, k, V, temperature, fallback_frac=0.5)
    ref = compare(inp, temperature, f"k={k} V={V} tau={temperature}")
    # the draws reach every outcome: some kept tokens, some fallbacks, some restarts
    assert (ref.n_accept > 0).any() and (ref.n_accept == 0).any()
    if V > 5:
        assert (ref.branch == 1).any()


def test_accept_full_vocab_size():
    """A 64K vocabulary at the c4 shape (16 sequences, k = 4, fallback for
    about 40%)."""
    for temperature in (0.0, 0.8):
        inp = accept_inputs(777, 16, 4, 65536, temperature)
        compare(inp, temperature, f"V=65536 tau={temperature}")


@pytest.mark.parametrize("B,k,V", [(12, 3, 70001), (4, 2, 300007)])
def test_accept_ragged_and_long_slices(B, k, V):
    """Vocabulary sizes that slice unevenly: 70001 gives 18 slices of 3904
    indices and a shorter last one (every per-index sweep has a ragged
    tail); 300007 hits the 64-slice cap, so slices of 4736 indices are longer
    than the 4096 the row statistics hold in registers and take the
    two-pass path."""
    for temperature in (0.0, 0.9):
        inp = accept_inputs(4242 + V, B, k, V, temperature, fallback_frac=0.5, draft_noise=1.5)
        print(f"[case] B={B} k={k} V={V} tau={temperature}", flush=True)
        compare(inp, temperature, f"B={B} k={k} V={V} tau={temperature}")


def test_accept_edge_cases():
    # tokens out of range, masked (-inf) logits, exact ties for greedy, V = 1
    inp = accept_inputs(31, 40, 3, 64, 0.9, fallback_frac=0.6)
    inp.tokens[0, 0, 0] = -1
    inp.tokens[1, 0, 0] = 64
    inp.tokens[2, 1, 0] = 1 << 30
    inp.target[3, 0, 0, 10:] = -np.inf       # most of a target row masked
    inp.draft[4, 0, 0, :32] = -np.inf        # most of a draft row masked
    compare(inp, 0.9, "edge sampling")
    g = accept_inputs(32, 40, 3, 64, 0.0, fallback_frac=0.6)
    g.target[:, :, :, 5] = g.target.max() + 1.0  # two equal maxima: the lower index wins
    g.target[:, :, :, 9] = g.target.max()
    g.tokens[:20] = 5
    g.tokens[20:30] = 9
    compare(g, 0.0, "greedy ties")
    one = accept_inputs(33, 8, 2, 1, 1.0, fallback_frac=0.5)
    ref = compare(one, 1.0, "V=1")
    assert np.all(ref.n_accept == 2) and np.all(ref.next_token == 0)


def test_accept_identical_rows_accept_everything():
    """Draft rows equal to the target rows: every drafted token is accepted
    (u q(t) < p(t) for u < 1 whenever p(t) > 0)."""
    inp = accept_inputs(44, 32, 4, 500, 1.0, fallback_frac=0.0)
    inp.draft[:, 0] = inp.target[:, 0, :4]
    ref = compare(inp, 1.0, "identical rows")
    assert np.all(ref.n_accept == 4)


def test_accept_then_commit():
    """The accept result drives ripe_commit (n_accept, src_row of the kept
    chain's group) for a RIPE cache; the committed rows are those of the
    chain the oracle keeps."""
    from oracle import ripe_oracle as ro
    from oracle import layout as olay
    B, R, W, Hkv, D, k, V = 6, 4, 8, 2, 64, 3, 50
    t_max = 64
    desc = rp.make_desc("ripe", "f32", R, W, B, t_max, Hkv, D, Hkv, max_rows=2 * B * k, max_groups=2 * B)
    cache = torch.zeros(rp.ripe_layout_bytes(desc), dtype=torch.uint8, device=DEV)
    rng = np.random.default_rng(5)
    n_rows = 2 * B * k
    kv_new = rng.standard_normal((2, R, n_rows, Hkv, D)).astype(np.float32)
    seq_len = np.array([0, 5, 9, 17, 30, 40], np.int32)
    # prefixes committed from kv_new rows first (rows 0.., a plain fill)
    oc = ro.LogicalCache("ripe", "f32", R, W, B, t_max, Hkv, D)
    sl = np.zeros(B, np.int32)
    fill = rng.standard_normal((2, R, 64, Hkv, D)).astype(np.float32)
    for b in range(B):
        if seq_len[b]:
            na = np.zeros(B, np.int32)
            na[b] = seq_len[b]
            rp.ripe_commit(desc, cache, sl, na, np.zeros(B, np.int32), torch.from_numpy(fill).to(DEV), 64)
            ro.commit(oc, na, np.zeros(B, np.int32), fill)
    inp = accept_inputs(55, B, k, V, 0.8, fallback_frac=0.5)
    n, br, nx = gpu_accept(inp, 0.8)
    ref = oa.accept(inp.target, inp.draft, inp.tokens, inp.has_fallback, inp.rand, 0.8)
    assert np.array_equal(n, ref.n_accept) and np.array_equal(br, ref.branch)
    primary = np.arange(B) * 2 * k
    fallback = primary + k
    na, src = rp.commit_args(n, br, primary, fallback)
    sl2 = rp.ripe_commit(desc, cache, sl.copy(), na, src, torch.from_numpy(kv_new).to(DEV), n_rows)
    torch.cuda.synchronize()
    ro.commit(oc, na, src, kv_new)
    assert np.array_equal(sl2, seq_len + n)
    ref_bytes = olay.encode(oc).view(np.uint32)
    got = cache.cpu().numpy().view(np.uint32)
    held = ref_bytes != np.float32(np.nan).view(np.uint32)
    assert np.array_equal(got[held], ref_bytes[held])
