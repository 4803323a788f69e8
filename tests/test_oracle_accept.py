"""Pins for the acceptance oracle (oracle.accept).

The pages' guarantee is that accepting each draft with probability
min(1, p/q) yields output that follows the autoregressive distribution
("Introspective Diffusion Language Models", section "Inference & ISD").  The
tests check that property of the oracle, not its formulas:

* exact integration over the 2**-24 uniform grid (the acceptance decision is
  monotone in u and the sampled token in u', so bisection finds every
  boundary): each committed token follows p_k given the earlier drafts were
  kept, the bonus follows p_K, and acceptance lengths follow the product of
  1 - TV(p_i, q_i);
* chi-square tests of the seeded Philox path over 10**6 seeds on a 16-token
  vocabulary;
* special cases: q == p, one-hot p, one-hot q (argmax proposals), greedy
  T = 0, and N = 1, which is plain categorical sampling (numpy searchsorted).
"""

import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest
from scipy import special, stats

from oracle.accept import accept_with_uniforms, isd_accept, softmax_t
from oracle.philox import isd_uniforms

GRID = 1 << 24
TOP = (GRID - 1) / GRID


def _first_false(pred):
    """Smallest k in [0, GRID] with pred(k / GRID) false; pred must be true-then-false."""
    lo, hi = 0, GRID
    while lo < hi:
        mid = (lo + hi) // 2
        if pred(mid / GRID):
            lo = mid + 1
        else:
            hi = mid
    return lo


def _rows(rng, V, N, T=1.0, scale=1.5):
    lc = rng.standard_normal((N, V)) * scale
    lm = rng.standard_normal((N - 1, V)) * scale
    P = [softmax_t(r, T) for r in lc]
    Q = [softmax_t(r, T) for r in lm]
    return lc, lm, P, Q


def _accepted_at(P, Q, drafts, i, u):
    K = len(Q)
    uu = [0.0] * K
    uu[i] = u
    n, _, _ = accept_with_uniforms(P, Q, drafts, uu, [0.0] * (K + 1))
    return n > i + 1


def _token_at(P, Q, drafts, i, u_i, u2):
    K = len(Q)
    uu = [0.0] * K
    if i < K:
        uu[i] = u_i
    vv = [0.0] * (K + 1)
    vv[i] = u2
    _, toks, _ = accept_with_uniforms(P, Q, drafts, uu, vv)
    return toks[i]


def _token_measure(P, Q, drafts, i, u_i, V):
    """Grid measure of u' giving each token at position i."""
    cum = [_first_false(lambda u2: _token_at(P, Q, drafts, i, u_i, u2) <= v) for v in range(V)]
    cum = np.array([0] + cum, dtype=np.float64)
    return np.diff(cum) / GRID


def _exact_position_law(P, Q, i, V, rng):
    """Exact law of the committed token at position i given drafts 0..i-1 kept."""
    K = len(Q)
    law = np.zeros(V)
    base = [int(rng.integers(V)) for _ in range(K)]  # earlier drafts: kept since u = 0 and p > 0
    for x in range(V):
        drafts = base[:i] + [x] + base[i + 1:]
        acc = _first_false(lambda u: _accepted_at(P, Q, drafts, i, u)) / GRID
        law[x] += Q[i][x] * acc
        if acc < 1.0:
            law += Q[i][x] * (1.0 - acc) * _token_measure(P, Q, drafts, i, TOP, V)
    return law


@pytest.mark.parametrize("V,N,seed", [(3, 2, 1), (4, 2, 2), (4, 3, 3), (3, 3, 4)])
def test_exact_committed_token_law(V, N, seed):
    rng = np.random.default_rng(seed)
    lc, lm, P, Q = _rows(rng, V, N)
    ref = [special.softmax(r) for r in lc]
    tol = 4 * V / GRID
    for i in range(N - 1):
        law = _exact_position_law(P, Q, i, V, rng)
        assert np.max(np.abs(law - ref[i])) < tol, (i, law, ref[i])
    # bonus: all drafts kept, token at position K follows p_K
    K = N - 1
    drafts = [int(rng.integers(V)) for _ in range(K)]
    bonus = _token_measure(P, Q, drafts, K, 0.0, V)
    assert np.max(np.abs(bonus - ref[K])) < tol
    # a list cut short after k drafts takes its bonus from clean row k
    for k in range(K):
        cut = drafts[:k] + [-1] * (K - k)
        law = _token_measure(P, Q, cut, k, 0.0, V)
        assert np.max(np.abs(law - ref[k])) < tol


@pytest.mark.parametrize("V,N,seed", [(4, 3, 5), (3, 4, 6)])
def test_exact_accept_length_law(V, N, seed):
    rng = np.random.default_rng(seed)
    lc, lm, P, Q = _rows(rng, V, N)
    K = N - 1
    base = [int(rng.integers(V)) for _ in range(K)]
    a = []
    for i in range(K):
        tot = 0.0
        for x in range(V):
            d = base[:i] + [x] + base[i + 1:]
            tot += Q[i][x] * _first_false(lambda u: _accepted_at(P, Q, d, i, u)) / GRID
        a.append(tot)
    sp = [special.softmax(r) for r in lc]
    for i in range(K):
        overlap = 1.0 - 0.5 * np.abs(sp[i] - special.softmax(lm[i])).sum()
        assert abs(a[i] - overlap) < 2 * V / GRID


def _chi2_worker(args):
    seeds, V, N, lc, lm, qprobs = args
    K = N - 1
    rng = np.random.default_rng(int(seeds[0]) + 7)
    counts = np.zeros((N, V), dtype=np.int64)
    lens = np.zeros(N + 1, dtype=np.int64)
    for s in seeds:
        drafts = np.array([[rng.choice(V, p=qprobs[i]) for i in range(K)]], dtype=np.int32)
        toks, n, _ = isd_accept(lc[None], lm[None], drafts, int(s), 1.0)
        n = int(n[0])
        lens[n] += 1
        for k in range(n):
            counts[k, toks[0, k]] += 1
    return counts, lens


def test_chi_square_seeded_path_1e6():
    V, N = 16, 4
    K = N - 1
    rng = np.random.default_rng(123)
    lc = rng.standard_normal((N, V)) * 1.2
    lm = lc[:K] + rng.standard_normal((K, V)) * 0.8
    P = [special.softmax(r) for r in lc]
    Qp = [special.softmax(r) for r in lm]
    total = 1_000_000
    workers = min(16, os.cpu_count() or 1)
    parts = np.array_split(np.arange(total, dtype=np.int64) * 2654435761 % (1 << 62), workers * 4)
    with ProcessPoolExecutor(workers) as ex:
        res = list(ex.map(_chi2_worker, [(p, V, N, lc, lm, Qp) for p in parts]))
    counts = sum(r[0] for r in res)
    lens = sum(r[1] for r in res)
    # position k is present iff the first k drafts were kept; it then follows p_k
    for k in range(N):
        n = counts[k].sum()
        expected = n * P[k]
        pval = stats.chisquare(counts[k], expected).pvalue
        assert pval > 1e-3, (k, pval)
    # acceptance lengths: P(len >= k+1) = prod_{i<k} (1 - TV(p_i, q_i))
    a = [1.0 - 0.5 * np.abs(P[i] - Qp[i]).sum() for i in range(K)]
    probs = np.array([np.prod(a[:k]) * ((1 - a[k]) if k < K else 1.0) for k in range(N)])
    pval = stats.chisquare(lens[1:], probs * total).pvalue
    assert pval > 1e-3
    mean = (lens * np.arange(N + 1)).sum() / total
    want = sum(np.prod(a[:k]) for k in range(N))
    sd = np.sqrt(((np.arange(1, N + 1) - want) ** 2 * probs).sum() / total)
    assert abs(mean - want) < 4 * sd


def test_identical_rows_always_accept():
    rng = np.random.default_rng(8)
    V, N, B = 32, 4, 200
    lm = (rng.standard_normal((B, N - 1, V)) * 2).astype(np.float32)
    lc = np.concatenate([lm, rng.standard_normal((B, 1, V)).astype(np.float32)], axis=1)
    drafts = rng.integers(0, V, size=(B, N - 1)).astype(np.int32)
    toks, lens, _ = isd_accept(lc, lm, drafts, 99, 1.0, dtype="f32")
    assert np.all(lens == N)
    assert np.array_equal(toks[:, :N - 1], drafts)


def test_one_hot_p_forces_token():
    rng = np.random.default_rng(9)
    V, N, B = 16, 3, 300
    lm = rng.standard_normal((B, N - 1, V))
    lc = rng.standard_normal((B, N, V))
    y = rng.integers(0, V, size=(B, N))
    for b in range(B):
        for i in range(N):
            lc[b, i, y[b, i]] = 1000.0  # exp(-1000) underflows: p is exactly one-hot
    drafts = rng.integers(0, V, size=(B, N - 1)).astype(np.int32)
    toks, lens, _ = isd_accept(lc, lm, drafts, 5, 1.0)
    for b in range(B):
        for k in range(lens[b]):
            assert toks[b, k] == y[b, k]


def test_one_hot_q_argmax_proposal():
    # q one-hot at x: kept iff u < p(x); the residual is p without x, renormalised.
    rng = np.random.default_rng(10)
    V = 6
    lc = rng.standard_normal((2, V))
    x = 2
    lm = np.full((1, V), -1000.0)
    lm[0, x] = 0.0
    P = [softmax_t(r, 1.0) for r in lc]
    Q = [softmax_t(r, 1.0) for r in lm]
    acc = _first_false(lambda u: _accepted_at(P, Q, [x], 0, u)) / GRID
    assert abs(acc - special.softmax(lc[0])[x]) <= 1 / GRID
    res = _token_measure(P, Q, [x], 0, TOP, V)
    want = special.softmax(lc[0]).copy()
    want[x] = 0
    want /= want.sum()
    assert np.max(np.abs(res - want)) < 2 * V / GRID


def test_greedy_temperature_zero():
    rng = np.random.default_rng(11)
    V, N, B = 50, 4, 300
    lc = rng.standard_normal((B, N, V)).astype(np.float32)
    lm = rng.standard_normal((B, N - 1, V)).astype(np.float32)
    # make some drafts agree with the clean argmax
    for b in range(0, B, 2):
        lm[b, 0] = lc[b, 0]
    drafts = lm.argmax(-1).astype(np.int32)
    toks, lens, _ = isd_accept(lc, lm, drafts, 3, 0.0, dtype="f32")
    am = lc.argmax(-1)
    for b in range(B):
        j = 0
        while j < N - 1 and drafts[b, j] == am[b, j]:
            j += 1
        assert lens[b] == j + 1
        assert list(toks[b, :j + 1]) == list(drafts[b, :j]) + [am[b, j]]


def test_n1_is_categorical_sampling():
    rng = np.random.default_rng(12)
    V, B = 40, 400
    lc = (rng.standard_normal((B, 1, V)) * 2).astype(np.float32)
    lm = np.zeros((B, 0, V), dtype=np.float32)
    drafts = np.zeros((B, 0), dtype=np.int32)
    seed = 0xABCDEF
    toks, lens, _ = isd_accept(lc, lm, drafts, seed, 1.0, dtype="f32")
    assert np.all(lens == 1)
    for b in range(B):
        p = special.softmax(lc[b, 0].astype(np.float64))
        u2 = isd_uniforms(seed, b, 0)[1]
        assert toks[b, 0] == np.searchsorted(np.cumsum(p), u2 * p.sum(), side="right")


def test_temperature_scales_logits():
    rng = np.random.default_rng(13)
    V, N, B = 24, 3, 50
    lc = rng.standard_normal((B, N, V))
    lm = rng.standard_normal((B, N - 1, V))
    drafts = rng.integers(0, V, size=(B, N - 1)).astype(np.int32)
    a = isd_accept(lc, lm, drafts, 21, 0.7)
    b = isd_accept(lc / 0.7, lm / 0.7, drafts, 21, 1.0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    for ia, ib in zip(a[2], b[2]):
        assert np.allclose(ia["p"], ib["p"], rtol=1e-12) and np.allclose(ia["q"], ib["q"], rtol=1e-12)


def test_draft_without_mass_under_p_is_rejected():
    """min(1, p(x)/q(x)) is 0 when p(x) = 0: such a draft is never kept, even
    when q(x) = 0 too (a draft no proposal could have made).  Greedy (T = 0):
    a draft that is the argmax of neither its clean nor its MASK row is
    rejected and the clean argmax is committed in its place.  Sampled: a
    draft whose logit is -1000 below both rows' maxima has p(x) = q(x) = 0
    exactly in float64 and is rejected for every u."""
    rng = np.random.default_rng(14)
    V, N, B = 20, 4, 60
    lc = rng.standard_normal((B, N, V)).astype(np.float32)
    lm = rng.standard_normal((B, N - 1, V)).astype(np.float32)
    am_c, am_m = lc.argmax(-1), lm.argmax(-1)
    drafts = np.empty((B, N - 1), dtype=np.int32)
    for b in range(B):
        for i in range(N - 1):
            drafts[b, i] = next(v for v in range(V) if v != am_c[b, i] and v != am_m[b, i])
    toks, lens, _ = isd_accept(lc, lm, drafts, 7, 0.0, dtype="f32")
    assert np.all(lens == 1)
    assert np.array_equal(toks[:, 0], am_c[:, 0])

    lc2, lm2 = lc.astype(np.float64), lm.astype(np.float64)
    x = 5
    lc2[:, 0, x] = -1000.0
    lm2[:, 0, x] = -1000.0
    d2 = np.full((B, N - 1), x, dtype=np.int32)
    _, lens2, infos = isd_accept(lc2, lm2, d2, 8, 1.0)
    assert all(info["p"][0] == 0.0 and info["q"][0] == 0.0 for info in infos)
    assert np.all(lens2 == 1)
    P = [softmax_t(r, 1.0) for r in lc2[0]]
    Q = [softmax_t(r, 1.0) for r in lm2[0]]
    for u in (0.0, 0.5, TOP):
        assert not _accepted_at(P, Q, list(d2[0]), 0, u)
