"""Pins of oracle.propose."""

import numpy as np
from scipy import stats

from oracle.accept import isd_accept
from oracle.philox import MASK64, philox4x64_10, propose_uniform
from oracle.propose import isd_propose, propose_row
from oracle.tpf import simulate_chain, tpf_closed_form


def test_uniform_stream_is_apart_from_acceptance():
    w_acc = philox4x64_10((2, 0, 0, 0), (7, 3))
    w_pro = philox4x64_10((2, 1, 0, 0), (7, 3))
    assert w_acc != w_pro
    assert propose_uniform(7, 3, 2) == float(w_pro[0] >> 40) * 2.0 ** -24


def test_grid_integration_follows_softmax():
    # Every uniform on the 2**-24 grid, bucketed by the draft it gives: the
    # mass per token is the softmax probability to within one grid step.
    rng = np.random.default_rng(5)
    z = rng.normal(0, 2, size=12)
    for T in (1.0, 0.6):
        p = np.exp((z - z.max()) / T)
        p /= p.sum()
        # the draft is monotone in u: find each token's u-interval by bisection
        edges = [0]
        for v in range(len(z)):
            lo, hi = edges[-1], 1 << 24
            while lo < hi:  # first grid point giving a draft > v
                mid = (lo + hi) // 2
                if propose_row(z, mid * 2.0 ** -24, T) > v:
                    hi = mid
                else:
                    lo = mid + 1
            edges.append(lo)
        mass = np.diff(edges) * 2.0 ** -24
        assert np.allclose(mass, p, atol=2.0 ** -23), (mass, p)


def test_chi_square_of_seeded_draws():
    V, K, n = 16, 2, 20000
    rng = np.random.default_rng(8)
    rows = rng.normal(0, 1.5, size=(1, K, V))
    drafts = np.array([[3, 4]], dtype=np.int32)
    counts = np.zeros((K, V))
    for s in range(n):
        d = isd_propose(rows, drafts, np.array([K + 1]), s, 1.0)
        for i in range(K):
            counts[i, d[0, i]] += 1
    for i in range(K):
        p = np.exp(rows[0, i] - rows[0, i].max())
        p /= p.sum()
        assert stats.chisquare(counts[i], p * n).pvalue > 1e-4


def test_greedy_and_fresh_steps():
    rows = np.array([[[0.0, 3.0, 3.0, 1.0], [5.0, 0.0, 0.0, 5.0]]])
    d = isd_propose(rows, np.array([[1, 2]]), np.array([3]), 0, 0.0)
    assert d.tolist() == [[1, 0]]  # argmax, lowest index on ties
    # a rejection (accept_len < k + 1): the next step is fresh
    assert isd_propose(rows, np.array([[1, 2]]), np.array([2]), 0, 1.0).tolist() == [[-1, -1]]
    # a fresh step (k = 0, accept_len 1) always continues
    d = isd_propose(rows, np.array([[-1, -1]]), np.array([1]), 0, 0.0)
    assert d.tolist() == [[1, 0]]
    # N = 1: nothing to propose
    assert isd_propose(np.zeros((2, 0, 4)), np.zeros((2, 0), dtype=np.int32),
                       np.array([1, 1]), 0, 1.0).shape == (2, 0)


def test_proposal_loop_reaches_closed_form():
    # Rows whose p and q overlap by exactly a: drafts proposed from q by the
    # proposal oracle, verified against p by the acceptance oracle, fresh and
    # verify steps alternating as the two oracles decide.
    V, N, a = 16, 4, 0.9
    K = N - 1
    rng = np.random.default_rng(77)
    r = rng.dirichlet(np.ones(V), size=K)
    s1 = np.zeros((K, V))
    s2 = np.zeros((K, V))
    s1[:, : V // 2] = rng.dirichlet(np.ones(V // 2), size=K)
    s2[:, V // 2:] = rng.dirichlet(np.ones(V - V // 2), size=K)
    P, Q = a * r + (1 - a) * s1, a * r + (1 - a) * s2
    bonus = rng.dirichlet(np.ones(V))
    lc = np.log(np.vstack([P, bonus]))[None]
    lm = np.log(Q)[None]
    state = {"drafts": np.full((1, K), -1, dtype=np.int32), "step": 0}

    def step(verify):
        state["step"] += 1
        d = state["drafts"]
        assert (d[0, 0] >= 0) == verify
        _, n, _ = isd_accept(lc, lm, d, state["step"], 1.0)
        state["drafts"] = isd_propose(lm, d, n, 10_000_000 + state["step"], 1.0)
        return int(n[0]), int(n[0]) == (K + 1 if verify else 1)

    m = simulate_chain(step, 20_000)
    assert abs(m - tpf_closed_form(a, N)) < 0.05


def _numpy_u(counter, key):
    """Uniform from word 0 of a Philox4x64-10 block, via numpy's own generator
    (it increments the 256-bit counter before producing a block)."""
    c = (sum(int(w) << (64 * i) for i, w in enumerate(counter)) - 1) % (1 << 256)
    bg = np.random.Philox(counter=np.array([(c >> (64 * i)) & MASK64 for i in range(4)],
                                           dtype=np.uint64),
                          key=np.array([int(k) & MASK64 for k in key], dtype=np.uint64))
    return (int(bg.random_raw(4)[0]) >> 40) * 2.0 ** -24


def test_draft_i_uses_its_own_counter():
    """Two equally likely tokens: draft i of sequence b is 1 exactly when its
    uniform, word 0 of counter (i, 1, 0, 0) under key (seed, b), is >= 1/2
    (computed here with numpy's Philox), so a shifted stream index fails."""
    B, K, seed = 4, 7, 123456789
    logits = np.zeros((B, K, 2))
    drafts = np.zeros((B, K), dtype=np.int32)
    out = isd_propose(logits, drafts, np.full(B, K + 1), seed, 1.0)
    want = np.array([[int(_numpy_u((i, 1, 0, 0), (seed, b)) >= 0.5) for i in range(K)]
                     for b in range(B)])
    assert np.array_equal(out, want)
    assert 0 < want.sum() < want.size  # both tokens occur, so the check has teeth
