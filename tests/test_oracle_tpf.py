"""Pins for the tokens-per-forward model (oracle.tpf) and, through it, for the
acceptance oracle's step semantics.

* golden: the pages' worked values (tests/golden/pages_worked_values.json);
* limits: p = 1 gives N tokens per forward, p = 0 gives 1;
* Monte Carlo: the fresh/verify chain with Bernoulli acceptance has the
  closed form as its mean;
* end to end: the same chain driven by the real acceptance oracle on
  16-token rows whose overlap sum(min(p, q)) is exactly 0.9 reaches the
  closed form at p = 0.9 (about 2.92 at N = 4).
"""

import json
import os

import numpy as np
import pytest

from oracle.accept import isd_accept
from oracle.tpf import bernoulli_step, compute_efficiency, simulate_chain, tpf_closed_form

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_worked_values.json")


def test_pages_worked_values():
    g = json.load(open(GOLDEN))
    w = g["tpf_idlm"]
    tpf = tpf_closed_form(w["p"], w["N"])
    assert round(tpf, w["tpf_printed_decimals"]) == w["tpf_printed"]
    assert 2 * w["N"] - 1 == w["queries_per_forward"] == g["queries_formula"]["queries"]
    eff = compute_efficiency(tpf, w["queries_per_forward"])
    assert round(eff, w["efficiency_printed_decimals"]) == w["efficiency_printed"]


@pytest.mark.parametrize("N", [2, 3, 4, 8, 16])
def test_limits(N):
    assert abs(tpf_closed_form(1.0, N) - N) < 1e-12
    assert abs(tpf_closed_form(0.0, N) - 1.0) < 1e-12
    ps = np.linspace(0, 1, 21)
    vals = [tpf_closed_form(p, N) for p in ps]
    assert all(b >= a for a, b in zip(vals, vals[1:]))  # more acceptance, more tokens


def test_n2_closed_form():
    # N = 2: one draft, commit 2 when kept (stay) or 1 (go fresh), fresh commits 1.
    for p in (0.1, 0.5, 0.9):
        assert abs(tpf_closed_form(p, 2) - 2.0 / (2.0 - p)) < 1e-15


@pytest.mark.parametrize("N,p", [(2, 0.5), (4, 0.9), (4, 0.5), (8, 0.9)])
def test_bernoulli_chain_matches_closed_form(N, p):
    rng = np.random.default_rng(N * 100 + int(p * 10))
    steps = 200_000
    m = simulate_chain(bernoulli_step(p, N, rng), steps)
    assert abs(m - tpf_closed_form(p, N)) < 0.02


def _rows_with_overlap(rng, V, a):
    """p = a*r + (1-a)*s1, q = a*r + (1-a)*s2 with s1, s2 on disjoint halves: sum(min(p, q)) = a."""
    r = rng.dirichlet(np.ones(V))
    s1 = np.zeros(V)
    s2 = np.zeros(V)
    s1[: V // 2] = rng.dirichlet(np.ones(V // 2))
    s2[V // 2:] = rng.dirichlet(np.ones(V - V // 2))
    return a * r + (1 - a) * s1, a * r + (1 - a) * s2


def test_real_acceptance_reaches_closed_form():
    V, N, a = 16, 4, 0.9
    K = N - 1
    rng = np.random.default_rng(2024)
    pairs = [_rows_with_overlap(rng, V, a) for _ in range(K)]
    for p, q in pairs:
        assert abs(np.minimum(p, q).sum() - a) < 1e-12
    bonus = rng.dirichlet(np.ones(V))
    lc = np.log(np.stack([p for p, _ in pairs] + [bonus]))[None]
    lm = np.log(np.stack([q for _, q in pairs]))[None]
    qrows = [q for _, q in pairs]
    step_no = [0]

    def step(verify):
        step_no[0] += 1
        if verify:
            d = [rng.choice(V, p=qrows[i]) for i in range(K)]
        else:
            d = [-1] * K
        toks, n, _ = isd_accept(lc, lm, np.array([d], dtype=np.int32), step_no[0], 1.0)
        n = int(n[0])
        if not verify:
            assert n == 1
        return n, n == N

    m = simulate_chain(step, 30_000)
    want = tpf_closed_form(a, N)
    assert abs(want - 2.919) < 1e-3
    assert abs(m - want) < 0.05
