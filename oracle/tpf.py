"""Tokens per forward (TPF) of strided decoding.  Test infrastructure.

The pages give, for stride N and per-draft acceptance rate p, the
memory-bound speedup estimate TPF = (2 + p + ... + p^(N-2)) / (2 - p^(N-1))
(speedup-explorer panel of "Introspective Diffusion Language Models" and
section "Speedup Factor Explorer" of the GeekNews summary; the extracted text
prints the exponents inline).  They work it at N = 4, p = 0.9: TPF about 2.9
with 2N-1 = 7 queries per forward and compute efficiency TPF^2 / 7 about 1.22
(section "How do DLMs perform as they approach compute-bound?").

The formula is the stationary mean of a two-state decode chain, which is how
this module reads it:

* verify state: the step carries K = N-1 drafts; each is kept with
  probability p in turn; the step commits the kept prefix plus one token (a
  resample at the first rejection, or the bonus when all K are kept).  All
  kept: stay.  A rejection: the MASK proposals of this step were conditioned
  on the rejected draft, so move to the fresh state.
* fresh state: no valid drafts; the step commits the anchor's token and
  proposes anew; move to the verify state.

Stationary weight of the verify state is 1 / (2 - p^(N-1)); the verify state
commits sum_{k<N} p^k on average and the fresh state 1, which gives the
formula.  ``simulate_chain`` runs the chain with any per-step acceptance
function, so tests can drive it with the real acceptance oracle.

Pinned in tests/test_oracle_tpf.py against the pages' worked values (golden
fixture), the limits p = 0 and p = 1, and Monte Carlo runs of the chain.
"""

import numpy as np


def tpf_closed_form(p, N):
    """(2 + p + ... + p^(N-2)) / (2 - p^(N-1)) for stride N >= 2."""
    if N < 2:
        raise ValueError("the strided-decoding formula needs N >= 2")
    num = 2.0 + sum(p ** k for k in range(1, N - 1))
    return num / (2.0 - p ** (N - 1))


def compute_efficiency(tpf, queries):
    """Useful output per unit of compute relative to AR decoding: TPF^2 / queries."""
    return tpf * tpf / queries


def simulate_chain(step, steps):
    """Run the fresh/verify chain for ``steps`` forwards.

    ``step(verify)`` performs one forward in the given state and returns
    (committed_tokens, all_drafts_kept).  Starts in the fresh state.
    Returns the mean committed tokens per forward.
    """
    verify = False
    total = 0
    for _ in range(steps):
        committed, all_kept = step(verify)
        total += committed
        verify = bool(verify and all_kept) or not verify
    return total / steps


def bernoulli_step(p, N, rng):
    """A chain step where each draft is kept independently with probability p."""
    K = N - 1

    def step(verify):
        if not verify:
            return 1, True
        for i in range(K):
            if rng.random() >= p:
                return i + 1, False
        return N, True

    return step
