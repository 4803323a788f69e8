"""Drafts for the next step, and the fresh / verify alternation.
Test infrastructure.

What the pages fix
------------------
* MASK positions propose the next tokens from the distribution q their rows
  give ("Introspective Diffusion Language Models", section "Inference & ISD";
  GeekNews summary, same section); argmax proposals are one serving option
  ("Serving (SGLang)").
* Decoding alternates steps that only propose with steps that verify and
  propose; the tokens-per-forward closed form of the speedup-explorer panel
  is the stationary mean of exactly that two-state chain (``oracle.tpf``).

Readings taken where the pages are silent
-----------------------------------------
* A step's MASK proposals are usable by the next step only if every draft
  this step listed was kept (accept_len == k + 1, k the listed drafts; k = 0
  is a fresh step, which always continues).  After a rejection the proposals
  were conditioned on a rejected token, so the next step is fresh: its draft
  list is all -1.
* Draft i is drawn from softmax(next_i / T) by inverse CDF (ascending
  vocabulary, smallest v whose running sum exceeds t = u * sum(w), guard: the
  last positive weight) with u = word 0 of the Philox4x64-10 block at counter
  (i, 1, 0, 0) under key (seed, b); T = 0 takes the argmax (lowest index).

Pinned in tests/test_oracle_propose.py: exact integration over the 2**-24
uniform grid (each draft follows softmax(next / T)), chi-square of the seeded
path, greedy and fresh-step special cases, and the tokens-per-forward closed
form reached by a loop of the real acceptance and proposal oracles.
"""

import numpy as np

from .accept import inverse_cdf, num_drafts
from .dtypes import to_f64
from .philox import propose_uniform


def propose_row(logits, u, T):
    """One draft from one float64 logit row given its uniform."""
    z = np.asarray(logits, dtype=np.float64)
    if T == 0:
        return int(np.argmax(z))
    w = np.exp((z - z.max()) / T)
    v, _, _ = inverse_cdf(w, u * w.sum())
    return v


def isd_propose(logits_next, drafts, accept_len, seed, T, dtype="f64"):
    """Next-step drafts int32 [B][K] (all -1 where the next step is fresh).

    logits_next [B][K][V] storage ``dtype``; drafts int [B][K] (this step's
    list); accept_len int [B] from the acceptance stage.
    """
    B, K, V = logits_next.shape
    out = np.full((B, K), -1, dtype=np.int32)
    for b in range(B):
        k = num_drafts(drafts[b]) if K else 0
        if int(accept_len[b]) != k + 1:
            continue
        for i in range(K):
            out[b, i] = propose_row(to_f64(logits_next[b, i], dtype), propose_uniform(seed, b, i), T)
    return out
