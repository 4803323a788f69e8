"""The ISD acceptance stage: p/q ratio test, residual resampling, truncation.
Test infrastructure.

What the pages fix
------------------
* MASK positions propose new tokens with a distribution q; clean positions
  verify the earlier tokens with the anchor distribution p
  ("Introspective Diffusion Language Models", section "Inference & ISD";
  GeekNews summary, section "Inference & ISD").
* A proposed token x is kept with probability min(1, p(x)/q(x)), and this is
  what makes the output follow the autoregressive distribution (same
  sections).
* Acceptance compounds along the stride: a later token is kept only if every
  earlier one was (ojeo.com article; the closed form in the speedup-explorer
  panel has the same structure).

Readings taken where the pages are silent
-----------------------------------------
* Rows.  The step has N clean rows (K = N-1 verifying rows plus the anchor of
  the position after the last draft) and K MASK rows: 2N-1 rows in all.  Clean
  row i gives p_i, the distribution that verifies draft i; MASK row i gives
  q_i, the distribution draft i was proposed from.  With all K drafts kept,
  clean row K supplies a bonus token, so a step commits up to N tokens, as
  the tokens-per-forward closed form requires (it reaches N at p = 1).
* Temperature.  p_i = softmax(clean_i / T) and q_i = softmax(mask_i / T) with
  the same T; T = 0 means greedy one-hot rows (lowest index wins ties), which
  is the argmax-proposal case of "Serving (SGLang)".
* Residual.  At the first rejected position j the committed token is drawn
  from normalize(max(0, p_j - q_j)), the only rule under which the output
  follows p; if that residual sums to zero, p_j is used.
* Comparison.  Draft i is kept iff p_i(x) > 0 and (p_i(x) >= q_i(x) or
  u_i * q_i(x) < p_i(x)), which is a draw with probability min(1, p/q)
  without a division; a token p gives no mass is never kept (min(1, 0/q) is
  0, and with q(x) = 0 as well such a draft could not have been proposed).
* Inverse CDF.  t = u' * sum(w); the token is the smallest v (ascending
  vocabulary order) whose running sum of w exceeds t; if rounding leaves
  none, the largest v with positive weight.
* Short draft lists.  A draft of -1 ends the list early (k < K drafts); the
  bonus then comes from clean row k.  k = 0 is the step right after a
  rejection, which commits exactly one token.
* Uniforms come from Philox4x64-10 (see ``oracle.philox``): u_i is word 0 and
  u'_i word 1 of the block at counter (i, 0, 0, 0) under key (seed, b).

``accept_with_uniforms`` is the step as a function of explicit uniforms; it
lets tests integrate the output distribution exactly over the 2**-24 grid.
``isd_accept`` wires in the Philox uniforms and loops over the batch.

Pinned in tests/test_oracle_accept.py: exact grid integration showing that
each committed token follows p (the pages' guarantee) and that acceptance
lengths follow the product of 1 - TV(p_i, q_i); chi-square tests of the
seeded path; the q == p, one-hot, greedy and N = 1 (plain categorical
sampling, numpy searchsorted) special cases; and the tokens-per-forward
closed form reached by the real acceptance loop (tests/test_oracle_tpf.py).
"""

import numpy as np

from .dtypes import to_f64
from .philox import isd_uniforms


def softmax_t(logits, T):
    """Temperature softmax of one float64 logit row; T == 0 gives argmax one-hot."""
    z = np.asarray(logits, dtype=np.float64)
    if T == 0:
        out = np.zeros_like(z)
        out[int(np.argmax(z))] = 1.0  # numpy argmax returns the lowest index on ties
        return out
    z = z / T
    e = np.exp(z - z.max())
    return e / e.sum()


def num_drafts(drafts):
    """Drafts before the first -1 terminator."""
    for i, x in enumerate(drafts):
        if int(x) < 0:
            return i
    return len(drafts)


def inverse_cdf(w, t):
    """Smallest index whose running sum of ``w`` exceeds ``t``.

    Also returns the running sums just before and at that index, so callers
    can see how far ``t`` sat from a boundary.
    """
    c = np.cumsum(w)
    hits = np.nonzero(c > t)[0]
    if hits.size:
        v = int(hits[0])
    else:
        v = int(np.nonzero(w > 0)[0][-1])
    lo = float(c[v - 1]) if v > 0 else 0.0
    return v, lo, float(c[v])


def accept_with_uniforms(P, Q, drafts, u, u2):
    """One sequence's acceptance as a function of explicit uniforms.

    P      list of N float64 probability rows (clean rows 0..N-1)
    Q      list of K = N-1 float64 probability rows (MASK rows)
    drafts K ints; -1 ends the list early
    u      K ratio-test uniforms (u[i] used for draft i)
    u2     K+1 sampling uniforms (u2[j] used at the resample/bonus index j)

    Returns (accept_len, tokens[N] padded with -1, info dict); info["w"] is
    the weight row the token was drawn from (unnormalised).
    """
    N = len(P)
    K = N - 1
    assert len(Q) == K and len(drafts) == K
    kp = num_drafts(drafts)
    info = {"p": [], "q": [], "u": [], "u2": []}
    j = kp
    for i in range(kp):
        x = int(drafts[i])
        p, q = float(P[i][x]), float(Q[i][x])
        info["p"].append(p)
        info["q"].append(q)
        info["u"].append(float(u[i]))
        info["u2"].append(float(u2[i]))
        if not (p > 0 and (p >= q or u[i] * q < p)):
            j = i
            break
    if j < kp:
        w = np.maximum(0.0, P[j] - Q[j])
        info["mode"] = "residual"
    else:
        w = np.asarray(P[kp], dtype=np.float64)
        info["mode"] = "bonus"
    if not w.sum() > 0:
        w = np.asarray(P[j], dtype=np.float64)
        info["mode"] += "-fallback"
    total = float(w.sum())
    t = float(u2[j]) * total
    v, lo, hi = inverse_cdf(w, t)
    tokens = [int(x) for x in drafts[:j]] + [v] + [-1] * (N - j - 1)
    info.update(j=j, total=total, t=t, cdf_lo=lo, cdf_hi=hi, u2_used=float(u2[j]), w=w)
    return j + 1, tokens, info


def isd_accept(logits_clean, logits_mask, drafts, seed, T, dtype="f64"):
    """The acceptance stage for a batch.

    logits_clean [B][N][V], logits_mask [B][N-1][V] in storage ``dtype``
    ("bf16" bit patterns, "f32" or "f64"); drafts int [B][N-1]; seed a
    64-bit integer; T >= 0.

    Returns (tokens int32 [B][N], accept_len int32 [B], infos list).
    """
    B, N, V = logits_clean.shape
    K = N - 1
    tokens = np.full((B, N), -1, dtype=np.int32)
    lens = np.zeros(B, dtype=np.int32)
    infos = []
    for b in range(B):
        P = [softmax_t(to_f64(logits_clean[b, i], dtype), T) for i in range(N)]
        Q = [softmax_t(to_f64(logits_mask[b, i], dtype), T) for i in range(K)]
        u, u2 = [], []
        for i in range(N):
            a, c = isd_uniforms(seed, b, i)
            u.append(a)
            u2.append(c)
        n, toks, info = accept_with_uniforms(P, Q, [int(x) for x in drafts[b]], u[:K], u2)
        lens[b] = n
        tokens[b] = toks
        infos.append(info)
    return tokens, lens, infos
