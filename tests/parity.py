"""Helpers shared by the GPU parity tests: run the oracle on a workload and
compare the library's outputs with it.

Tolerances (the oracle is float64; the library computes attention with bf16
MFMA and float32 softmax/accumulation; the acceptance's row statistics with
float32 exponentials summed in float64, its sampling weights wholly in
float64):

* attention: normwise per head vector, max|gpu - ref| / max|ref| over d,
  at most 2e-2 for bf16 storage and 1e-4 for float32 storage;
* p_i(x_i) and q_i(x_i): within 1e-5 absolute;
* accept lengths and committed tokens: equal, except at boundary decisions,
  which are counted and reported: a ratio test with |u - p/q| < 1e-6 (or
  |p - q| < 1e-6 q), or an inverse-CDF pick whose threshold t lies within
  1e-12 * sum(w) of a cumulative-sum boundary (float64 weights on both
  sides).

The library takes T as float32, so the oracle is evaluated at that same
value (float(np.float32(T))).
"""

import numpy as np

from oracle.accept import isd_accept as oracle_accept_batch
from oracle.attention import isd_attention, isd_attention_rows
from oracle.dtypes import to_f64

ATTN_TOL = {"bf16": 2e-2, "f32": 1e-4}
PROB_TOL = 1e-5
RATIO_BAND = 1e-6
CDF_BAND = 1e-12


def q_f64(w):
    return to_f64(w.q, w.qkv_dtype).reshape(w.q.shape)


def oracle_attention(w):
    return isd_attention(q_f64(w), w.kv_pages, w.page_table, w.ctx_lens, w.N, w.Hkv, w.qkv_dtype)


def oracle_attention_rows(w, picks):
    return isd_attention_rows(q_f64(w), w.kv_pages, w.page_table, w.ctx_lens, w.N, w.Hkv,
                              w.qkv_dtype, picks)


def normwise_err(got, ref):
    """max over head vectors of max|got - ref| / max|ref| (last axis = d)."""
    num = np.abs(got - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return float((num / den).max())


def t32(T):
    """The temperature as the library receives it (a float32)."""
    return float(np.float32(T))


def oracle_accept(w, seed=None, T=None):
    return oracle_accept_batch(w.logits_clean, w.logits_mask, w.draft_tokens,
                               w.seed if seed is None else seed, t32(w.T if T is None else T),
                               dtype=w.logits_dtype)


def _ratio_boundary(p, q, u):
    if abs(p - q) <= RATIO_BAND * max(q, 1e-300):
        return True
    return p < q and abs(u - p / q) < RATIO_BAND


def compare_accept(w, tokens, lens, debug, ref):
    """Compare GPU acceptance outputs with the oracle's.

    Returns dict(exact=..., boundary=[...], bad=[...], max_prob_err=...).
    ``debug`` is the library's [B][N+1][4] float64 record (or None).
    """
    o_tok, o_len, infos = ref
    exact, boundary, bad = 0, [], []
    max_prob_err = 0.0
    for b in range(w.B):
        info = infos[b]
        if debug is not None:
            for i, (p, q) in enumerate(zip(info["p"], info["q"])):
                if i < debug.shape[1] - 1 and not np.isnan(debug[b, i, 0]):
                    max_prob_err = max(max_prob_err, abs(debug[b, i, 0] - p),
                                       abs(debug[b, i, 1] - q))
        if lens[b] == o_len[b] and np.array_equal(tokens[b], o_tok[b]):
            exact += 1
            continue
        why = None
        if lens[b] != o_len[b]:
            i = min(int(lens[b]), int(o_len[b])) - 1  # first index where the decisions differ
            if i < len(info["p"]) and _ratio_boundary(info["p"][i], info["q"][i], info["u"][i]):
                why = ("ratio", b, i)
        else:
            t, lo, hi, tot = info["t"], info["cdf_lo"], info["cdf_hi"], info["total"]
            j = int(o_len[b]) - 1
            if np.array_equal(tokens[b][:j], o_tok[b][:j]) and \
                    min(abs(t - lo), abs(hi - t)) < CDF_BAND * tot:
                why = ("cdf", b, j)
        (boundary if why else bad).append(why or (b, list(tokens[b]), list(o_tok[b]),
                                                   int(lens[b]), int(o_len[b])))
    return dict(exact=exact, boundary=boundary, bad=bad, max_prob_err=max_prob_err)
