"""The GPU acceptance path keeps the pages' guarantee: committed tokens follow
the anchor distribution p ("Introspective Diffusion Language Models",
section "Inference & ISD").  10**6 sequences on a 16-token vocabulary, one
launch, drafts redrawn per sequence from q; chi-square per position and on
acceptance lengths, plus bit-exact agreement with the oracle on a subset."""

import numpy as np
import pytest
from scipy import special, stats

from parity import compare_accept
from oracle.accept import isd_accept as oracle_accept_batch

pytestmark = pytest.mark.gpu


def test_gpu_acceptance_follows_p_1e6():
    import torch

    from speculative_verify_isd_amd.lib import alloc_workspace, idlm_isd_accept, make_dims

    V, N, B = 16, 4, 1_000_000
    K = N - 1
    rng = np.random.default_rng(321)
    lc = (rng.standard_normal((N, V)) * 1.2).astype(np.float32)
    lm = (lc[:K] + rng.standard_normal((K, V)) * 0.8).astype(np.float32)
    P = [special.softmax(r.astype(np.float64)) for r in lc]
    Q = [special.softmax(r.astype(np.float64)) for r in lm]
    drafts = np.stack([np.minimum(np.searchsorted(np.cumsum(Q[i]), rng.random(B), side="right"),
                                  V - 1) for i in range(K)], axis=1).astype(np.int32)
    print(f"[case] gpu chi-square B={B} V={V} N={N}", flush=True)
    d = make_dims(B, N, 8, 8, 64, V, 1, 1, "bf16", "f32")
    ws = alloc_workspace(d)
    dev = "cuda"
    tlc = torch.from_numpy(np.broadcast_to(lc, (B, N, V)).copy()).to(dev)
    tlm = torch.from_numpy(np.broadcast_to(lm, (B, K, V)).copy()).to(dev)
    tdr = torch.from_numpy(drafts).to(dev)
    tok = torch.empty((B, N), dtype=torch.int32, device=dev)
    lens = torch.empty(B, dtype=torch.int32, device=dev)
    seed = 0x5EED
    idlm_isd_accept(d, tlc, tlm, tdr, seed, 1.0, tok, lens, None, ws)
    torch.cuda.synchronize()
    tok = tok.cpu().numpy()
    lens = lens.cpu().numpy()
    assert lens.min() >= 1 and lens.max() <= N
    for k in range(N):
        sel = lens > k
        counts = np.bincount(tok[sel, k], minlength=V)
        pval = stats.chisquare(counts, counts.sum() * P[k]).pvalue
        print(f"[chi2] position {k}: n={sel.sum()} p-value {pval:.3g}", flush=True)
        assert pval > 1e-3
    a = [1.0 - 0.5 * np.abs(P[i] - Q[i]).sum() for i in range(K)]
    probs = np.array([np.prod(a[:k]) * ((1 - a[k]) if k < K else 1.0) for k in range(N)])
    pval = stats.chisquare(np.bincount(lens, minlength=N + 1)[1:], probs * B).pvalue
    print(f"[chi2] accept lengths p-value {pval:.3g}", flush=True)
    assert pval > 1e-3
    # bit-exact agreement with the oracle on the first 3000 sequences
    n = 3000

    class Sub:
        B = n

    ref = oracle_accept_batch(np.broadcast_to(lc, (n, N, V)), np.broadcast_to(lm, (n, K, V)),
                              drafts[:n], seed, 1.0, dtype="f32")
    res = compare_accept(Sub, tok[:n], lens[:n], None, ref)
    print(f"[oracle] exact {res['exact']}/{n} boundary {res['boundary']}", flush=True)
    assert not res["bad"]
