"""GPU parity of idlm_isd_propose against oracle.propose, and the fresh /
verify decode loop run on the GPU (acceptance then proposal, step after
step) reaching the tokens-per-forward closed form."""

import numpy as np
import pytest

from oracle.dtypes import to_f64
from oracle.philox import propose_uniform
from oracle.propose import isd_propose
from oracle.tpf import tpf_closed_form
from speculative_verify_isd_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available()
    return torch


def _dev(torch, a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16" and a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def _boundary(row, dtype, T, seed, b, i, got, want):
    """Whether the oracle's t sits within 1e-6 of the total from a running-sum
    boundary between the two picks (a rounding tie)."""
    z = to_f64(row, dtype)
    w = np.exp((z - z.max()) / T)
    c = np.cumsum(w)
    t = propose_uniform(seed, b, i) * c[-1]
    lo, hi = min(got, want), max(got, want)
    return bool(np.min(np.abs(c[lo:hi] - t)) < 1e-6 * c[-1]) if hi > lo else False


def run_case(torch, B, N, V, dtype, T, seed, keep_frac=0.6):
    from speculative_verify_isd_amd import lib as L

    K = N - 1
    rng = np.random.default_rng(seed)
    nxt = rng.normal(0, 3, size=(B, K, V)).astype(np.float32)
    nxt_store = W.f32_to_bf16_bits(nxt) if dtype == "bf16" else nxt
    drafts = rng.integers(0, V, size=(B, K)).astype(np.int32)
    k = rng.integers(0, K + 1, size=B)  # listed drafts
    for b in range(B):
        drafts[b, k[b]:] = -1
    keep = rng.random(B) < keep_frac
    lens = np.where(keep, k + 1, np.maximum(1, rng.integers(1, K + 1, size=B))).astype(np.int32)
    lens = np.where(~keep & (lens == k + 1), np.maximum(1, k), lens).astype(np.int32)
    dims = L.make_dims(B, N, 8, 2, 64, V, 4, 4, "f32", dtype)
    ws = L.alloc_workspace(dims)
    out = torch.full((B, K), -7, dtype=torch.int32, device="cuda")
    L.idlm_isd_propose(dims, _dev(torch, nxt_store, dtype), _dev(torch, drafts, None),
                       _dev(torch, lens, None), seed, T, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = isd_propose(nxt_store, drafts, lens, seed, T, dtype=dtype)
    bad, ties = [], []
    for b in range(B):
        for i in range(K):
            if got[b, i] == want[b, i]:
                continue
            if T > 0 and want[b, i] >= 0 and got[b, i] >= 0 and \
                    _boundary(nxt_store[b, i], dtype, T, seed, b, i, int(got[b, i]), int(want[b, i])):
                ties.append((b, i))
            else:
                bad.append((b, i, int(got[b, i]), int(want[b, i])))
    fresh = int((want[:, 0] < 0).sum()) if K else 0
    print(f"[propose] B={B} N={N} V={V} {dtype} T={T}: exact {B * K - len(bad) - len(ties)}/"
          f"{B * K}, ties {ties}, fresh sequences {fresh}", flush=True)
    assert not bad, bad[:5]
    assert len(ties) <= 2
    return got


@pytest.mark.parametrize("B,N,V,dtype,T", [
    (16, 4, 151936, "bf16", 1.0), (64, 4, 151936, "bf16", 0.7), (8, 8, 151936, "bf16", 1.0),
    (16, 4, 151936, "bf16", 0.0), (12, 4, 512, "f32", 1.0), (12, 3, 1000, "f32", 1.0),
    (5, 4, 77, "bf16", 1.0), (3, 16, 5000, "bf16", 1.0),
    # nearly one-hot (most weights underflow) and nearly uniform proposals
    (16, 4, 5000, "bf16", 0.05), (16, 4, 5000, "bf16", 20.0),
])
def test_propose_matches_oracle(torch_cuda, B, N, V, dtype, T):
    run_case(torch_cuda, B, N, V, dtype, T, seed=B * 131 + N)


def test_propose_n1_is_a_no_op(torch_cuda):
    torch = torch_cuda
    from speculative_verify_isd_amd import lib as L

    dims = L.make_dims(4, 1, 8, 2, 64, 64, 4, 4, "f32", "f32")
    ws = L.alloc_workspace(dims)
    z = torch.zeros(1, dtype=torch.int32, device="cuda")
    L.idlm_isd_propose(dims, torch.zeros(1, device="cuda"), z, z, 1, 1.0, z, ws)
    torch.cuda.synchronize()


def test_decode_loop_reaches_closed_form(torch_cuda):
    """Rows whose p and q overlap by exactly a = 0.9 at every draft position;
    each step runs the acceptance on the current drafts, then the proposal on
    the same q rows.  The mean committed tokens per forward over all
    sequences and steps is the closed form (2 + p + p^2) / (2 - p^3) at N = 4."""
    torch = torch_cuda
    from speculative_verify_isd_amd import lib as L

    B, N, V, a, steps = 512, 4, 64, 0.9, 400
    K = N - 1
    rng = np.random.default_rng(2025)
    r = rng.dirichlet(np.ones(V), size=K)
    s1 = np.zeros((K, V))
    s2 = np.zeros((K, V))
    s1[:, : V // 2] = rng.dirichlet(np.ones(V // 2), size=K)
    s2[:, V // 2:] = rng.dirichlet(np.ones(V - V // 2), size=K)
    P, Q = a * r + (1 - a) * s1, a * r + (1 - a) * s2
    assert np.allclose(np.minimum(P, Q).sum(axis=1), a)
    bonus = rng.dirichlet(np.ones(V))
    lc = np.broadcast_to(np.log(np.vstack([P, bonus])).astype(np.float32), (B, N, V)).copy()
    lm = np.broadcast_to(np.log(Q).astype(np.float32), (B, K, V)).copy()
    dims = L.make_dims(B, N, 8, 2, 64, V, 4, 4, "f32", "f32")
    ws = L.alloc_workspace(dims)
    d_lc, d_lm = _dev(torch, lc, "f32"), _dev(torch, lm, "f32")
    drafts = torch.full((B, K), -1, dtype=torch.int32, device="cuda")
    nxt = torch.empty_like(drafts)
    toks = torch.empty((B, N), dtype=torch.int32, device="cuda")
    lens = torch.empty(B, dtype=torch.int32, device="cuda")
    total = torch.zeros(B, dtype=torch.int64, device="cuda")
    for step in range(steps):
        L.idlm_isd_accept(dims, d_lc, d_lm, drafts, step + 1, 1.0, toks, lens, None, ws)
        if step == 0:
            torch.cuda.synchronize()
            assert (lens == 1).all()  # a fresh start commits one token
        total += lens
        L.idlm_isd_propose(dims, d_lm, drafts, lens, 1_000_000 + step, 1.0, nxt, ws)
        drafts, nxt = nxt, drafts
    torch.cuda.synchronize()
    assert L.idlm_isd_read_status(ws) == 0
    tpf = float(total.sum().item()) / (B * steps)
    want = tpf_closed_form(a, N)
    print(f"[loop] GPU decode loop: {B} sequences x {steps} forwards, tokens per forward "
          f"{tpf:.4f} vs closed form {want:.4f}", flush=True)
    assert abs(tpf - want) < 0.02
