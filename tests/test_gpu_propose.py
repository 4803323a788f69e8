"""GPU parity of idlm_isd_propose against oracle.propose, and the fresh /
verify decode loop run on the GPU (acceptance then proposal, step after
step) reaching the tokens-per-forward closed form."""

import numpy as np
import pytest

from oracle.dtypes import to_f64
from oracle.philox import propose_uniform
from oracle.propose import isd_propose
from oracle.tpf import tpf_closed_form
from parity import CDF_BAND
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
    """Whether the oracle's t sits within CDF_BAND (1e-12) of the total from a
    running-sum boundary between the two picks: float64 weights on both
    sides, so only a tie to float64 rounding may pick differently."""
    z = to_f64(row, dtype)
    w = np.exp((z - z.max()) / T)
    c = np.cumsum(w)
    t = propose_uniform(seed, b, i) * c[-1]
    lo, hi = min(got, want), max(got, want)
    return bool(np.min(np.abs(c[lo:hi] - t)) < CDF_BAND * c[-1]) if hi > lo else False


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


def test_propose_many_draws_full_vocabulary(torch_cuda):
    """Thousands of proposal draws over 151936-entry bf16 rows (32 seeds of a
    B = 64, N = 4 batch, every sequence continuing): with float64 weights on
    both sides, no pick may differ from the oracle's outside the 1e-12 band."""
    torch = torch_cuda
    from speculative_verify_isd_amd import lib as L

    B, N, V, T, seeds = 64, 4, W.VOCAB, 1.0, 32
    K = N - 1
    rng = np.random.default_rng(4242)
    nxt = rng.normal(0, 3, size=(B, K, V)).astype(np.float32)
    nxt_store = W.f32_to_bf16_bits(nxt)
    drafts = rng.integers(0, V, size=(B, K)).astype(np.int32)
    lens = np.full(B, K + 1, dtype=np.int32)  # every draft kept: all continue
    dims = L.make_dims(B, N, 8, 2, 64, V, 4, 4, "f32", "bf16")
    ws = L.alloc_workspace(dims)
    d_nxt, d_drafts, d_lens = (_dev(torch, nxt_store, "bf16"), _dev(torch, drafts, None),
                               _dev(torch, lens, None))
    out = torch.full((B, K), -7, dtype=torch.int32, device="cuda")
    n, ties = 0, 0
    for s in range(seeds):
        seed = 0xD0C0 + 977 * s
        L.idlm_isd_propose(dims, d_nxt, d_drafts, d_lens, seed, T, out, ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        want = isd_propose(nxt_store, drafts, lens, seed, T, dtype="bf16")
        for b, i in zip(*np.nonzero(got != want)):
            assert _boundary(nxt_store[b, i], "bf16", T, seed, b, i, int(got[b, i]),
                             int(want[b, i])), (seed, b, i, int(got[b, i]), int(want[b, i]))
            ties += 1
        n += B * K
    print(f"[propose] {n} draws over V={V}: ties within 1e-12 {ties}", flush=True)
    assert ties <= 2


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


@pytest.mark.parametrize("B,steps", [(16, 6), (64, 3)])  # one / two sub-chunks per summing WG
@pytest.mark.parametrize("T", [1.0, 0.0])
def test_loop_with_mask_stats_matches_plain_acceptance(torch_cuda, T, B, steps):
    """A decode loop over changing logits (clean rows of step t = MASK rows of
    step t-1 plus N(0, 0.5^2), bonus and new MASK rows fresh): the proposals
    record their MASK rows' statistics, and the acceptance of their drafts
    with that record (only the N clean rows reduced) gives the same tokens
    and lengths as without it, and as the oracle."""
    torch = torch_cuda
    from speculative_verify_isd_amd import lib as L
    from oracle.accept import isd_accept as oracle_accept_batch

    N, V, sigma = 4, 151936, 0.5
    K = N - 1
    rng = np.random.default_rng(77 + int(T) + B)
    mask = [rng.normal(0, 3, (B, K, V)).astype(np.float32)]
    clean = [None]
    for t in range(1, steps + 1):
        c = np.empty((B, N, V), dtype=np.float32)
        c[:, :K] = mask[t - 1] + rng.normal(0, sigma, (B, K, V)).astype(np.float32)
        c[:, K] = rng.normal(0, 3, (B, V)).astype(np.float32)
        clean.append(W.f32_to_bf16_bits(c))
        mask.append(rng.normal(0, 3, (B, K, V)).astype(np.float32))
    mask = [W.f32_to_bf16_bits(m) for m in mask]
    dims = L.make_dims(B, N, 8, 2, 64, V, 4, 4, "bf16", "bf16")
    ws = L.alloc_workspace(dims)
    ms = L.alloc_mask_stats(dims)
    dev = lambda a: _dev(torch, a, "bf16")
    drafts = torch.full((B, K), -1, dtype=torch.int32, device="cuda")
    lens = torch.ones(B, dtype=torch.int32, device="cuda")
    nxt = torch.empty_like(drafts)
    toks_a, toks_b = (torch.empty((B, N), dtype=torch.int32, device="cuda") for _ in range(2))
    lens_a, lens_b = (torch.empty(B, dtype=torch.int32, device="cuda") for _ in range(2))
    verified = 0
    for t in range(1, steps + 1):
        d_prev, d_clean = dev(mask[t - 1]), dev(clean[t])
        L.idlm_isd_propose(dims, d_prev, drafts, lens, 500 + t, T, nxt, ws, mask_stats=ms)
        L.idlm_isd_accept(dims, d_clean, d_prev, nxt, t, T, toks_a, lens_a, None, ws)
        L.idlm_isd_accept(dims, d_clean, d_prev, nxt, t, T, toks_b, lens_b, None, ws,
                          mask_stats=ms)
        torch.cuda.synchronize()
        assert L.idlm_isd_read_status(ws) == 0
        ta, tb = toks_a.cpu().numpy(), toks_b.cpu().numpy()
        la, lb = lens_a.cpu().numpy(), lens_b.cpu().numpy()
        dr = nxt.cpu().numpy()
        assert np.array_equal(la, lb) and np.array_equal(ta, tb), t
        o_tok, o_len, _ = oracle_accept_batch(clean[t], mask[t - 1], dr, t, float(np.float32(T)),
                                              dtype="bf16")
        assert np.array_equal(o_len, la) and np.array_equal(o_tok, ta), t
        verified += int((dr[:, 0] >= 0).sum())
        drafts.copy_(nxt)
        lens.copy_(lens_a)
    print(f"[loop] B={B} T={T}: {steps} steps, {verified} verifying sequence-steps, mask-stats "
          f"acceptance identical to the plain one and to the oracle", flush=True)
    assert verified >= B  # the record was actually used

    # A record made at another temperature, or for other drafts, is flagged.
    d_prev = dev(mask[steps - 1])
    L.idlm_isd_propose(dims, d_prev, drafts, lens, 900, 0.7 if T else 1.0, nxt, ws, mask_stats=ms)
    L.idlm_isd_accept(dims, dev(clean[steps]), d_prev, nxt, 1, T, toks_b, lens_b, None, ws,
                      mask_stats=ms)
    torch.cuda.synchronize()
    flagged = L.idlm_isd_read_status(ws)
    verifying = bool((nxt[:, 0] >= 0).any().item())
    assert flagged == (7 if verifying else 0)


def test_loop_step_equals_step_then_propose(torch_cuda):
    """idlm_isd_loop_step (proposals on the acceptance's stream, beside the
    attention) against idlm_isd_step then idlm_isd_propose: attention
    output, tokens, lengths, next drafts and the MASK-row statistics record
    bit-identical, over two iterations, the second reading and rewriting one
    record in place."""
    torch = torch_cuda
    from speculative_verify_isd_amd import lib as L
    from speculative_verify_isd_amd.lib import DeviceStep

    w = W.named_workload("b16", 1)  # B*R*V = 17M logits: the step forks
    rng = np.random.default_rng(9)
    nxt_rows = [_dev(torch, W.f32_to_bf16_bits(rng.normal(0, 3, w.logits_mask.shape)
                                               .astype(np.float32)), "bf16") for _ in range(2)]
    B, K = w.B, w.N - 1
    a, b = DeviceStep(w), DeviceStep(w)
    ms_a = [L.alloc_mask_stats(a.dims), L.alloc_mask_stats(a.dims)]
    ms_b = L.alloc_mask_stats(b.dims)
    drafts_a, drafts_b = a.drafts.clone(), b.drafts.clone()
    nxt_a = torch.empty((B, K), dtype=torch.int32, device="cuda")
    nxt_b = torch.empty_like(nxt_a)
    for it in range(2):
        seed = 40 + it
        rec_in_a = ms_a[1 - it % 2] if it else None
        rec_in_b = ms_b if it else None
        a.step(seed=seed, drafts=drafts_a, mask_stats=rec_in_a)
        L.idlm_isd_propose(a.dims, nxt_rows[it], drafts_a, a.lens, seed, w.T, nxt_a, a.ws,
                           mask_stats=ms_a[it % 2])
        L.idlm_isd_loop_step(b.dims, b.q, b.kv, b.page_table, b.ctx_lens, b.lc, b.lm, drafts_b,
                             rec_in_b, nxt_rows[it], seed, w.N, w.T, b.tokens, b.lens, b.out,
                             nxt_b, ms_b, b.ws)
        torch.cuda.synchronize()
        assert L.idlm_isd_read_status(a.ws) == 0 and L.idlm_isd_read_status(b.ws) == 0
        for name, x, y in (("out", a.out, b.out), ("tokens", a.tokens, b.tokens),
                           ("lens", a.lens, b.lens), ("next", nxt_a, nxt_b),
                           ("record", ms_a[it % 2], ms_b)):
            bx = x.contiguous().view(torch.uint8).cpu().numpy().tobytes()
            by = y.contiguous().view(torch.uint8).cpu().numpy().tobytes()
            assert bx == by, (it, name)
        # next iteration: these drafts verified against the rows they came from
        a.lm, b.lm = nxt_rows[it], nxt_rows[it]
        drafts_a.copy_(nxt_a)
        drafts_b.copy_(nxt_b)
    print(f"[loop] loop step = step + propose over 2 iterations, "
          f"{int((nxt_b[:, 0] >= 0).sum().item())} sequences verifying next", flush=True)
