"""idlm_isd_accept_noalloc (static per-GPU scratch, no workspace, allocates
nothing) against idlm_isd_accept on the same inputs: tokens, lengths and the
debug record bit-identical, on calls in a row through the same scratch, the
later ones with smaller inputs, then a call whose draft ids are out of range
(the kernels' own bounds check sets the status)."""

import numpy as np
import pytest

from speculative_verify_isd_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available()
    return torch


def _both(torch, w, seed, T):
    from speculative_verify_isd_amd import lib as L
    from speculative_verify_isd_amd.lib import DeviceStep

    print(f"[case] noalloc {w.name} B={w.B} N={w.N} V={w.V} T={T} seed={seed}", flush=True)
    ds = DeviceStep(w)
    ds.accept(seed=seed, T=T)
    ref = (ds.tokens.clone(), ds.lens.clone(), ds.debug.clone())
    ref_status = L.idlm_isd_read_status(ds.ws)
    tok = torch.full_like(ds.tokens, -9)
    lens = torch.full_like(ds.lens, -9)
    dbg = torch.full_like(ds.debug, 7.0)
    status = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    L.idlm_isd_accept_noalloc(ds.dims, ds.lc, ds.lm, ds.drafts, seed, T, tok, lens, dbg, status)
    torch.cuda.synchronize()
    return ref, ref_status, (tok, lens, dbg), int(status.item())


def _bits_equal(a, b):
    return a.cpu().numpy().tobytes() == b.cpu().numpy().tobytes()


def test_noalloc_matches_workspace_entry_point(torch_cuda):
    torch = torch_cuda
    cases = [
        (W.named_workload("b16", 1), 11, 1.0),
        (W.make_workload("small", B=5, N=3, Hq=8, Hkv=8, D=64, V=3000, ctx_lens=[8] * 5,
                         T=0.7, seed=4), 12, 0.7),
        (W.make_workload("smaller", B=2, N=4, Hq=8, Hkv=8, D=64, V=700, ctx_lens=[9] * 2,
                         T=1.0, seed=5, logits_dtype="f32"), 13, 0.0),
    ]
    for w, seed, T in cases:
        ref, ref_status, got, status = _both(torch, w, seed, T)
        assert ref_status == 0 and status == 0
        for name, a, b in zip(("tokens", "lens", "debug"), ref, got):
            assert _bits_equal(a, b), (w.name, name)


def test_noalloc_flags_bad_drafts(torch_cuda):
    import dataclasses

    torch = torch_cuda
    w = W.make_workload("bad", B=4, N=4, Hq=8, Hkv=8, D=64, V=1000, ctx_lens=[8] * 4, T=1.0,
                        seed=6)
    drafts = w.draft_tokens.copy()
    drafts[2, 0] = w.V + 5  # out of range: clamped, flagged
    w = dataclasses.replace(w, draft_tokens=drafts)
    ref, ref_status, got, status = _both(torch, w, 21, 1.0)
    assert ref_status == 7 and status != 0
    good = [0, 1, 3]
    for a, b in zip(ref[:2], got[:2]):
        assert np.array_equal(a.cpu().numpy()[good], b.cpu().numpy()[good])
    # the next call through the same scratch starts from a clear status
    w2 = W.make_workload("after", B=3, N=4, Hq=8, Hkv=8, D=64, V=900, ctx_lens=[8] * 3, T=1.0,
                         seed=7)
    _, ref_status, _, status = _both(torch, w2, 22, 1.0)
    assert ref_status == 0 and status == 0


def test_noalloc_at_its_largest_batch(torch_cuda):
    """The largest batch the static scratch holds at N = 4, V = 151936
    (B = 1469; one more is refused with IDLM_ERR_SCRATCH, checked on the
    host): bit-identical to idlm_isd_accept.  Logits are seeded N(0, 3^2) bf16 made on the device,
    clean rows perturbed by N(0, 0.5^2); drafts drawn uniformly."""
    torch = torch_cuda
    from speculative_verify_isd_amd import lib as L

    B, N, V = 1469, 4, W.VOCAB
    K = N - 1
    dims = L.make_dims(B, N, 8, 8, 64, V, 1, 1, "bf16", "bf16")
    print(f"[case] noalloc largest batch B={B} N={N} V={V}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(1469)
    lm = (torch.randn((B, K, V), generator=g, device="cuda") * 3).to(torch.bfloat16)
    lc = torch.empty((B, N, V), dtype=torch.bfloat16, device="cuda")
    lc[:, :K] = (lm.float() + 0.5 * torch.randn((B, K, V), generator=g, device="cuda")).to(
        torch.bfloat16)
    lc[:, K] = (torch.randn((B, V), generator=g, device="cuda") * 3).to(torch.bfloat16)
    drafts = torch.randint(0, V, (B, K), generator=g, device="cuda", dtype=torch.int32)
    ws = L.alloc_workspace(dims)
    tok_a = torch.empty((B, N), dtype=torch.int32, device="cuda")
    len_a = torch.empty(B, dtype=torch.int32, device="cuda")
    dbg_a = torch.empty((B, N + 1, 4), dtype=torch.float64, device="cuda")
    tok_b, len_b, dbg_b = torch.full_like(tok_a, -9), torch.full_like(len_a, -9), \
        torch.full_like(dbg_a, 7.0)
    status = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    L.idlm_isd_accept(dims, lc, lm, drafts, 5, 1.0, tok_a, len_a, dbg_a, ws)
    L.idlm_isd_accept_noalloc(dims, lc, lm, drafts, 5, 1.0, tok_b, len_b, dbg_b, status)
    torch.cuda.synchronize()
    assert L.idlm_isd_read_status(ws) == 0 and int(status.item()) == 0
    for name, x, y in (("tokens", tok_a, tok_b), ("lens", len_a, len_b), ("debug", dbg_a, dbg_b)):
        assert x.cpu().numpy().tobytes() == y.cpu().numpy().tobytes(), name
    mean_len = float(len_a.float().mean().item())
    print(f"[noalloc] B={B}: identical to the workspace call; mean accept length {mean_len:.3f}",
          flush=True)
