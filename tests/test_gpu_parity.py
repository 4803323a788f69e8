"""GPU parity: libidlm_isd.so through its C ABI against the CPU oracle.

Small shapes and the named b1, b16, c64 (sigma = 0.5) and c64n8 workloads
compare every output element; the other sigma values of the c64 sweep
compare sampled attention rows and every acceptance output.  Tolerances are
in tests/parity.py.
"""

import numpy as np
import pytest

from parity import (ATTN_TOL, PROB_TOL, compare_accept, normwise_err, oracle_accept,
                    oracle_attention, oracle_attention_rows)
from speculative_verify_isd_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available()
    return torch


def run(w, torch):
    from speculative_verify_isd_amd.lib import DeviceStep

    print(f"[case] {w.name} B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} D={w.D} V={w.V} "
          f"T={w.T} ctx={list(w.ctx_lens[:6])}", flush=True)
    ds = DeviceStep(w)
    ds.attn()
    ds.accept()
    torch.cuda.synchronize()
    return ds


def check_accept(w, ds, allow_boundary=2):
    ref = oracle_accept(w)
    res = compare_accept(w, ds.tokens.cpu().numpy(), ds.lens.cpu().numpy(),
                         ds.debug.cpu().numpy(), ref)
    print(f"[accept] exact={res['exact']}/{w.B} boundary={res['boundary']} "
          f"max|dp|={res['max_prob_err']:.2e}", flush=True)
    assert not res["bad"], res["bad"]
    assert res["max_prob_err"] < PROB_TOL
    assert len(res["boundary"]) <= allow_boundary
    return ref


def check_attn_full(w, ds):
    ref = oracle_attention(w)
    err = normwise_err(ds.out_f64(), ref)
    print(f"[attn] normwise err {err:.3e}", flush=True)
    assert err < ATTN_TOL[w.qkv_dtype]


def small(name, B, N, Hq, Hkv, D, V, ctx, T=1.0, qkv="bf16", logits="bf16", seed=7, **kw):
    return W.make_workload(name, B=B, N=N, Hq=Hq, Hkv=Hkv, D=D, V=V, ctx_lens=ctx, T=T, seed=seed,
                           qkv_dtype=qkv, logits_dtype=logits, **kw)


def test_tiny_named_workload(torch_cuda):
    w = W.named_workload("tiny")
    ds = run(w, torch_cuda)
    check_attn_full(w, ds)
    check_accept(w, ds, allow_boundary=0)


@pytest.mark.parametrize("case", [
    # ragged contexts: minimum (ctx == R), page edges, odd page counts, several chunks
    dict(name="ragged", B=6, N=4, Hq=32, Hkv=8, D=128, V=1000, ctx=[7, 16, 17, 40, 300, 2053]),
    dict(name="d64", B=3, N=4, Hq=8, Hkv=2, D=64, V=4096, ctx=[9, 129, 777]),
    dict(name="wr2", B=2, N=4, Hq=32, Hkv=4, D=128, V=2048, ctx=[50, 1500]),       # 56 rows
    dict(name="n8g8", B=2, N=8, Hq=64, Hkv=8, D=128, V=3000, ctx=[15, 999]),        # 120 rows
    dict(name="n8g8d64", B=2, N=8, Hq=64, Hkv=8, D=64, V=3000, ctx=[15, 999]),
    # 120 rows over many short segments: LDS page buffers reused across pairs
    dict(name="n8g8seg", B=6, N=8, Hq=64, Hkv=8, D=128, V=2000,
         ctx=[15, 200, 33, 1000, 64, 517]),
    dict(name="n1", B=4, N=1, Hq=32, Hkv=8, D=128, V=5000, ctx=[1, 2, 16, 700]),    # plain decode
    dict(name="f32_128", B=2, N=4, Hq=16, Hkv=4, D=128, V=777, ctx=[7, 500], qkv="f32",
         logits="f32"),
    dict(name="f32_g120", B=2, N=8, Hq=64, Hkv=8, D=64, V=300, ctx=[15, 400], qkv="f32",
         logits="f32"),                                                             # 120 rows
    dict(name="mha", B=2, N=2, Hq=4, Hkv=4, D=128, V=64, ctx=[3, 260]),
    # the largest stride: 31 rows and 15 drafts per sequence; a 31-row tile and
    # a 124-row tile (two 64-row waves per run)
    dict(name="n16g1", B=3, N=16, Hq=4, Hkv=4, D=128, V=3000, ctx=[31, 500, 1777]),
    dict(name="n16g4", B=3, N=16, Hq=16, Hkv=4, D=128, V=3000, ctx=[31, 640, 1500]),
    # many short sequences: most pairs lie whole inside one run
    dict(name="b400", B=400, N=4, Hq=32, Hkv=8, D=128, V=1000,
         ctx=[7 + (37 * i) % 190 for i in range(400)]),
    # the largest tile, R * G = 128 (one KV head for 128 query heads), no padding rows
    dict(name="g128", B=2, N=1, Hq=128, Hkv=1, D=64, V=50, ctx=[1, 300]),
    # a one-token vocabulary: p = q = 1, every draft kept, the bonus token is 0
    dict(name="v1", B=3, N=4, Hq=8, Hkv=2, D=64, V=1, ctx=[7, 20, 100]),
])
def test_small_shapes_full_parity(torch_cuda, case):
    w = small(**case)
    ds = run(w, torch_cuda)
    check_attn_full(w, ds)
    check_accept(w, ds, allow_boundary=0)


def scale_k_pages(w, factor):
    """Multiplies the K block of page i of every sequence by factor(i) (the
    scores of its tokens scale by the same factor)."""
    for b in range(w.B):
        n = (int(w.ctx_lens[b]) + W.PAGE - 1) // W.PAGE
        for i in range(n):
            phys = w.page_table[b, i]
            k = W._store_to_f32(w.kv_pages[phys, 0], w.qkv_dtype) * np.float32(factor(i))
            w.kv_pages[phys, 0] = W.f32_to_bf16_bits(k)


@pytest.mark.parametrize("shape", [(4, 32, 8, 128), (4, 64, 8, 128), (8, 64, 8, 128), (4, 8, 2, 64)],
                         ids=["n4d128", "n4g8d128", "n8g8d128", "n4d64"])
@pytest.mark.parametrize("big", [6.0, 30.0])
def test_scores_outgrowing_the_first_page(torch_cuda, shape, big):
    """Every odd page's scores are `big` times larger: a segment that starts on
    an even page takes a softmax reference far below its later scores
    (weights up to ~2^35 or ~2^130 against it), so the kernel must detect it
    and stream the segment again from the true row max."""
    N, Hq, Hkv, D = shape
    w = small(f"rising{N}_{D}_{big:g}", B=4, N=N, Hq=Hq, Hkv=Hkv, D=D, V=512,
              ctx=[2 * N - 1, 40, 700, 2100])
    scale_k_pages(w, lambda i: big if i % 2 else 1.0)
    ds = run(w, torch_cuda)
    check_attn_full(w, ds)


@pytest.mark.parametrize("seed", range(8))
def test_random_shapes_and_score_scales(torch_cuda, seed):
    """Seeded random shapes over every attention tiling (32- and 64-row waves,
    one or two waves per run, D = 64 / 128, N = 1..16), ragged contexts, and
    for half of the cases K pages scaled by random factors up to 40 (so some
    segments outgrow their first page's reference and take the re-stream
    path, in no fixed pattern)."""
    rng = np.random.default_rng(1000 + seed)
    while True:
        N = int(rng.integers(1, 17))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 8]))
        if (2 * N - 1) * G <= 128:
            break
    D = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 9))
    ctx = [int(rng.integers(2 * N - 1, 2500)) for _ in range(B)]
    w = small(f"rand{seed}", B=B, N=N, Hq=G * Hkv, Hkv=Hkv, D=D, V=int(rng.integers(64, 4000)),
              ctx=ctx, seed=seed)
    if seed % 2:
        f = rng.uniform(0.2, 40.0, size=1 + max(ctx) // 16)
        scale_k_pages(w, lambda i: float(f[i]))
    ds = run(w, torch_cuda)
    check_attn_full(w, ds)
    check_accept(w, ds, allow_boundary=1)


@pytest.mark.parametrize("T", [0.05, 0.3, 2.5, 20.0])
def test_temperatures(torch_cuda, T):
    """Low T makes p and q nearly one-hot: most weights underflow and the
    residual sums of max(0, p - q) get tiny (down to ~1e-83 at T = 0.05 on
    these rows).  High T makes them nearly uniform."""
    w = small(f"temp{T}", B=16, N=4, Hq=8, Hkv=2, D=64, V=5000, ctx=[20] * 16, T=T, seed=11)
    ds = run(w, torch_cuda)
    check_accept(w, ds, allow_boundary=1)


@pytest.mark.parametrize("V", [2048 * 1024, 2048 * 1024 - 1])
def test_largest_vocabulary(torch_cuda, V):
    """The largest vocabulary the acceptance takes (1024 sub-chunks of 2048):
    every sub-chunk table is full; V - 1 takes the element-wise load path."""
    w = small(f"vmax{V}", B=6, N=4, Hq=8, Hkv=2, D=64, V=V, ctx=[8, 40, 17, 100, 33, 64],
              n_drafts=[3, 3, 3, 2, 3, 1])
    ds = run(w, torch_cuda)
    check_accept(w, ds, allow_boundary=1)


def test_greedy_and_short_draft_lists(torch_cuda):
    w = small("greedy", B=8, N=4, Hq=8, Hkv=2, D=64, V=3001, ctx=[20] * 8, T=0.0,
              n_drafts=[3, 0, 1, 2, 3, 0, 3, 3])
    ds = run(w, torch_cuda)
    check_accept(w, ds, allow_boundary=0)
    w = small("short", B=8, N=4, Hq=8, Hkv=2, D=64, V=3001, ctx=[20] * 8, T=0.8,
              n_drafts=[3, 0, 1, 2, 3, 0, 3, 3])
    ds = run(w, torch_cuda)
    check_accept(w, ds, allow_boundary=0)


def test_identical_rows_accept_everything(torch_cuda):
    w = small("ident", B=16, N=4, Hq=8, Hkv=2, D=64, V=20000, ctx=[30] * 16, sigma=0.0)
    ds = run(w, torch_cuda)
    assert np.all(ds.lens.cpu().numpy() == 4)
    check_accept(w, ds, allow_boundary=0)


def test_deterministic_and_reusable_workspace(torch_cuda):
    torch = torch_cuda
    w = small("det", B=4, N=4, Hq=32, Hkv=8, D=128, V=151936, ctx=[100, 5000, 3000, 64])
    ds = run(w, torch)
    out1, tok1, len1 = ds.out.clone(), ds.tokens.clone(), ds.lens.clone()
    for _ in range(3):
        ds.step()
    torch.cuda.synchronize()
    assert torch.equal(out1, ds.out) and torch.equal(tok1, ds.tokens) and torch.equal(len1, ds.lens)
    # a different seed gives a (generally) different draw, through the same workspace
    ds.accept(seed=w.seed + 1)
    ref = oracle_accept(w, seed=w.seed + 1)
    res = compare_accept(w, ds.tokens.cpu().numpy(), ds.lens.cpu().numpy(), None, ref)
    assert not res["bad"]


def test_step_joins_its_second_stream(torch_cuda):
    """idlm_isd_step runs the acceptance on a stream of its own: work enqueued
    on the caller's stream right after the step (no synchronisation) must see
    the step's outputs, equal to the two calls in sequence."""
    torch = torch_cuda
    rng = np.random.default_rng(3)
    ctx = [int(c) for c in rng.integers(256, 4096, size=16, endpoint=True)]
    w = small("fork", B=16, N=4, Hq=32, Hkv=8, D=128, V=151936, ctx=ctx)
    ds = run(w, torch)
    ref = (ds.tokens.clone(), ds.lens.clone(), ds.out.clone())
    for i in range(4):
        ds.tokens.fill_(-7)
        ds.lens.zero_()
        ds.out.zero_()
        ds.step()
        got = (ds.tokens.clone(), ds.lens.clone(), ds.out.clone())  # same stream, no sync
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), f"step {i}"
        assert torch.equal(got[2].view(torch.int16), ref[2].view(torch.int16)), f"step {i}"


def test_steps_from_two_host_threads(torch_cuda):
    """Two host threads run forked steps at once, each on its own stream and
    workspace; both share the library's second stream, and every result must
    equal the same step run alone."""
    import threading

    torch = torch_cuda
    from speculative_verify_isd_amd.lib import DeviceStep

    rng = np.random.default_rng(8)
    works = [small(f"thread{t}", B=16, N=4, Hq=32, Hkv=8, D=128, V=151936,
                   ctx=[int(c) for c in rng.integers(256, 3000, size=16, endpoint=True)], seed=40 + t)
             for t in range(2)]
    steps = [DeviceStep(w) for w in works]
    refs = []
    for ds in steps:
        ds.attn()
        ds.accept()
        torch.cuda.synchronize()
        refs.append((ds.tokens.clone(), ds.lens.clone(), ds.out.clone()))
    errors = []

    def worker(t):
        try:
            ds, ref = steps[t], refs[t]
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for i in range(6):
                    ds.tokens.fill_(-7)
                    ds.lens.zero_()
                    ds.step()
                    got = (ds.tokens.clone(), ds.lens.clone(), ds.out.clone())
                    stream.synchronize()
                    if not (torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
                            and torch.equal(got[2].view(torch.int16), ref[2].view(torch.int16))):
                        errors.append((t, i))
        except Exception as e:  # reported below, in the main thread
            errors.append((t, repr(e)))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors


def test_device_data_errors_are_flagged(torch_cuda):
    torch = torch_cuda
    from speculative_verify_isd_amd.lib import idlm_isd_read_status, idlm_isd_workspace_init

    w = small("baddata", B=2, N=4, Hq=8, Hkv=2, D=64, V=500, ctx=[40, 40])
    ds = run(w, torch)
    assert idlm_isd_read_status(ds.ws) == 0
    ds.page_table[0, 1] = 10 ** 6              # page id outside the pool
    ds.attn()
    assert idlm_isd_read_status(ds.ws) == 7
    idlm_isd_workspace_init(ds.ws)
    ds.page_table[0, 1] = int(w.page_table[0, 1])
    ds.ctx_lens[1] = 10 ** 6                   # context longer than the table allows
    ds.attn()
    assert idlm_isd_read_status(ds.ws) == 7
    idlm_isd_workspace_init(ds.ws)
    ds.ctx_lens[1] = 40
    ds.drafts[1, 0] = w.V                      # draft id outside the vocabulary
    ds.accept()
    assert idlm_isd_read_status(ds.ws) == 7
    idlm_isd_workspace_init(ds.ws)
    ds.drafts[1, 0] = int(w.draft_tokens[1, 0])
    ds.step()
    assert idlm_isd_read_status(ds.ws) == 0


def test_empty_batch(torch_cuda):
    torch = torch_cuda
    from speculative_verify_isd_amd.lib import alloc_workspace, idlm_isd_step, make_dims

    d = make_dims(0, 4, 32, 8, 128, 100, 4, 1)
    ws = alloc_workspace(d)
    e = torch.empty(0, device="cuda")
    z = torch.empty(0, dtype=torch.int32, device="cuda")
    idlm_isd_step(d, e.bfloat16(), e.bfloat16(), z, z, e.bfloat16(), e.bfloat16(), z, 1, 4, 1.0,
                  z, z, e.bfloat16(), ws)
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# named full-size workloads: every acceptance output, sampled attention rows
# ---------------------------------------------------------------------------
def _picks(w, n, seed):
    rng = np.random.default_rng(seed)
    order = np.argsort(w.ctx_lens)
    bs = [int(order[0]), int(order[-1])] + [int(x) for x in rng.integers(0, w.B, n - 2)]
    return [(b, int(rng.integers(0, w.R)) if k else w.R - 1, int(rng.integers(0, w.Hq)))
            for k, b in enumerate(bs)]


@pytest.mark.parametrize("name,sig", [("b1", 1), ("b16", 1), ("c64", 1), ("c64n8", 1),
                                      ("c64_dp8", 1), ("c64_tp8", 1)])
def test_named_full_size_every_head_vector(torch_cuda, name, sig):
    """Every attention head vector of the named workload against the oracle
    (every (b, KV head) pair and every merge of its split pieces), and every
    acceptance output."""
    w = W.named_workload(name, sig)
    ds = run(w, torch_cuda)
    got = ds.out_f64()
    ref = oracle_attention(w)
    err = normwise_err(got, ref)
    print(f"[attn] {w.B * w.R * w.Hq} head vectors of {w.D}, normwise err {err:.3e}", flush=True)
    assert err < ATTN_TOL["bf16"]
    check_accept(w, ds, allow_boundary=2)


@pytest.mark.parametrize("name,sig", [("c64", 0), ("c64", 2)])
def test_named_full_size_sampled_rows(torch_cuda, name, sig):
    """The other sigma values of the sweep (their attention inputs differ only
    by seed): sampled head vectors, every acceptance output."""
    w = W.named_workload(name, sig)
    ds = run(w, torch_cuda)
    # The extremes and random rows, plus one row of every sequence.
    rng = np.random.default_rng(11)
    picks = _picks(w, 6, 5) + [(b, int(rng.integers(0, w.R)), int(rng.integers(0, w.Hq)))
                               for b in range(w.B)]
    ref = oracle_attention_rows(w, picks)
    got = ds.out_f64()
    err = max(normwise_err(got[b, r, h], ref[n]) for n, (b, r, h) in enumerate(picks))
    print(f"[attn] sampled {len(picks)} head vectors, normwise err {err:.3e}", flush=True)
    assert err < ATTN_TOL["bf16"]
    check_accept(w, ds, allow_boundary=2)


# ---------------------------------------------------------------------------
# a large batch compared element by element: ~90k units over every wave-lane,
# with pairs split across several lanes (7-row tiles in 32-row waves, 56-row
# tiles in 64-row waves)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("Hq,D", [(8, 128), (64, 64)])
def test_large_batch_full(torch_cuda, Hq, D):
    rng = np.random.default_rng(23)
    ctx = rng.integers(12000, 16384, size=12, endpoint=True)
    w = small(f"large_hq{Hq}_d{D}", 12, 4, Hq, 8, D, 4096, ctx, seed=31)
    ds = run(w, torch_cuda)
    check_attn_full(w, ds)
    check_accept(w, ds)
