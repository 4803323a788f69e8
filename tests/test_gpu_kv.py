"""GPU parity of the KV append / rollback entry points against oracle.kv_cache:
pool, page table, contexts and free-page stack bit-exact; device-data
errors reported and leaving the state unchanged; attention over a cache the
library appended to equals the oracle's attention over the oracle's cache."""

import numpy as np
import pytest

from oracle.kv_cache import kv_append, kv_rollback
from parity import ATTN_TOL, normwise_err
from oracle.attention import isd_attention
from oracle.dtypes import to_f64
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


def _host(t, dtype):
    import torch

    if dtype == "bf16" and t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class Cache:
    def __init__(self, torch, ctx, N, Hkv, D, dtype, spare, max_pages, seed):
        from speculative_verify_isd_amd import lib as L

        self.L, self.torch, self.dtype = L, torch, dtype
        self.R = 2 * N - 1
        rng = np.random.default_rng(seed)
        (self.pool, self.table, self.stack, self.count, self.k_new,
         self.v_new) = W.make_cache_state(rng, ctx, max_pages, Hkv, D, self.R, dtype, spare)
        self.ctx = np.asarray(ctx, dtype=np.int32)
        B = len(ctx)
        self.dims = L.make_dims(B, N, Hkv, Hkv, D, 512, max_pages, self.pool.shape[0], dtype, dtype)
        self.ws = L.alloc_workspace(self.dims)
        self.d_pool = _dev(torch, self.pool, dtype)
        self.d_table = _dev(torch, self.table, None)
        self.d_stack = _dev(torch, self.stack, None)
        self.d_count = torch.tensor([self.count], dtype=torch.int32, device="cuda")
        self.d_ctx = _dev(torch, self.ctx, None)
        self.d_ctx2 = torch.zeros_like(self.d_ctx)
        self.d_k = _dev(torch, self.k_new, dtype)
        self.d_v = _dev(torch, self.v_new, dtype)

    def append(self, count=None, ctx=None):
        if count is not None:
            self.d_count.fill_(count)
        if ctx is not None:
            self.d_ctx.copy_(self.torch.from_numpy(np.asarray(ctx, dtype=np.int32)))
        self.L.idlm_isd_kv_append(self.dims, self.d_k, self.d_v, self.d_ctx, self.d_ctx2,
                                  self.d_pool, self.d_table, self.d_stack, self.d_count, self.ws)
        self.torch.cuda.synchronize()

    def state(self):
        return (_host(self.d_pool, self.dtype), self.d_table.cpu().numpy(),
                self.d_ctx2.cpu().numpy(), int(self.d_count.item()), self.d_stack.cpu().numpy())


CASES = [("bf16", 128, 4), ("bf16", 64, 8), ("f32", 64, 4), ("f32", 128, 1), ("bf16", 128, 16)]


@pytest.mark.parametrize("dtype,D,N", CASES)
def test_append_and_rollback_match_oracle(torch_cuda, dtype, D, N):
    torch = torch_cuda
    ctx = [0, 1, 15, 16, 17, 31, 32, 100, 257, 1000, 4090]
    c = Cache(torch, ctx, N, 2, D, dtype, spare=40, max_pages=300, seed=D + N)
    c.append()
    pool, table, ctx2, count, stack = c.state()
    o_pool, o_table, o_ctx, o_count, err = kv_append(c.pool, c.table, c.ctx, c.k_new, c.v_new,
                                                     c.stack, c.count, dtype)
    assert not err
    assert c.L.idlm_isd_read_status(c.ws) == 0
    assert np.array_equal(table, o_table) and np.array_equal(ctx2, o_ctx) and count == o_count
    assert np.array_equal(pool, o_pool), "pool differs"
    print(f"[kv] append {dtype} D={D} N={N}: {c.count - count} pages taken, pool bit-exact",
          flush=True)

    rng = np.random.default_rng(7)
    acc = rng.integers(1, N + 1, size=len(ctx)).astype(np.int32)
    d_acc = torch.from_numpy(acc).cuda()
    d_ctx3 = torch.zeros_like(c.d_ctx2)
    c.L.idlm_isd_kv_rollback(c.dims, c.d_ctx2, d_acc, d_ctx3, c.d_table, c.d_stack, c.d_count,
                             c.ws)
    torch.cuda.synchronize()
    r_table, r_ctx, r_stack, r_count, err = kv_rollback(o_table, o_ctx, acc, c.R, stack, count)
    assert not err
    assert c.L.idlm_isd_read_status(c.ws) == 0
    assert np.array_equal(c.d_table.cpu().numpy(), r_table)
    assert np.array_equal(d_ctx3.cpu().numpy(), r_ctx)
    assert int(c.d_count.item()) == r_count
    assert np.array_equal(c.d_stack.cpu().numpy()[:r_count], r_stack[:r_count])


def test_in_place_context_update(torch_cuda):
    torch = torch_cuda
    ctx = [5, 16, 40]
    c = Cache(torch, ctx, 4, 1, 64, "bf16", spare=8, max_pages=16, seed=3)
    c.d_ctx2 = c.d_ctx  # ctx_after is ctx_before
    c.append()
    assert c.d_ctx.cpu().numpy().tolist() == [x + 7 for x in ctx]
    acc = torch.tensor([1, 7, 3], dtype=torch.int32, device="cuda")
    c.L.idlm_isd_kv_rollback(c.dims, c.d_ctx, acc, c.d_ctx, c.d_table, c.d_stack, c.d_count, c.ws)
    torch.cuda.synchronize()
    assert c.d_ctx.cpu().numpy().tolist() == [6, 23, 43]


def test_device_data_errors_leave_state(torch_cuda):
    torch = torch_cuda
    ctx = [3, 14, 20]
    c = Cache(torch, ctx, 4, 1, 64, "bf16", spare=3, max_pages=8, seed=4)
    ctx_np = np.asarray(ctx)
    need = int((((ctx_np + 7 + 15) // 16) - ((ctx_np + 15) // 16)).sum())  # pages for 7 rows
    assert need >= 1
    c.append(count=need - 1)
    pool, table, ctx2, count, _ = c.state()
    assert c.L.idlm_isd_read_status(c.ws) == 7
    assert np.array_equal(pool, c.pool) and np.array_equal(table, c.table)
    assert ctx2.tolist() == ctx and count == need - 1
    print("[kv] too few free pages: reported, nothing written", flush=True)

    c2 = Cache(torch, ctx, 4, 1, 64, "bf16", spare=3, max_pages=8, seed=5)
    bad = [3, 14, 16 * 8 - 2]  # the last cannot take 7 more rows
    c2.append(ctx=bad)
    pool, table, ctx2, count, _ = c2.state()
    o_pool, o_table, o_ctx, o_count, err = kv_append(c2.pool, c2.table, bad, c2.k_new, c2.v_new,
                                                     c2.stack, c2.count, "bf16")
    assert err == {"bad_ctx"} and c2.L.idlm_isd_read_status(c2.ws) == 7
    assert np.array_equal(table, o_table) and np.array_equal(ctx2, o_ctx) and count == o_count
    assert np.array_equal(pool, o_pool)

    # rollback with an accept length out of range: clamped and reported
    c3 = Cache(torch, [20, 30], 4, 1, 64, "bf16", spare=4, max_pages=8, seed=6)
    c3.append()
    acc = torch.tensor([0, 99], dtype=torch.int32, device="cuda")
    out = torch.zeros_like(c3.d_ctx2)
    c3.L.idlm_isd_kv_rollback(c3.dims, c3.d_ctx2, acc, out, c3.d_table, c3.d_stack,
                              c3.d_count, c3.ws)
    torch.cuda.synchronize()
    assert out.cpu().numpy().tolist() == [21, 37]
    assert c3.L.idlm_isd_read_status(c3.ws) == 7


def test_attention_over_appended_cache(torch_cuda):
    torch = torch_cuda
    N, Hkv, G, D, dtype = 4, 2, 4, 128, "bf16"
    ctx = [9, 60, 300]
    c = Cache(torch, ctx, N, Hkv, D, dtype, spare=16, max_pages=32, seed=8)
    # same dims but with Hq = G * Hkv for attention
    L = c.L
    dims = L.make_dims(len(ctx), N, Hkv * G, Hkv, D, 512, 32, c.pool.shape[0], dtype, dtype)
    ws = L.alloc_workspace(dims)
    c.append()
    rng = np.random.default_rng(9)
    q = W._normal_store(rng, (len(ctx), c.R, Hkv * G, D), 1.0, dtype)
    d_q = _dev(torch, q, dtype)
    out = torch.zeros_like(d_q)
    L.idlm_isd_paged_attn(dims, d_q, c.d_pool, c.d_table, c.d_ctx2, out, ws)
    torch.cuda.synchronize()
    o_pool, o_table, o_ctx, _, err = kv_append(c.pool, c.table, c.ctx, c.k_new, c.v_new, c.stack,
                                               c.count, dtype)
    ref = isd_attention(to_f64(q, dtype).reshape(q.shape), o_pool, o_table, o_ctx, N, Hkv, dtype)
    err = normwise_err(out.to(torch.float64).cpu().numpy(), ref)
    print(f"[kv] attention over the appended cache: normwise err {err:.3e}", flush=True)
    assert err < ATTN_TOL[dtype]


def test_batch_over_one_work_group(torch_cuda):
    # B > 1024 takes the chunked bookkeeping path.
    torch = torch_cuda
    rng = np.random.default_rng(12)
    ctx = rng.integers(0, 60, size=1500)
    c = Cache(torch, ctx, 4, 1, 64, "bf16", spare=3000, max_pages=8, seed=13)
    c.append()
    pool, table, ctx2, count, stack = c.state()
    o_pool, o_table, o_ctx, o_count, err = kv_append(c.pool, c.table, c.ctx, c.k_new, c.v_new,
                                                     c.stack, c.count, "bf16")
    assert not err and c.L.idlm_isd_read_status(c.ws) == 0
    assert np.array_equal(table, o_table) and np.array_equal(ctx2, o_ctx) and count == o_count
    assert np.array_equal(pool, o_pool)
    acc = rng.integers(1, 5, size=1500).astype(np.int32)
    d_acc = torch.from_numpy(acc).cuda()
    out = torch.zeros_like(c.d_ctx2)
    c.L.idlm_isd_kv_rollback(c.dims, c.d_ctx2, d_acc, out, c.d_table, c.d_stack, c.d_count, c.ws)
    torch.cuda.synchronize()
    r_table, r_ctx, r_stack, r_count, err = kv_rollback(o_table, o_ctx, acc, c.R, stack, count)
    assert not err
    assert np.array_equal(c.d_table.cpu().numpy(), r_table)
    assert np.array_equal(out.cpu().numpy(), r_ctx) and int(c.d_count.item()) == r_count
    assert np.array_equal(c.d_stack.cpu().numpy()[:r_count], r_stack[:r_count])
    print(f"[kv] B=1500 chunked path: {c.count - count} pages taken, {r_count - count} freed",
          flush=True)
