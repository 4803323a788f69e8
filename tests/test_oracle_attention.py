"""Pins for the attention oracle (oracle.attention).

* brute force: pure-Python loops over tiny shapes, with the pool filled
  element by element from logical K/V through the documented page layout;
* library: torch scaled_dot_product_attention in float64 with an explicit
  causal-offset mask and GQA expansion;
* invariants: physical page permutation, constant V, a key that only the last
  row sees, and the N = 1 (plain decode) reduction.
"""

import math

import numpy as np
import pytest
import torch

from oracle.attention import isd_attention, isd_attention_rows

PAGE = 16


def _x(dtype):
    return 8 if dtype == "bf16" else 4


def _scatter_pool(Klog, Vlog, ctx_lens, max_pages, rng, dtype, slack=3):
    """Write logical K/V [B][Hkv][T][D] into a random page pool, one element at a time."""
    B, Hkv, T, D = Klog.shape
    x = _x(dtype)
    need = [(c + PAGE - 1) // PAGE for c in ctx_lens]
    P = sum(need) + slack
    slots = rng.permutation(P)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    o = 0
    for b in range(B):
        table[b, :need[b]] = slots[o:o + need[b]]
        o += need[b]
    pool = rng.standard_normal((P, 2, Hkv, PAGE * D)).astype(np.float32)  # junk in unused slots
    for b in range(B):
        for h in range(Hkv):
            for t in range(ctx_lens[b]):
                phys, s = table[b, t // PAGE], t % PAGE
                for d in range(D):
                    pool[phys, 0, h, ((d // x) * PAGE + s) * x + d % x] = Klog[b, h, t, d]
                    pool[phys, 1, h, d * PAGE + s] = Vlog[b, h, t, d]
    return pool, table


def _brute(q, Klog, Vlog, ctx_lens, N):
    B, R, Hq, D = q.shape
    Hkv = Klog.shape[1]
    G = Hq // Hkv
    out = np.zeros_like(q)
    for b in range(B):
        for hq in range(Hq):
            h = hq // G
            for r in range(R):
                pos = ctx_lens[b] - R + r
                sc = []
                for t in range(pos + 1):
                    s = 0.0
                    for d in range(D):
                        s += q[b, r, hq, d] * Klog[b, h, t, d]
                    sc.append(s / math.sqrt(D))
                mx = max(sc)
                e = [math.exp(s - mx) for s in sc]
                z = sum(e)
                for d in range(D):
                    out[b, r, hq, d] = sum(e[t] * Vlog[b, h, t, d] for t in range(pos + 1)) / z
    return out


def _case(seed, B, N, Hq, Hkv, D, ctx_lens):
    rng = np.random.default_rng(seed)
    R = 2 * N - 1
    T = max(ctx_lens)
    q = rng.standard_normal((B, R, Hq, D)).astype(np.float32).astype(np.float64)
    Klog = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    Vlog = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    max_pages = (T + PAGE - 1) // PAGE + 1
    pool, table = _scatter_pool(Klog, Vlog, ctx_lens, max_pages, rng, "f32")
    return q, Klog.astype(np.float64), Vlog.astype(np.float64), pool, table, np.array(ctx_lens)


@pytest.mark.parametrize("B,N,Hq,Hkv,D,ctx", [
    (1, 2, 2, 1, 4, [3]),
    (2, 3, 4, 2, 8, [5, 37]),
    (1, 4, 4, 1, 8, [40]),
    (2, 1, 2, 2, 4, [1, 17]),
])
def test_brute_force(B, N, Hq, Hkv, D, ctx):
    q, Klog, Vlog, pool, table, ctx = _case(10 + B + N, B, N, Hq, Hkv, D, ctx)
    got = isd_attention(q, pool, table, ctx, N, Hkv, "f32")
    want = _brute(q, Klog, Vlog, ctx, N)
    assert np.max(np.abs(got - want)) < 1e-12


def test_brute_force_bf16_layout():
    # bfloat16 storage uses 8-element chunks in the K block.
    rng = np.random.default_rng(5)
    B, N, Hq, Hkv, D, ctx = 1, 2, 2, 1, 16, [21]
    R = 2 * N - 1
    q = rng.standard_normal((B, R, Hq, D))
    Klog = rng.standard_normal((B, Hkv, 21, D)).astype(np.float32)
    Vlog = rng.standard_normal((B, Hkv, 21, D)).astype(np.float32)
    # round logical values to bfloat16 so the bit patterns are exact
    kb = (Klog.view(np.uint32) >> 16).astype(np.uint16)
    vb = (Vlog.view(np.uint32) >> 16).astype(np.uint16)
    Kf = (kb.astype(np.uint32) << 16).view(np.float32)
    Vf = (vb.astype(np.uint32) << 16).view(np.float32)
    pool32, table = _scatter_pool(Kf, Vf, ctx, 3, rng, "bf16")
    pool = (pool32.view(np.uint32) >> 16).astype(np.uint16)
    got = isd_attention(q, pool, table, np.array(ctx), N, Hkv, "bf16")
    want = _brute(q, Kf.astype(np.float64), Vf.astype(np.float64), ctx, N)
    assert np.max(np.abs(got - want)) < 1e-12


def _sdpa(q, Klog, Vlog, ctx_lens, N):
    B, R, Hq, D = q.shape
    Hkv = Klog.shape[1]
    G = Hq // Hkv
    out = np.zeros_like(q)
    for b in range(B):
        c = ctx_lens[b]
        Q = torch.from_numpy(q[b]).permute(1, 0, 2)                       # [Hq][R][D]
        Kt = torch.from_numpy(Klog[b, :, :c]).repeat_interleave(G, 0)     # [Hq][c][D]
        Vt = torch.from_numpy(Vlog[b, :, :c]).repeat_interleave(G, 0)
        pos = torch.arange(R)[:, None] + (c - R)
        mask = torch.arange(c)[None, :] <= pos                            # [R][c]
        o = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, attn_mask=mask)
        out[b] = o.permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("B,N,Hq,Hkv,D,ctx", [
    (3, 4, 8, 2, 16, [7, 100, 333]),
    (2, 8, 8, 1, 32, [15, 250]),
    (1, 1, 4, 4, 8, [64]),
])
def test_matches_torch_sdpa(B, N, Hq, Hkv, D, ctx):
    q, Klog, Vlog, pool, table, ctx = _case(20 + N, B, N, Hq, Hkv, D, ctx)
    got = isd_attention(q, pool, table, ctx, N, Hkv, "f32")
    want = _sdpa(q, Klog, Vlog, ctx, N)
    assert np.max(np.abs(got - want)) < 1e-12


def test_ctx_equal_rows_is_plain_causal():
    # With ctx == R the mask is the ordinary lower-triangular causal mask.
    B, N, Hq, Hkv, D = 1, 4, 4, 2, 8
    q, Klog, Vlog, pool, table, ctx = _case(31, B, N, Hq, Hkv, D, [7])
    got = isd_attention(q, pool, table, ctx, N, Hkv, "f32")
    Q = torch.from_numpy(q[0]).permute(1, 0, 2)
    Kt = torch.from_numpy(Klog[0]).repeat_interleave(2, 0)
    Vt = torch.from_numpy(Vlog[0]).repeat_interleave(2, 0)
    want = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, is_causal=True)
    assert np.max(np.abs(got[0] - want.permute(1, 0, 2).numpy())) < 1e-12


def test_page_permutation_invariance():
    q, Klog, Vlog, pool, table, ctx = _case(41, 2, 3, 4, 2, 8, [50, 77])
    a = isd_attention(q, pool, table, ctx, 3, 2, "f32")
    rng = np.random.default_rng(9)
    perm = rng.permutation(pool.shape[0])          # new slot of old page i is perm[i]
    pool2 = np.empty_like(pool)
    pool2[perm] = pool
    table2 = np.where(table >= 0, perm[np.maximum(table, 0)], -1)
    b = isd_attention(q, pool2, table2, ctx, 3, 2, "f32")
    assert np.array_equal(a, b)


def test_constant_v_gives_that_constant():
    B, N, Hq, Hkv, D = 1, 4, 4, 1, 8
    q, Klog, _, _, _, ctx = _case(51, B, N, Hq, Hkv, D, [45])
    vec = np.arange(D, dtype=np.float64) - 3.5
    Vlog = np.broadcast_to(vec, Klog.shape).copy()
    pool, table = _scatter_pool(Klog.astype(np.float32), Vlog.astype(np.float32), [45], 4,
                                np.random.default_rng(1), "f32")
    got = isd_attention(q, pool, table, np.array([45]), N, Hkv, "f32")
    assert np.max(np.abs(got - vec)) < 1e-13


def test_last_key_only_reaches_last_row():
    B, N, Hq, Hkv, D = 1, 4, 4, 2, 8
    R = 2 * N - 1
    q, Klog, Vlog, pool, table, ctx = _case(61, B, N, Hq, Hkv, D, [30])
    a = isd_attention(q, pool, table, ctx, N, Hkv, "f32")
    K2, V2 = Klog.copy(), Vlog.copy()
    K2[0, :, 29] += 3.0
    V2[0, :, 29] -= 5.0
    pool2, table2 = _scatter_pool(K2.astype(np.float32), V2.astype(np.float32), [30], 3,
                                  np.random.default_rng(2), "f32")
    b = isd_attention(q, pool2, table2, ctx, N, Hkv, "f32")
    assert np.array_equal(a[:, :R - 1], b[:, :R - 1])
    assert np.all(np.abs(a[:, R - 1] - b[:, R - 1]).max(axis=-1) > 1e-6)


def test_sampled_rows_match_full():
    q, Klog, Vlog, pool, table, ctx = _case(71, 2, 4, 8, 2, 8, [40, 90])
    full = isd_attention(q, pool, table, ctx, 4, 2, "f32")
    picks = [(0, 0, 0), (1, 6, 7), (1, 3, 2), (0, 6, 5)]
    rows = isd_attention_rows(q, pool, table, ctx, 4, 2, "f32", picks)
    # Same definition; the full evaluation forms each KV head's scores with
    # one matrix product, the sampled rows with one product per row, so the
    # two agree to float64 summation order.
    for n, (b, r, h) in enumerate(picks):
        np.testing.assert_allclose(rows[n], full[b, r, h], rtol=1e-13, atol=1e-15)
