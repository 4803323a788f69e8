"""Seeded synthetic inputs for the ISD step.

This module only draws random inputs in the step's storage formats.  It
holds none of the step's arithmetic (no softmax, attention or acceptance),
so both the GPU library's tests and the CPU oracle can consume what it
makes.  Everything is numpy ``Generator(PCG64(seed))``.

Storage formats (the library's boundary formats):

* bfloat16 tensors are uint16 bit patterns, rounded to nearest-even from
  float32 draws;
* ``kv_pages`` is the pool [P][2][Hkv][16*D]; its entries are i.i.d., so the
  draw does not depend on the intra-page layout;
* ``page_table`` int32 [B][max_pages], unused entries -1;
* ``ctx_lens`` int32 [B], counting the 2N-1 new rows;
* ``logits_clean`` [B][N][V], ``logits_mask`` [B][N-1][V];
* ``draft_tokens`` int32 [B][N-1], drawn from q = softmax(mask / T) with the
  Gumbel-max trick (argmax of mask / T plus Gumbel noise, an exact draw from
  that softmax that never forms it), or argmax at T = 0.

Named workloads (sizes of the step the library is built for):

tiny   B=1, N=4, Hq/Hkv=8/2, D=64, ctx 256, float32 everywhere, identity page
       table, V=512 logits ~ N(0, 2^2) on all 7 rows, T=1, step seed 0.
b1     B=1, N=4, 32/8 heads, D=128, bfloat16, ctx 4096 in 256 pages at a
       random permutation of 256 slots; V=151936, MASK rows ~ N(0, 3^2),
       verifying clean rows = MASK row + N(0, sigma^2) with sigma = 0.5, bonus
       clean row ~ N(0, 3^2); T=1.
b16    as b1 with B=16, ctx ~ U[1024, 8192], one shared pool with 10% slack
       and a random page permutation.
c64    as b1 with B=64, ctx ~ U[2048, 16384], sigma in {0.1, 0.5, 1.5}.
c64n8  B=64, N=8, 64/8 heads, D=128, bfloat16, ctx ~ U[4096, 32768],
       sigma = 0.5, T=0.7.

One GPU's share of c64 on eight GPUs:
c64_dp8  split by sequence: B=8 with the first 8 of c64's contexts.
c64_tp8  split by KV head: B=64 with c64's contexts, 4/1 heads.
"""

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

PAGE = 16
VOCAB = 151936


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (nearest-even) and return the bit
    patterns; NaN stays a quiet NaN with its sign (the bias would otherwise
    carry a NaN whose payload sits in the low half into infinity or zero)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) & np.uint32(0x8000)).astype(np.uint16) | np.uint16(0x7FC0)
    return out


def _normal_store(rng, shape, scale, dtype, block=1 << 24):
    """N(0, scale^2) draws in storage dtype.

    Large draws are cut into fixed blocks, each with its own PCG64 stream
    spawned from one seed taken from ``rng``; blocks fill in parallel threads
    (numpy releases the GIL), so the result depends only on the seed.
    """
    n = int(np.prod(shape))
    base = int(rng.integers(0, 2 ** 63))
    nblk = max(1, (n + block - 1) // block)
    seqs = np.random.SeedSequence(base).spawn(nblk)
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)

    def fill(i):
        s, e = i * block, min(n, (i + 1) * block)
        g = np.random.Generator(np.random.PCG64(seqs[i]))
        x = g.standard_normal(e - s, dtype=np.float32)
        x *= np.float32(scale)
        out[s:e] = x if dtype == "f32" else f32_to_bf16_bits(x)

    if nblk == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


def _store_to_f32(a, dtype):
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32)
    return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    name: str
    B: int
    N: int
    Hq: int
    Hkv: int
    D: int
    V: int
    T: float
    seed: int
    qkv_dtype: str
    logits_dtype: str
    q: np.ndarray
    kv_pages: np.ndarray
    page_table: np.ndarray
    ctx_lens: np.ndarray
    logits_clean: np.ndarray
    logits_mask: np.ndarray
    draft_tokens: np.ndarray
    meta: dict = field(default_factory=dict)

    @property
    def R(self):
        return 2 * self.N - 1

    @property
    def K(self):
        return self.N - 1

    @property
    def num_pages(self):
        return int(self.kv_pages.shape[0])

    @property
    def max_pages(self):
        return int(self.page_table.shape[1])


def make_pages(rng, ctx_lens, max_pages, Hkv, D, dtype, permute=True, slack=1.1, min_pages=None):
    """KV pool and page table for the given contexts.

    Each sequence gets ceil(ctx/16) distinct physical pages.  With ``permute``
    the pool holds ``slack`` times the pages needed and each sequence's pages
    are a random subset in random order; otherwise pages are assigned in
    order (identity table for B = 1).
    """
    need = [(int(c) + PAGE - 1) // PAGE for c in ctx_lens]
    total = sum(need)
    P = max(total, int(np.ceil(total * slack)) if permute else total)
    if min_pages is not None:
        P = max(P, min_pages)
    slots = rng.permutation(P) if permute else np.arange(P)
    table = np.full((len(ctx_lens), max_pages), -1, dtype=np.int32)
    o = 0
    for b, n in enumerate(need):
        table[b, :n] = slots[o:o + n]
        o += n
    pool = _normal_store(rng, (P, 2, Hkv, PAGE * D), 1.0, dtype)
    return pool, table


def make_cache_state(rng, ctx_before, max_pages, Hkv, D, R, dtype, spare):
    """A cache before a step's KV append: pool, page table for ``ctx_before``,
    a free-page stack (the unused pool pages in random order, int32
    [P] with the first ``free_count`` valid) and the step's new K/V rows
    [B][R][Hkv][D].  ``spare`` extra pages beyond what the contexts use."""
    ctx_before = np.asarray(ctx_before, dtype=np.int32)
    used = int(sum((int(c) + PAGE - 1) // PAGE for c in ctx_before))
    pool, table = make_pages(rng, ctx_before, max_pages, Hkv, D, dtype, permute=True, slack=1.0,
                             min_pages=used + spare)
    in_use = np.zeros(pool.shape[0], dtype=bool)
    in_use[table[table >= 0]] = True
    free = rng.permutation(np.nonzero(~in_use)[0]).astype(np.int32)
    stack = np.full(pool.shape[0], -1, dtype=np.int32)
    stack[:len(free)] = free
    B = len(ctx_before)
    k_new = _normal_store(rng, (B, R, Hkv, D), 1.0, dtype)
    v_new = _normal_store(rng, (B, R, Hkv, D), 1.0, dtype)
    return pool, table, stack, len(free), k_new, v_new


def sample_drafts(rng, logits_mask, dtype, T, n_drafts=None):
    """Draft tokens drawn from softmax(mask / T) by Gumbel-max (argmax at T = 0).

    ``n_drafts`` (optional int [B]) truncates sequence b's list to that many
    drafts, the rest set to -1.
    """
    B, K, V = logits_mask.shape
    out = np.full((B, K), -1, dtype=np.int32)
    for b in range(B):
        for i in range(K):
            z = _store_to_f32(logits_mask[b, i], dtype).astype(np.float64)
            if T > 0:
                z = z / T + rng.gumbel(size=V)
            out[b, i] = int(np.argmax(z))
    if n_drafts is not None:
        for b in range(B):
            out[b, int(n_drafts[b]):] = -1
    return out


def make_logits(rng, B, N, V, dtype, scale=3.0, sigma=0.5, independent=False):
    """Logit rows: MASK rows ~ N(0, scale^2); verifying clean rows are the MASK
    row plus N(0, sigma^2) noise; the bonus clean row is an independent
    N(0, scale^2) draw.  ``independent`` draws every row on its own."""
    K = N - 1
    mask32 = rng.standard_normal((B, K, V), dtype=np.float32) * np.float32(scale)
    clean32 = np.empty((B, N, V), dtype=np.float32)
    if independent:
        clean32[:] = rng.standard_normal((B, N, V), dtype=np.float32) * np.float32(scale)
    else:
        clean32[:, :K] = mask32 + rng.standard_normal((B, K, V), dtype=np.float32) * np.float32(sigma)
        clean32[:, K] = rng.standard_normal((B, V), dtype=np.float32) * np.float32(scale)
    if dtype == "f32":
        return clean32, mask32
    return f32_to_bf16_bits(clean32), f32_to_bf16_bits(mask32)


def make_workload(name, B, N, Hq, Hkv, D, V, ctx_lens, T, seed, qkv_dtype="bf16",
                  logits_dtype="bf16", sigma=0.5, logit_scale=3.0, independent_logits=False,
                  permute=True, slack=1.1, max_pages=None, n_drafts=None, step_seed=None):
    """Build a workload from explicit sizes and contexts."""
    rng = np.random.Generator(np.random.PCG64(seed))
    R = 2 * N - 1
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    assert ctx_lens.shape == (B,) and (B == 0 or ctx_lens.min() >= R)
    if max_pages is None:
        max_pages = max(1, (int(ctx_lens.max()) + PAGE - 1) // PAGE if B else 1)
    pool, table = make_pages(rng, ctx_lens, max_pages, Hkv, D, qkv_dtype, permute=permute,
                             slack=slack)
    q = _normal_store(rng, (B, R, Hq, D), 1.0, qkv_dtype)
    clean, mask = make_logits(rng, B, N, V, logits_dtype, logit_scale, sigma, independent_logits)
    drafts = sample_drafts(rng, mask, logits_dtype, T, n_drafts)
    return Workload(name=name, B=B, N=N, Hq=Hq, Hkv=Hkv, D=D, V=V, T=float(T),
                    seed=int(seed if step_seed is None else step_seed),
                    qkv_dtype=qkv_dtype, logits_dtype=logits_dtype, q=q, kv_pages=pool,
                    page_table=table, ctx_lens=ctx_lens, logits_clean=clean,
                    logits_mask=mask, draft_tokens=drafts,
                    meta={"sigma": sigma, "logit_scale": logit_scale, "input_seed": seed})


SIGMAS = (0.1, 0.5, 1.5)
# Perturbations that give a mean sum_v min(p, q) of about 0.97 / 0.9 / 0.6 at
# T = 1 (the acceptance rates the C = 64 configuration quotes for its sweep,
# which SIGMAS as written do not reach).
CALIBRATED_SIGMAS = (0.074, 0.25, 1.07)


def named_workload(name, sigma_index=1, sigma=None):
    """The five named workloads of the module docstring, plus one GPU's share
    of the C = 64 step on eight GPUs (c64_dp8 by sequence, c64_tp8 by KV
    head).  For the C = 64 workloads, ``sigma`` replaces the swept value
    SIGMAS[sigma_index] (same contexts and seeds; CALIBRATED_SIGMAS give the
    acceptance rates the configuration names)."""
    if name == "tiny":
        return make_workload("tiny", B=1, N=4, Hq=8, Hkv=2, D=64, V=512, ctx_lens=[256],
                             T=1.0, seed=1000, qkv_dtype="f32", logits_dtype="f32",
                             logit_scale=2.0, independent_logits=True, permute=False,
                             step_seed=0)
    if name == "b1":
        return make_workload("b1", B=1, N=4, Hq=32, Hkv=8, D=128, V=VOCAB, ctx_lens=[4096],
                             T=1.0, seed=2000, slack=1.0)
    rng = np.random.Generator(np.random.PCG64(77))
    if name == "b16":
        ctx = rng.integers(1024, 8192, size=16, endpoint=True)
        return make_workload("b16", B=16, N=4, Hq=32, Hkv=8, D=128, V=VOCAB, ctx_lens=ctx,
                             T=1.0, seed=3000)
    if name == "c64":
        ctx = rng.integers(2048, 16384, size=64, endpoint=True)
        label = "c64_s" if sigma is None else "c64_calibrated_s"
        sigma = SIGMAS[sigma_index] if sigma is None else float(sigma)
        return make_workload(f"{label}{sigma}", B=64, N=4, Hq=32, Hkv=8, D=128, V=VOCAB,
                             ctx_lens=ctx, T=1.0, seed=4000 + sigma_index, sigma=sigma,
                             max_pages=16384 // PAGE)
    if name in ("c64_dp8", "c64_tp8"):
        # One GPU's share of the C = 64 step on eight GPUs.  dp8: split by
        # sequence, the first 8 of the same context draws (the step needs no
        # exchange across GPUs).  tp8: split by KV head, all 64 sequences with
        # one KV head and its 4 query heads (the attention's share; the
        # vocabulary-split acceptance would need a cross-GPU exchange).
        ctx = rng.integers(2048, 16384, size=64, endpoint=True)
        sigma = SIGMAS[sigma_index] if sigma is None else float(sigma)
        if name == "c64_dp8":
            return make_workload(f"c64_dp8_s{sigma}", B=8, N=4, Hq=32, Hkv=8, D=128, V=VOCAB,
                                 ctx_lens=ctx[:8], T=1.0, seed=4100 + sigma_index, sigma=sigma,
                                 max_pages=16384 // PAGE)
        return make_workload(f"c64_tp8_s{sigma}", B=64, N=4, Hq=4, Hkv=1, D=128, V=VOCAB,
                             ctx_lens=ctx, T=1.0, seed=4200 + sigma_index, sigma=sigma,
                             max_pages=16384 // PAGE)
    if name == "c64n8":
        ctx = rng.integers(4096, 32768, size=64, endpoint=True)
        return make_workload("c64n8", B=64, N=8, Hq=64, Hkv=8, D=128, V=VOCAB, ctx_lens=ctx,
                             T=0.7, seed=5000, max_pages=32768 // PAGE)
    raise KeyError(name)
