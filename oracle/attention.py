"""Strictly causal GQA attention of the ISD step rows over a paged KV cache.
Test infrastructure.

What the pages fix
------------------
* Attention is strictly causal over every position, which is what lets the
  model run inside an ordinary autoregressive serving stack
  ("Introspective Diffusion Language Models", sections "Training" and
  "Serving (SGLang)"; GeekNews summary, section "I-DLM Yontemi").
* One forward handles 2N-1 query positions per sequence: at N=4 that is 7
  ("Introspective Diffusion Language Models", section "How do DLMs perform as
  they approach compute-bound?").
* The KV cache is paged ("Serving (SGLang)" on both README pages).

Readings taken where the pages are silent
-----------------------------------------
* Scores are q.k / sqrt(D); rotary embedding is applied before the cache, so q
  and k arrive rotated; no bias, window or soft-cap.
* Query head h reads KV head h // G with G = Hq / Hkv (grouped-query
  attention).
* ``ctx_lens[b]`` counts the R = 2N-1 new rows, whose K/V are already in the
  pages.  Row r sits at absolute position ctx - R + r and sees tokens
  0 .. ctx - R + r.

Paged layout (the library's; defined in include/idlm_isd.h)
-----------------------------------------------------------
``kv_pages`` has shape [P][2][Hkv][16*D]: for every physical page, a K block
and a V block per KV head, each holding 16 token slots.

* K block: 16-byte column chunks.  With x = 16 / element size (8 for
  bfloat16, 4 for float32), element (slot s, dim d) is at
  ((d // x) * 16 + s) * x + d % x.
* V block: transposed, element (slot s, dim d) is at d * 16 + s.

Logical token t of sequence b lives in physical page
``page_table[b][t // 16]`` at slot t % 16.

The oracle gathers K and V page by page through that map, widening each block
to float64 as it goes, and evaluates the definition directly: scores,
max-subtracted softmax, weighted sum.

Pinned in tests/test_oracle_attention.py: a pure-Python triple loop on tiny
shapes, torch's scaled_dot_product_attention in float64 with an explicit
offset mask, page-permutation invariance, constant-V, R=1 decode and
single-row key visibility.
"""

import math

import numpy as np

from .dtypes import to_f64

PAGE = 16


def chunk_elems(dtype):
    """Elements per 16-byte chunk of a K block."""
    if dtype == "bf16":
        return 8
    if dtype in ("f32",):
        return 4
    raise ValueError(f"unsupported KV dtype {dtype!r}")


def gather_kv(kv_pages, kv_dtype, page_table_row, ctx, h, D):
    """Logical K[ctx][D] and V[ctx][D] (float64) of one sequence and KV head.

    ``kv_pages`` is the pool [P][2][Hkv][16*D] in its storage dtype
    (``kv_dtype``: "bf16" bit patterns or "f32").  Page by page: the K block
    viewed as [D/x][16][x] holds K[s][c*x + i] at [c][s][i]; the V block
    viewed as [D][16] holds V[s][d] at [d][s].
    """
    x = chunk_elems(kv_dtype)
    npages = (ctx + PAGE - 1) // PAGE
    phys = np.asarray(page_table_row[:npages], dtype=np.int64)  # page p -> physical page
    # K blocks [page][D/x][16][x] -> [page][slot][D/x][x] = [page*16 + slot][D]
    kblk = to_f64(kv_pages[phys, 0, h], kv_dtype).reshape(npages, D // x, PAGE, x)
    K = kblk.transpose(0, 2, 1, 3).reshape(npages * PAGE, D)
    # V blocks [page][D][16] -> [page][slot][D]
    vblk = to_f64(kv_pages[phys, 1, h], kv_dtype).reshape(npages, D, PAGE)
    V = vblk.transpose(0, 2, 1).reshape(npages * PAGE, D)
    return K[:ctx], V[:ctx]


def isd_attention(q, kv_pages, page_table, ctx_lens, N, Hkv, kv_dtype):
    """Attention outputs of the 2N-1 step rows, float64 [B][R][Hq][D].

    q          float64 [B][R][Hq][D]
    kv_pages   [P][2][Hkv][16*D] in storage dtype ``kv_dtype``
    page_table int [B][max_pages]
    ctx_lens   int [B]
    """
    B, R, Hq, D = q.shape
    assert R == 2 * N - 1, "the step has 2N-1 query rows"
    assert Hq % Hkv == 0
    G = Hq // Hkv
    out = np.zeros((B, R, Hq, D), dtype=np.float64)
    for b in range(B):
        ctx = int(ctx_lens[b])
        assert R <= ctx <= PAGE * page_table.shape[1]
        # Row r sees tokens 0 .. ctx - R + r: the rest of its score row is
        # masked to -inf (weight exactly 0).  The G query heads of KV head h
        # (heads h*G .. h*G + G - 1) are evaluated together: score row
        # r*G + g belongs to row r and query head h*G + g.
        last = np.repeat(ctx - R + np.arange(R), G)
        hidden = np.arange(ctx)[None, :] > last[:, None]
        for h in range(Hkv):
            K, V = gather_kv(kv_pages, kv_dtype, page_table[b], ctx, h, D)
            qh = q[b, :, h * G:(h + 1) * G].reshape(R * G, D)
            scores = qh @ K.T / math.sqrt(D)  # [R*G][ctx]
            scores[hidden] = -np.inf
            e = np.exp(scores - scores.max(axis=1, keepdims=True))
            a = e / e.sum(axis=1, keepdims=True)
            out[b, :, h * G:(h + 1) * G] = (a @ V).reshape(R, G, D)
    return out


def isd_attention_rows(q, kv_pages, page_table, ctx_lens, N, Hkv, kv_dtype, picks):
    """The same definition evaluated only at sampled (b, r, hq) triples.

    Returns float64 [len(picks)][D].  Used at full sizes, where evaluating
    every row on the CPU would take too long.
    """
    B, R, Hq, D = q.shape
    G = Hq // Hkv
    cache = {}
    res = np.zeros((len(picks), D), dtype=np.float64)
    for n, (b, r, hq) in enumerate(picks):
        ctx = int(ctx_lens[b])
        h = hq // G
        if (b, h) not in cache:
            cache[(b, h)] = gather_kv(kv_pages, kv_dtype, page_table[b], ctx, h, D)
        K, V = cache[(b, h)]
        pos = ctx - R + r
        scores = K[: pos + 1] @ q[b, r, hq] / math.sqrt(D)
        e = np.exp(scores - scores.max())
        res[n] = (e / e.sum()) @ V[: pos + 1]
    return res
