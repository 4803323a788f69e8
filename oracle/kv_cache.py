"""KV-cache append and rollback around one ISD step.  Test infrastructure.

What the pages fix
------------------
* The cache is paged and serves continuous batching ("Introspective
  Diffusion Language Models" and its GeekNews summary, section "Serving
  (SGLang)").
* A step verifies the previous step's drafts and keeps only the accepted
  prefix: rows after the first rejection (the rejected draft, the drafts
  after it and the MASK rows) do not become context ("Inference & ISD").

Readings taken where the pages are silent
-----------------------------------------
* Append happens before attention: the step's R = 2N-1 rows get positions
  ctx_before .. ctx_before + R - 1 and the attention's ctx_lens is
  ctx_before + R.
* Rollback after acceptance keeps the anchor and the accepted drafts:
  the new context is ctx_lens - R + accept_len.  The resampled or bonus
  token is the next step's anchor, so its K/V comes with the next forward.
* Pages come from a free list used as a stack: a call needing T pages in
  total takes the top T entries, sequence by sequence in batch order, each
  sequence's pages in page order; rollback pushes the pages a sequence no
  longer needs in the same order.  Freed pages keep their stale contents.
* Bad input (a context out of range, an accept length outside [1, R], too
  few free pages, a free-list page id outside the pool) is reported, and the
  library leaves the affected state unchanged, as below.

Pinned in tests/test_oracle_kv_cache.py against the attention oracle's
gather (itself pinned against a brute-force scatter), conservation of the
page set, and the stack order.
"""

import numpy as np

from .attention import PAGE, chunk_elems


def pages_of(n):
    return (np.asarray(n, dtype=np.int64) + PAGE - 1) // PAGE


def kv_append(kv_pages, page_table, ctx_before, k_new, v_new, free_pages, free_count, kv_dtype):
    """Write the step rows' K/V into the cache.

    kv_pages   [P][2][Hkv][16*D] storage dtype (copied, not modified)
    page_table int [B][max_pages] (copied)
    ctx_before int [B]: tokens already cached
    k_new, v_new [B][R][Hkv][D] storage dtype
    free_pages int [capacity], stack; entries [0, free_count) are free
    Returns (kv_pages, page_table, ctx_after, free_count, errors) where errors
    is a set of strings; on "no_pages" / "bad_page" nothing is written.
    """
    pool = np.array(kv_pages, copy=True)
    table = np.array(page_table, copy=True)
    B, R, Hkv, D = k_new.shape
    max_pages = table.shape[1]
    P = pool.shape[0]
    x = chunk_elems(kv_dtype)
    ctx = np.asarray(ctx_before, dtype=np.int64)
    errors = set()
    valid = (ctx >= 0) & (ctx + R <= PAGE * max_pages)
    if not valid.all():
        errors.add("bad_ctx")
    need = np.where(valid, pages_of(ctx + R) - pages_of(ctx), 0)
    total = int(need.sum())
    if total > free_count:
        errors.add("no_pages")
        return pool, table, ctx.copy(), free_count, errors
    base = free_count - total
    taken = np.asarray(free_pages[base:free_count], dtype=np.int64)
    if ((taken < 0) | (taken >= P)).any():
        errors.add("bad_page")
        return pool, table, ctx.copy(), free_count, errors
    k = base
    for b in range(B):
        for i in range(int(need[b])):
            table[b, int(pages_of(ctx[b])) + i] = free_pages[k]
            k += 1
    for b in range(B):
        if not valid[b]:
            continue
        for r in range(R):
            t = int(ctx[b]) + r
            page, s = int(table[b, t // PAGE]), t % PAGE
            for h in range(Hkv):
                kblk = pool[page, 0, h].reshape(D // x, PAGE, x)  # views into pool
                vblk = pool[page, 1, h].reshape(D, PAGE)
                kblk[:, s, :] = k_new[b, r, h].reshape(D // x, x)
                vblk[:, s] = v_new[b, r, h]
    ctx_after = np.where(valid, ctx + R, ctx)
    return pool, table, ctx_after, base, errors


def kv_rollback(page_table, ctx_lens, accept_len, R, free_pages, free_count):
    """Truncate every sequence to its kept prefix and free unused pages.

    ctx_lens  int [B]: the step's context, R rows included
    accept_len int [B] in [1, R] (clamped otherwise, reported)
    free_pages stack with capacity len(free_pages)
    Returns (page_table, ctx_after, free_pages, free_count, errors).
    """
    table = np.array(page_table, copy=True)
    fp = np.array(free_pages, copy=True)
    B, max_pages = table.shape
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    acc = np.asarray(accept_len, dtype=np.int64)
    errors = set()
    valid = (ctx >= R) & (ctx <= PAGE * max_pages)
    if not valid.all():
        errors.add("bad_ctx")
    if ((acc < 1) | (acc > R)).any():
        errors.add("bad_len")
    acc = np.clip(acc, 1, R)
    keep = np.where(valid, ctx - R + acc, ctx)
    freed = np.where(valid, pages_of(ctx) - pages_of(keep), 0)
    total = int(freed.sum())
    if free_count + total > len(fp):
        errors.add("free_overflow")
        return table, ctx.copy(), fp, free_count, errors
    k = free_count
    for b in range(B):
        first = int(pages_of(keep[b]))
        for i in range(int(freed[b])):
            fp[k] = table[b, first + i]
            table[b, first + i] = -1
            k += 1
    return table, keep, fp, free_count + total, errors
