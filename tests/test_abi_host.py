"""The C ABI on the host: the library loads, exports every entry point that
include/idlm_isd.h declares, and validates sizes, temperature, pointers and
workspace before touching the GPU.  No kernel is launched here."""

import ctypes
import math
import os
import re

import pytest

from speculative_verify_isd_amd import lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "idlm_isd.h")


@pytest.fixture(scope="module")
def so():
    if not os.path.exists(L.LIB_PATH):
        from speculative_verify_isd_amd.build import build
        build()
    return L.load()


def declared_entry_points():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(idlm_isd_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_names():
    assert declared_entry_points() == sorted(L.ENTRY_POINTS)


def test_library_exports_every_declared_symbol(so):
    for name in declared_entry_points():
        assert hasattr(so, name), name


def good(**kw):
    base = dict(B=64, N=4, Hq=32, Hkv=8, D=128, V=151936, max_pages=1024, num_pages=40000)
    base.update(kw)
    return L.make_dims(**base)


def test_validate_accepts_the_step_shapes(so):
    for d in (good(), good(N=8, Hq=64), good(B=1, D=64, Hq=8, Hkv=2, V=512, qkv_dtype="f32",
                                              logits_dtype="f32"), good(N=1), good(B=0),
              good(N=16, Hq=4, Hkv=4), good(N=16, Hq=16, Hkv=4)):  # 31- and 124-row tiles
        assert L.idlm_isd_validate(d, 1.0) == 0
    assert L.idlm_isd_validate(good(), 0.0) == 0  # greedy


@pytest.mark.parametrize("kw,code", [
    (dict(N=0), 2), (dict(N=17), 2), (dict(Hq=30), 2), (dict(Hkv=0), 2), (dict(V=0), 2),
    (dict(B=-1), 2), (dict(max_pages=0), 2), (dict(num_pages=0), 2),
    (dict(D=96), 3), (dict(page_size=8), 3), (dict(N=9, Hq=64), 3),
])
def test_validate_rejects(so, kw, code):
    assert L.idlm_isd_validate(good(**kw), 1.0) == code
    assert L.idlm_isd_workspace_bytes(good(**kw)) == 0


def test_validate_rejects_bad_dtype(so):
    d = good()
    d.qkv_dtype = 5
    assert L.idlm_isd_validate(d, 1.0) == 2


@pytest.mark.parametrize("T", [-0.1, math.nan, math.inf])
def test_validate_rejects_temperature(so, T):
    assert L.idlm_isd_validate(good(), T) == 4


def test_null_dims(so):
    assert so.idlm_isd_validate(None, 1.0) == 1
    assert so.idlm_isd_workspace_bytes(None) == 0


def test_workspace_bytes_grow_with_batch(so):
    a = L.idlm_isd_workspace_bytes(good(B=16))
    b = L.idlm_isd_workspace_bytes(good(B=64))
    assert 0 < a < b
    assert b % 256 == 0


def test_entry_points_validate_before_launch(so):
    # All of these return before any HIP call: bad sizes, NULL or short workspace.
    d = good()
    n = L.idlm_isd_workspace_bytes(d)
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    assert so.idlm_isd_paged_attn(ctypes.byref(good(D=96)), fake, fake, fake, fake, fake,
                                  fake, n, None) == 3
    assert so.idlm_isd_paged_attn(ctypes.byref(d), fake, fake, fake, fake, fake, None, n,
                                  None) == 1
    assert so.idlm_isd_paged_attn(ctypes.byref(d), fake, fake, fake, fake, fake, fake, n - 256,
                                  None) == 5
    misaligned = ctypes.c_void_p((1 << 20) + 8)
    assert so.idlm_isd_accept(ctypes.byref(d), fake, fake, fake, 1, 1.0, fake, fake, None, None,
                              misaligned, n, None) == 5
    assert so.idlm_isd_accept(ctypes.byref(d), fake, fake, fake, 1, -1.0, fake, fake, None, None,
                              fake, n, None) == 4
    assert so.idlm_isd_accept(ctypes.byref(d), None, fake, fake, 1, 1.0, fake, fake, None, None,
                              fake, n, None) == 1
    # a misaligned MASK-row statistics record
    assert so.idlm_isd_accept(ctypes.byref(d), fake, fake, fake, 1, 1.0, fake, fake, None,
                              misaligned, fake, n, None) == 5
    assert so.idlm_isd_step(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, 1, 3, 1.0,
                            fake, fake, fake, None, fake, n, None) == 2  # N repeated must match
    assert so.idlm_isd_read_status(None, None, None) == 1
    assert so.idlm_isd_workspace_init(misaligned, 1024, None) == 5


def test_empty_batch_is_a_no_op(so):
    d = good(B=0)
    n = L.idlm_isd_workspace_bytes(d)
    fake = ctypes.c_void_p(1 << 20)
    assert so.idlm_isd_step(ctypes.byref(d), None, None, None, None, None, None, None, 1, 4, 1.0,
                            None, None, None, None, fake, n, None) == 0


def test_strerror(so):
    for code, name in L.STATUS.items():
        s = L.strerror(code)
        assert isinstance(s, str) and s
    assert L.strerror(99) == "unknown status"


def test_kv_append_rejects_before_launch(so):
    d = good()
    n = L.idlm_isd_workspace_bytes(d)
    fake = ctypes.c_void_p(1 << 20)
    a = [fake] * 8
    assert so.idlm_isd_kv_append(ctypes.byref(good(D=96)), *a, fake, n, None) == 3
    assert so.idlm_isd_kv_append(ctypes.byref(d), None, *a[1:], fake, n, None) == 1
    assert so.idlm_isd_kv_append(ctypes.byref(d), *a[:7], None, fake, n, None) == 1
    assert so.idlm_isd_kv_append(ctypes.byref(d), *a, fake, n - 256, None) == 5
    r = [fake] * 6
    assert so.idlm_isd_kv_rollback(ctypes.byref(d), None, *r[1:], fake, n, None) == 1
    assert so.idlm_isd_kv_rollback(ctypes.byref(d), *r, None, n, None) == 1
    assert so.idlm_isd_kv_rollback(ctypes.byref(good(N=0)), *r, fake, n, None) == 2
    e = good(B=0)
    ne = L.idlm_isd_workspace_bytes(e)
    assert so.idlm_isd_kv_append(ctypes.byref(e), *([None] * 8), fake, ne, None) == 0
    assert so.idlm_isd_kv_rollback(ctypes.byref(e), *([None] * 6), fake, ne, None) == 0


def test_gated_lora_validates_before_launch(so):
    ok = L.LoraDims(64, 4, 4096, 4096, 128)
    n = L.idlm_isd_lora_workspace_bytes(ok)
    assert n > 0 and n % 256 == 0
    for bad, code in ((L.LoraDims(64, 4, 4004, 4096, 128), 3), (L.LoraDims(64, 4, 4096, 4096, 100), 3),
                      (L.LoraDims(64, 0, 4096, 4096, 128), 2), (L.LoraDims(-1, 4, 4096, 64, 16), 2)):
        assert L.idlm_isd_lora_workspace_bytes(bad) == 0
        assert so.idlm_isd_gated_lora(ctypes.byref(bad), None, None, None, None, ctypes.c_float(1.0),
                                      None, None, 0, None) == code
    fake = ctypes.c_void_p(1 << 20)
    assert so.idlm_isd_gated_lora(ctypes.byref(ok), fake, fake, fake, fake, ctypes.c_float(1.0),
                                  fake, fake, n - 256, None) == 5
    assert so.idlm_isd_gated_lora(ctypes.byref(ok), None, fake, fake, fake, ctypes.c_float(1.0),
                                  fake, fake, n, None) == 1
    assert so.idlm_isd_gated_lora(ctypes.byref(ok), fake, ctypes.c_void_p((1 << 20) + 2), fake,
                                  fake, ctypes.c_float(1.0), fake, fake, n, None) == 3
    assert so.idlm_isd_gated_lora(ctypes.byref(ok), fake, fake, fake, fake,
                                  ctypes.c_float(float("nan")), fake, fake, n, None) == 2


# ---------------------------------------------------------------------------
# The Python binding's checks, on CPU tensors: the device check is stubbed to
# pass and the stream lookup (the last argument of every call) to raise, so
# every check runs and no call reaches the library.
# ---------------------------------------------------------------------------
class _Reached(Exception):
    pass


@pytest.fixture
def host_binding(so, monkeypatch):
    def stream():
        raise _Reached()

    monkeypatch.setattr(L, "_on_device", lambda t: True)
    monkeypatch.setattr(L, "_stream", stream)
    return L

def _binding_args():
    import torch

    B, N, Hq, Hkv, D, V, mp, P = 2, 4, 8, 2, 64, 100, 4, 8
    R, K = 2 * N - 1, N - 1
    d = L.make_dims(B, N, Hq, Hkv, D, V, mp, P)
    bf, i32 = torch.bfloat16, torch.int32
    t = {
        "q": torch.zeros(B * R * Hq * D, dtype=bf),
        "kv_pages": torch.zeros(P * 2 * Hkv * 16 * D, dtype=bf),
        "page_table": torch.zeros(B * mp, dtype=i32),
        "ctx_lens": torch.zeros(B, dtype=i32),
        "attn_out": torch.zeros(B * R * Hq * D, dtype=bf),
        "logits_clean": torch.zeros(B * N * V, dtype=bf),
        "logits_mask": torch.zeros(B * K * V, dtype=bf),
        "draft_tokens": torch.zeros(B * K, dtype=i32),
        "out_tokens": torch.zeros(B * N, dtype=i32),
        "out_accept_len": torch.zeros(B, dtype=i32),
        "workspace": torch.zeros(L.idlm_isd_workspace_bytes(d), dtype=torch.uint8),
    }
    return d, t


def _call_step(d, t):
    L.idlm_isd_step(d, t["q"], t["kv_pages"], t["page_table"], t["ctx_lens"], t["logits_clean"],
                    t["logits_mask"], t["draft_tokens"], 1, d.N, 1.0, t["out_tokens"],
                    t["out_accept_len"], t["attn_out"], t["workspace"])


def test_binding_names_a_short_tensor(host_binding):
    d, t = _binding_args()
    for name in ("q", "kv_pages", "page_table", "ctx_lens", "attn_out", "logits_clean",
                 "logits_mask", "draft_tokens", "out_tokens", "out_accept_len"):
        short = dict(t)
        short[name] = t[name][:-1]
        with pytest.raises(ValueError, match=name):
            _call_step(d, short)
    with pytest.raises(_Reached):  # every size right
        _call_step(d, t)
    with pytest.raises(ValueError, match="logits_mask"):  # N = 4 needs MASK rows
        _call_step(d, dict(t, logits_mask=t["logits_mask"][:0]))
    # B = 0 is a no-op: empty tensors pass
    d0 = L.make_dims(0, 4, 8, 2, 64, 100, 4, 8)
    with pytest.raises(_Reached):
        _call_step(d0, {k: (v if k == "workspace" else v[:0]) for k, v in t.items()})


def test_binding_checks_every_entry_points_sizes(host_binding):
    import torch

    d, t = _binding_args()
    with pytest.raises(ValueError, match="logits_next"):
        L.idlm_isd_propose(d, t["logits_mask"][:-1], t["draft_tokens"], t["out_accept_len"], 1,
                           1.0, t["draft_tokens"], t["workspace"])
    d1 = L.make_dims(2, 1, 8, 2, 64, 100, 4, 8)  # N = 1: a no-op that reads nothing
    with pytest.raises(_Reached):
        L.idlm_isd_propose(d1, t["q"][:0], t["ctx_lens"][:0], t["ctx_lens"][:0], 1, 1.0,
                           t["ctx_lens"][:0], t["workspace"])
    i32 = torch.int32
    with pytest.raises(ValueError, match="free_pages"):
        L.idlm_isd_kv_append(d, t["q"][:2 * 7 * 2 * 64], t["q"][:2 * 7 * 2 * 64], t["ctx_lens"],
                             t["ctx_lens"], t["kv_pages"], t["page_table"],
                             torch.zeros(d.num_pages - 1, dtype=i32), torch.zeros(1, dtype=i32),
                             t["workspace"])
    with pytest.raises(ValueError, match="k_new"):
        L.idlm_isd_kv_append(d, t["q"][:10], t["q"][:2 * 7 * 2 * 64], t["ctx_lens"],
                             t["ctx_lens"], t["kv_pages"], t["page_table"],
                             torch.zeros(d.num_pages, dtype=i32), torch.zeros(1, dtype=i32),
                             t["workspace"])
    with pytest.raises(ValueError, match="free_count"):
        L.idlm_isd_kv_rollback(d, t["ctx_lens"], t["out_accept_len"], t["ctx_lens"],
                               t["page_table"], torch.zeros(d.num_pages, dtype=i32),
                               torch.zeros(0, dtype=i32), t["workspace"])
    ld = L.LoraDims(2, 4, 64, 32, 16)
    M = 2 * 7
    bf = torch.bfloat16
    with pytest.raises(ValueError, match="lora_b"):
        L.idlm_isd_gated_lora(ld, torch.zeros(M * 32), torch.zeros(M * 64, dtype=bf),
                              torch.zeros(16 * 64, dtype=bf), torch.zeros(32 * 16 - 1, dtype=bf),
                              0.5, torch.zeros(M * 32, dtype=bf),
                              torch.zeros(64, dtype=torch.uint8))


# ---------------------------------------------------------------------------
# Sizes whose grids would not fit one dispatch, temperatures whose exponent
# scale would overflow float32, and the workspace's state region.
# ---------------------------------------------------------------------------
def test_validate_rejects_grids_beyond_one_dispatch(so):
    # 2^22 sequences of 7 rows of 8 logits: small in bytes, but the
    # acceptance's statistics grid would need 7 * 2^22 work-groups of 256.
    assert L.idlm_isd_validate(L.make_dims(1 << 22, 4, 1, 1, 64, 8, 1, 1), 1.0) == 3
    assert L.idlm_isd_workspace_bytes(L.make_dims(1 << 22, 4, 1, 1, 64, 8, 1, 1)) == 0
    assert L.idlm_isd_validate(L.make_dims(1 << 20, 4, 1, 1, 64, 8, 1, 1), 1.0) == 0


def test_gated_lora_rejects_grids_beyond_one_dispatch(so):
    huge = L.LoraDims(1 << 20, 2, 65536, 1, 256)  # down projection: > 2^32 work-items
    assert L.idlm_isd_lora_workspace_bytes(huge) == 0
    assert so.idlm_isd_gated_lora(ctypes.byref(huge), None, None, None, None,
                                  ctypes.c_float(1.0), None, None, 0, None) == 3
    assert L.idlm_isd_lora_workspace_bytes(L.LoraDims(1 << 20, 2, 4096, 512, 256)) > 0


@pytest.mark.parametrize("T,code", [(1e-39, 4), (2.0 ** -127, 4), (2.0 ** -126, 0),
                                    (3e38, 0), (0.0, 0)])
def test_temperature_range(so, T, code):
    # 0 < T < 2^-126 would make log2(e)/T overflow float32; 0 is greedy.
    assert L.idlm_isd_validate(good(), T) == code


def test_workspace_state_bytes(so):
    d = good()
    s = so.idlm_isd_workspace_state_bytes(ctypes.byref(d))
    assert s == 256  # the sticky status word, padded to the workspace alignment
    assert s < L.idlm_isd_workspace_bytes(d)
    assert so.idlm_isd_workspace_state_bytes(None) == 0
    assert so.idlm_isd_workspace_state_bytes(ctypes.byref(good(D=96))) == 0


def test_accept_probs_validates_before_launch(so):
    d = good()
    n = L.idlm_isd_workspace_bytes(d)
    fake = ctypes.c_void_p(1 << 20)
    f = ctypes.c_float
    assert so.idlm_isd_accept_probs(None, fake, fake, f(1.0), fake, n, fake, fake, fake,
                                    None) == 1
    assert so.idlm_isd_accept_probs(ctypes.byref(d), fake, fake, f(-1.0), fake, n, fake, fake,
                                    fake, None) == 4
    assert so.idlm_isd_accept_probs(ctypes.byref(d), fake, fake, f(1.0), fake, n - 256, fake,
                                    fake, fake, None) == 5
    assert so.idlm_isd_accept_probs(ctypes.byref(d), None, fake, f(1.0), fake, n, fake, fake,
                                    fake, None) == 1


def test_accept_noalloc_validates_before_launch(so):
    fake = ctypes.c_void_p(1 << 20)
    f = ctypes.c_float
    d = good()
    assert so.idlm_isd_accept_noalloc(None, fake, fake, fake, 1, f(1.0), fake, fake, None, None,
                                      None, None) == 1
    assert so.idlm_isd_accept_noalloc(ctypes.byref(d), fake, fake, fake, 1, f(-1.0), fake, fake,
                                      None, None, None, None) == 4
    assert so.idlm_isd_accept_noalloc(ctypes.byref(d), None, fake, fake, 1, f(1.0), fake, fake,
                                      None, None, None, None) == 1
    # The scratch need stated in the header: 256 bytes plus seven regions,
    # each rounded up to 256 bytes.  Sizes over 8 MiB are refused (8) before
    # anything is looked up; sizes within it reach the pointer checks (1).
    def need(B, N=4, V=151936):
        R, c8, c2 = 2 * N - 1, -(-V // 8192), -(-V // 2048)
        r = lambda x: -(-x // 256) * 256
        return 256 + sum(r(x) for x in (B * 64, B * R * 16 * c8, B * 32 * c2, B * R * 4,
                                         B * 256, B * R * 32, B * 8 * c2))
    last = max(B for B in range(1, 4096) if need(B) <= L.NOALLOC_SCRATCH_BYTES)
    assert last == 1471 and need(64) < 400_000
    for B, code in ((last, 1), (last + 1, 8), (4096, 8)):
        big = good(B=B)
        assert L.idlm_isd_validate(big, 1.0) == 0
        assert so.idlm_isd_accept_noalloc(ctypes.byref(big), None, fake, fake, 1, f(1.0), fake,
                                          fake, None, None, None, None) == code
    assert L.strerror(8) != "unknown status"
    z = good(B=0)
    assert so.idlm_isd_accept_noalloc(ctypes.byref(z), None, None, None, 1, f(1.0), None, None,
                                      None, None, None, None) == 0


def test_loop_step_validates_before_launch(so):
    d = good()
    n = L.idlm_isd_workspace_bytes(d)
    fake = ctypes.c_void_p(1 << 20)
    mis = ctypes.c_void_p((1 << 20) + 64)
    f = ctypes.c_float(1.0)
    args = lambda ms_next, nxt, ln: (fake, fake, fake, fake, fake, fake, fake, None, ln, 1, 4, f,
                                     fake, fake, fake, nxt, ms_next, fake, n, None)
    assert so.idlm_isd_loop_step(None, *args(None, fake, fake)) == 1
    assert so.idlm_isd_loop_step(ctypes.byref(d), *args(mis, fake, fake)) == 5
    assert so.idlm_isd_loop_step(ctypes.byref(d), *args(None, None, fake)) == 1
    assert so.idlm_isd_loop_step(ctypes.byref(d), *args(None, fake, None)) == 1
    z = good(B=0)
    assert so.idlm_isd_loop_step(ctypes.byref(z), None, None, None, None, None, None, None, None,
                                 None, 1, 4, f, None, None, None, None, None, fake,
                                 L.idlm_isd_workspace_bytes(z), None) == 0


def test_mask_stats_bytes(so):
    # header (256) + each MASK row's (max, sum) [B][K] + logits and drafts [B][K]
    d = good()
    K = 3
    r = lambda x: -(-x // 256) * 256
    assert L.idlm_isd_mask_stats_bytes(d) == 256 + r(64 * K * 16) + r(64 * K * 4) * 2
    assert L.idlm_isd_mask_stats_bytes(good(N=1)) == 256
    assert L.idlm_isd_mask_stats_bytes(good(D=96)) == 0
    assert so.idlm_isd_mask_stats_bytes(None) == 0
    fake = ctypes.c_void_p(1 << 20)
    n = L.idlm_isd_workspace_bytes(d)
    assert so.idlm_isd_propose(ctypes.byref(d), fake, fake, fake, 1, ctypes.c_float(1.0), fake,
                               ctypes.c_void_p((1 << 20) + 64), fake, n, None) == 5
