"""ctypes binding of libidlm_isd.so (C ABI in include/idlm_isd.h).

Argument marshalling only: every function here checks tensor dtypes,
contiguity, sizes (each tensor must hold at least the elements the sizes in
``dims`` imply, since the kernels index by those sizes) and devices, then
passes raw device pointers and torch's current HIP stream to the entry point
of the same name.  No step arithmetic happens in
Python and there is no fallback: if the library is missing, ``load()``
raises.
"""

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libidlm_isd.so")

IDLM_BF16 = 0
IDLM_F32 = 1

STATUS = {
    0: "IDLM_OK",
    1: "IDLM_ERR_NULL",
    2: "IDLM_ERR_DIMS",
    3: "IDLM_ERR_UNSUPPORTED",
    4: "IDLM_ERR_TEMPERATURE",
    5: "IDLM_ERR_WORKSPACE",
    6: "IDLM_ERR_HIP",
    7: "IDLM_ERR_DEVICE_DATA",
    8: "IDLM_ERR_SCRATCH",
}

# idlm_isd_accept_noalloc's static scratch per GPU (IDLM_ISD_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 8 << 20

# Every entry point declared in include/idlm_isd.h.
ENTRY_POINTS = (
    "idlm_isd_workspace_bytes",
    "idlm_isd_workspace_state_bytes",
    "idlm_isd_validate",
    "idlm_isd_workspace_init",
    "idlm_isd_paged_attn",
    "idlm_isd_mask_stats_bytes",
    "idlm_isd_accept",
    "idlm_isd_accept_probs",
    "idlm_isd_accept_noalloc",
    "idlm_isd_step",
    "idlm_isd_loop_step",
    "idlm_isd_propose",
    "idlm_isd_lora_workspace_bytes",
    "idlm_isd_gated_lora",
    "idlm_isd_kv_append",
    "idlm_isd_kv_rollback",
    "idlm_isd_read_status",
    "idlm_isd_strerror",
)


class IdlmError(RuntimeError):
    def __init__(self, code, where):
        self.code = int(code)
        super().__init__(f"{where}: {STATUS.get(self.code, self.code)} ({strerror(self.code)})")


class Dims(ctypes.Structure):
    """idlm_isd_dims."""

    _fields_ = [(n, ctypes.c_int32) for n in (
        "B", "N", "Hq", "Hkv", "D", "V", "page_size", "max_pages", "num_pages",
        "qkv_dtype", "logits_dtype")]


class LoraDims(ctypes.Structure):
    """idlm_isd_lora_dims."""
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "N", "H", "O", "rank")]


def make_dims(B, N, Hq, Hkv, D, V, max_pages, num_pages, qkv_dtype="bf16", logits_dtype="bf16",
              page_size=16):
    code = {"bf16": IDLM_BF16, "f32": IDLM_F32}
    return Dims(B, N, Hq, Hkv, D, V, page_size, max_pages, num_pages, code[qkv_dtype],
                code[logits_dtype])


_lib = None


def load():
    """Load libidlm_isd.so (once); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m speculative_verify_isd_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    D = ctypes.POINTER(Dims)
    i32, u64, f32, sz = ctypes.c_int32, ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "idlm_isd_workspace_bytes": (sz, [D]),
        "idlm_isd_workspace_state_bytes": (sz, [D]),
        "idlm_isd_validate": (i32, [D, f32]),
        "idlm_isd_workspace_init": (i32, [P, sz, P]),
        "idlm_isd_paged_attn": (i32, [D, P, P, P, P, P, P, sz, P]),
        "idlm_isd_accept": (i32, [D, P, P, P, u64, f32, P, P, P, P, P, sz, P]),
        "idlm_isd_mask_stats_bytes": (sz, [D]),
        "idlm_isd_accept_probs": (i32, [D, P, P, f32, P, sz, P, P, P, P]),
        "idlm_isd_accept_noalloc": (i32, [D, P, P, P, u64, f32, P, P, P, P, P, P]),
        "idlm_isd_step": (i32, [D, P, P, P, P, P, P, P, u64, i32, f32, P, P, P, P, P, sz, P]),
        "idlm_isd_loop_step": (i32, [D, P, P, P, P, P, P, P, P, P, u64, i32, f32, P, P, P, P, P,
                                     P, sz, P]),
        "idlm_isd_propose": (i32, [D, P, P, P, u64, f32, P, P, P, sz, P]),
        "idlm_isd_lora_workspace_bytes": (sz, [ctypes.POINTER(LoraDims)]),
        "idlm_isd_gated_lora": (i32, [ctypes.POINTER(LoraDims), P, P, P, P, f32, P, P, sz, P]),
        "idlm_isd_kv_append": (i32, [D, P, P, P, P, P, P, P, P, P, sz, P]),
        "idlm_isd_kv_rollback": (i32, [D, P, P, P, P, P, P, P, sz, P]),
        "idlm_isd_read_status": (i32, [P, P, ctypes.POINTER(i32)]),
        "idlm_isd_strerror": (ctypes.c_char_p, [i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def strerror(code):
    return load().idlm_isd_strerror(int(code)).decode()


def _check(code, where):
    if code != 0:
        raise IdlmError(code, where)


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------
def _torch():
    import torch

    return torch


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t, dtypes, name, allow_none=False, numel=None):
    """Device pointer of ``t`` after the checks; ``numel`` is the least
    number of elements the call will touch."""
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements; these sizes need {numel}")
    if not _on_device(t):
        raise TypeError(f"{name} must be a CUDA/HIP tensor")
    return ctypes.c_void_p(t.data_ptr())


def _on_device(t):
    return t.is_cuda


def _sizes(dims):
    """Element counts of the step's arrays for ``dims`` (idlm_isd.h layouts);
    all zero for B = 0, a call that reads and writes nothing."""
    B, N, V = dims.B, dims.N, dims.V
    R, K = 2 * N - 1, N - 1
    on = 1 if B > 0 else 0
    return {
        "q": B * R * dims.Hq * dims.D,
        "kv": on * dims.num_pages * 2 * dims.Hkv * 16 * dims.D,
        "kv_new": B * R * dims.Hkv * dims.D,
        "page_table": B * dims.max_pages,
        "B": B,
        "clean": B * N * V,
        "mask": B * K * V,
        "drafts": B * K,
        "tokens": B * N,
        "debug": B * (N + 1) * 4,
        "subw": B * ((V + 2047) // 2048),
        "pool": on * dims.num_pages,
        "one": on,
    }


def _fdt(dims_code):
    torch = _torch()
    return (torch.bfloat16,) if dims_code == IDLM_BF16 else (torch.float32,)


def _i32():
    return (_torch().int32,)


def idlm_isd_workspace_bytes(dims):
    return int(load().idlm_isd_workspace_bytes(ctypes.byref(dims)))


def idlm_isd_workspace_state_bytes(dims):
    return int(load().idlm_isd_workspace_state_bytes(ctypes.byref(dims)))


def idlm_isd_validate(dims, T):
    return int(load().idlm_isd_validate(ctypes.byref(dims), float(T)))


def alloc_workspace(dims, device="cuda"):
    """Allocate (256-byte aligned) and initialise a workspace for ``dims``."""
    torch = _torch()
    n = idlm_isd_workspace_bytes(dims)
    if n == 0:
        raise IdlmError(2, "idlm_isd_workspace_bytes")
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    ws = ws[off:off + n]
    idlm_isd_workspace_init(ws)
    return ws


def idlm_isd_workspace_init(ws):
    _check(load().idlm_isd_workspace_init(_ptr(ws, (_torch().uint8,), "workspace"),
                                          ws.numel(), _stream()), "idlm_isd_workspace_init")


def idlm_isd_paged_attn(dims, q, kv_pages, page_table, ctx_lens, attn_out, ws):
    ft = _fdt(dims.qkv_dtype)
    n = _sizes(dims)
    _check(load().idlm_isd_paged_attn(
        ctypes.byref(dims), _ptr(q, ft, "q", numel=n["q"]),
        _ptr(kv_pages, ft, "kv_pages", numel=n["kv"]),
        _ptr(page_table, _i32(), "page_table", numel=n["page_table"]),
        _ptr(ctx_lens, _i32(), "ctx_lens", numel=n["B"]),
        _ptr(attn_out, ft, "attn_out", numel=n["q"]), _ptr(ws, (_torch().uint8,), "workspace"),
        ws.numel(), _stream()), "idlm_isd_paged_attn")


def idlm_isd_mask_stats_bytes(dims):
    return int(load().idlm_isd_mask_stats_bytes(ctypes.byref(dims)))


def alloc_mask_stats(dims, device="cuda"):
    """A (256-byte aligned) MASK-row statistics record for ``dims``."""
    torch = _torch()
    n = idlm_isd_mask_stats_bytes(dims)
    if n == 0:
        raise IdlmError(2, "idlm_isd_mask_stats_bytes")
    m = torch.zeros(n + 256, dtype=torch.uint8, device=device)
    off = (-m.data_ptr()) % 256
    return m[off:off + n]


def _mstats(mask_stats, dims):
    return _ptr(mask_stats, (_torch().uint8,), "mask_stats", allow_none=True,
                numel=idlm_isd_mask_stats_bytes(dims) if mask_stats is not None else None)


def idlm_isd_accept(dims, logits_clean, logits_mask, draft_tokens, seed, T, out_tokens,
                    out_accept_len, out_debug, ws, mask_stats=None):
    ft = _fdt(dims.logits_dtype)
    torch = _torch()
    n = _sizes(dims)
    _check(load().idlm_isd_accept(
        ctypes.byref(dims), _ptr(logits_clean, ft, "logits_clean", numel=n["clean"]),
        _ptr(logits_mask, ft, "logits_mask", allow_none=True, numel=n["mask"]),
        _ptr(draft_tokens, _i32(), "draft_tokens", allow_none=True, numel=n["drafts"]),
        ctypes.c_uint64(int(seed) & ((1 << 64) - 1)), float(T),
        _ptr(out_tokens, _i32(), "out_tokens", numel=n["tokens"]),
        _ptr(out_accept_len, _i32(), "out_accept_len", numel=n["B"]),
        _ptr(out_debug, (torch.float64,), "out_debug", allow_none=True, numel=n["debug"]),
        _mstats(mask_stats, dims),
        _ptr(ws, (torch.uint8,), "workspace"), ws.numel(), _stream()), "idlm_isd_accept")


def idlm_isd_accept_noalloc(dims, logits_clean, logits_mask, draft_tokens, seed, T, out_tokens,
                            out_accept_len, out_debug=None, out_status=None, mask_stats=None):
    ft = _fdt(dims.logits_dtype)
    torch = _torch()
    n = _sizes(dims)
    _check(load().idlm_isd_accept_noalloc(
        ctypes.byref(dims), _ptr(logits_clean, ft, "logits_clean", numel=n["clean"]),
        _ptr(logits_mask, ft, "logits_mask", allow_none=True, numel=n["mask"]),
        _ptr(draft_tokens, _i32(), "draft_tokens", allow_none=True, numel=n["drafts"]),
        ctypes.c_uint64(int(seed) & ((1 << 64) - 1)), float(T),
        _ptr(out_tokens, _i32(), "out_tokens", numel=n["tokens"]),
        _ptr(out_accept_len, _i32(), "out_accept_len", numel=n["B"]),
        _ptr(out_debug, (torch.float64,), "out_debug", allow_none=True, numel=n["debug"]),
        _mstats(mask_stats, dims),
        _ptr(out_status, _i32(), "out_status", allow_none=True, numel=1), _stream()),
        "idlm_isd_accept_noalloc")


def idlm_isd_accept_probs(dims, logits_clean, logits_mask, T, ws, out_p=None, out_q=None,
                          out_subw=None):
    ft = _fdt(dims.logits_dtype)
    torch = _torch()
    n = _sizes(dims)
    f64 = (torch.float64,)
    _check(load().idlm_isd_accept_probs(
        ctypes.byref(dims), _ptr(logits_clean, ft, "logits_clean", numel=n["clean"]),
        _ptr(logits_mask, ft, "logits_mask", allow_none=True, numel=n["mask"]), float(T),
        _ptr(ws, (torch.uint8,), "workspace"), ws.numel(),
        _ptr(out_p, f64, "out_p", allow_none=True, numel=n["clean"]),
        _ptr(out_q, f64, "out_q", allow_none=True, numel=n["mask"]),
        _ptr(out_subw, f64, "out_subw", allow_none=True, numel=n["subw"]), _stream()),
        "idlm_isd_accept_probs")


def idlm_isd_step(dims, q, kv_pages, page_table, ctx_lens, logits_clean, logits_mask,
                  draft_tokens, seed, N, T, out_tokens, out_accept_len, attn_out, ws,
                  mask_stats=None):
    fq = _fdt(dims.qkv_dtype)
    fl = _fdt(dims.logits_dtype)
    torch = _torch()
    n = _sizes(dims)
    _check(load().idlm_isd_step(
        ctypes.byref(dims), _ptr(q, fq, "q", numel=n["q"]),
        _ptr(kv_pages, fq, "kv_pages", numel=n["kv"]),
        _ptr(page_table, _i32(), "page_table", numel=n["page_table"]),
        _ptr(ctx_lens, _i32(), "ctx_lens", numel=n["B"]),
        _ptr(logits_clean, fl, "logits_clean", numel=n["clean"]),
        _ptr(logits_mask, fl, "logits_mask", allow_none=True, numel=n["mask"]),
        _ptr(draft_tokens, _i32(), "draft_tokens", allow_none=True, numel=n["drafts"]),
        ctypes.c_uint64(int(seed) & ((1 << 64) - 1)), int(N), float(T),
        _ptr(out_tokens, _i32(), "out_tokens", numel=n["tokens"]),
        _ptr(out_accept_len, _i32(), "out_accept_len", numel=n["B"]),
        _ptr(attn_out, fq, "attn_out", numel=n["q"]), _mstats(mask_stats, dims),
        _ptr(ws, (torch.uint8,), "workspace"), ws.numel(), _stream()), "idlm_isd_step")


def idlm_isd_loop_step(dims, q, kv_pages, page_table, ctx_lens, logits_clean, logits_mask,
                       draft_tokens, mask_stats, logits_next, seed, N, T, out_tokens,
                       out_accept_len, attn_out, next_drafts, mask_stats_next, ws):
    fq = _fdt(dims.qkv_dtype)
    fl = _fdt(dims.logits_dtype)
    torch = _torch()
    n = _sizes(dims)
    _check(load().idlm_isd_loop_step(
        ctypes.byref(dims), _ptr(q, fq, "q", numel=n["q"]),
        _ptr(kv_pages, fq, "kv_pages", numel=n["kv"]),
        _ptr(page_table, _i32(), "page_table", numel=n["page_table"]),
        _ptr(ctx_lens, _i32(), "ctx_lens", numel=n["B"]),
        _ptr(logits_clean, fl, "logits_clean", numel=n["clean"]),
        _ptr(logits_mask, fl, "logits_mask", allow_none=True, numel=n["mask"]),
        _ptr(draft_tokens, _i32(), "draft_tokens", allow_none=True, numel=n["drafts"]),
        _mstats(mask_stats, dims),
        _ptr(logits_next, fl, "logits_next", allow_none=True, numel=n["mask"]),
        ctypes.c_uint64(int(seed) & ((1 << 64) - 1)), int(N), float(T),
        _ptr(out_tokens, _i32(), "out_tokens", numel=n["tokens"]),
        _ptr(out_accept_len, _i32(), "out_accept_len", numel=n["B"]),
        _ptr(attn_out, fq, "attn_out", numel=n["q"]),
        _ptr(next_drafts, _i32(), "next_drafts", allow_none=True, numel=n["drafts"]),
        _mstats(mask_stats_next, dims),
        _ptr(ws, (torch.uint8,), "workspace"), ws.numel(), _stream()), "idlm_isd_loop_step")


def idlm_isd_propose(dims, logits_next, draft_tokens, accept_len, seed, T, next_drafts, ws,
                     mask_stats=None):
    n = _sizes(dims)
    _check(load().idlm_isd_propose(
        ctypes.byref(dims),
        _ptr(logits_next, _fdt(dims.logits_dtype), "logits_next", numel=n["mask"]),
        _ptr(draft_tokens, _i32(), "draft_tokens", numel=n["drafts"]),
        _ptr(accept_len, _i32(), "accept_len", numel=n["B"] if dims.N > 1 else 0),  # N = 1: no-op
        ctypes.c_uint64(int(seed) & (2**64 - 1)), ctypes.c_float(float(T)),
        _ptr(next_drafts, _i32(), "next_drafts", numel=n["drafts"]),
        _mstats(mask_stats, dims),
        _ptr(ws, (_torch().uint8,), "workspace"),
        ctypes.c_size_t(ws.numel()), _stream()),
        "idlm_isd_propose")


def idlm_isd_lora_workspace_bytes(ldims):
    return int(load().idlm_isd_lora_workspace_bytes(ctypes.byref(ldims)))


def alloc_lora_workspace(ldims, device="cuda"):
    torch = _torch()
    n = idlm_isd_lora_workspace_bytes(ldims)
    if n == 0:
        raise IdlmError(2, "idlm_isd_lora_workspace_bytes")
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + n]


def idlm_isd_gated_lora(ldims, y_base, x, lora_a, lora_b, scale, y_out, ws):
    torch = _torch()
    bf = (torch.bfloat16,)
    M = ldims.B * (2 * ldims.N - 1)
    w = 1 if M > 0 else 0  # B = 0 reads no weights
    _check(load().idlm_isd_gated_lora(
        ctypes.byref(ldims), _ptr(y_base, (torch.float32,), "y_base", numel=M * ldims.O),
        _ptr(x, bf, "x", numel=M * ldims.H),
        _ptr(lora_a, bf, "lora_a", numel=w * ldims.rank * ldims.H),
        _ptr(lora_b, bf, "lora_b", numel=w * ldims.O * ldims.rank), ctypes.c_float(float(scale)),
        _ptr(y_out, bf, "y_out", numel=M * ldims.O), _ptr(ws, (torch.uint8,), "workspace"),
        ctypes.c_size_t(ws.numel()), _stream()),
        "idlm_isd_gated_lora")


def idlm_isd_kv_append(dims, k_new, v_new, ctx_before, ctx_after, kv_pages, page_table,
                       free_pages, free_count, ws):
    dt = _fdt(dims.qkv_dtype)
    n = _sizes(dims)
    _check(load().idlm_isd_kv_append(
        ctypes.byref(dims), _ptr(k_new, dt, "k_new", numel=n["kv_new"]),
        _ptr(v_new, dt, "v_new", numel=n["kv_new"]),
        _ptr(ctx_before, _i32(), "ctx_before", numel=n["B"]),
        _ptr(ctx_after, _i32(), "ctx_after", numel=n["B"]),
        _ptr(kv_pages, dt, "kv_pages", numel=n["kv"]),
        _ptr(page_table, _i32(), "page_table", numel=n["page_table"]),
        _ptr(free_pages, _i32(), "free_pages", numel=n["pool"]),
        _ptr(free_count, _i32(), "free_count", numel=n["one"]),
        _ptr(ws, (_torch().uint8,), "workspace"), ctypes.c_size_t(ws.numel()), _stream()),
        "idlm_isd_kv_append")


def idlm_isd_kv_rollback(dims, ctx_lens, accept_len, ctx_after, page_table, free_pages,
                         free_count, ws):
    n = _sizes(dims)
    _check(load().idlm_isd_kv_rollback(
        ctypes.byref(dims), _ptr(ctx_lens, _i32(), "ctx_lens", numel=n["B"]),
        _ptr(accept_len, _i32(), "accept_len", numel=n["B"]),
        _ptr(ctx_after, _i32(), "ctx_after", numel=n["B"]),
        _ptr(page_table, _i32(), "page_table", numel=n["page_table"]),
        _ptr(free_pages, _i32(), "free_pages", numel=n["pool"]),
        _ptr(free_count, _i32(), "free_count", numel=n["one"]),
        _ptr(ws, (_torch().uint8,), "workspace"),
        ctypes.c_size_t(ws.numel()), _stream()),
        "idlm_isd_kv_rollback")


def idlm_isd_read_status(ws):
    code = ctypes.c_int32(-1)
    _check(load().idlm_isd_read_status(_ptr(ws, (_torch().uint8,), "workspace"), _stream(),
                                       ctypes.byref(code)), "idlm_isd_read_status")
    return int(code.value)


# ---------------------------------------------------------------------------
# Workload upload (storage arrays -> device tensors of the boundary formats)
# ---------------------------------------------------------------------------
def _to_dev(a, dtype, device):
    torch = _torch()
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


class DeviceStep:
    """Device tensors and workspace for one workload, plus the step's calls."""

    def __init__(self, w, device="cuda"):
        torch = _torch()
        self.w = w
        self.dims = make_dims(w.B, w.N, w.Hq, w.Hkv, w.D, w.V, w.max_pages, max(1, w.num_pages),
                              w.qkv_dtype, w.logits_dtype)
        self.q = _to_dev(w.q, w.qkv_dtype, device)
        self.kv = _to_dev(w.kv_pages, w.qkv_dtype, device)
        self.page_table = torch.from_numpy(np.ascontiguousarray(w.page_table)).to(device)
        self.ctx_lens = torch.from_numpy(np.ascontiguousarray(w.ctx_lens)).to(device)
        self.lc = _to_dev(w.logits_clean, w.logits_dtype, device)
        self.lm = _to_dev(w.logits_mask, w.logits_dtype, device) if w.N > 1 else None
        self.drafts = torch.from_numpy(np.ascontiguousarray(w.draft_tokens)).to(device) \
            if w.N > 1 else None
        qdt = torch.bfloat16 if w.qkv_dtype == "bf16" else torch.float32
        self.out = torch.zeros(self.q.shape, dtype=qdt, device=device)
        self.tokens = torch.full((w.B, w.N), -7, dtype=torch.int32, device=device)
        self.lens = torch.zeros(w.B, dtype=torch.int32, device=device)
        self.debug = torch.zeros((w.B, w.N + 1, 4), dtype=torch.float64, device=device)
        self.ws = alloc_workspace(self.dims, device)

    def attn(self):
        idlm_isd_paged_attn(self.dims, self.q, self.kv, self.page_table, self.ctx_lens, self.out,
                            self.ws)

    def accept(self, seed=None, T=None, debug=True, drafts=None, mask_stats=None):
        idlm_isd_accept(self.dims, self.lc, self.lm, self.drafts if drafts is None else drafts,
                        self.w.seed if seed is None else seed, self.w.T if T is None else T,
                        self.tokens, self.lens, self.debug if debug else None, self.ws,
                        mask_stats=mask_stats)

    def probs(self, T=None):
        """(p [B][N][V], q [B][K][V], sub-chunk weights [B][ceil(V/2048)]) as
        float64 tensors, dumped from the last accept or step call."""
        torch = _torch()
        w = self.w
        dev = self.lc.device
        p = torch.empty((w.B, w.N, w.V), dtype=torch.float64, device=dev)
        q = torch.empty((w.B, max(w.N - 1, 0), w.V), dtype=torch.float64, device=dev)
        sw = torch.empty((w.B, (w.V + 2047) // 2048), dtype=torch.float64, device=dev)
        idlm_isd_accept_probs(self.dims, self.lc, self.lm, self.w.T if T is None else T, self.ws,
                              p, q if w.N > 1 else None, sw)
        return p, q, sw

    def step(self, seed=None, T=None, drafts=None, mask_stats=None):
        idlm_isd_step(self.dims, self.q, self.kv, self.page_table, self.ctx_lens, self.lc, self.lm,
                      self.drafts if drafts is None else drafts,
                      self.w.seed if seed is None else seed, self.w.N,
                      self.w.T if T is None else T, self.tokens, self.lens, self.out, self.ws,
                      mask_stats=mask_stats)

    def out_f64(self):
        return self.out.to(_torch().float64).cpu().numpy()
