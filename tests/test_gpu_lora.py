"""GPU parity of idlm_isd_gated_lora against oracle.lora: verify rows
bit-identical to the base-only output (and to the oracle); MASK rows within
one bfloat16 ulp of the float64 oracle plus the float32 accumulation bound
(which matters only near zero, where terms cancel), and almost all exact."""

import numpy as np
import pytest

from oracle.dtypes import bf16_bits_to_f64
from oracle.lora import f64_to_bf16_rne, gated_lora
from speculative_verify_isd_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available()
    return torch


def _bf(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).cuda()


def _bits(t):
    import torch

    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("B,N,H,O,rank", [
    (4, 4, 256, 200, 32), (64, 4, 4096, 512, 128), (3, 8, 512, 64, 16), (5, 1, 128, 96, 16),
    (2, 2, 1024, 1000, 256), (3, 16, 512, 256, 64),
])
def test_gated_lora_matches_oracle(torch_cuda, B, N, H, O, rank):
    torch = torch_cuda
    from speculative_verify_isd_amd import lib as L

    rng = np.random.default_rng(B * 7 + N + rank)
    M = B * (2 * N - 1)
    x = W.f32_to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    a = W.f32_to_bf16_bits((rng.standard_normal((rank, H)) / np.sqrt(H)).astype(np.float32))
    b = W.f32_to_bf16_bits((0.05 * rng.standard_normal((O, rank))).astype(np.float32))
    y = rng.standard_normal((M, O)).astype(np.float32)
    ld = L.LoraDims(B, N, H, O, rank)
    ws = L.alloc_lora_workspace(ld)
    d_y = torch.from_numpy(y).cuda()
    d_x, d_a, d_b = _bf(torch, x), _bf(torch, a), _bf(torch, b)
    out = torch.empty((M, O), dtype=torch.bfloat16, device="cuda")
    base = torch.empty_like(out)
    L.idlm_isd_gated_lora(ld, d_y, d_x, d_a, d_b, 2.0, out, ws)
    L.idlm_isd_gated_lora(ld, d_y, d_x, d_a, d_b, 0.0, base, ws)
    torch.cuda.synchronize()
    got, got0 = _bits(out), _bits(base)
    want = gated_lora(y, x, a, b, 2.0, N)
    verify = (np.arange(M) % (2 * N - 1)) < N
    base_rne = f64_to_bf16_rne(y.astype(np.float64))
    # verify rows: the base-only output, bit for bit
    assert np.array_equal(got[verify], base_rne[verify])
    assert np.array_equal(got[verify], got0[verify])
    assert np.array_equal(got0, base_rne)
    # MASK rows: float32 accumulation vs the float64 oracle, within one ulp
    if (~verify).any():
        g = bf16_bits_to_f64(got[~verify])
        w = bf16_bits_to_f64(want[~verify])
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(w), 1e-30))) - 7)
        # float32 accumulation of H + rank products: first-order bound
        # (H/32 MFMA steps + splits + rank terms) * 2^-24 * sum of |terms|,
        # taken generously as 2^-16 * sum of |terms|
        xm = np.abs(bf16_bits_to_f64(x[~verify]))
        mag = np.abs(y[~verify]) + 2.0 * (xm @ np.abs(bf16_bits_to_f64(a)).T) @ np.abs(
            bf16_bits_to_f64(b)).T
        over = np.abs(g - w) > ulp * 1.0001 + 2.0 ** -16 * mag
        if over.any():
            idx = np.argwhere(over)[:8]
            print("[lora] >1 ulp:", int(over.sum()), "of", over.size,
                  [(int(i), int(j), float(w[i, j]), float(g[i, j])) for i, j in idx], flush=True)
        assert not over.any()
        exact = float((got[~verify] == want[~verify]).mean())
        changed = float((got[~verify] != base_rne[~verify]).mean())
        print(f"[lora] B={B} N={N} H={H} O={O} rank={rank}: verify rows bit-exact, MASK rows "
              f"{exact:.4%} exact (rest within the bound), adapter changed {changed:.1%}", flush=True)
        assert exact > 0.98
    else:
        print(f"[lora] N=1: no MASK rows, output is the base rounding", flush=True)


def test_gated_lora_nan_and_inf_in_base(torch_cuda):
    """NaN (quiet, signalling, payload only in the low 16 bits, all ones) and
    +-Inf in y_base: verify rows round them as the oracle does (NaN keeps
    its sign as a quiet bf16 NaN, never collapsing to Inf or 0), MASK rows
    stay NaN / the same infinity after the adapter's finite addition."""
    torch = torch_cuda
    from speculative_verify_isd_amd import lib as L

    B, N, H, O, rank = 4, 4, 256, 200, 32
    M = B * (2 * N - 1)
    rng = np.random.default_rng(17)
    x = W.f32_to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    a = W.f32_to_bf16_bits((rng.standard_normal((rank, H)) / np.sqrt(H)).astype(np.float32))
    b = W.f32_to_bf16_bits((0.05 * rng.standard_normal((O, rank))).astype(np.float32))
    y = rng.standard_normal((M, O)).astype(np.float32)
    yb = y.view(np.uint32)
    specials = np.array([0x7FC00000, 0x7F800001, 0xFFFFFFFF, 0x7FFFFFFF, 0xFF800123,
                         0x7F800000, 0xFF800000], dtype=np.uint32)
    cells = rng.choice(M * O, size=7 * 12, replace=False)
    for n, c in enumerate(cells):
        yb.reshape(-1)[c] = specials[n % len(specials)]
    ld = L.LoraDims(B, N, H, O, rank)
    ws = L.alloc_lora_workspace(ld)
    out = torch.empty((M, O), dtype=torch.bfloat16, device="cuda")
    L.idlm_isd_gated_lora(ld, torch.from_numpy(y).cuda(), _bf(torch, x), _bf(torch, a),
                          _bf(torch, b), 2.0, out, ws)
    torch.cuda.synchronize()
    got = _bits(out)
    want = gated_lora(y, x, a, b, 2.0, N)
    verify = (np.arange(M) % (2 * N - 1)) < N
    assert np.array_equal(got[verify], want[verify])
    g = bf16_bits_to_f64(got)
    w = bf16_bits_to_f64(want)
    assert np.array_equal(np.isnan(g), np.isnan(w))
    inf = np.isinf(w)
    assert inf.sum() > 0 and np.array_equal(g[inf], w[inf])
    nan_cells = np.isnan(y)
    assert np.isnan(g[nan_cells]).all()  # every NaN input stays NaN
    # NaN outputs are the quiet pattern with the input's sign: 0x7FC0 / 0xFFC0
    assert set(np.unique(got[np.isnan(g)]).tolist()) <= {0x7FC0, 0xFFC0}
