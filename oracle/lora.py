"""R-ISD's gated LoRA at MASK rows, applied after the base projection.
Test infrastructure.

What the pages fix
------------------
* Residual ISD adds a gated LoRA adapter of rank 128 that is active only at
  MASK positions; verify positions use the base weights alone, which is what
  makes the output bit-for-bit that of the base autoregressive model
  ("Introspective Diffusion Language Models", section "Lossless R-ISD";
  GeekNews summary, section "Inference & ISD").

Readings taken where the pages are silent
-----------------------------------------
* Rows follow the step's order: in each sequence's block of R = 2N-1 rows the
  first N are clean (verify) rows and the last N-1 are MASK rows.
* The adapter's update of a MASK row is scale * (x A^T) B^T with A [rank][H]
  and B [O][rank], added to the base projection's float32 accumulator before
  its single rounding to bfloat16 (no intermediate rounding of x A^T).
* Verify rows are the base accumulator rounded to bfloat16, nothing else.
* Rounding is to nearest, ties to even.

Pinned in tests/test_oracle_lora.py: the rounding against an exhaustive
nearest-value search over bfloat16, verify rows independent of the adapter,
a rank-one closed form, a zero adapter giving the base output.
"""

import numpy as np

from .dtypes import bf16_bits_to_f64


def f64_to_bf16_rne(v):
    """Round float64 values to bfloat16 bit patterns, nearest even.

    Goes through float32 first only where that is exact for the purpose:
    the inputs here are float32 accumulators (exact in float64) or
    float64 sums, so the value is rounded directly from its float64 bits:
    a bfloat16 keeps 8 significant bits, so the float64 mantissa is rounded
    at bit 45 (52 - 7), ties to even, then repacked into 16 bits.
    """
    x = np.asarray(v, dtype=np.float64)
    u = x.view(np.uint64)
    sign = (u >> np.uint64(63)).astype(np.uint16)
    exp = ((u >> np.uint64(52)) & np.uint64(0x7FF)).astype(np.int64)
    man = u & np.uint64((1 << 52) - 1)
    out = np.zeros(x.shape, dtype=np.uint16)
    for idx in np.ndindex(x.shape):
        e, m, s = int(exp[idx]), int(man[idx]), int(sign[idx])
        if e == 0x7FF:  # inf / nan
            out[idx] = (s << 15) | 0x7F80 | (0x40 if m else 0)
            continue
        if e == 0 and m == 0:
            out[idx] = s << 15
            continue
        # value = (1.m) * 2^(e-1023) for normals (float64 subnormals are far
        # below bfloat16's range and round to zero)
        if e == 0:
            out[idx] = s << 15
            continue
        E = e - 1023 + 127  # bfloat16 (float32) biased exponent
        full = (1 << 52) | m  # 53-bit significand
        if E >= 1:
            keep, shift = 8, 45  # 1 + 7 stored bits
        else:  # bfloat16 subnormal: fewer significant bits
            shift = 45 + (1 - E)
            E = 0
        if shift >= 60:
            out[idx] = s << 15
            continue
        q, rem = full >> shift, full & ((1 << shift) - 1)
        half = 1 << (shift - 1)
        if rem > half or (rem == half and (q & 1)):
            q += 1
        if E == 0:
            # subnormal: q is the stored mantissa (may carry into the exponent)
            bits = q
        else:
            if q >> 8:  # carry out of the significand
                q >>= 1
                E += 1
            bits = (E << 7) | (q & 0x7F)
        if (bits >> 7) >= 0xFF:
            bits = 0x7F80  # overflow to infinity
        out[idx] = (s << 15) | bits
    return out


def gated_lora(y_base, x, lora_a, lora_b, scale, N):
    """bfloat16 bit patterns [M][O] of the gated projection.

    y_base  float32 [M][O]: the base projection's accumulator
    x       bfloat16 bits [M][H]; lora_a bf16 bits [rank][H]; lora_b bf16 bits [O][rank]
    Rows are sequences' blocks of R = 2N-1; row r of a block is a MASK row iff r >= N.
    """
    M, O = y_base.shape
    R = 2 * N - 1
    assert M % R == 0
    y = np.asarray(y_base, dtype=np.float32).astype(np.float64)
    mask = (np.arange(M) % R) >= N
    if mask.any():
        xa = bf16_bits_to_f64(x[mask]) @ bf16_bits_to_f64(lora_a).T  # [Mm][rank]
        delta = xa @ bf16_bits_to_f64(lora_b).T  # [Mm][O]
        y[mask] = y[mask] + float(scale) * delta
    return f64_to_bf16_rne(y)
