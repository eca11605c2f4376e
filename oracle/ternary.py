"""Ternary W2A8 linear of the paper's §III-D (Eq. 4) -- test infrastructure only.

Eq. 4, restated: every activation row x_m gets a scale
alpha_m = max(||x_m||_inf, 1e-5) / 127; its int8 codes are
a_mj = clip(round(x_mj / alpha_m), -128, 127) with ties rounded to even; the
output is y_mn = alpha_m * beta * sum_j a_mj q_nj with q in {-1, 0, +1}, the sum
kept in 32-bit integers and the scaled result rounded to bfloat16 (nearest,
ties to even).

Readings where the page leaves a step open:
  * the quantizer runs in float32 with IEEE division, x / alpha (not
    x * (1 / alpha)), and alpha = max(absmax, 1e-5) / 127 is itself an IEEE
    float32 division;
  * the scale is applied as bf16(float(acc) * (alpha_m * beta)), each product
    rounded to float32; float(acc) is exact because |acc| < 2^24 here;
  * beta is one scale per weight tensor (one output group), the per-tensor form,
    in the model; w2a8_linear_grouped takes the page's group-wise beta_g(n),
    output channel n in group n // group_size;
  * packing: code = q + 1 in {0, 1, 2} (3 is invalid), four codes per byte,
    element 4j + i of a row in bits 2i..2i+1 of byte j (least significant
    first); rows are [out, in], in a multiple of 4.
"""
from __future__ import annotations

import numpy as np

_F32 = np.float32


def bf16_round(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); float32 result.

    The bfloat16 format keeps the top 16 bits of a float32.  Rounding to nearest
    with ties to even adds 0x7FFF plus the lowest kept bit before truncating.
    NaNs stay NaN.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=_F32))
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    out = rounded.view(_F32).copy()
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.nan
    return out.reshape(x.shape)


def quantize_rows(x):
    """Per-row absmax int8 quantization of Eq. 4 (float32 arithmetic).

    x: [M, K] (converted to float32).  Returns (a int8 [M, K], alpha float32 [M]).
    """
    x = np.asarray(x, dtype=_F32)
    absmax = np.max(np.abs(x), axis=-1)
    alpha = (np.maximum(absmax, _F32(1e-5)) / _F32(127.0)).astype(_F32)
    scaled = (x / alpha[..., None]).astype(_F32)          # IEEE float32 division
    a = np.clip(np.rint(scaled), -128, 127).astype(np.int8)  # rint: ties to even
    return a, alpha


def w2a8_accumulate(a, q) -> np.ndarray:
    """acc[m, n] = sum_j a[m, j] * q[n, j] in exact integer arithmetic (int32 result).

    Computed with a float32 BLAS product when every partial sum is an integer of
    magnitude below 2^24 (then each float32 operation is exact whatever the
    summation order), else with float64 (exact below 2^53).
    """
    a = np.asarray(a)
    q = np.asarray(q)
    K = a.shape[-1]
    bound = 128 * int(np.max(np.abs(q))) * K if q.size else 0
    if bound < (1 << 24):
        acc = a.astype(_F32) @ q.astype(_F32).T
    else:
        assert bound < (1 << 53)
        acc = a.astype(np.float64) @ q.astype(np.float64).T
    return acc.astype(np.int64).astype(np.int32)


def w2a8_linear(x, q, beta) -> np.ndarray:
    """y = bf16(alpha_m * beta * sum_j a_mj q_nj) for x [M, K], q [N, K]; float32 result."""
    a, alpha = quantize_rows(x)
    acc = w2a8_accumulate(a, q)
    scale = (alpha * _F32(beta)).astype(_F32)
    y = (acc.astype(_F32) * scale[:, None]).astype(_F32)
    return bf16_round(y)


def w2a8_linear_grouped(x, q, betas, group_size: int) -> np.ndarray:
    """Eq. 4 with group-wise weight scales: y_mn = bf16(float(acc_mn) * (alpha_m * beta_g(n)))
    with g(n) = n // group_size, betas [N / group_size]; float32 products, as w2a8_linear."""
    a, alpha = quantize_rows(x)
    acc = w2a8_accumulate(a, q)
    n = np.arange(np.shape(q)[0])
    beta_n = np.asarray(betas, dtype=_F32)[n // group_size]
    scale = (alpha[:, None] * beta_n[None, :]).astype(_F32)
    return bf16_round((acc.astype(_F32) * scale).astype(_F32))


def pack_ternary(q) -> np.ndarray:
    """[N, K] codes in {-1, 0, 1} -> [N, K/4] uint8, four 2-bit codes per byte."""
    q = np.asarray(q)
    if q.ndim != 2 or q.shape[1] % 4:
        raise ValueError("ternary rows must be [out, in] with in % 4 == 0")
    if q.size and (q.min() < -1 or q.max() > 1):
        raise ValueError("ternary values must be -1, 0 or +1")
    codes = (q.astype(np.int16) + 1).astype(np.uint8).reshape(q.shape[0], -1, 4)
    packed = np.zeros(codes.shape[:2], dtype=np.uint8)
    for i in range(4):
        packed |= (codes[:, :, i] << (2 * i)).astype(np.uint8)
    return packed


def unpack_ternary(packed) -> np.ndarray:
    """Inverse of pack_ternary; raises ValueError on the invalid code 3."""
    packed = np.asarray(packed, dtype=np.uint8)
    codes = np.stack([(packed >> (2 * i)) & 3 for i in range(4)], axis=-1)
    if np.any(codes == 3):
        raise ValueError("invalid ternary code 3")
    return (codes.astype(np.int8) - 1).reshape(packed.shape[0], -1)
