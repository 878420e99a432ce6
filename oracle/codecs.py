"""Closed KV profiles: quantize and dequantize (oracle side, NumPy).

The pages fix the profiles and their plane inventory ("Paged KV Context Store"
page: closed-profile paragraph, X-extent list) but defer the exact codec to a
header they do not contain.  The reading implemented here:

* all codec arithmetic is IEEE fp32, correctly rounded (NumPy float32);
* BF16: the input bits are stored unchanged (no FP16 conversion on write);
* INT8-G64: per 64 contiguous head_dim elements a = max|x|, s = a/127,
  q = clamp(round_half_even(x/s), -127, 127); s == 0 gives codes 0;
* FP8-E4M3FN-row256: one scale per row (X = 1), s = a/448,
  code = E4M3FN(x/s) rounded half-to-even with saturation to +-448;
* NVFP4-G16: per 16 elements the E4M3 scale is S = E4M3FN(a/6), and each
  element is E2M1(x/value(S)) rounded half-to-even, saturating at +-6;
  element 2k is the low nibble of byte k; value(S) == 0 gives codes 0;
* FP8/FP4 codes keep the sign of the quotient (so -0 encodes as the sign bit);
* dequantization is one fp32 multiply: value(code) * scale;
* 2-byte scale planes (the D256 payload table's sizes): the INT8-G64 and
  FP8-row scale is stored as IEEE binary16, s16 = f16(a/127) (or a/448),
  the fp32 quotient rounded half-to-even to binary16 and saturated at the
  largest finite binary16 (65504); the codes are taken against the stored
  scale (x / float(s16)), so a code times its stored scale is the value the
  consumer reconstructs; s16 == 0 gives codes 0.

The two minifloat formats are taken from their published definitions (OCP
8-bit floating point spec for E4M3FN: bias 7, no infinities, 0x7F/0xFF NaN,
max 448; OCP MX spec for E2M1: values {0, .5, 1, 1.5, 2, 3, 4, 6}).  Encoding
here is a nearest-value search over the enumerated grid, ties to the even code.
"""

from __future__ import annotations

import numpy as np

F32 = np.float32


# ---------------------------------------------------------------- bf16 ------
def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 values (exact)."""
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ------------------------------------------------------------ minifloats ----
def _e4m3fn_grid() -> np.ndarray:
    """Value of each non-negative E4M3FN code 0x00..0x7E (0x7F is NaN)."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        if e == 0:
            vals.append(m * 2.0 ** -9)             # subnormal: m/8 * 2^(1-7)
        else:
            vals.append((1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


E4M3FN_GRID = _e4m3fn_grid()
E4M3FN_MAX = float(E4M3FN_GRID[-1])               # 448
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def _nearest_even(a: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the grid value nearest to a (a >= 0, a <= grid[-1]); ties -> even index."""
    k = np.searchsorted(grid, a, side="left")
    k = np.clip(k, 1, len(grid) - 1)
    lo, hi = grid[k - 1], grid[k]
    d_lo, d_hi = a - lo, hi - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (k % 2 == 0))
    return np.where(take_hi, k, k - 1)


def encode_e4m3fn(y) -> np.ndarray:
    """fp32 -> E4M3FN code (uint8), round half to even, saturate to +-448."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)
    sat = a >= E4M3FN_MAX
    idx = _nearest_even(np.minimum(a, E4M3FN_MAX), E4M3FN_GRID)
    idx = np.where(sat, 0x7E, idx).astype(np.uint8)
    sign = np.where(np.signbit(y), 0x80, 0).astype(np.uint8)
    return idx | sign


def decode_e4m3fn(code) -> np.ndarray:
    """E4M3FN code -> float32 value (NaN code decodes to NaN)."""
    code = np.asarray(code, dtype=np.uint8)
    mag = code & 0x7F
    val = np.where(mag == 0x7F, np.nan, E4M3FN_GRID[np.minimum(mag, 0x7E)])
    return np.where(code & 0x80, -val, val).astype(np.float32)


def encode_e2m1(y) -> np.ndarray:
    """fp32 -> E2M1 nibble (uint8, sign in bit 3), round half to even, saturate at +-6."""
    y = np.asarray(y, dtype=np.float32)
    a = np.minimum(np.abs(y).astype(np.float64), 6.0)
    idx = _nearest_even(a, E2M1_GRID).astype(np.uint8)
    sign = np.where(np.signbit(y), 8, 0).astype(np.uint8)
    return idx | sign


def decode_e2m1(nib) -> np.ndarray:
    nib = np.asarray(nib, dtype=np.uint8)
    val = E2M1_GRID[nib & 7]
    return np.where(nib & 8, -val, val).astype(np.float32)


# -------------------------------------------------------------- profiles ----
def _absmax(xg: np.ndarray) -> np.ndarray:
    return np.max(np.abs(xg), axis=-1)


F16_MAX = F32(65504.0)


def to_f16_bits(s32: np.ndarray) -> np.ndarray:
    """fp32 scales -> binary16 bits (uint16), round half to even, saturated at 65504."""
    return np.minimum(np.asarray(s32, dtype=np.float32), F16_MAX).astype(np.float16).view(np.uint16)


def scale_values(scales: np.ndarray) -> np.ndarray:
    """A scale plane's data as float32: fp32 as is, binary16 bits (uint16) widened exactly."""
    scales = np.asarray(scales)
    if scales.dtype == np.uint16:
        return scales.view(np.float16).astype(np.float32)
    return scales.astype(np.float32)


def quant_int8_g64(x: np.ndarray, scale_bytes: int = 4):
    """x float32 [..., D] -> (codes int8 [..., D], scales [..., D/64]: float32, or
    binary16 bits (uint16) when scale_bytes == 2)."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    xg = x.reshape(x.shape[:-1] + (D // 64, 64))
    s = (_absmax(xg) / F32(127)).astype(np.float32)
    stored = s if scale_bytes == 4 else to_f16_bits(s)
    sv = scale_values(stored)
    with np.errstate(divide="ignore", invalid="ignore"):
        qf = np.rint((xg / sv[..., None]).astype(np.float32))
    q = np.where(sv[..., None] == 0, 0, np.clip(qf, -127, 127)).astype(np.int8)
    return q.reshape(x.shape), stored


def dequant_int8_g64(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    D = codes.shape[-1]
    qg = codes.astype(np.float32).reshape(codes.shape[:-1] + (D // 64, 64))
    return (qg * scale_values(scales)[..., None]).astype(np.float32).reshape(codes.shape)


def quant_fp8_row(x: np.ndarray, scale_bytes: int = 4):
    """x float32 [..., D] -> (codes uint8 E4M3FN [..., D], scales [..., 1]: float32,
    or binary16 bits (uint16) when scale_bytes == 2)."""
    x = np.asarray(x, dtype=np.float32)
    s = (_absmax(x) / F32(E4M3FN_MAX)).astype(np.float32)[..., None]
    stored = s if scale_bytes == 4 else to_f16_bits(s)
    sv = scale_values(stored)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = (x / sv).astype(np.float32)
    codes = np.where(sv == 0, np.uint8(0), encode_e4m3fn(np.where(sv == 0, F32(0), y)))
    return codes.astype(np.uint8), stored


def dequant_fp8_row(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    return (decode_e4m3fn(codes) * scale_values(scales)).astype(np.float32)


def quant_nvfp4_g16(x: np.ndarray):
    """x float32 [..., D] -> (packed uint8 [..., D/2], E4M3 scales uint8 [..., D/16])."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    xg = x.reshape(x.shape[:-1] + (D // 16, 16))
    s_code = encode_e4m3fn((_absmax(xg) / F32(6)).astype(np.float32))
    vs = decode_e4m3fn(s_code)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        y = (xg / vs).astype(np.float32)
    nib = np.where(vs == 0, np.uint8(0), encode_e2m1(np.where(vs == 0, F32(0), y))).astype(np.uint8)
    nib = nib.reshape(x.shape)
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return packed, s_code


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out


def dequant_nvfp4_g16(packed: np.ndarray, s_code: np.ndarray) -> np.ndarray:
    vals = decode_e2m1(unpack_nibbles(packed))
    D = vals.shape[-1]
    vg = vals.reshape(vals.shape[:-1] + (D // 16, 16))
    return (vg * decode_e4m3fn(s_code)[..., None]).astype(np.float32).reshape(vals.shape)


def quantize(kind: str, x_bf16: np.ndarray, scale_bytes: int = 4) -> tuple[np.ndarray, np.ndarray | None]:
    """Quantize bf16 rows [..., D] for one side; returns (code plane data, scale data).
    scale_bytes (4 or 2) applies to the INT8-G64 and FP8-row scales."""
    if kind == "bf16":
        return np.asarray(x_bf16, dtype=np.uint16).copy(), None
    x = bf16_to_f32(x_bf16)
    if kind == "int8_g64":
        return quant_int8_g64(x, scale_bytes)
    if kind == "fp8_row":
        return quant_fp8_row(x, scale_bytes)
    if kind == "nvfp4_g16":
        return quant_nvfp4_g16(x)
    raise ValueError(kind)


def dequantize(kind: str, code: np.ndarray, scale: np.ndarray | None) -> np.ndarray:
    """Code/scale plane data -> float32 values [..., D]."""
    if kind == "bf16":
        return bf16_to_f32(code)
    if kind == "int8_g64":
        return dequant_int8_g64(code, scale)
    if kind == "fp8_row":
        return dequant_fp8_row(code, scale)
    if kind == "nvfp4_g16":
        return dequant_nvfp4_g16(code, scale)
    raise ValueError(kind)
