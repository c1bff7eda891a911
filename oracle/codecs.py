"""Oracle codecs: exact decoding of the stored weight formats to float64.

Test infrastructure only (see oracle/__init__.py).

* bf16: the upper 16 bits of an IEEE binary32.
* Q8_0 (graysoft.dev "Lucebox Kimi-K3-DSpark Q8_0 GGUF", "Conversion result":
  output format MOSTLY_Q8_0): blocks of 32 consecutive weights along a row,
  each stored as an fp16 scale d followed by 32 signed bytes q; weight = d * q.
  34 bytes per 32 weights; the printed file size pins this (tests).
* FP8 E4M3FN, per output channel (huggingface.co "Kimi-K3-DSpark-NVFP4",
  "Limitations": the per-channel weight-only FP8 path): OCP 8-bit E4M3 with
  bias 7, no infinities, 0x7F/0xFF = NaN, largest finite 448; weight = s_n * v.
* MXFP4 (huggingface.co "Kimi-K3-DSpark-NVFP4", "Drift-limited acceptance
  ceiling" and "Detail": the 4-bit MX variant measured beside NVFP4), as the
  OCP Microscaling (MX) format defines it: blocks of 32 consecutive weights
  along a row share one E8M0 scale X = 2^(e - 127) (code 255 = NaN); each
  weight is an FP4 E2M1 element (sign, 2 exponent bits with bias 1, 1 mantissa
  bit: +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}); weight = X * element.  The pages fix
  no byte layout; the stored one here is 17 bytes per block: the scale code,
  then 16 bytes with element 2i in the low nibble of byte i and element
  2i + 1 in the high nibble.

Encoders are here only so that tests can state round-trip properties; the
draft pass itself only ever decodes.
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------- bf16 ----
def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_encode(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest, ties to even (finite inputs).

    Written as: take the two neighbouring bf16 values (truncated and one ulp up)
    and keep the closer one; on a tie keep the one with an even last bit.
    """
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    u = x32.view(np.uint32)
    lo = (u >> np.uint32(16)).astype(np.uint32)
    rem = u & np.uint32(0xFFFF)
    half = np.uint32(0x8000)
    up = (rem > half) | ((rem == half) & ((lo & np.uint32(1)) == 1))
    return (lo + up.astype(np.uint32)).astype(np.uint16)


# ---------------------------------------------------------------- Q8_0 ----
Q8_BLOCK = 32
Q8_BYTES = 34


def q8_0_decode(blocks: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """[rows, cols/32*34] uint8 -> float64 [rows, cols]; weight = fp16(d) * q."""
    nb = cols // Q8_BLOCK
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(rows, nb, Q8_BYTES)
    d = b[:, :, 0:2].copy().view(np.float16).astype(np.float64)  # [rows, nb, 1]
    q = b[:, :, 2:].copy().view(np.int8).astype(np.float64)      # [rows, nb, 32]
    return (d * q).reshape(rows, cols)


def q8_0_encode(w: np.ndarray) -> np.ndarray:
    """float32 [rows, K] -> 34-byte blocks.

    Per block: amax = max |x| (fp32); d = amax / 127 in fp32; q = x / d in fp32,
    rounded half away from zero and clamped to [-127, 127]; the stored scale is
    d rounded to fp16 (nearest even).  An all-zero block stores d = 0, q = 0.
    """
    x = np.ascontiguousarray(w, dtype=np.float32)
    rows, K = x.shape
    nb = K // Q8_BLOCK
    xb = x.reshape(rows, nb, Q8_BLOCK)
    amax = np.max(np.abs(xb), axis=2, keepdims=True)
    d = (amax / np.float32(127)).astype(np.float32)
    safe = np.where(d == 0, np.float32(1), d)
    r = (xb / safe).astype(np.float32)
    q = np.trunc(r + np.copysign(np.float32(0.5), r))
    q = np.where(d == 0, 0, np.clip(q, -127, 127)).astype(np.int8)
    out = np.empty((rows, nb, Q8_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = d.astype(np.float16).view(np.uint8)
    out[:, :, 2:] = q.view(np.uint8)
    return out.reshape(rows, nb * Q8_BYTES)


# ---------------------------------------------------------- FP8 E4M3FN ----
def e4m3fn_value(code: int) -> float:
    """One OCP E4M3FN code -> its real value (NaN for 0x7F / 0xFF)."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** (1 - 7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def fp8_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """uint8 codes [rows, K] and fp32 per-row scales -> float64 [rows, K]."""
    v = _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]
    return v * np.asarray(scales, dtype=np.float32).astype(np.float64)[:, None]


def e4m3fn_encode(x: np.ndarray) -> np.ndarray:
    """float -> E4M3FN code: nearest finite value, ties to the even code,
    saturating at +-448 (inputs beyond 448 in magnitude map to +-448)."""
    x = np.asarray(x, dtype=np.float64)
    pos_codes = np.arange(0, 0x7F)                   # 0 .. 448, increasing
    pos_vals = _E4M3_TABLE[pos_codes]
    a = np.minimum(np.abs(x), 448.0)
    i = np.searchsorted(pos_vals, a, side="left")     # pos_vals[i-1] < a <= pos_vals[i]
    i = np.clip(i, 1, len(pos_vals) - 1)
    lo_v, hi_v = pos_vals[i - 1], pos_vals[i]
    pick_hi = (hi_v - a < a - lo_v) | ((hi_v - a == a - lo_v) & (pos_codes[i] % 2 == 0))
    c = np.where(pick_hi, pos_codes[i], pos_codes[i - 1])
    c = np.where(a == 0, 0, c)
    return (c | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


# --------------------------------------------------------------- MXFP4 ----
MX_BLOCK = 32
MX_BYTES = 17


def e2m1_value(code: int) -> float:
    """One FP4 E2M1 code (4 bits) -> its real value."""
    s = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return s * (m / 2.0)                      # subnormal: m * 2^(1 - bias) / 2
    return s * (1.0 + m / 2.0) * 2.0 ** (e - 1)


def e8m0_value(code: int) -> float:
    """One E8M0 scale code -> 2^(code - 127); 255 is NaN."""
    return float("nan") if code == 255 else 2.0 ** (int(code) - 127)


_E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
_E8M0_TABLE = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)


def mxfp4_decode(blocks: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """[rows, cols/32*17] uint8 -> float64 [rows, cols]; weight = X * element."""
    nb = cols // MX_BLOCK
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(rows, nb, MX_BYTES)
    x = _E8M0_TABLE[b[:, :, 0]][..., None]             # [rows, nb, 1]
    packed = b[:, :, 1:]
    codes = np.empty((rows, nb, MX_BLOCK), dtype=np.uint8)
    codes[:, :, 0::2] = packed & 0x0F
    codes[:, :, 1::2] = packed >> 4
    return (x * _E2M1_TABLE[codes]).reshape(rows, cols)


def e2m1_encode(r: np.ndarray) -> np.ndarray:
    """float -> E2M1 code: nearest element, ties to the even code (mantissa
    bit 0), magnitudes above 6 saturate to +-6."""
    r = np.asarray(r, dtype=np.float64)
    pos = _E2M1_TABLE[:8]                                # 0 .. 6, increasing
    a = np.minimum(np.abs(r), 6.0)
    i = np.clip(np.searchsorted(pos, a, side="left"), 1, 7)
    lo_v, hi_v = pos[i - 1], pos[i]
    pick_hi = (hi_v - a < a - lo_v) | ((hi_v - a == a - lo_v) & (i % 2 == 0))
    c = np.where(pick_hi, i, i - 1)
    c = np.where(a == 0, 0, c)
    return (c | np.where(np.signbit(r) & (c != 0), 0x8, 0)).astype(np.uint8)


def mxfp4_encode(w: np.ndarray) -> np.ndarray:
    """float32 [rows, K] -> 17-byte blocks, by the MX conversion rule: the
    shared exponent is floor(log2(amax)) - 2 (2 = exponent of the largest
    power of two in E2M1), clamped to the E8M0 range [-127, 127]; elements are
    x / X rounded to E2M1 (nearest, ties to even, saturating).  An all-zero
    block stores exponent -127 and zero elements."""
    x = np.ascontiguousarray(w, dtype=np.float32).astype(np.float64)
    rows, K = x.shape
    nb = K // MX_BLOCK
    xb = x.reshape(rows, nb, MX_BLOCK)
    amax = np.max(np.abs(xb), axis=2)
    _, e = np.frexp(amax)                                # amax = f 2^e, f in [0.5, 1)
    shared = np.where(amax > 0, e - 1 - 2, -127)
    shared = np.clip(shared, -127, 127)
    codes = e2m1_encode(xb / np.ldexp(1.0, shared)[..., None])
    out = np.empty((rows, nb, MX_BYTES), dtype=np.uint8)
    out[:, :, 0] = (shared + 127).astype(np.uint8)
    out[:, :, 1:] = codes[:, :, 0::2] | (codes[:, :, 1::2] << 4)
    return out.reshape(rows, nb * MX_BYTES)


# ------------------------------------------------------------ dispatch ----
def decode(stored) -> np.ndarray:
    """A stored tensor (attributes fmt, shape, data, scales) -> float64."""
    fmt, shape = stored.fmt, tuple(stored.shape)
    if fmt == "f32":
        return np.asarray(stored.data, dtype=np.float32).astype(np.float64).reshape(shape)
    if fmt == "bf16":
        return bf16_decode(stored.data).reshape(shape)
    if fmt == "q8_0":
        return q8_0_decode(stored.data, shape[0], shape[1])
    if fmt == "fp8_e4m3":
        return fp8_decode(stored.data, stored.scales)
    if fmt == "mxfp4":
        return mxfp4_decode(stored.data, shape[0], shape[1])
    raise ValueError(fmt)


def decode_rows(stored, r0: int, r1: int) -> np.ndarray:
    """Rows [r0, r1) of a stored 2-D tensor -> float64 (same arithmetic as decode)."""
    fmt, (rows, cols) = stored.fmt, tuple(stored.shape)
    if fmt == "f32":
        return np.asarray(stored.data[r0:r1], dtype=np.float32).astype(np.float64)
    if fmt == "bf16":
        return bf16_decode(stored.data[r0:r1])
    if fmt == "q8_0":
        return q8_0_decode(stored.data[r0:r1], r1 - r0, cols)
    if fmt == "fp8_e4m3":
        return fp8_decode(stored.data[r0:r1], stored.scales[r0:r1])
    if fmt == "mxfp4":
        return mxfp4_decode(stored.data[r0:r1], r1 - r0, cols)
    raise ValueError(fmt)
