"""Storage encoders: float32 rows -> the planes' byte formats (oracle; test infrastructure only).

Written from the format definitions (OCP 8-bit floating point specification
for E4M3 "FN"; OCP Microscaling specification v1.0 for E2M1 and E8M0) and the
planes' layouts:

* FP8 rows with one float32 scale per row (the index plane's 128 + 4 bytes,
  "DeepSeek-V4.1-Flash 架构解剖", special module "indexer", key side):
  scale = amax / 448 (1 for an all-zero row), codes = E4M3(x / scale).
* FP4 rows with one E8M0 scale per 32 elements (the MXFP4 index plane of the
  same page and of "DeepSeek-V4.1-Flash 结构说明" §5.3): scale = 2^e with
  e = ceil(log2(amax / 6)) clamped to [-127, 127] (e = -127 for an all-zero
  block), codes = E2M1(x / scale).
* Packed FP4 rows with one E4M3 scale per 16 elements (the 288-byte main rows,
  anatomy page, "换成 packed FP4 主池"): scale = E4M3(amax / 6) clamped to
  [2^-9, 448], codes = E2M1(x / scale).

Roundings: E4M3 and E2M1 round to nearest, ties to the even code, saturating
at the largest finite magnitude (448, 6).

Every value that decides a code (the scale, x / scale) is formed in float32
with correctly rounded IEEE operations, and the rounding itself is then exact
(a float32 value is exact in float64), so an implementation that forms the
same float32 values takes the same decisions.  The scale choices are readings
(the pages fix the layouts, not how a scale is picked); they are the ones the
synthetic-input encoders use.

Pins (tests/test_oracle_quantize.py): every E4M3 and E2M1 code round-trips
through the decoders in ``formats``; each rounding against brute force over
the whole code table (nearest value, ties to the even code); saturation; the
scale rules on crafted rows.
"""

import numpy as np

from . import formats

_F32 = np.float32


def e4m3_encode(y):
    """float32 array -> E4M3-FN codes (uint8): nearest, ties to even, saturating at +-448 (infinities too);
    NaN -> 0x7F (with its sign bit)."""
    y = np.asarray(y, dtype=np.float32)
    a_in = np.abs(y.astype(np.float64))
    finite = np.isfinite(a_in)
    a = np.where(finite, a_in, 0.0)
    sign = (np.signbit(y)).astype(np.uint8) << 7
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormals: multiples of 2^-9 (mantissa codes 0..7; a rounding up to 8 is 2^-6, code 0x08)
    code = np.where(sub, np.rint(a * 2.0 ** 9).astype(np.int64), code)
    m, e = np.frexp(np.where(sub, 1.0, a))            # a = m * 2^e, m in [0.5, 1)
    e = e - 1                                          # a = (2m) * 2^e, 2m in [1, 2)
    k = np.rint((2.0 * m - 1.0) * 8.0).astype(np.int64)  # 3 mantissa bits, exact ties to even
    carry = k == 8
    e = np.where(carry, e + 1, e)
    k = np.where(carry, 0, k)
    norm_code = ((e + 7) << 3) | k
    code = np.where(sub, code, norm_code)
    code = np.minimum(code, 0x7E)                      # saturate at 448 (0x7F is NaN)
    code = np.where(np.isinf(a_in), 0x7E, code)        # infinities saturate too
    code = np.where(np.isnan(a_in), 0x7F, code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e2m1_encode(y):
    """float32 array -> E2M1 codes (uint8, 0..15): nearest magnitude, ties to the even code, saturating at 6."""
    y = np.asarray(y, dtype=np.float32)
    a = np.minimum(np.abs(y.astype(np.float64)), 6.0)
    mags = np.array([formats.e2m1_value(c) for c in range(8)], dtype=np.float64)
    d = np.abs(a[..., None] - mags)                     # distance to every magnitude
    best = d.min(axis=-1, keepdims=True)
    near = d == best
    # ties: the even code among the nearest
    even = near & (np.arange(8) % 2 == 0)
    code = np.where(even.any(axis=-1), even.argmax(axis=-1), near.argmax(axis=-1))
    sign = np.signbit(y).astype(np.int64) << 3
    return (code | sign).astype(np.uint8)


def _amax(x, axis=-1):
    return np.max(np.abs(np.asarray(x, dtype=np.float32)), axis=axis)


def fp8_rows(x):
    """float32 [..., D] -> (codes uint8 [..., D], scale float32 [...])."""
    x = np.asarray(x, dtype=np.float32)
    amax = _amax(x)
    scale = np.where(amax > 0, (amax / _F32(448.0)).astype(np.float32), _F32(1.0)).astype(np.float32)
    y = (x / scale[..., None]).astype(np.float32)
    return e4m3_encode(y), scale


def _e8m0_exponent(v):
    """ceil(log2(v)) of positive float32 values, exactly (frexp of the float32 value)."""
    m, e = np.frexp(np.asarray(v, dtype=np.float32).astype(np.float64))  # v = m 2^e, m in [0.5, 1)
    return np.where(m == 0.5, e - 1, e)


def fp4_e8m0_rows(x):
    """float32 [..., D] -> (packed uint8 [..., D/2], E8M0 uint8 [..., D/32])."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    xb = x.reshape(*x.shape[:-1], d // 32, 32)
    amax = _amax(xb)
    v = (amax / _F32(6.0)).astype(np.float32)
    e = np.where(amax > 0, _e8m0_exponent(np.where(amax > 0, v, _F32(1.0))), -127)
    e = np.clip(e, -127, 127)
    sc = np.ldexp(np.float32(1.0), e.astype(np.int32)).astype(np.float32)
    y = (xb / sc[..., None]).astype(np.float32)
    codes = e2m1_encode(y).reshape(*x.shape[:-1], d)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


def nvfp4_rows(x):
    """float32 [..., D] -> rows uint8 [..., D/2 + D/16]: packed E2M1, then one E4M3 scale per 16."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    xb = x.reshape(*x.shape[:-1], d // 16, 16)
    amax = _amax(xb)
    v = np.clip((amax / _F32(6.0)).astype(np.float32), _F32(2.0 ** -9), _F32(448.0))
    sc_code = e4m3_encode(v)
    sc = formats.decode_fp8_values(sc_code).astype(np.float32)
    y = (xb / sc[..., None]).astype(np.float32)
    codes = e2m1_encode(y).reshape(*x.shape[:-1], d)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return np.concatenate([packed, sc_code], axis=-1)
