"""Storage-format decoders, float64 (oracle; test infrastructure only).

Each decoder is written from the published definition of the format, not from
any implementation:

* bfloat16: the upper 16 bits of an IEEE-754 binary32.
* FP8-E4M3, OCP "FN" variant (OCP 8-bit floating point specification, 2023):
  1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities; S.1111.111 is
  NaN; largest finite magnitude 448; subnormals 2^-6 * m/8.
* FP4-E2M1 (OCP Microscaling specification v1.0): 1 sign, 2 exponent (bias 1),
  1 mantissa bit; magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* E8M0 (same specification): an unsigned biased exponent, value 2^(e-127);
  e = 255 is NaN.

Layouts decoded here are the ones the stored planes use:

* FP8 rows: ``codes[N, D]`` uint8 with one float32 scale per row
  (the index plane of "DeepSeek-V4.1-Flash 架构解剖", special module
  "压缩平面与候选块": 128 FP8 values plus one FP32 scale = 132 B per row; the
  FP8 SWA ring uses the same per-row form).
* FP4 rows: ``packed[N, D/2]`` uint8, element 2i in the low nibble and 2i+1 in
  the high nibble, with one E8M0 byte per 32 consecutive elements in
  ``scales[N, D/32]`` (MXFP4 block size 32).  The pages' FP4 index plane
  (68 B per row: 64 bytes of E2M1 plus one E8M0 per 32, "DeepSeek-V4.1-Flash
  结构说明" §5.3; "万字长文解析DeekSeekV4.1flash" §10.6) and FP4 indexer query
  are this format.
* Packed FP4 main rows of the pages' 890 B/token configuration: 288 bytes per
  512-element row, the 256 bytes of E2M1 (packed as above) followed by 32
  E4M3 scales, one per 16 consecutive elements, with no second-level scale
  ("DeepSeek-V4.1-Flash 架构解剖", "换成 packed FP4 主池"; the essay §10.7).
* FP8 SWA rows of that configuration: 528 bytes per 512-element row, 512
  E4M3 codes followed by 16 E8M0 scales, one per 32 elements (the anatomy
  page, same section).

Pins (tests/test_oracle_formats.py): every FP8 code against torch's
independent float8_e4m3fn conversion and against spot values fixed by the
specification; the 16 E2M1 codes against the specification's value list
(tests/golden/e2m1_values.json); E8M0 against exact powers of two; bf16
against torch's bfloat16 conversion.
"""

import numpy as np


def bf16_to_f64(u16):
    """Decode raw bfloat16 bit patterns (uint16 array) to float64 exactly."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def e4m3fn_value(code):
    """Value of one FP8-E4M3-FN code (0..255) from the bit-field definition."""
    code = int(code)
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def e4m3fn_table():
    """All 256 FP8-E4M3-FN values, indexed by code."""
    return np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def e2m1_value(code):
    """Value of one FP4-E2M1 code (0..15): sign bit 3, exponent bits 2..1, mantissa bit 0."""
    code = int(code)
    sign = -1.0 if (code >> 3) & 1 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:
        mag = man * 0.5  # subnormal: 2^(1-1) * m/2
    else:
        mag = (1.0 + man * 0.5) * 2.0 ** (exp - 1)
    return sign * mag


def e2m1_table():
    """All 16 FP4-E2M1 values, indexed by code."""
    return np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e8m0_to_f64(u8):
    """Decode E8M0 scale bytes: 2^(e-127), with e = 255 mapping to NaN."""
    e = np.asarray(u8, dtype=np.int64)
    out = np.ldexp(1.0, e - 127).astype(np.float64)
    return np.where(e == 255, np.nan, out)


_E4M3 = None
_E2M1 = None


def decode_fp8_rows(codes, row_scale):
    """FP8-E4M3 rows times their float32 row scale -> float64 [N, D]."""
    global _E4M3
    if _E4M3 is None:
        _E4M3 = e4m3fn_table()
    codes = np.asarray(codes, dtype=np.uint8)
    scale = np.asarray(row_scale, dtype=np.float32).astype(np.float64)
    return _E4M3[codes] * scale[..., None]


def decode_fp8_values(codes):
    """FP8-E4M3 codes to float64 with no scale."""
    global _E4M3
    if _E4M3 is None:
        _E4M3 = e4m3fn_table()
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def decode_fp4_rows(packed, scales):
    """Packed FP4-E2M1 rows with one E8M0 scale per 32 elements -> float64 [N, D]."""
    global _E2M1
    if _E2M1 is None:
        _E2M1 = e2m1_table()
    packed = np.asarray(packed, dtype=np.uint8)
    n, half = packed.shape[-2], packed.shape[-1]
    d = 2 * half
    lo = packed & 0x0F
    hi = packed >> 4
    codes = np.empty(packed.shape[:-1] + (d,), dtype=np.uint8)
    codes[..., 0::2] = lo
    codes[..., 1::2] = hi
    vals = _E2M1[codes]
    sc = e8m0_to_f64(scales)  # [..., N, D/32]
    assert sc.shape[-1] * 32 == d and sc.shape[-2] == n
    return vals * np.repeat(sc, 32, axis=-1)


def _unpack_e2m1(packed):
    """Packed E2M1 bytes [..., B] -> codes [..., 2B] (element 2i = low nibble of byte i)."""
    packed = np.asarray(packed, dtype=np.uint8)
    codes = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.uint8)
    codes[..., 0::2] = packed & 0x0F
    codes[..., 1::2] = packed >> 4
    return codes


def decode_nvfp4_rows(rows):
    """288-byte-per-512 rows: packed E2M1 then one E4M3 scale per 16 elements -> float64 [..., D]."""
    global _E2M1, _E4M3
    if _E2M1 is None:
        _E2M1 = e2m1_table()
    if _E4M3 is None:
        _E4M3 = e4m3fn_table()
    rows = np.asarray(rows, dtype=np.uint8)
    nb = rows.shape[-1]
    assert (nb * 16) % 9 == 0
    d = nb * 16 // 9                       # D/2 value bytes + D/16 scale bytes
    vals = _E2M1[_unpack_e2m1(rows[..., : d // 2])]
    scales = _E4M3[rows[..., d // 2: d // 2 + d // 16]]
    return vals * np.repeat(scales, 16, axis=-1)


def decode_fp8_e8m0_rows(rows):
    """528-byte-per-512 rows: E4M3 codes then one E8M0 scale per 32 elements -> float64 [..., D]."""
    global _E4M3
    if _E4M3 is None:
        _E4M3 = e4m3fn_table()
    rows = np.asarray(rows, dtype=np.uint8)
    nb = rows.shape[-1]
    assert (nb * 32) % 33 == 0
    d = nb * 32 // 33                      # D value bytes + D/32 scale bytes
    vals = _E4M3[rows[..., :d]]
    scales = e8m0_to_f64(rows[..., d: d + d // 32])
    return vals * np.repeat(scales, 32, axis=-1)
