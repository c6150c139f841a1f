"""Pins for oracle.formats against the format specifications and torch's independent conversions."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_all_codes_match_torch_conversion():
    codes = torch.arange(256, dtype=torch.int64).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = formats.e4m3fn_table()
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(ours))
    assert np.array_equal(ref[~nan_ref], ours[~nan_ref])
    # signed zeros are distinct codes with the same value; the sign bit must still be honoured
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_e4m3_spot_values_from_spec():
    g = json.load(open(os.path.join(GOLDEN, "e4m3_spot_values.json")))
    t = formats.e4m3fn_table()
    for code, val in g["values"].items():
        assert t[int(code, 16)] == val, code
    for code in g["nan_codes"]:
        assert math.isnan(t[int(code, 16)])
    finite = t[~np.isnan(t)]
    assert finite.max() == 448.0 and finite.min() == -448.0


def test_e2m1_table_from_spec():
    g = json.load(open(os.path.join(GOLDEN, "e2m1_values.json")))
    t = formats.e2m1_table()
    assert np.array_equal(t, np.array(g["codes_to_values"]))
    assert math.copysign(1.0, t[8]) == -1.0


def test_e8m0_powers_of_two():
    e = np.array([0, 1, 100, 126, 127, 128, 200, 254, 255])
    v = formats.e8m0_to_f64(e)
    assert v[4] == 1.0 and v[3] == 0.5 and v[5] == 2.0
    assert v[0] == 2.0 ** -127 and v[7] == 2.0 ** 127
    assert math.isnan(v[8])
    assert np.all(v[:-1] == np.ldexp(1.0, e[:-1] - 127))


def test_bf16_matches_torch():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(4096, generator=g) * 100
    b = x.to(torch.bfloat16)
    bits = b.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(formats.bf16_to_f64(bits), b.to(torch.float64).numpy())


def test_fp4_rows_nibble_order_and_block_scale():
    # element e of the row carries code e % 16; element 2i is the low nibble of byte i
    d = 64
    codes = np.arange(d) % 16
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)[None, :]
    scales = np.array([[127, 129]], dtype=np.uint8)  # block 0 scale 1, block 1 scale 4
    out = formats.decode_fp4_rows(packed, scales)[0]
    t = np.array(json.load(open(os.path.join(GOLDEN, "e2m1_values.json")))["codes_to_values"])
    expect = t[codes] * np.where(np.arange(d) < 32, 1.0, 4.0)
    assert np.array_equal(out, expect)


def test_fp8_rows_scale():
    codes = np.array([[0x38, 0x40, 0xB8]], dtype=np.uint8)  # 1, 2, -1
    out = formats.decode_fp8_rows(codes, np.array([0.25], dtype=np.float32))
    assert np.array_equal(out, np.array([[0.25, 0.5, -0.25]]))


def test_nvfp4_rows_layout_group16_e4m3_scales():
    """288-byte rows: 256 bytes of packed E2M1 (element 2i low nibble), then one E4M3 scale per 16 elements."""
    d = 512
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 16, d)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    # scales per group of 16: E4M3 codes of 1, 2, 0.5, -1.5, 448 (largest), 2^-9 (smallest subnormal), cycling
    sc_codes = np.array([0x38, 0x40, 0x30, 0xBC, 0x7E, 0x01] * 6, dtype=np.uint8)[: d // 16]
    sc_vals = np.array([1.0, 2.0, 0.5, -1.5, 448.0, 2.0 ** -9] * 6)[: d // 16]
    row = np.concatenate([packed, sc_codes])[None, :]
    assert row.shape[1] == 288
    out = formats.decode_nvfp4_rows(row)[0]
    t = np.array(json.load(open(os.path.join(GOLDEN, "e2m1_values.json")))["codes_to_values"])
    expect = t[codes] * np.repeat(sc_vals, 16)
    assert np.array_equal(out, expect)
    # a swapped nibble order or a group of 32 would give different values
    assert not np.array_equal(out, t[np.stack([codes[1::2], codes[0::2]], 1).reshape(-1)] * np.repeat(sc_vals, 16))
    assert not np.array_equal(out, t[codes] * np.repeat(sc_vals[: d // 32], 32))


def test_fp8_e8m0_rows_layout():
    """528-byte rows: 512 E4M3 codes, then one E8M0 scale per 32 elements."""
    d = 512
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 256, d).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38                     # no NaN codes
    e8 = np.array([127, 128, 126, 1, 254, 120, 130, 127] * 2, dtype=np.uint8)
    row = np.concatenate([codes, e8])[None, :]
    assert row.shape[1] == 528
    out = formats.decode_fp8_e8m0_rows(row)[0]
    expect = formats.decode_fp8_values(codes) * np.repeat(np.ldexp(1.0, e8.astype(np.int64) - 127), 32)
    assert np.array_equal(out, expect)
    # spot values fixed by the specifications: code 0x40 = 2.0, E8M0 128 = 2^1
    r2 = np.concatenate([np.full(d, 0x40, np.uint8), np.full(16, 128, np.uint8)])[None, :]
    assert np.all(formats.decode_fp8_e8m0_rows(r2) == 4.0)
