"""Pins of oracle.quantize: round trips, brute-force nearest-value rounding, saturation, scale rules."""
import numpy as np
import pytest
import torch

import oracle
from oracle import formats, quantize

E4M3 = formats.e4m3fn_table()
E2M1 = formats.e2m1_table()


def _brute_nearest(y, table, codes, max_mag):
    """Nearest finite table value to each y (ties -> even code), saturating at max_mag; brute force."""
    out = []
    for v in np.asarray(y, dtype=np.float64).ravel():
        a = min(abs(v), max_mag)
        cand = [(abs(table[c] - a), c % 2, c) for c in codes if table[c] >= 0 and np.isfinite(table[c])]
        d, _, c = min(cand)
        out.append(c | (0x80 if table is E4M3 and np.signbit(v) else 0) | (0x8 if table is E2M1 and np.signbit(v) else 0))
    return np.array(out, dtype=np.uint8).reshape(np.shape(y))


def test_e4m3_every_code_round_trips():
    codes = np.array([c for c in range(256) if not np.isnan(E4M3[c])], dtype=np.uint8)
    vals = E4M3[codes].astype(np.float32)
    got = quantize.e4m3_encode(vals)
    # -0 encodes as 0x80, +0 as 0x00: both decode to zero
    assert np.array_equal(formats.decode_fp8_values(got), E4M3[codes])
    nz = vals != 0
    assert np.array_equal(got[nz], codes[nz])


def test_e4m3_rounding_against_brute_force():
    rng = np.random.default_rng(0)
    y = np.concatenate([rng.standard_normal(3000) * 50, rng.standard_normal(2000) * 0.01,
                        rng.uniform(-600, 600, 1000), rng.uniform(-2 ** -6, 2 ** -6, 1000)]).astype(np.float32)
    # exact midpoints between neighbouring codes (ties) in both ranges
    pos = np.sort(E4M3[[c for c in range(0x7F)]])
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    y = np.concatenate([y, mids, -mids]).astype(np.float32)
    want = _brute_nearest(y, E4M3, range(0x7F), 448.0)
    got = quantize.e4m3_encode(y)
    # compare values (the sign of zero aside)
    assert np.array_equal(formats.decode_fp8_values(got), formats.decode_fp8_values(want))


def test_e4m3_matches_torch_float8_cast_inside_range():
    """torch's float8_e4m3fn cast (round to nearest even) agrees wherever it does not overflow."""
    rng = np.random.default_rng(1)
    y = (rng.standard_normal(20000) * 30).astype(np.float32)
    y = y[np.abs(y) <= 448]
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = quantize.e4m3_encode(y)
    assert np.array_equal(formats.decode_fp8_values(got), formats.decode_fp8_values(ref))


def test_e4m3_saturates_and_nan():
    got = quantize.e4m3_encode(np.array([448, 463.9, 464, 1e9, -1e9, np.inf, np.nan], dtype=np.float32))
    assert list(got[:5]) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    assert got[5] == 0x7E and (got[6] & 0x7F) == 0x7F


def test_e2m1_rounding_against_brute_force():
    rng = np.random.default_rng(2)
    mags = E2M1[:8]
    mids = ((mags[1:] + mags[:-1]) / 2)
    y = np.concatenate([rng.uniform(-8, 8, 5000), mids, -mids, mags, -mags, [7.0, -100.0]]).astype(np.float32)
    want = _brute_nearest(y, E2M1, range(8), 6.0)
    got = quantize.e2m1_encode(y)
    assert np.array_equal(E2M1[got], E2M1[want])
    # ties at the spec's midpoints go to the even code: 0.25->0, 0.75->1.0, 1.25->1.0, 1.75->2, 2.5->2, 3.5->4, 5->4
    t = quantize.e2m1_encode(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32))
    assert list(E2M1[t]) == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]


def test_fp8_rows_scale_rule_and_error_bound():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 128)).astype(np.float32)
    x[3] = 0.0
    codes, scale = quantize.fp8_rows(x)
    assert scale[3] == 1.0 and np.all(codes[3] == 0)
    amax = np.max(np.abs(x), axis=1)
    assert np.array_equal(scale[amax > 0], (amax[amax > 0] / np.float32(448)).astype(np.float32))
    dec = formats.decode_fp8_rows(codes, scale)
    # the row maximum maps to 448 exactly (up to the float32 rounding of amax / scale)
    assert np.all(np.abs(np.max(np.abs(dec), axis=1)[amax > 0] - amax[amax > 0]) <= 2 ** -3 * amax[amax > 0])
    # relative error of E4M3 rounding: at most half a step (2^-4) for normal values
    big = np.abs(x) >= 2 ** -6 * scale[:, None]
    err = np.abs(dec - x)[big] / np.abs(x)[big]
    assert err.max() <= 2 ** -4 + 1e-7


def test_fp4_e8m0_rows_scale_rule():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((20, 128)).astype(np.float32)
    x[1, :32] = 0.0
    x[2, 32:64] = 3.0          # amax / 6 = 0.5 exactly: scale 2^-1
    x[2, 64:96] = 3.0001       # just above: scale 2^0
    packed, e8 = quantize.fp4_e8m0_rows(x)
    assert e8[1, 0] == 0
    assert e8[2, 1] == 127 - 1 and e8[2, 2] == 127
    dec = formats.decode_fp4_rows(packed, e8)
    blocks = x.reshape(20, 4, 32)
    amax = np.abs(blocks).max(axis=2)
    sc = formats.e8m0_to_f64(e8)
    # every block's scaled maximum lies in (3, 6]: the scale is the smallest power of two that fits 6
    ok = amax > 0
    assert np.all(amax[ok] / sc[ok] <= 6.0) and np.all(amax[ok] / sc[ok] > 3.0)
    assert np.all(np.abs(dec - x) <= np.repeat(sc, 32, axis=1) * 1.0 + 1e-12)


def test_nvfp4_rows_layout_and_scale_rule():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((10, 512)).astype(np.float32)
    x[4, :16] = 0.0
    rows = quantize.nvfp4_rows(x)
    assert rows.shape == (10, 288)
    sc = formats.decode_fp8_values(rows[:, 256:])
    assert sc[4, 0] == 2.0 ** -9          # an all-zero group takes the smallest scale
    dec = formats.decode_nvfp4_rows(rows)
    assert np.all(dec[4, :16] == 0)
    g = np.abs(x.reshape(10, 32, 16)).max(axis=2)
    want = formats.decode_fp8_values(quantize.e4m3_encode(np.clip(g / np.float32(6), 2 ** -9, 448).astype(np.float32)))
    assert np.array_equal(sc, want)


def test_encoders_agree_with_the_input_generators():
    """The synthetic-input encoders (workloads/gen.py, torch) and these encoders implement the same rules."""
    from workloads.gen import encode_fp4_rows, encode_fp8_rows, encode_nvfp4_rows
    rng = np.random.default_rng(6)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    t = torch.from_numpy(x)
    c8, s8 = encode_fp8_rows(t)
    o8, os8 = quantize.fp8_rows(x)
    assert np.array_equal(s8.numpy(), os8)
    assert np.array_equal(formats.decode_fp8_rows(c8.numpy(), s8.numpy()), formats.decode_fp8_rows(o8, os8))
    p4, e4 = encode_fp4_rows(t)
    op4, oe4 = quantize.fp4_e8m0_rows(x)
    assert np.array_equal(e4.numpy(), oe4) and np.array_equal(p4.numpy(), op4)
    assert np.array_equal(encode_nvfp4_rows(t).numpy(), quantize.nvfp4_rows(x))
