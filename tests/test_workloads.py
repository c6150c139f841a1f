"""Checks of the synthetic input generator (storage formats and shapes), CPU only."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import formats
from workloads import CONFIGS, make_inputs
from workloads.gen import encode_fp4_rows, encode_fp8_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_fp4_encoder_picks_nearest_grid_point():
    g = torch.Generator().manual_seed(0)
    x = torch.randn(64, 512, generator=g) / 22.6
    packed, sc = encode_fp4_rows(x)
    dec = formats.decode_fp4_rows(packed.numpy(), sc.numpy())
    xb = x.double().numpy().reshape(64, 16, 32)
    s = formats.e8m0_to_f64(sc.numpy())[..., None]
    grid = np.unique(np.abs(formats.e2m1_table()))
    cand = np.sign(xb)[..., None] * grid * s[..., None]
    best = np.abs(cand - xb[..., None]).min(axis=-1)
    assert np.allclose(np.abs(dec.reshape(64, 16, 32) - xb), best, atol=1e-12)
    assert np.all(np.abs(xb / s) <= 6.0 + 1e-12)


def test_fp8_encoder_within_half_ulp():
    g = torch.Generator().manual_seed(1)
    x = torch.randn(32, 128, generator=g)
    codes, sc = encode_fp8_rows(x)
    dec = formats.decode_fp8_rows(codes.numpy(), sc.numpy())
    rel = np.abs(dec - x.double().numpy()) / np.maximum(np.abs(x.double().numpy()), 2 ** -6 * sc.numpy()[:, None])
    assert rel.max() <= 2 ** -4 + 1e-9


def test_row_bytes_match_pages():
    g = json.load(open(os.path.join(GOLDEN, "byte_counts.json")))
    cfg = CONFIGS["full_decode_64k"]
    assert cfg.dim * 2 == g["bf16_main_row_bytes"]
    assert CONFIGS["lowp_full_decode_1m"].idx_dim + 4 == g["fp8_index_row_bytes"]
    rc = CONFIGS["reindex_decode_1m"]
    assert rc.n_blocks == g["n_blocks"] and rc.block_rows == g["block_rows"] and rc.width == g["reindex_width"]


def test_candidates_ascending_distinct_with_newest_block():
    cfg = CONFIGS["reindex_decode_1m"].replace(batch=6, q_tokens=6, context=5000, n_blocks=64, ragged=True)
    x = make_inputs(cfg, 3)
    for r in range(6):
        c = x["cand"][r].numpy()
        nv = (int(x["pos"][r]) + 1) // cfg.ratio
        valid = c[c >= 0]
        assert np.all(np.diff(valid) > 0)
        assert np.all(c[len(valid):] == -1)
        if nv > 0:
            assert valid[-1] == (nv + 7) // 8 - 1
            assert len(valid) == min(64, (nv + 7) // 8)


@pytest.mark.parametrize("name", ["tiny_full_fp32"])
def test_shapes(name):
    cfg = CONFIGS[name]
    x = make_inputs(cfg, 0)
    assert x["main"].shape == (cfg.n_main_rows, cfg.dim)
    assert x["layers"][0]["swa"].shape == (cfg.context, cfg.dim)
    assert x["layers"][0]["q"].shape == (cfg.q_tokens, cfg.heads, cfg.dim)
