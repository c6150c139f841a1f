"""Pins for oracle.attention: dense equivalence, textbook softmax, closed forms, invariants."""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import attention, geometry, rope


def _inverse_rope_complex(x, pos, freqs):
    r = 2 * len(freqs)
    y = x.copy()
    z = x[..., -r::2] + 1j * x[..., -r + 1::2]
    z = z * np.exp(-1j * pos * freqs)
    y[..., -r::2], y[..., -r + 1::2] = z.real, z.imag
    return y


def _tiny_problem(seed, T=40, D=16, H=3, W=4, m=2, R=4):
    rng = np.random.default_rng(seed)
    N = T // m
    return dict(
        q=rng.standard_normal((T, H, D)), main=rng.standard_normal((N, D)), swa=rng.standard_normal((T, D)),
        sink=rng.standard_normal(H), pos=np.arange(T), T=T, D=D, H=H, W=W, m=m,
        freqs=rope.inv_freq(R, 10000.0), tau=1.0 / math.sqrt(D), N=N)


def test_sparse_equals_dense_masked_when_topk_covers_all():
    p = _tiny_problem(0)
    k = p["N"]  # k >= every n_vis
    idx = np.full((p["T"], k), -1)
    for r in range(p["T"]):
        nv = (r + 1) // p["m"]
        idx[r, :nv] = np.arange(nv)
    ours = attention.prefill(p["q"], p["pos"], idx, p["main"], p["swa"], 0, p["W"], p["sink"], p["tau"], p["freqs"], p["m"])
    # dense: every SWA row and every compressed row as keys, masked, with a sink column appended
    keys = np.concatenate([p["swa"], p["main"]], axis=0)
    for r in range(p["T"]):
        mask = np.zeros(keys.shape[0], dtype=bool)
        mask[max(0, r - p["W"] + 1): r + 1] = True
        mask[p["T"]: p["T"] + (r + 1) // p["m"]] = True
        logits = p["tau"] * p["q"][r] @ keys.T
        logits[:, ~mask] = -np.inf
        full = np.concatenate([logits, p["sink"][:, None]], axis=1)
        prob = scipy.special.softmax(full, axis=1)
        dense = prob[:, :-1] @ keys
        assert np.allclose(ours[r], _inverse_rope_complex(dense, r, p["freqs"]), atol=1e-12, rtol=1e-12)


def test_sink_minus_inf_is_textbook_softmax_attention():
    rng = np.random.default_rng(1)
    H, D, E = 4, 32, 11
    q, rows = rng.standard_normal((H, D)), rng.standard_normal((E, D))
    tau = 1 / math.sqrt(D)
    ours = attention.sink_attention(q, rows, np.full(H, -np.inf), tau)
    qt = torch.from_numpy(q)[None, :, None, :]
    kt = torch.from_numpy(rows)[None, None].expand(1, H, E, D)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=tau)[0, :, 0].numpy()
    assert np.allclose(ours, ref, atol=1e-12)


def test_mass_plus_sink_is_one():
    rng = np.random.default_rng(2)
    q, rows, sink = rng.standard_normal((5, 8)) * 3, rng.standard_normal((20, 8)), rng.standard_normal(5) * 4
    pr, ps = attention.sink_softmax_weights(q, rows, sink, 0.5)
    assert np.allclose(pr.sum(axis=1) + ps, 1.0, atol=1e-14)
    assert np.all(pr >= 0) and np.all(ps > 0)


def test_single_entry_and_constant_rows():
    rng = np.random.default_rng(3)
    H, D = 4, 16
    q, v, sink = rng.standard_normal((H, D)), rng.standard_normal(D), rng.standard_normal(H)
    tau = 0.25
    s = tau * q @ v
    psink = 1.0 / (1.0 + np.exp(s - sink))
    assert np.allclose(attention.sink_attention(q, v[None], sink, tau), (1 - psink)[:, None] * v[None], atol=1e-14)
    E = 7
    psink7 = np.exp(sink) / (np.exp(sink) + E * np.exp(s))
    out = attention.sink_attention(q, np.repeat(v[None], E, axis=0), sink, tau)
    assert np.allclose(out, (1 - psink7)[:, None] * v[None], atol=1e-13)


def test_zero_query_gives_uniform_weights():
    rng = np.random.default_rng(4)
    rows, sink = rng.standard_normal((9, 8)), rng.standard_normal(3)
    out = attention.sink_attention(np.zeros((3, 8)), rows, sink, 1.0)
    expect = rows.sum(axis=0)[None] / (9 + np.exp(sink))[:, None]
    assert np.allclose(out, expect, atol=1e-14)


def test_joint_softmax_differs_from_two_softmaxes():
    rng = np.random.default_rng(5)
    q, a, b, sink = rng.standard_normal((2, 8)), rng.standard_normal((4, 8)), rng.standard_normal((6, 8)), np.zeros(2)
    joint = attention.sink_attention(q, np.concatenate([a, b]), sink, 1.0)
    separate = attention.sink_attention(q, a, sink, 1.0) + attention.sink_attention(q, b, sink, 1.0)
    assert not np.allclose(joint, separate, atol=1e-3)


def test_repeated_index_counts_twice_and_masks_hold():
    p = _tiny_problem(6, T=32)
    r = 31
    nv = (r + 1) // p["m"]
    idx = np.array([[3, 3, 5, -1, nv, nv + 3, 1 << 20]])
    main = p["main"].copy()
    rows = attention.entries_prefill(r, idx[0], main, p["swa"], 0, p["W"], p["m"])
    assert rows.shape[0] == p["W"] + 3
    assert np.array_equal(rows[p["W"]], main[3]) and np.array_equal(rows[p["W"] + 1], main[3])
    # rows the query may not see do not influence the result
    big = np.concatenate([main, np.zeros((1 << 20, p["D"]))[:0]], axis=0)
    out1 = attention.prefill(p["q"][r:r + 1], p["pos"][r:r + 1], idx[:, :4], main, p["swa"], 0, p["W"], p["sink"], p["tau"], p["freqs"], p["m"])
    main2 = main.copy()
    main2[nv:] = 1e6
    out2 = attention.prefill(p["q"][r:r + 1], p["pos"][r:r + 1], idx, main2, p["swa"], 0, p["W"], p["sink"], p["tau"], p["freqs"], p["m"])
    assert np.allclose(out1, out2, atol=1e-12)


def test_decode_ring_equals_prefill_window():
    p = _tiny_problem(7, T=37, W=8)
    W = p["W"]
    for r in [0, 3, 7, 8, 20, 36]:
        ring = np.zeros((W, p["D"]))
        for t in range(r + 1):
            ring[t % W] = p["swa"][t]        # slot = position mod W
        nv = (r + 1) // p["m"]
        idx = np.arange(nv)[None]
        a = attention.decode(p["q"][r:r + 1], np.array([r]), idx, lambda _: p["main"], lambda _: ring,
                             p["sink"], p["tau"], p["freqs"], p["m"])
        b = attention.prefill(p["q"][r:r + 1], np.array([r]), idx, p["main"], p["swa"], 0, W,
                              p["sink"], p["tau"], p["freqs"], p["m"])
        assert np.allclose(a, b, atol=1e-13)


def test_constant_stored_row_comes_back_unrotated():
    # a stored row c rotated at the query's position returns c*(1 - p_sink) after the inverse rotation
    rng = np.random.default_rng(8)
    H, D, R = 2, 16, 8
    freqs = rope.inv_freq(R, 10000.0)
    c = rng.standard_normal(D)
    pos = 37
    stored = rope.rotate_tail(c, pos, freqs)
    q, sink = rng.standard_normal((H, D)), rng.standard_normal(H)
    out = attention.attend(q, pos, np.repeat(stored[None], 3, axis=0), sink, 0.5, freqs)
    s = 0.5 * q @ stored
    psink = np.exp(sink) / (np.exp(sink) + 3 * np.exp(s))
    assert np.allclose(out, (1 - psink)[:, None] * c[None], atol=1e-13)


def test_nan_entry_row_gives_nan_output():
    """An entry row holding a NaN scores NaN against every head; one softmax over all entries then
    makes every output element NaN.  A NaN in a ring slot outside the window changes nothing."""
    rng = np.random.default_rng(21)
    H, D, W = 2, 8, 4
    q = rng.standard_normal((H, D))
    sink = rng.standard_normal(H)
    ring = rng.standard_normal((W, D))
    plane = rng.standard_normal((6, D))
    freqs = rope.inv_freq(4, 10000.0)
    idx = np.array([0, 2, -1])
    pos = 5   # ring slots hold positions 4, 5, 2, 3: all valid
    base = attention.attend(q, pos, attention.entries_decode(pos, idx, plane, ring, 1), sink, 0.3, freqs)
    assert np.all(np.isfinite(base))
    bad = plane.copy()
    bad[2, 5] = np.nan
    out = attention.attend(q, pos, attention.entries_decode(pos, idx, bad, ring, 1), sink, 0.3, freqs)
    assert np.all(np.isnan(out))
    # position 1: slots 2 and 3 were never written (positions -2, -1); a NaN there is not an entry
    ring2 = ring.copy()
    ring2[3, 0] = np.nan
    a = attention.attend(q, 1, attention.entries_decode(1, idx, plane, ring, 1), sink, 0.3, freqs)
    b = attention.attend(q, 1, attention.entries_decode(1, idx, plane, ring2, 1), sink, 0.3, freqs)
    assert np.array_equal(a, b) and np.all(np.isfinite(b))
