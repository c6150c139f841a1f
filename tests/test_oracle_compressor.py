"""Pins of oracle.compressor against closed forms, library routines and invariants."""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
from oracle import compressor, rope

FREQS = rope.inv_freq(64, 160000.0, 16.0, 65536)


def _weights(rng, d_in=96, wscale=0.1):
    return dict(wkv=rng.standard_normal((512, d_in)) * wscale, wgate=rng.standard_normal((512, d_in)) * wscale,
                norm_w=1.0 + 0.1 * rng.standard_normal(512), wk=rng.standard_normal((128, 512)) * 0.05,
                knorm_w=1.0 + 0.1 * rng.standard_normal(128))


def test_pool_weights_are_scipy_softmax_over_the_group():
    rng = np.random.default_rng(0)
    kvs = rng.standard_normal((2, 512))
    s = rng.standard_normal((2, 512)) * 3
    w = softmax(s, axis=0)
    assert np.allclose(compressor.pool(kvs, s), (w * kvs).sum(axis=0), rtol=1e-13, atol=1e-13)


def test_pool_special_cases():
    rng = np.random.default_rng(1)
    kvs = rng.standard_normal((2, 64))
    # equal scores: the plain mean
    assert np.allclose(compressor.pool(kvs, np.zeros((2, 64))), kvs.mean(axis=0), rtol=0, atol=1e-15)
    # a score far above the other selects its token (per channel)
    s = np.zeros((2, 64))
    s[0, :32] = 800.0
    s[1, 32:] = 800.0
    out = compressor.pool(kvs, s)
    assert np.array_equal(out[:32], kvs[0, :32]) and np.array_equal(out[32:], kvs[1, 32:])
    # adding a constant to a channel's scores changes nothing; the result lies between the two values
    s = rng.standard_normal((2, 64))
    shift = rng.standard_normal(64) * 50
    assert np.allclose(compressor.pool(kvs, s), compressor.pool(kvs, s + shift), rtol=1e-12, atol=1e-12)
    out = compressor.pool(kvs, s)
    assert np.all(out >= kvs.min(axis=0) - 1e-15) and np.all(out <= kvs.max(axis=0) + 1e-15)


def test_rms_norm_closed_forms():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((5, 512)) * 7
    out = compressor.rms_norm(v, np.ones(512), 0.0)
    assert np.allclose(np.sqrt(np.mean(out ** 2, axis=1)), 1.0, rtol=1e-14)
    # scale invariance without eps, and eps shrinks a tiny row instead of blowing it up
    assert np.allclose(compressor.rms_norm(3.5 * v, np.ones(512), 0.0), out, rtol=1e-13)
    tiny = np.full(512, 1e-6)
    assert np.allclose(compressor.rms_norm(tiny, np.ones(512), 1e-6), tiny / np.sqrt(1e-12 + 1e-6))
    # the weight multiplies channel by channel
    w = rng.standard_normal(512)
    assert np.allclose(compressor.rms_norm(v, w, 0.0), out * w, rtol=1e-13)


def test_ratio1_row_is_normalised_projection_rotated_at_its_position():
    rng = np.random.default_rng(3)
    W = _weights(rng)
    x = rng.standard_normal((1, 96))
    p = 123457
    rows, _, _ = compressor.compress_call(x, [p], [0], 1, W["wkv"], None, W["norm_w"], 1e-6, W["wk"],
                                          W["knorm_w"], 1e-6, FREQS)
    j, main, key, latent = rows[0]
    kv = x[0] @ W["wkv"].T
    want = kv / np.sqrt(np.mean(kv ** 2) + 1e-6) * W["norm_w"]
    assert j == p
    assert np.allclose(latent, want, rtol=1e-13)
    # rotation: the first 448 dims are untouched, each tail pair keeps its norm, the inverse undoes it
    assert np.array_equal(main[:448], latent[:448])
    pr = lambda a: np.hypot(a[448::2], a[449::2])
    assert np.allclose(pr(main), pr(latent), rtol=1e-13)
    assert np.allclose(rope.rotate_tail(main, p, FREQS, inverse=True), latent, rtol=1e-12, atol=1e-13)
    # the index key comes from the pre-rotation latent (not from the rotated main row)
    k0 = latent @ W["wk"].T
    k0 = k0 / np.sqrt(np.mean(k0 ** 2) + 1e-6) * W["knorm_w"]
    assert np.allclose(rope.rotate_tail(key, p, FREQS, inverse=True), k0, rtol=1e-12, atol=1e-13)
    k_wrong = main @ W["wk"].T
    k_wrong = k_wrong / np.sqrt(np.mean(k_wrong ** 2) + 1e-6) * W["knorm_w"]
    assert not np.allclose(rope.rotate_tail(key, p, FREQS, inverse=True), k_wrong, rtol=1e-6)


def test_ratio2_groups_rotate_at_the_first_position_and_pair_tokens():
    rng = np.random.default_rng(4)
    W = _weights(rng)
    x = rng.standard_normal((6, 96))
    pos = np.arange(10, 16)                     # groups 5, 6, 7 complete inside the call
    rows, tk, ts = compressor.compress_call(x, pos, np.zeros(6, int), 2, W["wkv"], W["wgate"], W["norm_w"], 1e-6,
                                            W["wk"], W["knorm_w"], 1e-6, FREQS, np.zeros((1, 512)),
                                            np.zeros((1, 512)))
    assert sorted(rows) == [1, 3, 5]
    for r in (1, 3, 5):
        j, main, key, latent = rows[r]
        assert j == pos[r] // 2
        kvs = x[r - 1:r + 1] @ W["wkv"].T
        sc = x[r - 1:r + 1] @ W["wgate"].T
        pooled = (softmax(sc, axis=0) * kvs).sum(axis=0)
        want = pooled / np.sqrt(np.mean(pooled ** 2) + 1e-6) * W["norm_w"]
        assert np.allclose(latent, want, rtol=1e-12)
        assert np.allclose(rope.rotate_tail(main, 2 * j, FREQS, inverse=True), latent, rtol=1e-12, atol=1e-13)
        # rotating at the group's second position would be a different row
        assert not np.allclose(main, rope.rotate_tail(latent, 2 * j + 1, FREQS), rtol=1e-6)
    # the tail state is untouched: no even position ended the call
    assert np.all(tk == 0) and np.all(ts == 0)


def test_tail_state_split_equals_one_call():
    """A sequence fed in chunks of odd lengths (groups straddling calls) writes the rows of one call."""
    rng = np.random.default_rng(5)
    W = _weights(rng)
    x = rng.standard_normal((11, 96))
    pos = np.arange(3, 14)
    args = (W["wkv"], W["wgate"], W["norm_w"], 1e-6, W["wk"], W["knorm_w"], 1e-6, FREQS)
    tail0 = rng.standard_normal((1, 512)), rng.standard_normal((1, 512))
    whole, _, _ = compressor.compress_call(x, pos, np.zeros(11, int), 2, *args, *tail0)
    got = {}
    tk, ts = tail0
    start = 0
    for n in (2, 3, 1, 5):
        rows, tk, ts = compressor.compress_call(x[start:start + n], pos[start:start + n], np.zeros(n, int), 2,
                                                *args, tk, ts)
        for r, v in rows.items():
            got[start + r] = v
        start += n
    assert sorted(got) == sorted(whole)
    for r in whole:
        for a, b in zip(got[r][1:], whole[r][1:]):
            assert np.allclose(a, b, rtol=1e-13, atol=1e-14)
    # the first row (position 3, odd) completed group 1 with the given tail state
    kvs = np.stack([tail0[0][0], x[0] @ W["wkv"].T])
    sc = np.stack([tail0[1][0], x[0] @ W["wgate"].T])
    pooled = (softmax(sc, axis=0) * kvs).sum(axis=0)
    assert np.allclose(whole[0][3], pooled / np.sqrt(np.mean(pooled ** 2) + 1e-6) * W["norm_w"], rtol=1e-12)


def test_batched_decode_sequences_are_independent():
    """Many sequences, one token each: each row only uses its own sequence's tail state."""
    rng = np.random.default_rng(6)
    W = _weights(rng)
    n = 8
    x = rng.standard_normal((n, 96))
    pos = rng.integers(0, 1000, n)
    args = (W["wkv"], W["wgate"], W["norm_w"], 1e-6, W["wk"], W["knorm_w"], 1e-6, FREQS)
    tk, ts = rng.standard_normal((n, 512)), rng.standard_normal((n, 512))
    rows, tk2, ts2 = compressor.compress_call(x, pos, np.arange(n), 2, *args, tk, ts)
    for r in range(n):
        if pos[r] % 2:
            one, _, _ = compressor.compress_call(x[r:r + 1], pos[r:r + 1], [0], 2, *args, tk[r:r + 1], ts[r:r + 1])
            assert np.allclose(rows[r][1], one[0][1], rtol=1e-13)
            assert np.array_equal(tk2[r], tk[r])
        else:
            assert r not in rows
            assert np.allclose(tk2[r], x[r] @ W["wkv"].T) and np.allclose(ts2[r], x[r] @ W["wgate"].T)
