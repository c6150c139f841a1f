"""Partial RoPE with YaRN frequencies, and its inverse (oracle; test infrastructure only).

What the pages fix ("DeepSeek-V4.1-Flash 结构说明", section 6.1-6.3; anatomy
page "DeepSeek-V4.1-Flash 架构解剖", CSA2 attention bullets):

* only the last R = 64 of the 512 latent dims rotate; the first 448 are NoPE;
* adjacent dims (2i, 2i+1) form one complex pair rotated by e^{i p theta_i}
  with 32 frequencies theta_i = base^(-2i/64);
* one frequency table per layer: base 10000 without YaRN for ratio-0 layers,
  base 160000 with YaRN (factor 16, original length 65536) for every layer
  with a compressed branch;
* the output of attention is multiplied by the conjugate phase at the query's
  own position on its rope tail (inverse rotation), because V is the rotated
  latent.

The YaRN segment formula itself did not survive on the pages (section 6.3
keeps only "three segments by how many turns the dim makes within the
training length 65536").  Reading taken: the NTK-by-parts rule of the YaRN
paper (Peng et al., 2023) with alpha = 1, beta = 32 and no attention
temperature change (section 6.3 says softmax_scale stays 512^-0.5):
r_i = L / lambda_i with lambda_i = 2*pi / theta_i; gamma = 0 for r < alpha,
1 for r > beta, linear in between; theta'_i = (1-gamma) theta_i / s + gamma theta_i.

Pins (tests/test_oracle_rope.py): inverse(rotate(x)) = x; the rotated pair
equals complex multiplication by exp(i p theta); q.k on the rope tail depends
only on the position difference; YaRN with factor 1 equals plain RoPE; the
YaRN table reproduces the three segments (high frequencies unchanged, low
frequencies divided by s).
"""

import math

import numpy as np


def inv_freq(rope_dim, theta, yarn_factor=1.0, yarn_orig_len=0, beta_fast=32.0, beta_slow=1.0):
    """Per-pair angular frequencies (float64, length rope_dim/2)."""
    half = rope_dim // 2
    base = np.array([theta ** (-2.0 * i / rope_dim) for i in range(half)], dtype=np.float64)
    if yarn_factor == 1.0 or yarn_orig_len <= 0:
        return base
    out = np.empty(half, dtype=np.float64)
    for i in range(half):
        wavelength = 2.0 * math.pi / base[i]
        r = yarn_orig_len / wavelength
        if r < beta_slow:
            gamma = 0.0
        elif r > beta_fast:
            gamma = 1.0
        else:
            gamma = (r - beta_slow) / (beta_fast - beta_slow)
        out[i] = (1.0 - gamma) * base[i] / yarn_factor + gamma * base[i]
    return out


def rotate_tail(x, pos, freqs, inverse=False):
    """Rotate the last 2*len(freqs) dims of x (float64, [..., D]) at absolute position ``pos``.

    Pair (2i, 2i+1) of the tail is multiplied by exp(+i*pos*freqs[i]), or by
    its conjugate when ``inverse``.
    """
    x = np.array(x, dtype=np.float64, copy=True)
    r = 2 * len(freqs)
    d = x.shape[-1]
    base = d - r
    for i in range(len(freqs)):
        phi = float(pos) * float(freqs[i])
        c, s = math.cos(phi), math.sin(phi)
        if inverse:
            s = -s
        a = x[..., base + 2 * i].copy()
        b = x[..., base + 2 * i + 1].copy()
        x[..., base + 2 * i] = a * c - b * s
        x[..., base + 2 * i + 1] = a * s + b * c
    return x
