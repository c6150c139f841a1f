"""Pins for oracle.geometry: closed forms against brute-force simulation and the printed prefix formulas."""
import json
import os

import numpy as np
import pytest

from oracle import geometry

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _completed_groups(pos, m):
    # brute force: a group is visible once every token in it has been reached
    return sum(1 for j in range(pos // m + 2) if all(t <= pos for t in range(j * m, j * m + m)))


@pytest.mark.parametrize("m", [1, 2, 3])
def test_n_visible_equals_completed_groups(m):
    for pos in range(0, 2048):
        assert geometry.n_visible(pos, m) == _completed_groups(pos, m)


@pytest.mark.parametrize("window", [16, 128])
def test_ring_slots_match_write_simulation(window):
    ring = [-1] * window
    for pos in range(0, 3 * window + 5):
        ring[pos % window] = pos          # decode overwrites slot pos mod W, then attends
        assert list(geometry.ring_slot_positions(pos, window)) == ring


@pytest.mark.parametrize("window", [16, 128])
def test_linear_window_count(window):
    for pos in range(0, 400):
        w = geometry.linear_window_positions(pos, window)
        assert len(w) == min(pos + 1, window)
        assert w[-1] == pos and (len(w) == 1 or np.all(np.diff(w) == 1))


def _uncovered(pos, window, m):
    wset = set(geometry.linear_window_positions(pos, window).tolist())
    nv = geometry.n_visible(pos, m)
    return [t for t in range(pos + 1) if t not in wset and geometry.compressed_rows_covering(t, m) >= nv]


@pytest.mark.parametrize("window,m", [(16, 1), (16, 2), (128, 1), (128, 2), (2, 2)])
def test_no_token_invisible_to_both_branches(window, m):
    for pos in range(0, 1024):
        assert _uncovered(pos, window, m) == []


def test_invariant_checker_is_not_vacuous():
    # a window shorter than a group leaves tokens unseen by both branches
    assert any(_uncovered(pos, 1, 4) for pos in range(16))


def test_printed_prefix_closed_forms():
    g = json.load(open(os.path.join(GOLDEN, "visibility.json")))
    for c in g["cases"]:
        w = len(geometry.linear_window_positions(c["pos"], 128))
        nv = int(geometry.n_visible(c["pos"], c["ratio"]))
        assert w == c["window_rows"]
        assert nv == c["compressed_visible"]
        assert min(nv, 512) == c["selected_slots"]
        assert w + min(nv, 512) == c["full_prefix"] <= 640
