"""CPU pins of oracle.recurrence: the reverse linear recurrence and the cumsum
backward of rlx-cpu 0.2.17 training_bwd.rs cumsum_backward_row."""
import json
import os

import numpy as np
import pytest

from oracle import recurrence as rec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "reverse_scan_T4.json")


def test_cumsum_backward_row_matches_numpy_suffix_sums():
    rng = np.random.default_rng(0)
    dy = rng.standard_normal(37)
    inc = np.cumsum(dy[::-1])[::-1]                     # library suffix sum
    assert np.allclose(rec.cumsum_backward_row(dy, False), inc, rtol=0, atol=1e-12)
    assert np.allclose(rec.cumsum_backward_row(dy, True), inc - dy, rtol=0, atol=1e-12)


def test_cumsum_backward_is_the_transpose_of_cumsum():
    """<cumsum(v), w> = <v, cumsum_bwd(w)> for the inclusive and exclusive forward sums."""
    rng = np.random.default_rng(1)
    v, w = rng.standard_normal(50), rng.standard_normal(50)
    inc = np.cumsum(v)
    exc = inc - v
    assert abs(inc @ w - v @ rec.cumsum_backward_row(w, False)) < 1e-10
    assert abs(exc @ w - v @ rec.cumsum_backward_row(w, True)) < 1e-10


@pytest.mark.parametrize("exclusive", [False, True])
def test_unit_decay_is_the_row_cumsum_backward(exclusive):
    rng = np.random.default_rng(2)
    b = rng.standard_normal((2, 19, 3))
    x = rec.reverse_linear_scan(None, b, exclusive)
    ones = rec.reverse_linear_scan(np.ones_like(b), b, exclusive)
    for i in range(2):
        for c in range(3):
            assert np.allclose(x[i, :, c], rec.cumsum_backward_row(b[i, :, c], exclusive), atol=1e-12)
    assert np.array_equal(x, ones)


def test_explicit_sum_over_later_steps():
    """x_t = sum_{j >= t} (prod_{t < r <= j} a_r) b_j, by brute force."""
    rng = np.random.default_rng(3)
    a = rng.uniform(0.2, 1.1, (1, 12, 2))
    b = rng.standard_normal((1, 12, 2))
    want = np.zeros_like(b)
    for t in range(12):
        for j in range(t, 12):
            want[:, t] += np.prod(a[:, t + 1:j + 1], axis=1) * b[:, j]
    assert np.allclose(rec.reverse_linear_scan(a, b, False), want, rtol=1e-12, atol=1e-12)
    assert np.allclose(rec.reverse_linear_scan(a, b, True), want - b, rtol=1e-12, atol=1e-12)


def test_adjoint_of_the_forward_recurrence():
    """The inclusive sweep is the transpose of h_t = a_t h_{t-1} + v_t (h_{-1} = 0):
    <h(v), w> = <v, x(w)> (the adjoint of mamba-rs Phase B3 for one state)."""
    rng = np.random.default_rng(4)
    a = rng.uniform(0.1, 1.0, (2, 30, 4))
    v, w = rng.standard_normal((2, 30, 4)), rng.standard_normal((2, 30, 4))
    h = np.zeros_like(v)
    prev = np.zeros((2, 4))
    for t in range(30):
        prev = a[:, t] * prev + v[:, t]
        h[:, t] = prev
    assert abs(np.sum(h * w) - np.sum(v * rec.reverse_linear_scan(a, w))) < 1e-10


def test_hand_worked_example():
    """tests/golden/reverse_scan_T4.json: T = 4 values worked by hand."""
    g = json.load(open(GOLDEN))
    a = np.array(g["a"], dtype=np.float64)[None, :, None]
    b = np.array(g["b"], dtype=np.float64)[None, :, None]
    assert np.allclose(rec.reverse_linear_scan(a, b, False)[0, :, 0], g["inclusive"], atol=1e-15)
    assert np.allclose(rec.reverse_linear_scan(a, b, True)[0, :, 0], g["exclusive"], atol=1e-15)
    assert np.allclose(rec.reverse_linear_scan(None, b, False)[0, :, 0], g["inclusive_unit_decay"], atol=1e-15)


def test_empty_and_single_step():
    assert rec.reverse_linear_scan(None, np.zeros((2, 0, 3))).shape == (2, 0, 3)
    b = np.array([[[1.5, -2.0]]])
    assert np.array_equal(rec.reverse_linear_scan(np.full_like(b, 7.0), b), b)
    assert np.array_equal(rec.reverse_linear_scan(None, b, True), np.zeros_like(b))
