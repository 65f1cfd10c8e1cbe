"""Pins of the diagnostics oracle (output RSE, mask Jaccard) against closed
forms and hand-worked examples."""
import numpy as np
import pytest

import oracle
import synth


def _bf16(x):
    return synth.f32_to_bf16(np.asarray(x, np.float32))


def test_rse_zero_for_identical_and_one_for_the_mean():
    rng = np.random.default_rng(1)
    y = _bf16(rng.standard_normal((2, 3, 17, 8)))
    assert np.all(oracle.output_rse(y, y) == 0.0)
    # a prediction that is the reference's own mean explains nothing: RSE = 1
    yf = synth.bf16_to_f32(y).astype(np.float64)
    mean = yf.mean(axis=(2, 3), keepdims=True)
    np.testing.assert_allclose(oracle.output_rse(np.broadcast_to(mean, yf.shape), yf), 1.0, rtol=1e-12)


def test_rse_of_a_shift_and_scale_invariance():
    rng = np.random.default_rng(2)
    y = rng.standard_normal((1, 2, 9, 4))
    var = ((y - y.mean(axis=(2, 3), keepdims=True)) ** 2).sum(axis=(2, 3))
    # y + c: the numerator is n c^2
    np.testing.assert_allclose(oracle.output_rse(y + 0.25, y), 36 * 0.0625 / var, rtol=1e-12)
    t = y + 0.1 * rng.standard_normal(y.shape)
    np.testing.assert_allclose(oracle.output_rse(3.0 * t, 3.0 * y), oracle.output_rse(t, y), rtol=1e-12)


def test_rse_hand_example():
    # reference (1, 2, 3, 4): mean 2.5, spread 5; test (1, 2, 3, 6): error 4
    ref = np.array([1.0, 2.0, 3.0, 4.0]).reshape(1, 1, 2, 2)
    tst = np.array([1.0, 2.0, 3.0, 6.0]).reshape(1, 1, 2, 2)
    assert oracle.output_rse(tst, ref)[0, 0] == pytest.approx(0.8, rel=1e-15)
    # a constant reference: 0/0 -> 0, x/0 -> inf
    c = np.ones((1, 1, 2, 2))
    assert oracle.output_rse(c, c)[0, 0] == 0.0
    assert oracle.output_rse(c + 1, c)[0, 0] == np.inf


def _csr(rows):
    rp = np.zeros(len(rows) + 1, np.int32)
    rp[1:] = np.cumsum([len(r) for r in rows])
    ci = np.array([j for r in rows for j in r], np.int32)
    return rp, ci


def test_jaccard_hand_example_and_conventions():
    # one head, 4 x 4 blocks
    a = _csr([[0, 1], [1, 2, 3], [], [3]])
    b = _csr([[0], [2, 3], [1], [3]])
    # intersections 1 + 2 + 0 + 1 = 4; unions 2 + 3 + 1 + 1 = 7
    assert oracle.mask_jaccard(1, 1, 4, *a, *b)[0, 0] == pytest.approx(4 / 7)
    assert oracle.mask_jaccard(1, 1, 4, *b, *a)[0, 0] == pytest.approx(4 / 7)
    assert oracle.mask_jaccard(1, 1, 4, *a, *a)[0, 0] == 1.0
    e = _csr([[], [], [], []])
    assert oracle.mask_jaccard(1, 1, 4, *e, *e)[0, 0] == 1.0
    assert oracle.mask_jaccard(1, 1, 4, *a, *e)[0, 0] == 0.0
    # repeats count once; indices outside [0, nB) are ignored
    d = _csr([[0, 1, 1, 7], [1, 2, 3, -1], [], [3, 3]])
    assert oracle.mask_jaccard(1, 1, 4, *d, *a)[0, 0] == 1.0


def test_jaccard_per_head_layout():
    # two heads: the second head's rows follow the first head's
    a = _csr([[0], [1], [0, 1], [0, 1]])
    b = _csr([[0], [1], [1], []])
    j = oracle.mask_jaccard(1, 2, 2, *a, *b)
    # head 1: intersections 1 + 0, unions 2 + 2
    assert j[0, 0] == 1.0 and j[0, 1] == pytest.approx(0.25)
