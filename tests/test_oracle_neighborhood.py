"""Pins of the 2-D neighbourhood attention oracle (window starts, the masked
forward, tile-major order, block layout) against hand examples, closed forms
and special cases that reduce to dense or block-sparse attention."""
import math

import numpy as np
import pytest

import oracle
import synth


def test_window_start_hand_examples():
    assert [oracle.na_start(i, 8, 3, 1) for i in range(8)] == [0, 0, 1, 2, 3, 4, 5, 5]
    assert [oracle.na_start(i, 9, 3, 3) for i in range(9)] == [0, 0, 0, 3, 3, 3, 6, 6, 6]
    assert [oracle.na_start(i, 8, 4, 2) for i in range(8)] == [0, 0, 1, 1, 3, 3, 4, 4]


@pytest.mark.parametrize("L,k,s", [(16, 5, 1), (16, 4, 1), (20, 7, 3), (12, 12, 1), (32, 8, 8), (33, 9, 4)])
def test_window_start_properties(L, k, s):
    st = [oracle.na_start(i, L, k, s) for i in range(L)]
    assert all(0 <= a <= L - k for a in st)                    # the window stays inside the axis
    assert all(st[i] <= st[i + 1] for i in range(L - 1))      # and moves forward with the query
    for i in range(L):
        if s == 1 and k % 2 == 1 and k // 2 <= i < L - k // 2:
            assert st[i] == i - k // 2                         # interior: centred on the query
        assert st[i] == st[(i // s) * s]                       # a stride group shares one window
    if L % k == 0 and s == k:
        assert st == [(i // k) * k for i in range(L)]          # blocked attention


def test_permutation_hand_example():
    perm = oracle.tile_permutation(2, (4, 4), (2, 2))
    assert perm.tolist() == [0, 1, 2, 3, 6, 7, 4, 5, 8, 9, 10, 11, 14, 15, 12, 13, 16, 17]
    p2 = oracle.tile_permutation(64, (16, 32), (8, 16))
    assert sorted(p2.tolist()) == list(range(64 + 16 * 32))


def _geom_inputs(B, H, T, R, C, D, seed):
    q, k, v = synth.random_qkv(B, H, T + R * C, D, seed=seed)
    return q, k, v


def test_full_window_is_dense_attention():
    T, R, C, D = 16, 6, 8, 32
    q, k, v = _geom_inputs(1, 2, T, R, C, D, 5)
    N = T + R * C
    O, L = oracle.forward_neighborhood(q, k, v, T, (R, C), (R, C), (1, 1))
    rp = np.arange(0, 2 * N + 1, N, dtype=np.int32)[:3]                 # block = N: one block per head
    rp = np.array([0, 1, 2], np.int32)
    ci = np.zeros(2, np.int32)
    Od, Ld = oracle.forward(q, k, v, N, rp, ci)
    np.testing.assert_allclose(O, Od, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L, Ld, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("window,stride", [((3, 5), (1, 1)), ((4, 4), (2, 2)), ((6, 8), (3, 4))])
def test_kept_counts_and_window_centres(window, stride):
    """With Q = 0 every kept key gets the same weight: LSE = ln(#kept keys) and
    O is the mean of the kept values.  V carries each image token's row and
    column (text values 0)."""
    T, R, C, D = 4, 9, 11, 8
    N = T + R * C
    q = np.zeros((1, 1, N, D), np.float32)
    k = synth.bf16_to_f32(synth.random_qkv(1, 1, N, D, seed=7)[1])
    v = np.zeros((1, 1, N, D), np.float32)
    idx = np.arange(R * C)
    v[0, 0, T:, 0] = idx // C
    v[0, 0, T:, 1] = idx % C
    O, L = oracle.forward_neighborhood(synth.f32_to_bf16(q), synth.f32_to_bf16(k), synth.f32_to_bf16(v), T,
                                       (R, C), window, stride)
    (kh, kw), (sh, sw) = window, stride
    np.testing.assert_allclose(np.exp(L[0, 0, :T]), N, rtol=1e-12)            # text queries: every key
    np.testing.assert_allclose(np.exp(L[0, 0, T:]), T + kh * kw, rtol=1e-12)  # image queries: text + window
    for p in range(R * C):
        r, c = divmod(p, C)
        r0, c0 = oracle.na_start(r, R, kh, sh), oracle.na_start(c, C, kw, sw)
        # the mean row / column of a kh x kw window starting at (r0, c0), diluted by the T text keys
        w = kh * kw / (T + kh * kw)
        assert O[0, 0, T + p, 0] == pytest.approx(w * (r0 + (kh - 1) / 2), abs=1e-12)
        assert O[0, 0, T + p, 1] == pytest.approx(w * (c0 + (kw - 1) / 2), abs=1e-12)


def test_layout_of_blocked_attention_is_perfectly_block_sparse():
    # window = stride = 2 x 2 tiles of 4 x 8: every kept block pair is full
    T, R, C, th, tw = 32, 16, 32, 4, 8
    rp, ci, fl = oracle.neighborhood_layout(T, (R, C), (th, tw), (8, 16), (8, 16))
    nB = (T + R * C) // (th * tw)
    assert np.all(fl == 0)
    tb = T // (th * tw)
    counts = np.diff(rp)
    assert np.all(counts[:tb] == nB) and np.all(counts[tb:] == tb + 2 * 2)


@pytest.mark.parametrize("window,stride", [((8, 16), (8, 16)), ((5, 9), (1, 1)), ((8, 12), (4, 4))])
def test_block_sparse_forward_on_the_layout_matches(window, stride):
    """The block layout (flags ignored) in tile-major order keeps every pair
    the neighbourhood mask keeps; where every kept block pair is full the
    block-sparse forward on the permuted inputs equals the neighbourhood
    forward, and otherwise it sees a superset of keys."""
    T, R, C, th, tw, D = 32, 16, 32, 4, 8, 16
    N = T + R * C
    q, k, v = _geom_inputs(1, 1, T, R, C, D, 9)
    perm = oracle.tile_permutation(T, (R, C), (th, tw))
    rp, ci, fl = oracle.neighborhood_layout(T, (R, C), (th, tw), window, stride)
    On, Ln = oracle.forward_neighborhood(q, k, v, T, (R, C), window, stride)
    qp, kp, vp = (np.ascontiguousarray(a[:, :, perm]) for a in (q, k, v))
    Ob, Lb = oracle.forward(qp, kp, vp, th * tw, rp, ci)
    if np.all(fl == 0):
        np.testing.assert_allclose(Ob, On[:, :, perm], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(Lb, Ln[:, :, perm], rtol=1e-12, atol=1e-12)
    else:
        assert np.all(Lb >= Ln[:, :, perm] - 1e-12)        # more keys: LSE cannot drop
        assert np.any(Lb > Ln[:, :, perm] + 1e-6)
