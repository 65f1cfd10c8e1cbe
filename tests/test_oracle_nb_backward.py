"""Pins for the oracle's backward of 2-D neighbourhood attention (GNA
notes, 1.1), natural token order.

  * Central differences of L = sum(O * G) through the oracle's own fp64
    neighbourhood forward, on sampled entries of Q, K and V.
  * Blocked attention (window = stride, a whole number of tiles per axis)
    keeps whole tiles only: the gradient must equal the block-sparse
    backward on the tile-major tokens with the block layout the oracle
    derives by brute force.
  * The fp64 forward agrees with the bf16-input neighbourhood forward.
"""
import numpy as np
import pytest

import oracle
from synth import bf16_to_f32, random_qkv

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _f64(u16):
    return bf16_to_f32(u16).astype(np.float64)


@pytest.mark.parametrize("T,grid,window,stride", [(4, (6, 8), (3, 5), (1, 1)), (0, (5, 7), (4, 3), (2, 3)),
                                                  (2, (4, 4), (4, 2), (1, 2))])
def test_gradient_is_the_central_difference(T, grid, window, stride):
    B, H, D = 1, 2, 8
    N = T + grid[0] * grid[1]
    rng = np.random.default_rng(1000 + N)
    q, k, v = (rng.standard_normal((B, H, N, D)) for _ in range(3))
    G = rng.standard_normal((B, H, N, D))
    dQ, dK, dV = oracle.backward_neighborhood(q, k, v, G, T, grid, window, stride)
    h = 1e-6

    def loss(qq, kk, vv):
        O, _ = oracle.forward_neighborhood_f64(qq, kk, vv, T, grid, window, stride)
        return float(np.sum(O * G))

    for which, grad in ((0, dQ), (1, dK), (2, dV)):
        for _ in range(12):
            idx = (0, int(rng.integers(H)), int(rng.integers(N)), int(rng.integers(D)))
            xs = [q.copy(), k.copy(), v.copy()]
            xs[which][idx] += h
            lp = loss(*xs)
            xs[which][idx] -= 2 * h
            lm = loss(*xs)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * (1 + abs(fd)), (which, idx, fd, grad[idx])


def test_blocked_window_equals_block_sparse_backward():
    # tiles 2 x 4 (block 8), window = stride = (2, 8): each query sees the two
    # whole tiles of its aligned 2 x 8 group, plus the text keys
    T, grid, tile, window = 8, (4, 16), (2, 4), (2, 8)
    B, H, D = 1, 2, 8
    N = T + grid[0] * grid[1]
    q, k, v = random_qkv(B, H, N, D, seed=1101)
    G = random_qkv(B, H, N, D, seed=1102)[0]
    want = oracle.backward_neighborhood(q, k, v, G, T, grid, window, window)
    perm = oracle.tile_permutation(T, grid, tile)
    rp, ci, flags = oracle.neighborhood_layout(T, grid, tile, window, window)
    assert np.all(flags == 0)                                      # whole tiles only
    nB = N // 8
    rp_all = np.concatenate([rp[:-1] + h * rp[-1] for h in range(B * H)] + [[B * H * rp[-1]]]).astype(np.int32)
    ci_all = np.tile(ci, B * H)
    got = oracle.backward(*(x[:, :, perm] for x in (q, k, v, G)), 8, rp_all, ci_all)
    inv = np.argsort(perm)
    for a, b in zip(got, want):
        np.testing.assert_allclose(a[:, :, inv], b, rtol=1e-12, atol=1e-12)
    assert rp_all.shape == (B * H * nB + 1,)


def test_fp64_forward_matches_bf16_input_forward():
    T, grid, window, stride = 3, (5, 6), (3, 3), (2, 1)
    N = T + 30
    q, k, v = random_qkv(1, 2, N, 16, seed=1111)
    O1, L1 = oracle.forward_neighborhood(q, k, v, T, grid, window, stride)
    O2, L2 = oracle.forward_neighborhood_f64(_f64(q), _f64(k), _f64(v), T, grid, window, stride)
    np.testing.assert_allclose(O2, O1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L2, L1, rtol=1e-12, atol=1e-13)


def test_token_mask_changes_the_gradient():
    # the sliding-window case of the GPU parity tests: the block-sparse
    # gradient over the same blocks without the token mask misses the masked
    # gradient by far more than the GPU tolerance (2e-2 of the largest
    # element), so that parity holds only if the kernels mask
    T, grid, tile, window, stride, D = 128, (16, 32), (8, 16), (5, 9), (1, 1), 64
    B, H = 1, 2
    N = T + grid[0] * grid[1]
    q, k, v = random_qkv(B, H, N, D, seed=1201)
    g = random_qkv(B, H, N, D, seed=1202)[0]
    want = oracle.backward_neighborhood(q, k, v, g, T, grid, window, stride)
    perm = oracle.tile_permutation(T, grid, tile)
    rp, ci, flags = oracle.neighborhood_layout(T, grid, tile, window, stride)
    assert flags.mean() > 0.5
    rp_all = np.concatenate([rp[:-1] + h * rp[-1] for h in range(B * H)] + [[B * H * rp[-1]]]).astype(np.int32)
    got = oracle.backward(*(x[:, :, perm] for x in (q, k, v, g)), 128, rp_all, np.tile(ci, B * H))
    inv = np.argsort(perm)
    for a, b in zip(got, want):
        assert np.abs(a[:, :, inv] - b).max() > 0.2 * np.abs(b).max()


def test_dq_rows_are_the_full_gradient_rows():
    T, grid, window, stride = 4, (6, 8), (3, 5), (1, 2)
    N = T + grid[0] * grid[1]
    q, k, v = random_qkv(1, 2, N, 8, seed=1401)
    g = random_qkv(1, 2, N, 8, seed=1402)[0]
    dq, _, _ = oracle.backward_neighborhood(q, k, v, g, T, grid, window, stride)
    rows = np.array([0, 3, 4, 30, N - 1, N, 2 * N - 1])
    got = oracle.backward_neighborhood_dq_rows(q, k, v, g, T, grid, window, stride, rows)
    np.testing.assert_array_equal(got, dq.reshape(-1, 8)[rows])


def test_fp64_forward_rows_are_the_full_forward_rows():
    T, grid, window, stride = 4, (6, 8), (3, 5), (2, 1)
    N = T + grid[0] * grid[1]
    rng = np.random.default_rng(1501)
    q, k, v = (rng.standard_normal((1, 2, N, 8)) for _ in range(3))
    O, L = oracle.forward_neighborhood_f64(q, k, v, T, grid, window, stride)
    rows = np.array([0, 3, 4, 30, N - 1, N, 2 * N - 1])
    Or, Lr = oracle.forward_neighborhood_f64(q, k, v, T, grid, window, stride, rows=rows)
    np.testing.assert_array_equal(Or, O.reshape(-1, 8)[rows])
    np.testing.assert_array_equal(Lr, L.reshape(-1)[rows])
