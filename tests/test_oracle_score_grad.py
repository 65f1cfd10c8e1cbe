"""Pins for the oracle's gradient of the projected block score
(block-sparse DiT write-up, 2.2: the projection W is trained jointly with
the model, which needs dL/dW of S_ij = (W^T qbar_i) . (W^T kbar_j)).

The gradient is checked against finite differences of the oracle's own
score function (itself pinned in test_oracle_pins.py), never against a
retyped formula.  L(W) = sum(dS * S(W)) is quadratic in W, so a central
difference with a step that is exact in fp32 is exact up to fp64
rounding; L is linear in each token of Q and of K, so a one-token forward
difference is exact too.  A transposed dS, a dropped query or key term, a
missing 1/n_i or a wrong W orientation all fail here.
"""
import numpy as np
import pytest

import oracle
from synth import f32_to_bf16, bf16_to_f32

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _case(B, H, N, D, r, block, seed):
    rng = np.random.default_rng(seed)
    q = f32_to_bf16(rng.standard_normal((B, H, N, D)).astype(np.float32))
    k = f32_to_bf16(rng.standard_normal((B, H, N, D)).astype(np.float32))
    # W on a 2^-8 grid inside (-2, 2): W +- 2^-4 is exact in fp32
    w = (rng.integers(-511, 512, size=(D, r)) / 256.0).astype(np.float32)
    nB = -(-N // block)
    dS = rng.standard_normal((B, H, nB, nB))
    return q, k, w, dS


def _loss(q, k, w, dS, block):
    return float(np.sum(dS * oracle.scores_meanpool_proj(q, k, block, w)))


@pytest.mark.parametrize("B,H,N,D,r,block,seed", [(2, 2, 37, 8, 3, 8, 801), (1, 3, 16, 6, 1, 4, 802)])
def test_dw_is_the_central_difference(B, H, N, D, r, block, seed):
    q, k, w, dS = _case(B, H, N, D, r, block, seed)
    dW, _, _ = oracle.score_grad(q, k, block, w, dS)
    h = 2.0 ** -4
    fd = np.empty((D, r))
    for d in range(D):
        for m in range(r):
            wp, wm = w.copy(), w.copy()
            wp[d, m] += h
            wm[d, m] -= h
            assert wp[d, m] - w[d, m] == h and w[d, m] - wm[d, m] == h
            fd[d, m] = (_loss(q, k, wp, dS, block) - _loss(q, k, wm, dS, block)) / (2 * h)
    scale = np.abs(fd).max()
    np.testing.assert_allclose(dW, fd, rtol=0, atol=1e-10 * scale)


@pytest.mark.parametrize("side", ["q", "k"])
def test_pooled_gradients_are_token_differences(side):
    # L is linear in every token, and a token of block i moves the pooled
    # mean by delta / n_i: (L(x') - L(x)) * n_i / delta = dL/dbar_i[d]
    B, H, N, D, r, block = 1, 2, 21, 5, 3, 8          # blocks of 8, 8, 5
    q, k, w, dS = _case(B, H, N, D, r, block, 811)
    _, dq, dk = oracle.score_grad(q, k, block, w, dS)
    g = dq if side == "q" else dk
    L0 = _loss(q, k, w, dS, block)
    checked = 0
    for h in range(H):
        for t in (0, 7, 8, 16, 20):                    # first, last of a block; the ragged tail
            for d in range(D):
                x = (q if side == "q" else k).copy()
                v = bf16_to_f32(x[0, h, t, d:d + 1])[0]
                x[0, h, t, d] = f32_to_bf16(np.array([v + 1.0], np.float32))[0]
                delta = float(bf16_to_f32(x[0, h, t, d:d + 1])[0]) - float(v)
                L1 = _loss(x, k, w, dS, block) if side == "q" else _loss(q, x, w, dS, block)
                i = t // block
                n_i = min(block, N - i * block)
                np.testing.assert_allclose((L1 - L0) * n_i / delta, g[0, h, i, d], rtol=1e-9, atol=1e-9)
                checked += 1
    assert checked == H * 5 * D


def test_gradient_is_linear_in_ds_and_zero_for_zero():
    q, k, w, dS = _case(1, 2, 24, 4, 2, 8, 821)
    z = oracle.score_grad(q, k, 8, w, np.zeros_like(dS))
    assert all(np.all(a == 0) for a in z)
    a = oracle.score_grad(q, k, 8, w, dS)
    b = oracle.score_grad(q, k, 8, w, -2.0 * dS)
    for x, y in zip(a, b):
        np.testing.assert_allclose(y, -2.0 * x, rtol=1e-12, atol=1e-12)
