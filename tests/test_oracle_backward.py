"""Pins of the backward oracle: finite differences of the fp64 forward,
torch autograd (float64, CPU) on dense masked attention, and the closed-form
sums of dV and dK."""
import numpy as np
import pytest
import torch

import oracle
import synth


def _case(B, H, N, D, block, seed, density=0.6):
    rng = np.random.default_rng(seed)
    q, k, v, g = (rng.standard_normal((B, H, N, D)) for _ in range(4))
    nB = -(-N // block)
    rp, ci = synth.random_block_lists(B, H, nB, seed=seed + 1, density=density, empty_rows=1, full_rows=1)
    return q, k, v, g, rp, ci


def test_backward_matches_finite_differences():
    B, H, N, D, block = 1, 2, 13, 4, 4          # ragged last block, an empty row
    q, k, v, g, rp, ci = _case(B, H, N, D, block, 601)
    dQ, dK, dV = oracle.backward(q, k, v, g, block, rp, ci, scale=0.7)

    def loss(q_, k_, v_):
        O, _ = oracle.forward_f64(q_, k_, v_, block, rp, ci, scale=0.7)
        return float((O * g).sum())
    eps = 1e-6
    rng = np.random.default_rng(602)
    for name, x, grad in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert grad[idx] == pytest.approx(fd, rel=1e-6, abs=1e-8), (name, idx)


def test_backward_matches_torch_autograd_dense():
    B, H, N, D, block = 2, 2, 24, 8, 8
    q, k, v, g, rp, ci = _case(B, H, N, D, block, 611, density=0.5)
    dQ, dK, dV = oracle.backward(q, k, v, g, block, rp, ci)
    # the same mask at token level, through torch's float64 autograd
    nB = N // block
    mask = np.zeros((B, H, N, N), bool)
    for bh in range(B * H):
        b, h = divmod(bh, H)
        for i in range(nB):
            for e in range(rp[bh * nB + i], rp[bh * nB + i + 1]):
                j = ci[e]
                mask[b, h, i * block:(i + 1) * block, j * block:(j + 1) * block] = True
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    z = (tq @ tk.transpose(-1, -2)) / np.sqrt(D)
    z = z.masked_fill(~torch.tensor(mask), float("-inf"))
    p = torch.softmax(z, dim=-1)
    p = torch.nan_to_num(p, nan=0.0)                     # rows with no kept key
    o = p @ tv
    (o * torch.tensor(g)).sum().backward()
    np.testing.assert_allclose(dQ, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dK, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dV, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_backward_closed_form_sums():
    """Each kept row's probabilities sum to 1, so the dV rows of a head sum to
    the dO rows of its non-empty rows; the dS of a row sums to 0, so the dK
    rows of a head sum to 0."""
    B, H, N, D, block = 1, 3, 40, 8, 8
    q, k, v, g, rp, ci = _case(B, H, N, D, block, 621)
    dQ, dK, dV = oracle.backward(q, k, v, g, block, rp, ci)
    _, L = oracle.forward_f64(q, k, v, block, rp, ci)
    live = np.isfinite(L)[..., None]
    np.testing.assert_allclose(dV.sum(axis=2), (g * live).sum(axis=2), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(dK.sum(axis=2), 0.0, atol=1e-10)
    assert np.all(dQ[~np.isfinite(L)] == 0.0)


def test_forward_f64_matches_the_bf16_oracle():
    B, H, N, D, block = 1, 2, 70, 16, 32
    q, k, v = synth.random_qkv(B, H, N, D, seed=631)
    rp, ci = synth.random_block_lists(B, H, 3, seed=632, density=0.6)
    O, L = oracle.forward(q, k, v, block, rp, ci)
    O2, L2 = oracle.forward_f64(q, k, v, block, rp, ci)
    np.testing.assert_allclose(O2, O, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L2[np.isfinite(L)], L[np.isfinite(L)], rtol=1e-12)


def test_dq_rows_are_the_full_gradient_rows():
    # the per-row dQ (for full-size checks) is the full backward's dQ,
    # including an empty row and the ragged last block
    q, k, v = synth.random_qkv(2, 2, 200, 16, seed=3)
    g = synth.random_qkv(2, 2, 200, 16, seed=4)[0]
    rp, ci = synth.random_block_lists(2, 2, 4, seed=5, density=0.5, empty_rows=1)
    dq, _, _ = oracle.backward(q, k, v, g, 64, rp, ci)
    rows = np.array([0, 5, 63, 64, 199, 200, 401, 799])
    got = oracle.backward_dq_rows(q, k, v, g, 64, rp, ci, rows)
    np.testing.assert_array_equal(got, dq.reshape(-1, 16)[rows])
