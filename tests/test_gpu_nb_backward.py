"""GPU parity of the backward of 2-D neighbourhood (GNA) attention against the
fp64 oracle gradient under the token mask.

Natural-order inputs are permuted to tile-major order on the GPU, the
forward and the backward run there (the partially covered entries masked
per token in both backward kernels), and dQ, dK, dV are permuted back.
Tolerances as for the block-sparse backward (tests/test_gpu_backward.py):
max 2e-2 of each gradient's largest element, mean 1e-2 of its mean
magnitude (bf16 P, dS, O and gradients)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import block_sparse_attention_18_amd as bsa
from helpers import bf16_bits, bf16_to_f64, dev, to_dev_bf16

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

MAX_REL = 2e-2
MEAN_REL = 1e-2


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check_grad(g, want, name):
    d = np.abs(g - want)
    mx = float(d.max()) / max(float(np.abs(want).max()), 1e-30)
    mean = float(d.mean()) / max(float(np.abs(want).mean()), 1e-30)
    _log(f"  {name}: max {mx:.2e} of max|g|, mean {mean:.2e} of mean|g|")
    assert mx <= MAX_REL and mean <= MEAN_REL, name


def _backward_natural(q, k, v, g, nb):
    B, H, N, D = q.shape
    qd, kd, vd, gd = (bsa.permute_tokens(to_dev_bf16(a), nb) for a in (q, k, v, g))
    rp, ci, fl = bsa.build_neighborhood_layout(B, H, nb, device=dev())
    Op, Lp = bsa.forward_neighborhood(qd, kd, vd, rp, ci, fl, nb)
    dq, dk, dv = bsa.backward_neighborhood(qd, kd, vd, Op, gd, rp, ci, fl, nb, Lp)
    out = [bsa.permute_tokens(x, nb, inverse=True) for x in (dq, dk, dv)]
    torch.cuda.synchronize()
    return out, fl


GEOMS = [
    # T, grid, tile, window, stride, D
    (128, (16, 32), (8, 16), (5, 9), (1, 1), 64),          # sliding window, mostly partial tiles
    (0, (32, 32), (8, 16), (16, 32), (16, 32), 128),       # stride = window: no partial tile
    (64, (16, 24), (8, 8), (8, 12), (4, 4), 64),           # block 64, a stride between
    (256, (32, 64), (8, 16), (12, 20), (2, 3), 128),       # uneven strides, window not a tile multiple
    (128, (8, 16), (8, 16), (8, 16), (1, 1), 64),          # window = whole grid: dense
    (64, (24, 16), (8, 8), (3, 16), (1, 1), 128),          # block 64 at D 128, window spanning whole rows
    (0, (8, 256), (1, 128), (3, 40), (1, 1), 128),         # one-row tiles 128 wide
    (128, (16, 128), (2, 64), (5, 70), (1, 2), 64),        # tiles 64 wide, window wider than a tile
    (64, (8, 128), (1, 64), (3, 20), (2, 1), 128),         # block 64, one-row tiles 64 wide
    (128, (16, 64), (4, 32), (6, 20), (1, 1), 128),        # tiles 32 wide
]


@pytest.mark.parametrize("T,grid,tile,window,stride,D", GEOMS)
def test_backward_matches_oracle(T, grid, tile, window, stride, D):
    _log(f"nb backward T={T} grid={grid} tile={tile} window={window} stride={stride} D={D}")
    B, H = 1, 2
    N = T + grid[0] * grid[1]
    nb = bsa.neighborhood(T, grid, tile, window, stride)
    q, k, v = synth.random_qkv(B, H, N, D, seed=1201)
    g = synth.random_qkv(B, H, N, D, seed=1202)[0]
    (dq, dk, dv), fl = _backward_natural(q, k, v, g, nb)
    wq, wk, wv = oracle.backward_neighborhood(q, k, v, g, T, grid, window, stride)
    _check_grad(bf16_to_f64(dq), wq, "dQ")
    _check_grad(bf16_to_f64(dk), wk, "dK")
    _check_grad(bf16_to_f64(dv), wv, "dV")
    if window == stride:
        assert int(fl.sum().item()) == 0


def test_backward_peaked_logits_and_determinism():
    # logits of sigma 3 (sharper rows) and two calls agreeing bit for bit
    T, grid, tile, window, stride, D = 128, (16, 32), (8, 16), (7, 11), (1, 2), 128
    B, H = 1, 2
    N = T + grid[0] * grid[1]
    nb = bsa.neighborhood(T, grid, tile, window, stride)
    q, k, _ = synth.random_qkv(B, H, N, D, seed=1211, scale=3.0)
    v = synth.random_qkv(B, H, N, D, seed=1212)[2]
    g = synth.random_qkv(B, H, N, D, seed=1213)[0]
    a, _ = _backward_natural(q, k, v, g, nb)
    b, _ = _backward_natural(q, k, v, g, nb)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(bf16_bits(x), bf16_bits(y))
    wq, wk, wv = oracle.backward_neighborhood(q, k, v, g, T, grid, window, stride)
    _check_grad(bf16_to_f64(a[0]), wq, "dQ")
    _check_grad(bf16_to_f64(a[1]), wk, "dK")
    _check_grad(bf16_to_f64(a[2]), wv, "dV")


@pytest.mark.parametrize("stride", [(1, 1), (32, 32)])
def test_backward_full_g1_workload_sampled_rows_and_sums(stride):
    """The full 2-D neighbourhood workload G1 (FLUX 2048², 24 heads, window
    32 x 32, tiles 8 x 16) as bench.py runs it (natural-order tensors): sampled dQ rows against the
    oracle row by row, and the column-sum identities of dK (zero) and dV (the
    sum of dO), bounded as for the 2K arrow workload (2e-3 of the sum of
    magnitudes)."""
    wl = synth.WORKLOADS["G1"]
    x = synth.make_inputs(wl)
    B, H, N, D = wl.B, wl.H, wl.N, wl.D
    T = wl.text_len
    nb = bsa.neighborhood(T, wl.nb_grid, wl.nb_tile, wl.nb_window, stride)
    g = synth.random_qkv(B, H, N, D, seed=1220)[0]
    _log(f"nb backward full G1 stride {stride}")
    # natural-order forward and backward, as bench.py --backward runs them
    qd, kd, vd, gd = (to_dev_bf16(a) for a in (x["q"], x["k"], x["v"], g))
    rp, ci, fl = bsa.build_neighborhood_layout(B, H, nb, device=dev())
    O, L = bsa.forward_neighborhood(qd, kd, vd, rp, ci, fl, nb, natural=True)
    dq, dk, dv = bsa.backward_neighborhood(qd, kd, vd, O, gd, rp, ci, fl, nb, L, natural=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1221)
    rows = np.concatenate([[0, T - 1, T, T + 127, N - 1, (H - 1) * N + T + 5000],
                           rng.integers(0, H, 42) * N + rng.integers(0, N, 42)]).astype(np.int64)
    want = oracle.backward_neighborhood_dq_rows(x["q"], x["k"], x["v"], g, T, wl.nb_grid, wl.nb_window, stride,
                                                rows)
    _check_grad(bf16_to_f64(dq).reshape(-1, D)[rows], want, "dQ rows")
    gk, gv = bf16_to_f64(dk), bf16_to_f64(dv)
    go = synth.bf16_to_f32(g).astype(np.float64)
    dk_sum = np.abs(gk.sum(axis=2)) / np.abs(gk).sum(axis=2)
    dv_err = np.abs(gv.sum(axis=2) - go.sum(axis=2)) / np.abs(gv).sum(axis=2)
    _log(f"  sum dK / sum |dK|: max {dk_sum.max():.2e}; |sum dV - sum dO| / sum |dV|: max {dv_err.max():.2e}")
    assert dk_sum.max() <= 2e-3 and dv_err.max() <= 2e-3


def test_backward_full_g1_workload_is_deterministic():
    """The full G1 natural-order backward three times on the same inputs:
    the gradients agree bit for bit.  (Each tile copy must have landed in LDS
    before the barrier that hands the tile to the other waves; a missing
    wait there once left dQ rows differing from run to run at this size.)"""
    wl = synth.WORKLOADS["G1"]
    x = synth.make_inputs(wl)
    B, H, N, D = wl.B, wl.H, wl.N, wl.D
    nb = bsa.neighborhood(wl.text_len, wl.nb_grid, wl.nb_tile, wl.nb_window, wl.nb_stride)
    g = synth.random_qkv(B, H, N, D, seed=1225)[0]
    _log("nb backward full G1: determinism over three runs")
    qd, kd, vd, gd = (to_dev_bf16(a) for a in (x["q"], x["k"], x["v"], g))
    rp, ci, fl = bsa.build_neighborhood_layout(B, H, nb, device=dev())
    O, L = bsa.forward_neighborhood(qd, kd, vd, rp, ci, fl, nb, natural=True)
    runs = []
    for _ in range(3):
        got = bsa.backward_neighborhood(qd, kd, vd, O, gd, rp, ci, fl, nb, L, natural=True)
        torch.cuda.synchronize()
        runs.append([bf16_bits(t) for t in got])
    for r in (1, 2):
        for name, a, b in zip(("dQ", "dK", "dV"), runs[0], runs[r]):
            np.testing.assert_array_equal(a, b, err_msg=f"{name}, run {r} against run 0")


@pytest.mark.parametrize("T,grid,tile,window,stride,D", GEOMS)
def test_natural_order_backward_equals_the_permuted_path(T, grid, tile, window, stride, D):
    """bsa_backward_neighborhood_natural takes natural-order Q, K, V, O, dO and
    LSE (those of the natural-order forward) and writes natural-order dQ, dK,
    dV: the same arithmetic on the same tiles as the tile-major backward, so
    the gradients equal its permuted-back ones bit for bit."""
    _log(f"nb backward natural T={T} grid={grid} tile={tile} window={window} stride={stride} D={D}")
    B, H = 1, 2
    N = T + grid[0] * grid[1]
    nb = bsa.neighborhood(T, grid, tile, window, stride)
    q, k, v = synth.random_qkv(B, H, N, D, seed=1231)
    g = synth.random_qkv(B, H, N, D, seed=1232)[0]
    want, _ = _backward_natural(q, k, v, g, nb)
    qd, kd, vd, gd = (to_dev_bf16(a) for a in (q, k, v, g))
    rp, ci, fl = bsa.build_neighborhood_layout(B, H, nb, device=dev())
    O, L = bsa.forward_neighborhood(qd, kd, vd, rp, ci, fl, nb, natural=True)
    got = bsa.backward_neighborhood(qd, kd, vd, O, gd, rp, ci, fl, nb, L, natural=True)
    torch.cuda.synchronize()
    for name, x, y in zip(("dQ", "dK", "dV"), got, want):
        np.testing.assert_array_equal(bf16_bits(x), bf16_bits(y), err_msg=name)
