"""GPU parity of 2-D neighbourhood (GNA) attention: the tile-major
permutation (bit-exact), the block layout and flags (bit-exact against the
oracle's brute-force layout) and the forward on natural-order inputs
(permute, forward, permute back) against the oracle's masked softmax."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import block_sparse_attention_18_amd as bsa
from helpers import bf16_bits, bf16_to_f64, check_forward, dev, sample_rows, to_dev_bf16

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


GEOMS = [
    # T, grid, tile, window, stride, D
    (128, (16, 32), (8, 16), (5, 9), (1, 1), 64),          # sliding window, mostly partial tiles
    (0, (32, 32), (8, 16), (16, 32), (16, 32), 128),       # stride = window: perfectly block-sparse
    (64, (16, 24), (8, 8), (8, 12), (4, 4), 64),           # block 64, a stride between
    (256, (32, 64), (8, 16), (12, 20), (2, 3), 128),       # uneven strides, window not a tile multiple
    (128, (8, 16), (8, 16), (8, 16), (1, 1), 64),          # window = whole grid: dense
    (0, (8, 256), (1, 128), (3, 40), (1, 1), 128),         # one-row tiles 128 wide
    (128, (16, 128), (2, 64), (5, 70), (1, 2), 64),        # tiles 64 wide, window wider than a tile
    (64, (8, 128), (1, 64), (3, 20), (2, 1), 128),         # block 64, one-row tiles 64 wide
    (128, (16, 64), (4, 32), (6, 20), (1, 1), 128),        # tiles 32 wide
]


@pytest.mark.parametrize("T,grid,tile,window,stride,D", GEOMS)
def test_permutation_and_layout_bit_exact(T, grid, tile, window, stride, D):
    _log(f"permute/layout T={T} grid={grid} tile={tile} window={window} stride={stride}")
    B, H = 2, 2
    N = T + grid[0] * grid[1]
    nb = bsa.neighborhood(T, grid, tile, window, stride)
    x = synth.random_qkv(B, H, N, D, seed=501)[0]
    lse = np.random.default_rng(502).standard_normal((B, H, N)).astype(np.float32)
    perm = oracle.tile_permutation(T, grid, tile)
    xd, ld = to_dev_bf16(x), torch.from_numpy(lse).to(dev())
    y, ly = bsa.permute_tokens(xd, nb, lse=ld)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_bits(y), x[:, :, perm])
    np.testing.assert_array_equal(ly.cpu().numpy(), lse[:, :, perm])
    z, lz = bsa.permute_tokens(y, nb, inverse=True, lse=ly)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_bits(z), x)
    np.testing.assert_array_equal(lz.cpu().numpy(), lse)
    rp, ci, fl = bsa.build_neighborhood_layout(B, H, nb, device=dev())
    torch.cuda.synchronize()
    rpo, cio, flo = oracle.neighborhood_layout(T, grid, tile, window, stride)
    nnz = int(rpo[-1])
    nB = len(rpo) - 1
    want_rp = np.concatenate([[0]] + [rpo[1:] + h * nnz for h in range(B * H)])
    np.testing.assert_array_equal(rp.cpu().numpy(), want_rp)
    np.testing.assert_array_equal(ci.cpu().numpy()[:B * H * nnz], np.tile(cio, B * H))
    np.testing.assert_array_equal(fl.cpu().numpy()[:B * H * nnz], np.tile(flo.astype(np.int32), B * H))
    assert nB == N // (tile[0] * tile[1])


def _forward_natural(q, k, v, nb, split=None):
    B, H, N, D = q.shape
    qd, kd, vd = (bsa.permute_tokens(to_dev_bf16(a), nb) for a in (q, k, v))
    rp, ci, fl = bsa.build_neighborhood_layout(B, H, nb, device=dev())
    Op, Lp = bsa.forward_neighborhood(qd, kd, vd, rp, ci, fl, nb, split=split)
    O, L = bsa.permute_tokens(Op, nb, inverse=True, lse=Lp)
    torch.cuda.synchronize()
    return O, L


@pytest.mark.parametrize("T,grid,tile,window,stride,D", GEOMS)
def test_forward_matches_oracle(T, grid, tile, window, stride, D):
    _log(f"forward T={T} grid={grid} tile={tile} window={window} stride={stride} D={D}")
    B, H = 1, 2
    N = T + grid[0] * grid[1]
    nb = bsa.neighborhood(T, grid, tile, window, stride)
    q, k, v = synth.random_qkv(B, H, N, D, seed=511)
    O, L = _forward_natural(q, k, v, nb)
    Oo, Lo = oracle.forward_neighborhood(q, k, v, T, grid, window, stride)
    check_forward(bf16_to_f64(O), L.cpu().numpy().astype(np.float64), Oo, Lo, "neighbourhood")


def test_forward_split_rows_and_large_logits():
    """Long text rows split over several workgroups, and logits of sigma 3 (the
    row max of a partial tile is taken over all of its keys)."""
    T, grid, tile, window, stride, D = 256, (32, 32), (8, 16), (7, 11), (1, 1), 128
    B, H = 1, 3
    N = T + grid[0] * grid[1]
    nb = bsa.neighborhood(T, grid, tile, window, stride)
    q, k, _ = synth.random_qkv(B, H, N, D, seed=521, scale=3.0)
    v = synth.random_qkv(B, H, N, D, seed=522)[2]
    split = {"chunk_blocks": 3, "max_chunks": 4, "max_split_rows": 64}
    O, L = _forward_natural(q, k, v, nb, split=split)
    Oo, Lo = oracle.forward_neighborhood(q, k, v, T, grid, window, stride)
    check_forward(bf16_to_f64(O), L.cpu().numpy().astype(np.float64), Oo, Lo, "neighbourhood split")


@pytest.mark.slow
@pytest.mark.parametrize("stride", [(1, 1), (16, 16), (32, 32)])
def test_workload_g1(stride):
    """The full G1 workload in the launch configuration bench.py times: the
    natural-order forward with the long-row split the bench takes from the
    geometry (rows whole at stride 1, split at stride 32)."""
    wl = synth.WORKLOADS["G1"]
    x = synth.make_inputs(wl)
    B, H, N, D = wl.B, wl.H, wl.N, wl.D
    nb = bsa.neighborhood(wl.text_len, wl.nb_grid, wl.nb_tile, wl.nb_window, stride)
    rp, ci, fl = bsa.build_neighborhood_layout(B, H, nb, device=dev())
    split = bsa.neighborhood_split_policy(B, H, nb, wl.block)
    _log(f"G1 stride {stride}: split {split}")
    O, L = bsa.forward_neighborhood(*(to_dev_bf16(a) for a in (x["q"], x["k"], x["v"])), rp, ci, fl, nb,
                                    split=split, natural=True)
    torch.cuda.synchronize()
    must = [((0 * H + h) * N + t) for h in (0, H - 1) for t in (0, 511, 512, 600, N // 2, N - 1)]
    rows = sample_rows(B, H, N, 256, 530, must)
    Oo, Lo = oracle.forward_neighborhood(x["q"], x["k"], x["v"], wl.text_len, wl.nb_grid, wl.nb_window, stride,
                                         rows=rows)
    Og = bf16_to_f64(O).reshape(-1, D)[rows]
    Lg = L.cpu().numpy().reshape(-1)[rows].astype(np.float64)
    mx, mean = check_forward(Og, Lg, Oo, Lo, f"G1 stride {stride}")
    _log(f"G1 stride {stride}: {len(rows)} rows, max|dO|={mx:.2e} mean|dO|={mean:.2e}")


@pytest.mark.parametrize("T,grid,tile,window,stride,D", GEOMS)
@pytest.mark.parametrize("split", [False, True])
def test_natural_order_forward_equals_the_permuted_path(T, grid, tile, window, stride, D, split):
    """bsa_forward_neighborhood_natural gathers the tiles from natural-order
    Q, K, V and scatters O, LSE itself: the same arithmetic on the same tiles
    as permute -> forward -> permute back, so the results agree bit for bit
    (with long rows split as well)."""
    _log(f"natural T={T} grid={grid} tile={tile} window={window} stride={stride} D={D} split={split}")
    B, H = 1, 2
    N = T + grid[0] * grid[1]
    nb = bsa.neighborhood(T, grid, tile, window, stride)
    q, k, v = synth.random_qkv(B, H, N, D, seed=541)
    sp = {"chunk_blocks": 2, "max_chunks": 4, "max_split_rows": 64} if split else None
    O1, L1 = _forward_natural(q, k, v, nb, split=dict(sp) if sp else None)
    rp, ci, fl = bsa.build_neighborhood_layout(B, H, nb, device=dev())
    O2, L2 = bsa.forward_neighborhood(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), rp, ci, fl, nb,
                                      split=dict(sp) if sp else None, natural=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_bits(O2), bf16_bits(O1))
    np.testing.assert_array_equal(L2.cpu().numpy(), L1.cpu().numpy())
    Oo, Lo = oracle.forward_neighborhood(q, k, v, T, grid, window, stride)
    check_forward(bf16_to_f64(O2), L2.cpu().numpy().astype(np.float64), Oo, Lo, "natural")
