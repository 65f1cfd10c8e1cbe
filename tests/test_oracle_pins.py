"""Pins for the fp64 CPU oracle.

The oracle is the yardstick for the GPU path, so it is itself checked
against things other than its own formulas: closed forms, invariants that
the pages' definitions imply, brute force on tiny inputs, and independent
library routines (torch's CPU scaled_dot_product_attention in float64,
Python's sorted).  Each case is chosen so that a plausible slip (a dropped
term, a wrong sign or index, a transposed operand, a wrong divisor) fails.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from synth import bf16_to_f32, f32_to_bf16, random_qkv, random_block_lists, random_scores

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _bf(x):
    return f32_to_bf16(np.asarray(x, dtype=np.float32))


def _f64(u16):
    return bf16_to_f32(u16).astype(np.float64)


def _csr_to_mask(row_ptr, col_idx, B, H, nB):
    m = np.zeros((B, H, nB, nB), dtype=bool)
    for r in range(B * H * nB):
        b, h, i = r // (H * nB), (r // nB) % H, r % nB
        m[b, h, i, col_idx[row_ptr[r]:row_ptr[r + 1]]] = True
    return m


def _token_mask(block_mask, N, block):
    """Expand a [.., nB, nB] block mask to [.., N, N]."""
    idx = np.arange(N) // block
    return block_mask[..., idx[:, None], idx[None, :]]


# ---------------------------------------------------------------------------
# pooling and projected scores (block-sparse DiT write-up, 2.2)
# ---------------------------------------------------------------------------
def test_pool_constant_blocks_and_ragged_tail():
    # block i holds the constant vector c_i; the last block is partial
    B, H, D, block = 1, 2, 8, 4
    N = 3 * block + 3
    rng = np.random.default_rng(0)
    consts = rng.integers(-8, 9, size=(B, H, 4, D)).astype(np.float32) / 4
    x = np.repeat(consts, block, axis=2)[:, :, :N]
    out = oracle.pool_mean(_bf(x), block)
    assert out.shape == (B, H, 4, D)
    np.testing.assert_array_equal(out, consts.astype(np.float64))
    # a partial block of distinct values averages over the tokens it holds
    x2 = np.zeros((1, 1, 6, 1), np.float32)
    x2[0, 0, 4:, 0] = [1.0, 2.0]
    x2[0, 0, :4, 0] = [1.0, 2.0, 3.0, 6.0]
    out2 = oracle.pool_mean(_bf(x2), 4)
    np.testing.assert_array_equal(out2[0, 0, :, 0], [3.0, 1.5])


@pytest.mark.parametrize("N,block", [(32, 8), (35, 8)])
def test_identity_projection_equals_avgpool_of_logits(N, block):
    # bilinearity: mean_{t in i, s in j} Q_t . K_s = qbar_i . kbar_j, so with
    # W = I the score is the block average of the raw logit matrix
    B, H, D = 2, 2, 16
    q, k, _ = random_qkv(B, H, N, D, seed=11)
    S = oracle.scores_meanpool_proj(q, k, block, np.eye(D, dtype=np.float32))
    Z = np.einsum("bhtd,bhsd->bhts", _f64(q), _f64(k))
    nB = -(-N // block)
    ref = np.zeros((B, H, nB, nB))
    for i in range(nB):
        for j in range(nB):
            ref[:, :, i, j] = Z[:, :, i * block:(i + 1) * block, j * block:(j + 1) * block].mean(axis=(2, 3))
    np.testing.assert_allclose(S, ref, rtol=1e-12, atol=1e-12)


def test_projection_orientation_and_columns():
    # W has two nonzero columns: e_3 and 2*e_10 -> S_ij = a_i[3] b_j[3] + 4 a_i[10] b_j[10]
    B, H, D, block, nb = 1, 1, 16, 4, 5
    rng = np.random.default_rng(1)
    a = rng.integers(-8, 9, size=(nb, D)).astype(np.float32) / 8
    bb = rng.integers(-8, 9, size=(nb, D)).astype(np.float32) / 8
    q = _bf(np.repeat(a, block, axis=0)[None, None])
    k = _bf(np.repeat(bb, block, axis=0)[None, None])
    w = np.zeros((D, 2), np.float32)
    w[3, 0] = 1.0
    w[10, 1] = 2.0
    S = oracle.scores_meanpool_proj(q, k, block, w)[0, 0]
    ref = np.outer(a[:, 3], bb[:, 3]) + 4 * np.outer(a[:, 10], bb[:, 10])
    np.testing.assert_array_equal(S, ref.astype(np.float64))
    # S is not symmetric in general: query blocks index rows, key blocks columns
    assert not np.allclose(S, S.T)


def test_orthogonal_projection_preserves_scores():
    # (W^T q).(W^T k) = q.k for an orthogonal W (Householder reflection)
    B, H, N, D, block = 1, 2, 24, 8, 8
    q, k, _ = random_qkv(B, H, N, D, seed=12)
    u = np.arange(1, D + 1, dtype=np.float64)
    u /= np.linalg.norm(u)
    Wh = (np.eye(D) - 2 * np.outer(u, u)).astype(np.float32)
    S1 = oracle.scores_meanpool_proj(q, k, block, np.eye(D, dtype=np.float32))
    S2 = oracle.scores_meanpool_proj(q, k, block, Wh)
    np.testing.assert_allclose(S1, S2, rtol=1e-5, atol=1e-6)


# ---------------------------------------------------------------------------
# exact block scores (SparseD notes, isolated selection: avgpool of A)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,block", [(64, 16), (70, 16)])
def test_exact_scores_row_mass(N, block):
    # rows of A sum to one, hence sum_j n_j S_ij = 1 for every query block i
    B, H, D = 1, 2, 16
    q, k, _ = random_qkv(B, H, N, D, seed=13)
    S = oracle.scores_exact_avgpool(q, k, block)
    nB = -(-N // block)
    n = np.array([min(block, N - j * block) for j in range(nB)], dtype=np.float64)
    np.testing.assert_allclose((S * n).sum(-1), 1.0, rtol=1e-12)
    assert (S > 0).all()


def test_exact_scores_uniform_when_queries_vanish():
    # Q = 0 -> every logit is 0 -> A uniform 1/N -> every block average is 1/N
    B, H, N, D, block = 1, 1, 40, 8, 8
    _, k, _ = random_qkv(B, H, N, D, seed=14)
    q = np.zeros_like(k)
    S = oracle.scores_exact_avgpool(q, k, block)
    np.testing.assert_allclose(S, 1.0 / N, rtol=1e-14)


def test_exact_scores_match_library_softmax():
    # the same quantity from torch.softmax in float64 (an independent routine)
    B, H, N, D, block = 1, 2, 48, 16, 16
    q, k, _ = random_qkv(B, H, N, D, seed=15)
    S = oracle.scores_exact_avgpool(q, k, block)
    Z = torch.from_numpy(_f64(q)) @ torch.from_numpy(_f64(k)).transpose(-1, -2) / math.sqrt(D)
    A = torch.softmax(Z, dim=-1)
    ref = F.avg_pool2d(A, kernel_size=block).numpy()
    np.testing.assert_allclose(S, ref, rtol=1e-10, atol=1e-14)


def test_exact_scores_key_shift_invariance_and_dominant_key():
    # adding one vector u to every key adds Q_t.u to a whole logit row: A unchanged
    B, H, N, D, block = 1, 1, 32, 8, 8
    rng = np.random.default_rng(2)
    q = rng.integers(-4, 5, size=(B, H, N, D)).astype(np.float32) / 4
    k = rng.integers(-4, 5, size=(B, H, N, D)).astype(np.float32) / 4
    u = rng.integers(-2, 3, size=(D,)).astype(np.float32) / 4
    S1 = oracle.scores_exact_avgpool(_bf(q), _bf(k), block)
    S2 = oracle.scores_exact_avgpool(_bf(q), _bf(k + u), block)
    np.testing.assert_allclose(S1, S2, rtol=1e-12, atol=1e-15)
    # one key aligned with every query dominates: its block takes ~1/block
    q3 = np.tile(np.ones(D, np.float32), (B, H, N, 1))
    k3 = np.zeros((B, H, N, D), np.float32)
    k3[0, 0, 13] = 8.0
    S3 = oracle.scores_exact_avgpool(_bf(q3), _bf(k3), block)[0, 0]
    np.testing.assert_allclose(S3[:, 1], 1.0 / block, rtol=1e-6)
    assert S3[:, [0, 2, 3]].max() < 1e-6


def test_exact_scores_row_subset():
    B, H, N, D, block = 2, 2, 48, 8, 16
    q, k, _ = random_qkv(B, H, N, D, seed=16)
    S = oracle.scores_exact_avgpool(q, k, block)
    rows = [5, 0, 11]
    Sr = oracle.scores_exact_avgpool(q, k, block, rows=rows)
    np.testing.assert_array_equal(Sr, S.reshape(-1, S.shape[-1])[rows])


# ---------------------------------------------------------------------------
# top-k selection (write-up 2.2/2.3, SparseD isolated selection)
# ---------------------------------------------------------------------------
def _brute_select(S, text_blocks, groups):
    B, H, nB, _ = S.shape
    out = []
    for b in range(B):
        for h in range(H):
            for i in range(nB):
                if i < text_blocks:
                    out.append(list(range(nB)))
                    continue
                keep = set(range(min(text_blocks, nB)))
                for (c0, c1, kk) in groups:
                    order = sorted(range(c0, c1), key=lambda j: (-S[b, h, i, j], j))
                    keep.update(order[:kk])
                out.append(sorted(keep))
    return out


@pytest.mark.parametrize("tie_levels", [0, 3])
@pytest.mark.parametrize("groups,text_blocks", [(((0, 8, 4),), 1),
                                                (((2, 12, 3),), 2),
                                                (((0, 9, 3), (9, 12, 2)), 0)])
def test_select_matches_sorted(groups, text_blocks, tie_levels):
    nB = max(c1 for (_, c1, _) in groups)
    S = random_scores(2, 3, nB, seed=17 + tie_levels, tie_levels=tie_levels)
    row_ptr, col_idx = oracle.select(S, text_blocks, groups)
    ref = _brute_select(S.astype(np.float64), text_blocks, groups)
    got = [col_idx[row_ptr[x]:row_ptr[x + 1]].tolist() for x in range(len(ref))]
    assert got == ref


def test_select_ties_lower_index_and_signed_zero():
    # all-equal scores: the lowest columns of every group win; -0.0 ties +0.0
    S = np.zeros((1, 1, 6, 6), np.float32)
    S[0, 0, 3] = [-0.0, 0.0, -0.0, 0.0, -0.0, 0.0]
    row_ptr, col_idx = oracle.select(S, 0, ((0, 6, 2),))
    for x in range(6):
        assert col_idx[row_ptr[x]:row_ptr[x + 1]].tolist() == [0, 1]
    # strictly ordered scores: the largest k win regardless of position
    S2 = np.array([[[[1.0, 5.0, 3.0, 4.0, 2.0]]]], np.float32)
    rp, ci = oracle.select_rows(S2[0, 0], [0], 0, ((0, 5, 2),))
    assert ci.tolist() == [1, 3]


def test_select_nan_scores_rank_last():
    """A NaN score ranks after every number, -inf included; NaNs among
    themselves by lower column (the selection's defined order for scores
    that carry no evidence)."""
    nan, inf = float("nan"), float("inf")
    row = np.array([nan, 2.0, -inf, nan, 0.5, -1.0, nan, 3.0], np.float32)
    order = [7, 1, 4, 5, 2, 0, 3, 6]          # numbers by value, then NaNs by column
    for kk in range(len(row) + 1):
        rp, ci = oracle.select_rows(row[None, :], [0], 0, ((0, 8, kk),))
        assert ci.tolist() == sorted(order[:kk])
    # a row of NaNs only: the lowest columns
    rp, ci = oracle.select_rows(np.full((1, 6), nan, np.float32), [0], 0, ((0, 6, 2),))
    assert ci.tolist() == [0, 1]


def test_select_forced_text_and_counts():
    nB, tb, kk = 10, 3, 4
    S = random_scores(1, 2, nB, seed=18)
    row_ptr, col_idx = oracle.select(S, tb, ((tb, nB, kk),))
    counts = np.diff(row_ptr)
    for x in range(2 * nB):
        cols = col_idx[row_ptr[x]:row_ptr[x + 1]]
        assert np.all(np.diff(cols) > 0)
        if x % nB < tb:
            assert counts[x] == nB
        else:
            # disjoint from the text columns: exactly T_b + k
            assert counts[x] == tb + kk and set(range(tb)) <= set(cols.tolist())
    # k equal to the width keeps everything
    rp, ci = oracle.select(S, 0, ((0, nB, nB),))
    assert np.all(np.diff(rp) == nB)


def test_select_group_union_is_disjoint():
    # SparseD isolated selection: prefill and generation budgets add up
    nB = 16
    S = random_scores(1, 1, nB, seed=19)
    rp, ci = oracle.select(S, 0, ((0, 12, 4), (12, 16, 2)))
    for x in range(nB):
        cols = ci[rp[x]:rp[x + 1]]
        assert len(cols) == 6
        assert (cols < 12).sum() == 4 and (cols >= 12).sum() == 2


# ---------------------------------------------------------------------------
# arrow layout (DiTFastAttnV2 notes, head-wise arrow attention)
# ---------------------------------------------------------------------------
def _arrow_count_closed_form(nB, tb, w):
    n_img = nB - tb
    if w >= n_img - 1:
        return nB * nB
    return tb * nB + n_img * tb + n_img * (2 * w + 1) - w * (w + 1)


@pytest.mark.parametrize("nB,tb,w,expect", [(36, 4, 1, 366), (132, 4, 8, 3144),
                                            (132, 4, 18, 5434), (132, 4, 127, 17424),
                                            (10, 0, 0, 10), (7, 7, 2, 49)])
def test_arrow_count_closed_form(nB, tb, w, expect):
    assert _arrow_count_closed_form(nB, tb, w) == expect
    rp, ci = oracle.arrow(1, 1, nB, tb, np.array([oracle.HEAD_ARROW]), np.array([w]))
    assert rp[-1] == expect


def test_arrow_regions_and_modes():
    B, H, nB, tb, w = 2, 3, 12, 2, 2
    modes = np.array([oracle.HEAD_ARROW, oracle.HEAD_FULL, oracle.HEAD_SKIP], np.int8)
    rp, ci = oracle.arrow(B, H, nB, tb, modes, np.full(H, w, np.int32))
    m = _csr_to_mask(rp, ci, B, H, nB)
    a = m[0, 0]
    # the three regions that involve text are dense
    assert a[:tb, :].all() and a[:, :tb].all()
    # vision-vision region is exactly the band |i - j| <= w
    vv = a[tb:, tb:]
    ii, jj = np.meshgrid(np.arange(nB - tb), np.arange(nB - tb), indexing="ij")
    np.testing.assert_array_equal(vv, np.abs(ii - jj) <= w)
    assert m[:, 1].all()            # FULL
    assert not m[:, 2].any()        # SKIP rows are empty
    np.testing.assert_array_equal(m[0], m[1])
    assert rp[-1] == B * (_arrow_count_closed_form(nB, tb, w) + nB * nB)


def test_arrow_sparsity_brackets_page_figure():
    # DiTFastAttnV2 reports attention sparsity 0.68 for FLUX at 2048^2; on the
    # 2048^2 token grid (132 blocks of 128, 4 text blocks) the windows w = 18
    # and w = 19 bracket that figure, while w = 8 is far sparser
    nB, tb = 132, 4
    sp = {w: 1 - _arrow_count_closed_form(nB, tb, w) / nB ** 2 for w in range(0, 64)}
    assert sp[18] > 0.68 > sp[19]
    assert abs(sp[18] - (1 - 5434 / 17424)) < 1e-12
    assert abs(sp[8] - 0.8196) < 1e-4


# ---------------------------------------------------------------------------
# forward: dense softmax restricted to the kept blocks
# ---------------------------------------------------------------------------
def _sdpa_masked(q, k, v, mask_tok, scale):
    """torch CPU float64 attention with a boolean mask; LSE by logsumexp."""
    Q, K, V = (torch.from_numpy(_f64(x)) for x in (q, k, v))
    M = torch.from_numpy(mask_tok)
    O = F.scaled_dot_product_attention(Q, K, V, attn_mask=M, scale=scale)
    Z = (Q @ K.transpose(-1, -2)) * scale
    Z = Z.masked_fill(~M, float("-inf"))
    L = torch.logsumexp(Z, dim=-1)
    return O.numpy(), L.numpy()


@pytest.mark.parametrize("N,block", [(64, 16), (75, 16)])
def test_forward_all_blocks_equals_dense_attention(N, block):
    B, H, D = 2, 2, 16
    q, k, v = random_qkv(B, H, N, D, seed=20)
    nB = -(-N // block)
    rp = np.arange(0, B * H * nB + 1, dtype=np.int32) * nB
    ci = np.tile(np.arange(nB, dtype=np.int32), B * H * nB)
    O, L = oracle.forward(q, k, v, block, rp, ci)
    Od, Ld = _sdpa_masked(q, k, v, np.ones((N, N), bool), 1 / math.sqrt(D))
    np.testing.assert_allclose(O, Od, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(L, Ld, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("N,block", [(96, 16), (90, 16)])
def test_forward_random_block_mask_matches_masked_sdpa(N, block):
    B, H, D = 2, 3, 16
    q, k, v = random_qkv(B, H, N, D, seed=21)
    nB = -(-N // block)
    rp, ci = random_block_lists(B, H, nB, seed=22, density=0.4, empty_rows=0, full_rows=2)
    O, L = oracle.forward(q, k, v, block, rp, ci, scale=0.3)
    tok = _token_mask(_csr_to_mask(rp, ci, B, H, nB), N, block)
    Od, Ld = _sdpa_masked(q, k, v, tok, 0.3)
    np.testing.assert_allclose(O, Od, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(L, Ld, rtol=1e-12, atol=1e-12)


def test_forward_softmax_rows_sum_to_one_and_constant_values():
    B, H, N, D, block = 1, 2, 64, 8, 16
    q, k, _ = random_qkv(B, H, N, D, seed=23)
    nB = N // block
    rp, ci = random_block_lists(B, H, nB, seed=24, density=0.5, empty_rows=0, full_rows=1)
    ones = _bf(np.ones((B, H, N, D), np.float32))
    O, _ = oracle.forward(q, k, ones, block, rp, ci)
    np.testing.assert_allclose(O, 1.0, rtol=1e-13)
    c = np.broadcast_to(np.linspace(-2, 2, D, dtype=np.float32), (B, H, N, D))
    O2, _ = oracle.forward(q, k, _bf(c), block, rp, ci)
    np.testing.assert_allclose(O2, np.broadcast_to(_f64(_bf(c)), O2.shape), rtol=1e-12, atol=1e-13)


def test_forward_ignores_unselected_blocks_and_lse_bounds():
    B, H, N, D, block = 1, 2, 64, 8, 16
    q, k, v = random_qkv(B, H, N, D, seed=25)
    nB = N // block
    rp, ci = random_block_lists(B, H, nB, seed=26, density=0.4, empty_rows=0, full_rows=0)
    O, L = oracle.forward(q, k, v, block, rp, ci)
    mask = _csr_to_mask(rp, ci, B, H, nB)
    # perturb K and V everywhere a query block does not look: only blocks no
    # query block of that head keeps can be changed without touching any row
    k2, v2 = k.copy(), v.copy()
    unused = ~mask.any(axis=2)           # [B,H,nB] key blocks unused by every row
    changed = 0
    for b in range(B):
        for h in range(H):
            for j in np.nonzero(unused[b, h])[0]:
                k2[b, h, j * block:(j + 1) * block] = _bf(np.full((block, D), 7.0))
                v2[b, h, j * block:(j + 1) * block] = _bf(np.full((block, D), -3.0))
                changed += 1
    O2, L2 = oracle.forward(q, k2, v2, block, rp, ci)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(L, L2)
    # max z <= LSE <= max z + ln(#kept keys)
    Z = np.einsum("bhtd,bhsd->bhts", _f64(q), _f64(k)) / math.sqrt(D)
    tok = _token_mask(mask, N, block)
    Zm = np.where(tok, Z, -np.inf)
    zmax = Zm.max(-1)
    nk = tok.sum(-1)
    assert np.all(L >= zmax - 1e-12) and np.all(L <= zmax + np.log(nk) + 1e-12)


def test_forward_single_block_is_dense_attention_over_that_block():
    B, H, N, D, block = 1, 1, 48, 8, 16
    q, k, v = random_qkv(B, H, N, D, seed=27)
    nB = N // block
    # every query block keeps only key block (i + 1) mod nB
    rp = np.arange(nB + 1, dtype=np.int32)
    ci = np.array([(i + 1) % nB for i in range(nB)], np.int32)
    O, L = oracle.forward(q, k, v, block, rp, ci)
    for i in range(nB):
        j = (i + 1) % nB
        sl_q = slice(i * block, (i + 1) * block)
        sl_k = slice(j * block, (j + 1) * block)
        Od, Ld = _sdpa_masked(q[:, :, sl_q], k[:, :, sl_k], v[:, :, sl_k],
                              np.ones((block, block), bool), 1 / math.sqrt(D))
        np.testing.assert_allclose(O[:, :, sl_q], Od, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(L[:, :, sl_q], Ld, rtol=1e-12)


def test_forward_two_token_closed_form():
    # N = 2, block 1, D = 1, both keys kept:
    # O_0 = (e^{z00} v0 + e^{z01} v1) / (e^{z00} + e^{z01}), z = q k scale
    q = _bf(np.array([1.5, -0.5], np.float32).reshape(1, 1, 2, 1))
    k = _bf(np.array([2.0, 0.25], np.float32).reshape(1, 1, 2, 1))
    v = _bf(np.array([3.0, -1.0], np.float32).reshape(1, 1, 2, 1))
    rp = np.array([0, 2, 3], np.int32)
    ci = np.array([0, 1, 1], np.int32)       # row 1 keeps only key 1
    O, L = oracle.forward(q, k, v, 1, rp, ci, scale=1.0)
    z00, z01 = 1.5 * 2.0, 1.5 * 0.25
    o0 = (math.exp(z00) * 3.0 + math.exp(z01) * -1.0) / (math.exp(z00) + math.exp(z01))
    assert O[0, 0, 0, 0] == pytest.approx(o0, rel=1e-15)
    assert L[0, 0, 0] == pytest.approx(math.log(math.exp(z00) + math.exp(z01)), rel=1e-15)
    assert O[0, 0, 1, 0] == -1.0 and L[0, 0, 1] == pytest.approx(-0.5 * 0.25, rel=1e-15)


def test_forward_empty_row_and_skip_heads():
    B, H, N, D, block = 1, 2, 32, 8, 16
    q, k, v = random_qkv(B, H, N, D, seed=28)
    nB = N // block
    rp = np.array([0, 0, 2, 2, 2], np.int32)      # head 0: row 0 empty, row 1 dense
    ci = np.array([0, 1], np.int32)
    cache = _bf(np.random.default_rng(3).standard_normal((B, H, N, D)).astype(np.float32))
    lse_c = np.random.default_rng(4).standard_normal((B, H, N)).astype(np.float32)
    modes = np.array([oracle.HEAD_FULL, oracle.HEAD_SKIP], np.int8)
    O, L = oracle.forward(q, k, v, block, rp, ci, modes=modes, o_cache=cache, lse_cache=lse_c)
    assert np.all(O[0, 0, :block] == 0.0) and np.all(np.isneginf(L[0, 0, :block]))
    np.testing.assert_array_equal(O[0, 1], _f64(cache[0, 1]))
    np.testing.assert_array_equal(L[0, 1], lse_c[0, 1].astype(np.float64))


def test_forward_row_subset_matches_full():
    B, H, N, D, block = 2, 2, 48, 8, 16
    q, k, v = random_qkv(B, H, N, D, seed=29)
    nB = N // block
    rp, ci = random_block_lists(B, H, nB, seed=30)
    O, L = oracle.forward(q, k, v, block, rp, ci)
    rows = [0, 17, 95, 191, 100]
    Or, Lr = oracle.forward(q, k, v, block, rp, ci, rows=rows)
    np.testing.assert_array_equal(Or, O.reshape(-1, D)[rows])
    np.testing.assert_array_equal(Lr, L.reshape(-1)[rows])


def test_forward_rejects_bad_block_lists():
    B, H, N, D, block = 1, 1, 32, 8, 16
    q, k, v = random_qkv(B, H, N, D, seed=31)
    with pytest.raises(ValueError):
        oracle.forward(q, k, v, block, np.array([0, 1, 2], np.int32), np.array([0, 2], np.int32))
