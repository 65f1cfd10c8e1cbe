"""GPU parity: every step of the HIP path against the fp64 CPU oracle.

Small cases span several tiles, ragged tails, empty and full rows, strided
and aliased tensors; the five workloads run at full size with the oracle
evaluated on sampled rows (or whole small parts).  Oracle inputs never come
from the GPU: block lists fed to both sides are built by the oracle or by
the seeded generator."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import block_sparse_attention_18_amd as bsa
from helpers import (bf16_bits, bf16_to_f64, check_csr_valid, check_forward, check_selection,
                     csr_rows, dev, sample_rows, to_dev_bf16)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def _run_forward(q, k, v, block, rp, ci, **kw):
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    O, L = bsa.forward(qd, kd, vd, block, _i32(rp), _i32(ci), **kw)
    torch.cuda.synchronize()
    return O, L


# ---------------------------------------------------------------------------
# forward, small shapes
# ---------------------------------------------------------------------------
FWD_CASES = [
    (2, 3, 4 * 64 + 17, 64, 64, 101),
    (1, 2, 5 * 128 + 3, 128, 128, 102),
    (2, 2, 3 * 128, 64, 128, 103),
    (1, 3, 6 * 64, 128, 64, 104),
    (1, 1, 40, 128, 128, 105),          # a single partial block
    (1, 3, 1, 64, 64, 106),             # one token: rows empty or holding the token itself
]


@pytest.mark.parametrize("B,H,N,D,block,seed", FWD_CASES)
def test_forward_random_block_lists(B, H, N, D, block, seed):
    _log(f"forward B={B} H={H} N={N} D={D} block={block}")
    q, k, v = synth.random_qkv(B, H, N, D, seed=seed)
    nB = -(-N // block)
    rp, ci = synth.random_block_lists(B, H, nB, seed=seed + 1, density=0.5, empty_rows=1, full_rows=2)
    O, L = _run_forward(q, k, v, block, rp, ci)
    Oo, Lo = oracle.forward(q, k, v, block, rp, ci)
    check_forward(bf16_to_f64(O), L.cpu().numpy().astype(np.float64), Oo, Lo, "random")
    # rows of an empty block row are exactly zero with LSE = -inf
    empty = [x for x in range(B * H * nB) if rp[x] == rp[x + 1]]
    for x in empty:
        bh, i = divmod(x, nB)
        b, h = divmod(bh, H)
        t0, t1 = i * block, min(N, (i + 1) * block)
        assert torch.all(O[b, h, t0:t1] == 0)
        assert torch.all(torch.isneginf(L[b, h, t0:t1]))


def test_forward_scale_and_large_logits():
    B, H, N, D, block = 1, 2, 3 * 128, 128, 128
    # large logits (Q, K with sigma 3), unit-scale V as in every workload
    q, k, _ = synth.random_qkv(B, H, N, D, seed=110, scale=3.0)
    _, _, v = synth.random_qkv(B, H, N, D, seed=112)
    nB = N // block
    rp, ci = synth.random_block_lists(B, H, nB, seed=111, density=0.6)
    O, L = _run_forward(q, k, v, block, rp, ci, scale=0.2)
    Oo, Lo = oracle.forward(q, k, v, block, rp, ci, scale=0.2)
    check_forward(bf16_to_f64(O), L.cpu().numpy().astype(np.float64), Oo, Lo, "scale 0.2")


@pytest.mark.parametrize("N", [3 * 128 + 40, 4 * 128])
def test_forward_large_logits_and_large_v(N):
    """Large logits (Q, K of standard deviation 3, scale 0.2) with V of
    standard deviation 3: the O bounds scale with V (relative tolerance).
    Whole blocks and a ragged last block."""
    B, H, D, block = 1, 2, 128, 128
    q, k, _ = synth.random_qkv(B, H, N, D, seed=113, scale=3.0)
    _, _, v = synth.random_qkv(B, H, N, D, seed=114, scale=3.0)
    nB = -(-N // block)
    rp, ci = synth.random_block_lists(B, H, nB, seed=116, density=0.7)
    O, L = _run_forward(q, k, v, block, rp, ci, scale=0.2)
    Oo, Lo = oracle.forward(q, k, v, block, rp, ci, scale=0.2)
    check_forward(bf16_to_f64(O), L.cpu().numpy().astype(np.float64), Oo, Lo, "large V", v_scale=3.0)


# Whole blocks at block 128, D 128 (the shape of the arrow and long-context
# workloads): odd and single-block grids, sparse and mostly empty lists.
WHOLE_CASES = [
    # B, H, nB, density, empty rows, full rows, seed
    (1, 2, 5, 0.5, 1, 2, 300),      # odd number of blocks
    (2, 3, 8, 0.3, 2, 1, 301),      # sparse rows
    (1, 1, 1, 1.0, 0, 1, 302),      # a single block
    (1, 4, 12, 0.8, 3, 3, 303),
    (1, 2, 6, 0.05, 4, 0, 304),     # mostly empty rows
]


@pytest.mark.parametrize("B,H,nB,dens,er,fr,seed", WHOLE_CASES)
def test_forward_whole_blocks(B, H, nB, dens, er, fr, seed):
    N, D, block = nB * 128, 128, 128
    _log(f"whole blocks B={B} H={H} nB={nB} density={dens}")
    q, k, v = synth.random_qkv(B, H, N, D, seed=seed)
    rp, ci = synth.random_block_lists(B, H, nB, seed=seed + 1, density=dens, empty_rows=er, full_rows=fr)
    O, L = _run_forward(q, k, v, block, rp, ci)
    Oo, Lo = oracle.forward(q, k, v, block, rp, ci)
    check_forward(bf16_to_f64(O), L.cpu().numpy().astype(np.float64), Oo, Lo, "whole blocks")
    for x in [x for x in range(B * H * nB) if rp[x] == rp[x + 1]]:
        bh, i = divmod(x, nB)
        b, h = divmod(bh, H)
        assert torch.all(O[b, h, i * block:(i + 1) * block] == 0)
        assert torch.all(torch.isneginf(L[b, h, i * block:(i + 1) * block]))


def test_forward_ignores_out_of_range_columns():
    """Column indices outside [0, nB) are ignored (the ABI's rule): the
    result equals the forward on the list without them."""
    B, H, nB, D, block = 1, 2, 6, 128, 128
    N = nB * block
    q, k, v = synth.random_qkv(B, H, N, D, seed=310)
    rp, ci = synth.random_block_lists(B, H, nB, seed=311, density=0.5, empty_rows=1, full_rows=1)
    rows = csr_rows(rp, ci)
    bad = []
    for x, r in enumerate(rows):     # an invalid index before and after the valid ones
        bad.append(([-3] if x % 2 else []) + r + ([nB + 7] if x % 3 == 0 else []))
    rpb = np.zeros(len(bad) + 1, np.int32)
    rpb[1:] = np.cumsum([len(r) for r in bad])
    cib = np.array([c for r in bad for c in r] or [0], np.int32)
    O, L = _run_forward(q, k, v, block, rpb, cib)
    O1, L1 = _run_forward(q, k, v, block, rp, ci)
    assert torch.equal(O.view(torch.int16), O1.view(torch.int16))
    assert torch.equal(L, L1)


def test_forward_whole_blocks_strided_and_skip():
    B, H, nB, D, block = 2, 4, 7, 128, 128
    N = nB * block
    q, k, v = synth.random_qkv(B, H, N, D, seed=320)
    rp, ci = synth.random_block_lists(B, H, nB, seed=321, density=0.6, empty_rows=1, full_rows=2)
    modes = np.array([bsa.HEAD_SKIP, bsa.HEAD_FULL, bsa.HEAD_SKIP, bsa.HEAD_ARROW], np.int8)
    cache = synth.random_qkv(B, H, N, D, seed=322)[0]

    def strided(a):
        t = to_dev_bf16(np.ascontiguousarray(a.transpose(0, 2, 1, 3)))
        return t.permute(0, 2, 1, 3)
    out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=dev()).permute(0, 2, 1, 3)
    O, L = bsa.forward(strided(q), strided(k), strided(v), block, _i32(rp), _i32(ci), head_modes=modes,
                       o_cache=to_dev_bf16(cache), out=out)
    torch.cuda.synchronize()
    Oo, Lo = oracle.forward(q, k, v, block, rp, ci)
    comp = modes != bsa.HEAD_SKIP
    check_forward(bf16_to_f64(O)[:, comp], L.cpu().numpy()[:, comp].astype(np.float64), Oo[:, comp],
                  Lo[:, comp], "strided whole blocks")
    np.testing.assert_array_equal(bf16_bits(O)[:, ~comp], cache[:, ~comp])
    # no LSE cache: the binding's own LSE tensor marks SKIP heads NaN
    assert torch.isnan(L[:, torch.from_numpy(~comp)]).all()


def test_forward_very_negative_logits_and_empty_last_subtile():
    """Every logit far below zero (about -260 in log2 units) with a last block
    of 40 keys, whose second 64-key sub-tile holds no key: that sub-tile must
    not raise the running reference max, or every probability underflows."""
    B, H, N, D, block = 1, 2, 2 * 128 + 40, 128, 128
    rng = np.random.default_rng(115)
    u = rng.choice([-1.0, 1.0], size=(B, H, 1, D))
    q = synth.f32_to_bf16((4.0 * u + 0.3 * rng.standard_normal((B, H, N, D))).astype(np.float32))
    k = synth.f32_to_bf16((-4.0 * u + 0.3 * rng.standard_normal((B, H, N, D))).astype(np.float32))
    v = synth.f32_to_bf16(rng.standard_normal((B, H, N, D)).astype(np.float32))
    nB = -(-N // block)
    rp = np.arange(0, B * H * nB * nB + 1, nB, dtype=np.int32)        # every row dense
    ci = np.tile(np.arange(nB, dtype=np.int32), B * H * nB)
    O, L = _run_forward(q, k, v, block, rp, ci)
    Oo, Lo = oracle.forward(q, k, v, block, rp, ci)
    assert np.all(np.isfinite(Lo)) and Lo.max() < -150.0
    check_forward(bf16_to_f64(O), L.cpu().numpy().astype(np.float64), Oo, Lo, "negative logits")


def test_forward_strided_skip_and_alias():
    B, H, N, D, block = 2, 4, 3 * 64 + 5, 64, 64
    q, k, v = synth.random_qkv(B, H, N, D, seed=120)
    nB = -(-N // block)
    rp, ci = synth.random_block_lists(B, H, nB, seed=121, density=0.5)
    modes = np.array([bsa.HEAD_FULL, bsa.HEAD_SKIP, bsa.HEAD_ARROW, bsa.HEAD_SKIP], np.int8)
    cache = synth.f32_to_bf16(np.random.default_rng(5).standard_normal((B, H, N, D)).astype(np.float32))
    lse_c = np.random.default_rng(6).standard_normal((B, H, N)).astype(np.float32)

    # [B, N, H, D] storage viewed as [B, H, N, D]: non-contiguous strides
    def strided(a):
        t = to_dev_bf16(np.ascontiguousarray(a.transpose(0, 2, 1, 3)))
        return t.permute(0, 2, 1, 3)
    qd, kd, vd = strided(q), strided(k), strided(v)
    out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=dev()).permute(0, 2, 1, 3)
    oc = to_dev_bf16(cache)
    lc = torch.from_numpy(lse_c).to(dev())
    O, L = bsa.forward(qd, kd, vd, block, _i32(rp), _i32(ci), head_modes=modes, o_cache=oc,
                       lse_cache=lc, out=out)
    torch.cuda.synchronize()
    Oo, Lo = oracle.forward(q, k, v, block, rp, ci, modes=modes, o_cache=cache, lse_cache=lse_c)
    comp = modes != bsa.HEAD_SKIP
    check_forward(bf16_to_f64(O)[:, comp], L.cpu().numpy()[:, comp].astype(np.float64),
                  Oo[:, comp], Lo[:, comp], "strided")
    # skip heads: bit-exact copies of the caches
    Ob = bf16_bits(O)
    np.testing.assert_array_equal(Ob[:, ~comp], cache[:, ~comp])
    np.testing.assert_array_equal(L.cpu().numpy()[:, ~comp], lse_c[:, ~comp])

    # in place: o_cache aliases the output -> skip heads keep their contents
    o2 = to_dev_bf16(cache)
    O2, _ = bsa.forward(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), block, _i32(rp), _i32(ci),
                        head_modes=modes, o_cache=o2, out=o2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_bits(O2)[:, ~comp], cache[:, ~comp])
    np.testing.assert_array_equal(bf16_bits(O2)[:, comp], Ob[:, comp])


SPLIT_CASES = [
    # B, H, N, D, block, chunk_blocks, max_chunks, max_split_rows, seed
    (2, 3, 9 * 128 + 40, 128, 128, 2, 4, 64, 200),     # many split rows, ragged tail
    (1, 2, 12 * 64, 64, 64, 3, 3, 4, 201),             # pool smaller than the long rows
    (1, 2, 10 * 128, 64, 128, 4, 2, 100, 202),
    (2, 2, 7 * 64 + 3, 128, 64, 1, 64, 1000, 203),     # a chunk per block, empty chunks
]


@pytest.mark.parametrize("B,H,N,D,block,cb,mc,msr,seed", SPLIT_CASES)
def test_forward_split_long_rows(B, H, N, D, block, cb, mc, msr, seed):
    _log(f"split B={B} H={H} N={N} D={D} block={block} chunk={cb} chunks={mc} pool={msr}")
    q, k, v = synth.random_qkv(B, H, N, D, seed=seed)
    nB = -(-N // block)
    rp, ci = synth.random_block_lists(B, H, nB, seed=seed + 1, density=0.6, empty_rows=2, full_rows=4)
    split = {"chunk_blocks": cb, "max_chunks": mc, "max_split_rows": msr}
    O, L = _run_forward(q, k, v, block, rp, ci, split=split)
    Oo, Lo = oracle.forward(q, k, v, block, rp, ci)
    check_forward(bf16_to_f64(O), L.cpu().numpy().astype(np.float64), Oo, Lo, "split")
    O1, L1 = _run_forward(q, k, v, block, rp, ci)
    assert float((O.float() - O1.float()).abs().max()) <= 2e-2
    # the plan's bookkeeping: items and split rows as the host expects
    lens = np.diff(rp)
    order = [(bh * nB + i) for i in range(nB) for bh in range(B * H)]
    want = [min(mc, -(-int(lens[r]) // cb)) if lens[r] > cb else 1 for r in order]
    n_split = min(msr, sum(1 for x in want if x > 1))
    counts = split["workspace"][:8].view(torch.int32).cpu().numpy()
    assert counts[1] == n_split
    ranked = 0
    n_items = 0
    for x in want:
        if x > 1 and ranked < msr:
            ranked += 1
            n_items += x
        else:
            n_items += 1
    assert counts[0] == n_items


def test_forward_split_with_skip_heads_keeps_lse():
    B, H, N, D, block = 1, 3, 6 * 128, 128, 128
    q, k, v = synth.random_qkv(B, H, N, D, seed=210)
    nB = N // block
    rp, ci = synth.random_block_lists(B, H, nB, seed=211, density=0.9, empty_rows=0, full_rows=6)
    modes = np.array([bsa.HEAD_FULL, bsa.HEAD_SKIP, bsa.HEAD_ARROW], np.int8)
    cache = synth.random_qkv(B, H, N, D, seed=212)[0]
    lse = torch.full((B, H, N), 123.0, dtype=torch.float32, device=dev())
    split = {"chunk_blocks": 1, "max_chunks": 6, "max_split_rows": 100}
    O, L = _run_forward(q, k, v, block, rp, ci, head_modes=modes, o_cache=to_dev_bf16(cache), lse=lse,
                        split=split)
    Oo, Lo = oracle.forward(q, k, v, block, rp, ci)
    comp = modes != bsa.HEAD_SKIP
    check_forward(bf16_to_f64(O)[:, comp], L.cpu().numpy()[:, comp].astype(np.float64), Oo[:, comp],
                  Lo[:, comp], "split+skip")
    np.testing.assert_array_equal(bf16_bits(O)[:, ~comp], cache[:, ~comp])
    assert torch.all(L[:, 1] == 123.0)
    # rows of the skip head are never split
    assert split["workspace"][:8].view(torch.int32).cpu().numpy()[1] == 2 * nB


def test_forward_is_deterministic():
    B, H, N, D, block = 1, 4, 8 * 128, 128, 128
    q, k, v = synth.random_qkv(B, H, N, D, seed=130)
    rp, ci = synth.random_block_lists(B, H, N // block, seed=131, density=0.5)
    O1, L1 = _run_forward(q, k, v, block, rp, ci)
    O2, L2 = _run_forward(q, k, v, block, rp, ci)
    assert torch.equal(O1.view(torch.int16), O2.view(torch.int16))
    assert torch.equal(L1, L2)


# ---------------------------------------------------------------------------
# arrow layout
# ---------------------------------------------------------------------------
ARROW_CASES = [
    (1, 3, 4608, 128, 512, [1, 0, 2], [1, 0, 0]),
    (2, 4, 4396, 128, 300, [1, 1, 0, 2], [0, 5, 0, 0]),      # ragged text and tail
    (1, 2, 16896, 128, 512, [1, 1], [8, 200]),
    (1, 2, 1000, 64, 0, [1, 1], [2, 0]),                      # no text at all
    (1, 1, 640, 64, 640, [1], [1]),                           # text only
]


@pytest.mark.parametrize("B,H,N,block,text_len,modes,wins", ARROW_CASES)
def test_arrow_layout_matches_oracle(B, H, N, block, text_len, modes, wins):
    nB = -(-N // block)
    tb = -(-text_len // block)
    rp, ci = bsa.build_arrow_layout(B, H, N, block, text_len, modes, wins, device=dev())
    torch.cuda.synchronize()
    rpo, cio = oracle.arrow(B, H, nB, tb, np.array(modes, np.int8), np.array(wins, np.int32))
    np.testing.assert_array_equal(rp.cpu().numpy(), rpo)
    np.testing.assert_array_equal(ci.cpu().numpy(), cio)


# ---------------------------------------------------------------------------
# top-k selection on given scores (bit-exact: both sides read the same fp32)
# ---------------------------------------------------------------------------
SELECT_CASES = [
    (1, 2, 8, 1, ((0, 8, 4),), 0),
    (2, 3, 68, 4, ((4, 68, 16),), 0),
    (1, 2, 68, 4, ((4, 68, 16),), 3),                         # many exact ties
    (1, 2, 512, 0, ((0, 480, 144), (480, 512, 10)), 0),
    (1, 1, 1024, 2, ((2, 1024, 300),), 5),
    (1, 2, 100, 0, ((0, 100, 100), (0, 1, 1)), 0),            # k = width; overlapping groups
    (1, 2, 70, 70, ((0, 70, 3),), 0),                         # every row is a text row
    # disjoint groups clear of the text columns (row lengths in closed form,
    # one kernel): a gap, a k = 0 group, k = width
    (2, 2, 37, 3, ((3, 20, 5), (25, 37, 12), (20, 25, 0)), 2),
    (1, 3, 9, 2, (), 0),                                      # no groups: text columns only
]


@pytest.mark.parametrize("B,H,nB,tb,groups,ties", SELECT_CASES)
def test_select_matches_oracle(B, H, nB, tb, groups, ties):
    S = synth.random_scores(B, H, nB, seed=140 + nB + ties, tie_levels=ties)
    if ties:
        S[..., ::7] = -0.0
        S[..., 1::7] = 0.0
    rp, ci = bsa.select_topk(torch.from_numpy(S).to(dev()), tb, groups)
    torch.cuda.synchronize()
    rpo, cio = oracle.select(S, tb, groups)
    rp = rp.cpu().numpy()
    np.testing.assert_array_equal(rp, rpo)
    np.testing.assert_array_equal(ci.cpu().numpy()[:rp[-1]], cio)


@pytest.mark.parametrize("B,H,nB,tb,groups", [
    (1, 2, 68, 4, ((4, 68, 16),)),
    (1, 2, 512, 0, ((0, 480, 144), (480, 512, 10))),
    (1, 1, 300, 3, ((5, 300, 290), (0, 40, 7))),             # overlapping groups
])
def test_select_nan_and_infinite_scores(B, H, nB, tb, groups):
    """NaN ranks below every number (-inf included), NaNs by lower column;
    +-inf and NaN runs longer than a group's budget."""
    S = synth.random_scores(B, H, nB, seed=145 + nB, tie_levels=2)
    r = np.random.default_rng(146)
    m = r.random(S.shape)
    S[m < 0.15] = np.nan
    S[(m >= 0.15) & (m < 0.2)] = -np.inf
    S[(m >= 0.2) & (m < 0.22)] = np.inf
    S[..., -1, :] = np.nan                    # a row of NaNs only
    rp, ci = bsa.select_topk(torch.from_numpy(S).to(dev()), tb, groups)
    torch.cuda.synchronize()
    rpo, cio = oracle.select(S, tb, groups)
    rp = rp.cpu().numpy()
    np.testing.assert_array_equal(rp, rpo)
    np.testing.assert_array_equal(ci.cpu().numpy()[:rp[-1]], cio)


# ---------------------------------------------------------------------------
# block scores
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,H,N,D,block,r", [
    (2, 3, 5 * 64 + 9, 64, 64, 32), (1, 2, 4 * 128, 128, 128, 32), (1, 2, 3 * 128 + 1, 64, 128, 32),
    (1, 2, 7 * 64 + 5, 128, 64, 32),          # block 64 at D 128
    (1, 1, 300 * 64 + 3, 64, 64, 19),         # 301 blocks: several 16 x 128 score tiles, r not a multiple of 4
    (1, 1, 140 * 128, 128, 128, 64),          # the widest r, 140 x 140 scores
])
def test_meanpool_scores_and_selection(B, H, N, D, block, r):
    q, k, _ = synth.random_qkv(B, H, N, D, seed=150 + N)
    w = np.random.default_rng(151).standard_normal((D, r)).astype(np.float32) / math.sqrt(D)
    S = bsa.pool_scores(to_dev_bf16(q), to_dev_bf16(k), block, bsa.SCORE_MEANPOOL_PROJ,
                        w=torch.from_numpy(w).to(dev()))
    torch.cuda.synchronize()
    So = oracle.scores_meanpool_proj(q, k, block, w)
    Sg = S.cpu().numpy().astype(np.float64)
    scale = np.abs(So).max(axis=-1, keepdims=True)
    assert np.all(np.abs(Sg - So) <= 1e-5 * scale + 1e-7)
    nB = So.shape[-1]
    tb, groups = 1, ((1, nB, max(1, nB // 3)),)
    rp, ci = bsa.select_topk(S, tb, groups)
    torch.cuda.synchronize()
    rpo, cio = oracle.select(So, tb, groups)
    rp = rp.cpu().numpy()
    g_rows = csr_rows(rp, ci.cpu().numpy())
    qb = np.tile(np.arange(nB), B * H)
    check_selection(g_rows, csr_rows(rpo, cio), So.reshape(-1, nB), qb, tb, groups)


@pytest.mark.parametrize("B,H,N,D,block", [(1, 2, 6 * 64 + 10, 64, 64), (1, 2, 5 * 128, 128, 128),
                                           (2, 1, 3 * 128 + 77, 128, 128),
                                           # last block of 40 keys: its second 64-key sub-tile is empty
                                           (1, 2, 3 * 128 + 40, 128, 128)])
def test_exact_scores_small(B, H, N, D, block):
    q, k, _ = synth.random_qkv(B, H, N, D, seed=160 + N, scale=1.5)
    S = bsa.pool_scores(to_dev_bf16(q), to_dev_bf16(k), block, bsa.SCORE_EXACT_AVGPOOL)
    torch.cuda.synchronize()
    So = oracle.scores_exact_avgpool(q, k, block)
    Sg = S.cpu().numpy().astype(np.float64)
    scale = np.abs(So).max(axis=-1, keepdims=True)
    err = np.abs(Sg - So) / scale
    assert err.max() <= 2e-5, f"max rel err {err.max():.2e}"
    # a workspace of a single slot gives the same bits (persistent workgroups)
    nB = So.shape[-1]
    ws = torch.empty(nB * block * 4, dtype=torch.uint8, device=dev())
    S1 = bsa.pool_scores(to_dev_bf16(q), to_dev_bf16(k), block, bsa.SCORE_EXACT_AVGPOOL, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(S, S1)


# ---------------------------------------------------------------------------
# the five workloads at full size
# ---------------------------------------------------------------------------
def _workload_forward_check(wl, x, rp, ci, n_sample, seed, must_blocks=(), modes=None, split=None):
    """The forward on the workload against the oracle: on every computed row
    when n_sample is None, else on a seeded sample plus the rows of
    must_blocks."""
    B, H, N, D, block = wl.B, wl.H, wl.N, wl.D, wl.block
    kw = {} if split is None else {"split": split}
    if modes is not None:
        kw.update(head_modes=modes, o_cache=to_dev_bf16(x["o_cache"]) if "o_cache" in x else None,
                  lse_cache=torch.from_numpy(x["lse_cache"]).to(dev()) if "lse_cache" in x else None)
    O, L = _run_forward(x["q"], x["k"], x["v"], block, rp, ci, **kw)
    must = []
    for (b, h, i) in must_blocks:
        t0 = i * block
        must += [((b * H + h) * N + t) for t in range(t0, min(N, t0 + block))]
    if n_sample is None:
        rows = np.arange(B * H * N, dtype=np.int64)
    else:
        rows = sample_rows(B, H, N, n_sample, seed, must)
    if modes is not None:
        rows = rows[modes[(rows // N) % H] != bsa.HEAD_SKIP]
    Oo, Lo = oracle.forward(x["q"], x["k"], x["v"], block, rp, ci, rows=rows)
    Og = bf16_to_f64(O).reshape(-1, D)[rows]
    Lg = L.cpu().numpy().reshape(-1)[rows].astype(np.float64)
    mx, mean = check_forward(Og, Lg, Oo, Lo, wl.name)
    _log(f"{wl.name}: {len(rows)} rows, max|dO|={mx:.2e} mean|dO|={mean:.2e}")
    return O, L


@pytest.mark.slow
def test_workload_c1_full_chain():
    wl = synth.WORKLOADS["C1"]
    x = synth.make_inputs(wl)
    nB, tb = wl.n_blocks, wl.text_blocks
    qd, kd = to_dev_bf16(x["q"]), to_dev_bf16(x["k"])
    S = bsa.pool_scores(qd, kd, wl.block, wl.score_mode, w=torch.from_numpy(x["w"]).to(dev()))
    rp, ci = bsa.select_topk(S, tb, wl.groups)
    torch.cuda.synchronize()
    So = oracle.scores_meanpool_proj(x["q"], x["k"], wl.block, x["w"])
    rpo, cio = oracle.select(So, tb, wl.groups)
    rpg, cig = rp.cpu().numpy(), ci.cpu().numpy()
    check_csr_valid(rpg, cig[:rpg[-1]], nB)
    g_rows = csr_rows(rpg, cig)
    qb = np.tile(np.arange(nB), wl.B * wl.H)
    differ = check_selection(g_rows, csr_rows(rpo, cio), So.reshape(-1, nB), qb, tb, wl.groups)
    counts = np.diff(rpo)
    assert counts[0] == nB and set(counts[1:nB].tolist()) <= {4, 5}
    # forward on the oracle's block list, every row
    O, L = _run_forward(x["q"], x["k"], x["v"], wl.block, rpo, cio)
    Oo, Lo = oracle.forward(x["q"], x["k"], x["v"], wl.block, rpo, cio)
    check_forward(bf16_to_f64(O), L.cpu().numpy().astype(np.float64), Oo, Lo, "C1")
    if differ == 0:   # GPU list identical: the end-to-end GPU chain gives the same bits
        O2, _ = bsa.forward(qd, kd, to_dev_bf16(x["v"]), wl.block, rp, ci)
        torch.cuda.synchronize()
        assert torch.equal(O.view(torch.int16), O2.view(torch.int16))


@pytest.mark.slow
@pytest.mark.parametrize("name", ["C2", "C4"])
def test_workload_arrow(name):
    wl = synth.WORKLOADS[name]
    x = synth.make_inputs(wl)
    modes, wins = x["head_modes"], x["head_windows"]
    nB, tb = wl.n_blocks, wl.text_blocks
    rp, ci = bsa.build_arrow_layout(wl.B, wl.H, wl.N, wl.block, wl.text_len, modes, wins, device=dev())
    torch.cuda.synchronize()
    rpo, cio = oracle.arrow(wl.B, wl.H, nB, tb, modes, wins)
    np.testing.assert_array_equal(rp.cpu().numpy(), rpo)
    np.testing.assert_array_equal(ci.cpu().numpy(), cio)
    comp_heads = [h for h in range(wl.H) if modes[h] != bsa.HEAD_SKIP]
    must = [(0, comp_heads[0], 0), (0, comp_heads[-1], nB - 1), (0, comp_heads[len(comp_heads) // 2], nB // 2)]
    O, L = _workload_forward_check(wl, x, rpo, cio, None, seed=170, modes=modes)
    # the same forward with long rows split over several workgroups
    # the same forward with long rows split over several workgroups (forced:
    # the policy may judge a split not worth it for this workload)
    plan = bsa.arrow_split_policy(wl.B, wl.H, wl.N, wl.block, wl.text_len, modes, wins) or \
        {"chunk_blocks": 33 if name == "C4" else 9, "max_chunks": 4, "max_split_rows": 1000}
    O2, L2 = _workload_forward_check(wl, x, rpo, cio, 384, seed=171, must_blocks=must, modes=modes,
                                     split=plan)
    assert float((O.float() - O2.float()).abs().max()) <= 2e-2
    skip = modes == bsa.HEAD_SKIP
    if skip.any():
        np.testing.assert_array_equal(bf16_bits(O)[:, skip], x["o_cache"][:, skip])
        np.testing.assert_array_equal(L.cpu().numpy()[:, skip], x["lse_cache"][:, skip])


@pytest.mark.slow
def test_workload_c3_content_driven():
    wl = synth.WORKLOADS["C3"]
    x = synth.make_inputs(wl)
    nB, tb = wl.n_blocks, wl.text_blocks
    S = bsa.pool_scores(to_dev_bf16(x["q"]), to_dev_bf16(x["k"]), wl.block, wl.score_mode,
                        w=torch.from_numpy(x["w"]).to(dev()))
    rp, ci = bsa.select_topk(S, tb, wl.groups)
    torch.cuda.synchronize()
    So = oracle.scores_meanpool_proj(x["q"], x["k"], wl.block, x["w"])
    Sg = S.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(Sg - So) <= 1e-5 * np.abs(So).max(axis=-1, keepdims=True) + 1e-7)
    rpo, cio = oracle.select(So, tb, wl.groups)
    rpg, cig = rp.cpu().numpy(), ci.cpu().numpy()
    check_csr_valid(rpg, cig[:rpg[-1]], nB)
    g_rows = csr_rows(rpg, cig)
    qb = np.tile(np.arange(nB), wl.B * wl.H)
    differ = check_selection(g_rows, csr_rows(rpo, cio), So.reshape(-1, nB), qb, tb, wl.groups)
    _log(f"C3: {differ} of {len(qb)} rows differ only by near-ties")
    assert rpo[-1] == wl.B * wl.H * (tb * nB + (nB - tb) * (tb + 16))
    _workload_forward_check(wl, x, rpo, cio, None, seed=171)
    plan = {"chunk_blocks": 20, "max_chunks": 4, "max_split_rows": 128}
    _workload_forward_check(wl, x, rpo, cio, 512, seed=172, must_blocks=[(1, 15, 0), (0, 3, 1)], split=plan)


@pytest.mark.slow
def test_workload_c5_exact_selection_and_forward():
    wl = synth.WORKLOADS["C5"]
    _log("C5: generating inputs")
    x = synth.make_inputs(wl)
    nB, tb = wl.n_blocks, wl.text_blocks
    qd, kd = to_dev_bf16(x["q"]), to_dev_bf16(x["k"])
    _log("C5: exact scores on the GPU")
    S = bsa.pool_scores(qd, kd, wl.block, wl.score_mode)
    rp, ci = bsa.select_topk(S, tb, wl.groups)
    torch.cuda.synchronize()
    rpg, cig = rp.cpu().numpy(), ci.cpu().numpy()
    check_csr_valid(rpg, cig[:rpg[-1]], nB)
    assert np.all(np.diff(rpg) == 154)
    # selection, every row, bit-exact: the oracle's top-k on the GPU's own fp32 scores
    Sg_all = S.cpu().numpy()
    rps, cis = oracle.select(Sg_all, tb, wl.groups)
    np.testing.assert_array_equal(rpg, rps)
    np.testing.assert_array_equal(cig[:rpg[-1]], cis)
    # the exact scores of 256 query-block rows, 8 per head (the first, the
    # last two and five seeded others), computed by the oracle in fp64
    r = np.random.default_rng(180)
    rows = []
    for bh in range(wl.B * wl.H):
        own = {0, nB - 2, nB - 1} | set(r.choice(np.arange(1, nB - 2), size=5, replace=False).tolist())
        rows += [bh * nB + i for i in sorted(own)]
    assert len(rows) >= 256
    _log(f"C5: oracle exact scores for {len(rows)} query blocks")
    So = oracle.scores_exact_avgpool(x["q"], x["k"], wl.block, rows=rows)
    Sg = Sg_all.reshape(-1, nB)[rows].astype(np.float64)
    rel = np.abs(Sg - So) / np.abs(So).max(axis=-1, keepdims=True)
    assert rel.max() <= 2e-5, f"C5 exact score rel err {rel.max():.2e}"
    np.testing.assert_allclose(So.sum(-1) * wl.block, 1.0, rtol=1e-9)
    # the GPU selection of those rows against the oracle's on its own fp64 scores
    qb = [row % nB for row in rows]
    rpo, cio = oracle.select_rows(So, qb, tb, wl.groups)
    g_rows = [cig[rpg[row]:rpg[row + 1]].tolist() for row in rows]
    differ = check_selection(g_rows, csr_rows(rpo, cio), So, qb, tb, wl.groups, nB=nB)
    _log(f"C5: {differ} of {len(rows)} scored rows differ only by near-ties")
    del S, qd, kd
    torch.cuda.empty_cache()
    # the end-to-end chain: the forward on the GPU's own block list
    _workload_forward_check(wl, x, rpg, cig[:rpg[-1]], 8192, seed=182,
                            must_blocks=[(0, 7, 0), (0, 31, nB - 1), (0, 0, nB - 2)])
