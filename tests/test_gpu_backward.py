"""GPU parity of the backward (dQ, dK, dV) against the fp64 oracle gradient.

The GPU backward runs on the GPU forward's O and LSE; the oracle computes
the exact gradient from Q, K, V and dO alone.  P and dS are rounded to bf16
for the MFMAs (relative 2^-9 each), Delta = rowsum(dO * O) uses the bf16 O,
and the gradients are rounded to bf16: each gradient element carries a
relative error of a few 2^-9 (measured 2-5e-3 on N(0,1) inputs).  In
sharply peaked rows dS = P (dP - Delta) cancels, and the 2^-9 error of Delta
from the bf16 O grows relative to dS by about 1 / (1 - P_max) (measured
1.0e-2 of max|dK| at logit sigma ~7).  The tolerances, relative to each
gradient tensor's size: max 2e-2 of its largest element, mean 1e-2 of its
mean magnitude."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import block_sparse_attention_18_amd as bsa
from helpers import bf16_to_f64, dev, to_dev_bf16

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

MAX_REL = 2e-2
MEAN_REL = 1e-2


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def _check_grad(g, want, name):
    d = np.abs(g - want)
    mx = float(d.max()) / max(float(np.abs(want).max()), 1e-30)
    mean = float(d.mean()) / max(float(np.abs(want).mean()), 1e-30)
    _log(f"  {name}: max {mx:.2e} of max|g|, mean {mean:.2e} of mean|g|")
    assert mx <= MAX_REL and mean <= MEAN_REL, name
    return mx, mean


def _run(q, k, v, g, block, rp, ci, scale=None):
    qd, kd, vd, gd = (to_dev_bf16(a) for a in (q, k, v, g))
    rpd, cid = _i32(rp), _i32(ci)
    O, L = bsa.forward(qd, kd, vd, block, rpd, cid, scale=scale)
    dq, dk, dv = bsa.backward(qd, kd, vd, O, gd, block, rpd, cid, L, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


CASES = [
    (1, 2, 4 * 64 + 17, 64, 64, 701),
    (2, 2, 3 * 128 + 40, 128, 128, 702),
    (1, 3, 5 * 64, 128, 64, 703),
    (2, 1, 4 * 128, 64, 128, 704),
    (1, 3, 33, 128, 128, 706),          # one partial block, its second sub-tile empty
]


@pytest.mark.parametrize("B,H,N,D,block,seed", CASES)
def test_backward_random_block_lists(B, H, N, D, block, seed):
    _log(f"backward B={B} H={H} N={N} D={D} block={block}")
    q, k, v = synth.random_qkv(B, H, N, D, seed=seed)
    g = synth.random_qkv(B, H, N, D, seed=seed + 50)[0]
    nB = -(-N // block)
    rp, ci = synth.random_block_lists(B, H, nB, seed=seed + 1, density=0.5, empty_rows=1, full_rows=2)
    dq, dk, dv = _run(q, k, v, g, block, rp, ci)
    wq, wk, wv = oracle.backward(q, k, v, g, block, rp, ci)
    _check_grad(bf16_to_f64(dq), wq, "dQ")
    _check_grad(bf16_to_f64(dk), wk, "dK")
    _check_grad(bf16_to_f64(dv), wv, "dV")


def test_backward_one_token():
    # N = 1: a non-empty row keeps only the token itself, so P = 1, O = V,
    # Delta = dO . V = dP and dS = 0 exactly: dQ = dK = 0 and dV = dO (to
    # fp32 rounding of the two equal dot products).  An empty row gives zeros.
    B, H, N, D, block = 1, 3, 1, 64, 64
    q, k, v = synth.random_qkv(B, H, N, D, seed=705)
    g = synth.random_qkv(B, H, N, D, seed=755)[0]
    rp = np.array([0, 1, 1, 2], np.int32)                  # heads 0 and 2 keep the block, head 1 is empty
    ci = np.array([0, 0], np.int32)
    dq, dk, dv = _run(q, k, v, g, block, rp, ci)
    gq, gk, gv = (bf16_to_f64(t) for t in (dq, dk, dv))
    qf, kf, vf, gf = (bf16_to_f64(to_dev_bf16(a)) for a in (q, k, v, g))
    scale = 1.0 / np.sqrt(D)
    for h in (0, 2):
        np.testing.assert_allclose(gv[0, h], gf[0, h], rtol=2 ** -8, atol=0)
        # dP and Delta are the same D products (exact in fp32) summed in two
        # orders: |dS| <= 2 D 2^-24 sum |dO V| (4x margin below); dQ = scale dS K,
        # dK = scale dS Q
        ds = 4 * 2 * D * 2.0 ** -24 * float(np.abs(gf[0, h, 0] * vf[0, h, 0]).sum())
        assert np.abs(gq[0, h]).max() <= scale * ds * np.abs(kf[0, h]).max()
        assert np.abs(gk[0, h]).max() <= scale * ds * np.abs(qf[0, h]).max()
    assert np.all(gq[0, 1] == 0) and np.all(gk[0, 1] == 0) and np.all(gv[0, 1] == 0)
    wq, wk, wv = oracle.backward(q, k, v, g, block, rp, ci)
    np.testing.assert_allclose(gv, wv, rtol=2 ** -8, atol=1e-12)


def test_backward_scale_large_logits_and_determinism():
    B, H, N, D, block = 1, 2, 3 * 128, 128, 128
    q, k, _ = synth.random_qkv(B, H, N, D, seed=711, scale=2.0)
    v, g = synth.random_qkv(B, H, N, D, seed=712)[1:]
    rp, ci = synth.random_block_lists(B, H, 3, seed=713, density=0.7)
    dq, dk, dv = _run(q, k, v, g, block, rp, ci, scale=0.15)
    wq, wk, wv = oracle.backward(q, k, v, g, block, rp, ci, scale=0.15)
    _check_grad(bf16_to_f64(dq), wq, "dQ")
    _check_grad(bf16_to_f64(dk), wk, "dK")
    _check_grad(bf16_to_f64(dv), wv, "dV")
    dq2, dk2, dv2 = _run(q, k, v, g, block, rp, ci, scale=0.15)
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.slow
def test_backward_arrow_2k_shape_two_heads():
    """The 2K MMDiT arrow layout (N = 16896, window 8) on two heads."""
    wl = synth.WORKLOADS["C4"].replace(H=2, arrow_counts=(2, 0, 0))
    x = synth.make_inputs(wl)
    g = synth.random_qkv(wl.B, wl.H, wl.N, wl.D, seed=720)[0]
    rp, ci = oracle.arrow(wl.B, wl.H, wl.n_blocks, wl.text_blocks, x["head_modes"], x["head_windows"])
    dq, dk, dv = _run(x["q"], x["k"], x["v"], g, wl.block, rp, ci)
    wq, wk, wv = oracle.backward(x["q"], x["k"], x["v"], g, wl.block, rp, ci)
    _check_grad(bf16_to_f64(dq), wq, "dQ")
    _check_grad(bf16_to_f64(dk), wk, "dK")
    _check_grad(bf16_to_f64(dv), wv, "dV")


def test_backward_full_2k_workload_sampled_rows_and_sums():
    """The full 2K MMDiT workload (24 heads, arrow w = 8) as bench.py times it:
    sampled dQ rows against the oracle row by row, and two identities that
    hold at any size.  Every row of P sums to one, so the keys' dV add up to
    the sum of dO over the (non-empty) query rows; every row of dS sums to
    zero, so the keys' dK add up to zero.  Both sums keep rounding that is
    random in sign (Delta from the bf16 O, P and dS rounded to bf16), summed
    over 16896 tokens: bounded by 2e-3 of the sum of magnitudes (measured
    1.6e-4 for dK, 9.4e-5 for dV)."""
    wl = synth.WORKLOADS["C4"]
    x = synth.make_inputs(wl)
    B, H, N, D = wl.B, wl.H, wl.N, wl.D
    g = synth.random_qkv(B, H, N, D, seed=730)[0]
    rp, ci = oracle.arrow(B, H, wl.n_blocks, wl.text_blocks, x["head_modes"], x["head_windows"])
    _log("backward full C4")
    dq, dk, dv = _run(x["q"], x["k"], x["v"], g, wl.block, rp, ci)
    rng = np.random.default_rng(731)
    rows = np.concatenate([[0, 511, 512, N - 1, (H - 1) * N + 600],
                           (rng.integers(0, H, 59) * N + rng.integers(0, N, 59))]).astype(np.int64)
    want = oracle.backward_dq_rows(x["q"], x["k"], x["v"], g, wl.block, rp, ci, rows)
    _check_grad(bf16_to_f64(dq).reshape(-1, D)[rows], want, "dQ rows")
    gk, gv = bf16_to_f64(dk), bf16_to_f64(dv)
    go = synth.bf16_to_f32(g).astype(np.float64)
    dk_sum = np.abs(gk.sum(axis=2)) / np.abs(gk).sum(axis=2)          # [B, H, D]
    dv_err = np.abs(gv.sum(axis=2) - go.sum(axis=2)) / np.abs(gv).sum(axis=2)
    _log(f"  sum dK / sum |dK|: max {dk_sum.max():.2e}; |sum dV - sum dO| / sum |dV|: max {dv_err.max():.2e}")
    assert dk_sum.max() <= 2e-3 and dv_err.max() <= 2e-3
