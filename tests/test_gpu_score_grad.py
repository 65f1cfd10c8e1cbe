"""GPU parity of bsa_score_grad (gradient of the mean-pool / projection
block score) against the fp64 oracle.

Tolerance.  The GPU path is fp32 throughout: block means over <= 128
tokens, projections over D terms, g over nB terms and dW over
2 * B * H * nB outer products.  Each is a sum of random-sign terms, so the
error is a few fp32 ulps of the larger terms; we allow 1e-4 of the largest
element (elementwise) and 1e-5 of the mean magnitude on average.  The
result is deterministic: two calls agree bit for bit.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import block_sparse_attention_18_amd as bsa
from helpers import dev, to_dev_bf16

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _close(got, ref, what):
    got = got.astype(np.float64)
    scale = np.abs(ref).max()
    err = np.abs(got - ref)
    assert err.max() <= 1e-4 * scale + 1e-30, f"{what}: max err {err.max():.3e} vs scale {scale:.3e}"
    assert err.mean() <= 1e-5 * np.abs(ref).mean() + 1e-30, f"{what}: mean err {err.mean():.3e}"


def _run(q, k, block, w, dS, pooled=True):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())
    dw, dqp, dkp = bsa.score_grad(to_dev_bf16(q), to_dev_bf16(k), block, t(w), t(dS), pooled=pooled)
    torch.cuda.synchronize()
    cpu = lambda x: None if x is None else x.cpu().numpy()
    return cpu(dw), cpu(dqp), cpu(dkp)


@pytest.mark.parametrize("B,H,N,D,r,block,seed", [
    (1, 2, 512, 64, 32, 64, 901),            # the C1 shape
    (2, 3, 5 * 64 + 9, 64, 32, 64, 902),     # ragged last block
    (1, 3, 1000, 128, 17, 128, 903),         # odd r, ragged
    (2, 2, 777, 128, 64, 64, 904),           # widest r
    (1, 1, 130, 64, 1, 128, 905),            # r = 1, two blocks, the second of 2 tokens
    (1, 1, 5, 128, 8, 64, 906),              # a single partial block
])
def test_score_grad_matches_oracle(B, H, N, D, r, block, seed):
    _log(f"score_grad B={B} H={H} N={N} D={D} r={r} block={block}")
    q, k, _ = synth.random_qkv(B, H, N, D, seed=seed)
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((D, r)) / math.sqrt(D)).astype(np.float32)
    nB = -(-N // block)
    dS = rng.standard_normal((B, H, nB, nB)).astype(np.float32)
    dw, dqp, dkp = _run(q, k, block, w, dS)
    rw, rq, rk = oracle.score_grad(q, k, block, w, dS.astype(np.float64))
    _close(dw, rw, "dW")
    _close(dqp, rq, "dqbar")
    _close(dkp, rk, "dkbar")
    # without the pooled gradients dW is the same, and the call is deterministic
    dw2, a, b = _run(q, k, block, w, dS, pooled=False)
    assert a is None and b is None
    np.testing.assert_array_equal(dw, dw2)


def test_score_grad_content_driven_workload_shape():
    # the content-driven DiT workload: B=2, H=16, N=4352, D=64, block 64, r=32,
    # its own W, and an upstream gradient of a distillation-style loss
    # (scores pulled towards the exact block averages: dS = S - S_exact)
    wl = synth.WORKLOADS["C3"]
    x = synth.make_inputs(wl)
    _log(f"score_grad workload {wl.name}")
    S = oracle.scores_meanpool_proj(x["q"], x["k"], wl.block, x["w"])
    rng = np.random.default_rng(931)
    dS = (S - S.mean(axis=-1, keepdims=True) + 0.1 * rng.standard_normal(S.shape)).astype(np.float32)
    dw, dqp, dkp = _run(x["q"], x["k"], wl.block, x["w"], dS)
    rw, rq, rk = oracle.score_grad(x["q"], x["k"], wl.block, x["w"], dS.astype(np.float64))
    _close(dw, rw, "dW")
    _close(dqp, rq, "dqbar")
    _close(dkp, rk, "dkbar")
    dw2, _, _ = _run(x["q"], x["k"], wl.block, x["w"], dS)
    np.testing.assert_array_equal(dw, dw2)


def test_score_grad_strided_inputs():
    # q, k through strided [B, N, H, D] views give the same gradient
    B, H, N, D, r, block = 2, 3, 300, 64, 32, 64
    q, k, _ = synth.random_qkv(B, H, N, D, seed=941)
    rng = np.random.default_rng(941)
    w = (rng.standard_normal((D, r)) / math.sqrt(D)).astype(np.float32)
    nB = -(-N // block)
    dS = torch.from_numpy(rng.standard_normal((B, H, nB, nB)).astype(np.float32)).to(dev())
    wt = torch.from_numpy(w).to(dev())
    qs = to_dev_bf16(np.ascontiguousarray(q.transpose(0, 2, 1, 3))).permute(0, 2, 1, 3)
    ks = to_dev_bf16(np.ascontiguousarray(k.transpose(0, 2, 1, 3))).permute(0, 2, 1, 3)
    a = bsa.score_grad(qs, ks, block, wt, dS)
    b = bsa.score_grad(to_dev_bf16(q), to_dev_bf16(k), block, wt, dS)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
