"""The workspace-free block-score entry point (bsa_pool_scores_noalloc)
against the entry point with a caller workspace (bsa_pool_scores): the same
kernels, so the same bits, on two calls in a row with the second smaller
(the static scratch keeps the first call's contents)."""
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


def _w(D, r, seed):
    return torch.from_numpy((np.random.default_rng(seed).standard_normal((D, r)) / math.sqrt(D))
                            .astype(np.float32)).to(dev())


@pytest.mark.parametrize("mode", [bsa.SCORE_MEANPOOL_PROJ, bsa.SCORE_EXACT_AVGPOOL])
def test_noalloc_matches_workspace_entry_point(mode):
    shapes = [(2, 16, 4352, 64, 64, 32), (1, 2, 512, 128, 128, 17)] if mode == bsa.SCORE_MEANPOOL_PROJ \
        else [(1, 4, 9 * 128, 128, 128, 0), (1, 2, 3 * 64 + 10, 64, 64, 0)]
    for call, (B, H, N, D, block, r) in enumerate(shapes):
        _log(f"noalloc mode={mode} call={call} B={B} H={H} N={N} D={D} block={block}")
        q, k, _ = synth.random_qkv(B, H, N, D, seed=400 + call, scale=1.5)
        qd, kd = to_dev_bf16(q), to_dev_bf16(k)
        w = _w(D, r, 401 + call) if r else None
        nB = -(-N // block)
        out = torch.full((B, H, nB, nB), float("nan"), dtype=torch.float32, device=dev())
        S1 = bsa.pool_scores_noalloc(qd, kd, block, mode, w=w, out=out)
        S0 = bsa.pool_scores(qd, kd, block, mode, w=w)
        torch.cuda.synchronize()
        assert S1.data_ptr() == out.data_ptr()
        assert torch.equal(S1, S0), f"call {call}: differs from bsa_pool_scores"
        # and to the oracle's bar
        So = oracle.scores_meanpool_proj(q, k, block, w.cpu().numpy()) if r else \
            oracle.scores_exact_avgpool(q, k, block)
        rel = np.abs(S1.cpu().numpy().astype(np.float64) - So) / np.abs(So).max(axis=-1, keepdims=True)
        assert rel.max() <= (1e-5 if r else 2e-5), f"call {call}: rel err {rel.max():.2e}"
