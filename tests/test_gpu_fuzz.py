"""Seeded random cases beside the hand-picked ones: shapes, ragged tails,
block and head sizes, tensor strides, head modes, long-row splits and column
groups drawn from a fixed seed, each checked against the fp64 oracle (block
lists and layouts bit for bit, outputs within the forward's tolerances).
Every input comes from numpy generators; nothing fed to the oracle is read
back from the GPU except the outputs under test."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import block_sparse_attention_18_amd as bsa
from helpers import bf16_bits, bf16_to_f64, check_forward, check_csr_valid, dev, to_dev_bf16
from test_gpu_fp8 import _pow2_inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def _strided(a):
    """[B, N, H, D] storage viewed as [B, H, N, D]."""
    t = to_dev_bf16(np.ascontiguousarray(a.transpose(0, 2, 1, 3)))
    return t.permute(0, 2, 1, 3)


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------
def _forward_case(seed):
    r = np.random.default_rng(seed)
    block = int(r.choice([64, 128]))
    D = int(r.choice([64, 128]))
    B = int(r.integers(1, 3))
    H = int(r.integers(1, 4))
    N = int(r.integers(1, 6 * block))
    return dict(block=block, D=D, B=B, H=H, N=N,
                density=float(r.uniform(0.1, 1.0)),
                empty=int(r.integers(0, 3)), full=int(r.integers(0, 3)),
                strided=bool(r.random() < 0.5),
                modes=bool(r.random() < 0.5),
                lse_cache=bool(r.random() < 0.5),
                split=bool(r.random() < 0.35),
                scale=float(r.uniform(0.05, 0.3)) if r.random() < 0.5 else None,
                mode_draw=r.integers(0, 3, size=H).astype(np.int8),
                chunk=int(r.integers(1, 4)), chunks=int(r.integers(2, 5)), pool=int(r.integers(1, 64)))


@pytest.mark.parametrize("seed", range(900, 960))
def test_fuzz_forward(seed):
    c = _forward_case(seed)
    B, H, N, D, block = c["B"], c["H"], c["N"], c["D"], c["block"]
    _log(f"fuzz forward seed={seed} B={B} H={H} N={N} D={D} block={block} strided={c['strided']} "
         f"modes={c['modes']} split={c['split']} scale={c['scale']}")
    q, k, v = synth.random_qkv(B, H, N, D, seed=seed)
    nB = -(-N // block)
    rp, ci = synth.random_block_lists(B, H, nB, seed=seed + 1000, density=c["density"],
                                      empty_rows=min(c["empty"], B * H * nB),
                                      full_rows=min(c["full"], max(0, B * H * nB - c["empty"])))
    modes = c["mode_draw"] if c["modes"] else None
    kw, okw = {}, {}
    if modes is not None:
        cache = synth.random_qkv(B, H, N, D, seed=seed + 2000)[0]
        lse_c = np.random.default_rng(seed + 3000).standard_normal((B, H, N)).astype(np.float32)
        kw.update(head_modes=modes, o_cache=to_dev_bf16(cache))
        okw.update(modes=modes, o_cache=cache)
        if c["lse_cache"]:
            kw["lse_cache"] = torch.from_numpy(lse_c).to(dev())
            okw["lse_cache"] = lse_c
    if c["scale"] is not None:
        kw["scale"] = c["scale"]
        okw["scale"] = c["scale"]
    if c["split"]:
        kw["split"] = {"chunk_blocks": c["chunk"], "max_chunks": c["chunks"], "max_split_rows": c["pool"]}
    mk = _strided if c["strided"] else to_dev_bf16
    out = None
    if c["strided"]:
        out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=dev()).permute(0, 2, 1, 3)
    O, L = bsa.forward(mk(q), mk(k), mk(v), block, _i32(rp), _i32(ci), out=out, **kw)
    torch.cuda.synchronize()
    Oo, Lo = oracle.forward(q, k, v, block, rp, ci, **okw)
    comp = np.ones(H, bool) if modes is None else modes != bsa.HEAD_SKIP
    Og, Lg = bf16_to_f64(O), L.cpu().numpy().astype(np.float64)
    check_forward(Og[:, comp], Lg[:, comp], Oo[:, comp], Lo[:, comp], f"fuzz {seed}")
    if modes is not None and (~comp).any():
        np.testing.assert_array_equal(bf16_bits(O)[:, ~comp], okw["o_cache"][:, ~comp])
        if c["lse_cache"]:
            np.testing.assert_array_equal(L.cpu().numpy()[:, ~comp], okw["lse_cache"][:, ~comp])
        else:
            assert torch.isnan(L[:, torch.from_numpy(~comp)]).all()


# ---------------------------------------------------------------------------
# arrow layout
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(1000, 1040))
def test_fuzz_arrow_layout(seed):
    r = np.random.default_rng(seed)
    block = int(r.choice([64, 128]))
    B, H = int(r.integers(1, 3)), int(r.integers(1, 6))
    N = int(r.integers(1, 40 * block))
    text_len = int(r.integers(0, N + 1)) if r.random() < 0.8 else 0
    modes = r.integers(0, 3, size=H).astype(np.int8)
    wins = r.integers(0, 12, size=H).astype(np.int32)
    _log(f"fuzz arrow seed={seed} B={B} H={H} N={N} block={block} text={text_len}")
    nB, tb = -(-N // block), -(-text_len // block)
    rp, ci = bsa.build_arrow_layout(B, H, N, block, text_len, modes, wins, device=dev())
    torch.cuda.synchronize()
    rpo, cio = oracle.arrow(B, H, nB, tb, modes, wins)
    np.testing.assert_array_equal(rp.cpu().numpy(), rpo)
    np.testing.assert_array_equal(ci.cpu().numpy()[:rpo[-1]], cio)


# ---------------------------------------------------------------------------
# top-k selection on given scores
# ---------------------------------------------------------------------------
def _random_groups(r, nB, tb):
    groups = []
    for _ in range(int(r.integers(0, 4))):
        a = int(r.integers(0, nB))
        b = int(r.integers(a + 1, nB + 1))
        k = int(r.choice([0, b - a, int(r.integers(0, b - a + 1))]))
        groups.append((a, b, k))
    if r.random() < 0.5:
        # disjoint groups clear of the text columns: the one-kernel path
        cuts = np.sort(r.choice(np.arange(tb, nB + 1), size=min(3, nB - tb + 1), replace=False))
        groups = [(int(a), int(b), int(r.integers(0, b - a + 1))) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
    return groups


@pytest.mark.parametrize("seed", range(1100, 1140))
def test_fuzz_select(seed):
    r = np.random.default_rng(seed)
    B, H = int(r.integers(1, 3)), int(r.integers(1, 4))
    nB = int(r.integers(1, 300))
    tb = int(r.integers(0, nB + 1)) if r.random() < 0.7 else 0
    groups = _random_groups(r, nB, tb)
    ties = int(r.choice([0, 0, 2, 5]))
    _log(f"fuzz select seed={seed} B={B} H={H} nB={nB} tb={tb} groups={groups} ties={ties}")
    S = synth.random_scores(B, H, nB, seed=seed, tie_levels=ties)
    rp, ci = bsa.select_topk(torch.from_numpy(S).to(dev()), tb, groups)
    torch.cuda.synchronize()
    rpo, cio = oracle.select(S, tb, groups)
    rpg = rp.cpu().numpy()
    np.testing.assert_array_equal(rpg, rpo)
    np.testing.assert_array_equal(ci.cpu().numpy()[:rpg[-1]], cio)
    check_csr_valid(rpg, ci.cpu().numpy()[:rpg[-1]], nB)


# ---------------------------------------------------------------------------
# fused mean-pool scores and selection
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(1200, 1220))
def test_fuzz_select_meanpool(seed):
    r = np.random.default_rng(seed)
    block = int(r.choice([64, 128]))
    D = int(r.choice([64, 128]))
    B, H = int(r.integers(1, 3)), int(r.integers(1, 3))
    nB = int(r.integers(1, 40))
    N = int(r.integers((nB - 1) * block + 1, nB * block + 1))
    rr = int(r.integers(1, 65))
    tb = int(r.integers(0, nB + 1)) if r.random() < 0.7 else 0
    cuts = np.sort(r.choice(np.arange(tb, nB + 1), size=min(3, nB - tb + 1), replace=False))
    groups = [(int(a), int(b), int(r.integers(0, b - a + 1))) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
    _log(f"fuzz select_meanpool seed={seed} B={B} H={H} N={N} D={D} block={block} r={rr} tb={tb} groups={groups}")
    assert bsa.select_meanpool_applies(nB, rr, tb, groups)
    q, k, _ = synth.random_qkv(B, H, N, D, seed=seed)
    w = np.random.default_rng(seed + 1).standard_normal((D, rr)).astype(np.float32)
    wd = torch.from_numpy(w).to(dev())
    qd, kd = to_dev_bf16(q), to_dev_bf16(k)
    scores = torch.empty((B, H, nB, nB), dtype=torch.float32, device=dev())
    rp, ci = bsa.select_meanpool(qd, kd, block, wd, tb, groups, scores=scores)
    S2 = bsa.pool_scores(qd, kd, block, bsa.SCORE_MEANPOOL_PROJ, w=wd)
    torch.cuda.synchronize()
    # the fused scores equal the two-call scores bit for bit, and both are
    # the oracle's within fp32 summation error
    assert torch.equal(scores, S2)
    So = oracle.scores_meanpool_proj(q, k, block, w)
    Sg = scores.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(Sg - So) <= 1e-5 * np.abs(So).max(axis=-1, keepdims=True) + 1e-7)
    # the selection is the oracle's top-k of the GPU's own fp32 scores
    rpo, cio = oracle.select(scores.cpu().numpy(), tb, groups)
    rpg = rp.cpu().numpy()
    np.testing.assert_array_equal(rpg, rpo)
    np.testing.assert_array_equal(ci.cpu().numpy()[:rpg[-1]], cio)


# ---------------------------------------------------------------------------
# FP8 forward on the exact-weight construction (logits small integers in
# log2 units, so E4M3 holds every probability and the output must match the
# FP8 oracle to bf16 rounding)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(1300, 1324))
def test_fuzz_forward_fp8_exact_weights(seed):
    r = np.random.default_rng(seed)
    block = int(r.choice([64, 128]))
    D = int(r.choice([64, 128]))
    B, H = int(r.integers(1, 3)), int(r.integers(1, 4))
    N = int(r.integers(1, 6 * block))
    q_exp = int(r.integers(-2, 4))
    k_exps = (0, 1) if r.random() < 0.5 else (0,)
    nch = int(r.integers(1, 3 if 1 in k_exps else 5))
    use_modes = bool(r.random() < 0.5)
    split = bool(r.random() < 0.35)
    _log(f"fuzz fp8 seed={seed} B={B} H={H} N={N} D={D} block={block} q_exp={q_exp} k_exps={k_exps} "
         f"nch={nch} modes={use_modes} split={split}")
    q, k, v, scale = _pow2_inputs(B, H, N, D, seed, q_exp, k_exps, nch)
    nB = -(-N // block)
    rp, ci = synth.random_block_lists(B, H, nB, seed=seed + 1, density=float(r.uniform(0.2, 1.0)),
                                      empty_rows=min(1, B * H * nB), full_rows=min(1, max(0, B * H * nB - 1)))
    qkv = bsa.quantize_fp8(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v))
    ref = oracle.quantize_fp8(q, k, v)
    kw = {"scale": scale}
    modes = r.integers(0, 3, size=H).astype(np.int8) if use_modes else None
    if modes is not None:
        cache = synth.random_qkv(B, H, N, D, seed=seed + 2)[0]
        lse_c = np.random.default_rng(seed + 3).standard_normal((B, H, N)).astype(np.float32)
        kw.update(head_modes=modes, o_cache=to_dev_bf16(cache), lse_cache=torch.from_numpy(lse_c).to(dev()))
    if split:
        kw["split"] = {"chunk_blocks": int(r.integers(1, 4)), "max_chunks": int(r.integers(2, 5)),
                       "max_split_rows": int(r.integers(1, 64))}
    O, L = bsa.forward_fp8(qkv, block, _i32(rp), _i32(ci), **kw)
    torch.cuda.synchronize()
    Oo, Lo = oracle.forward_fp8(*ref, block, rp, ci, scale=scale)
    comp = np.ones(H, bool) if modes is None else modes != bsa.HEAD_SKIP
    Og, Lg = bf16_to_f64(O), L.cpu().numpy().astype(np.float64)
    vmax = np.abs(synth.bf16_to_f32(v)).max(axis=2, keepdims=True)
    tol = 2.0 ** -8 * np.abs(Oo) + 1e-4 * vmax
    bad = (np.abs(Og - Oo) > tol)[:, comp]
    assert not bad.any(), f"{bad.sum()} outputs off; worst {np.abs(Og - Oo)[:, comp].max():.3e}"
    fin = np.isfinite(Lo[:, comp])
    np.testing.assert_array_equal(np.isfinite(Lg[:, comp]), fin)
    np.testing.assert_allclose(Lg[:, comp][fin], Lo[:, comp][fin], rtol=0, atol=3e-5)
    if modes is not None and (~comp).any():
        np.testing.assert_array_equal(bf16_bits(O)[:, ~comp], cache[:, ~comp])
        np.testing.assert_array_equal(L.cpu().numpy()[:, ~comp], lse_c[:, ~comp])


# ---------------------------------------------------------------------------
# 2-D neighbourhood geometries: permutation and layout bit for bit, and the
# natural-order forward against the oracle's per-token masked softmax
# ---------------------------------------------------------------------------
def _random_geometry(r):
    block = int(r.choice([64, 128]))
    tw = int(r.choice([8, 16, 32, 64] + ([128] if block == 128 else [])))
    th = block // tw
    R = th * int(r.integers(1, max(2, 48 // th + 1)))
    C = tw * int(r.integers(1, max(2, 256 // tw + 1)))
    while R * C > 4096:
        R, C = (R - th, C) if R > th else (R, C - tw)
    T = block * int(r.integers(0, 3))
    window = (int(r.integers(1, R + 1)), int(r.integers(1, C + 1)))
    stride = (int(r.integers(1, min(4, window[0]) + 1)), int(r.integers(1, min(4, window[1]) + 1)))
    return T, (R, C), (th, tw), window, stride, block


@pytest.mark.parametrize("seed", range(1400, 1424))
def test_fuzz_neighborhood(seed):
    r = np.random.default_rng(seed)
    T, grid, tile, window, stride, block = _random_geometry(r)
    D = int(r.choice([64, 128]))
    B, H = int(r.integers(1, 3)), int(r.integers(1, 3))
    N = T + grid[0] * grid[1]
    _log(f"fuzz neighbourhood seed={seed} T={T} grid={grid} tile={tile} window={window} stride={stride} D={D}")
    nb = bsa.neighborhood(T, grid, tile, window, stride)
    q, k, v = synth.random_qkv(B, H, N, D, seed=seed)
    perm = oracle.tile_permutation(T, grid, tile)
    y = bsa.permute_tokens(to_dev_bf16(q), nb)
    rp, ci, fl = bsa.build_neighborhood_layout(B, H, nb, device=dev())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_bits(y), q[:, :, perm])
    rpo, cio, flo = oracle.neighborhood_layout(T, grid, tile, window, stride)
    nnz = int(rpo[-1])
    want_rp = np.concatenate([[0]] + [rpo[1:] + h * nnz for h in range(B * H)])
    np.testing.assert_array_equal(rp.cpu().numpy(), want_rp)
    np.testing.assert_array_equal(ci.cpu().numpy()[:B * H * nnz], np.tile(cio, B * H))
    np.testing.assert_array_equal(fl.cpu().numpy()[:B * H * nnz], np.tile(flo.astype(np.int32), B * H))
    # the forward on natural-order tensors (gathered and scattered by the kernel)
    O, L = bsa.forward_neighborhood(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), rp, ci, fl, nb, natural=True)
    torch.cuda.synchronize()
    Oo, Lo = oracle.forward_neighborhood(q, k, v, T, grid, window, stride)
    check_forward(bf16_to_f64(O), L.cpu().numpy().astype(np.float64), Oo, Lo, f"neighbourhood fuzz {seed}")


# ---------------------------------------------------------------------------
# backward, exact avgpool scores and the score gradient
# ---------------------------------------------------------------------------
def _rel_close(got, want, max_rel, mean_rel, what):
    d = np.abs(got - want)
    mx = float(d.max()) / max(float(np.abs(want).max()), 1e-30)
    mean = float(d.mean()) / max(float(np.abs(want).mean()), 1e-30)
    assert mx <= max_rel and mean <= mean_rel, f"{what}: max {mx:.2e}, mean {mean:.2e}"


@pytest.mark.parametrize("seed", range(1500, 1516))
def test_fuzz_backward(seed):
    """Tolerances as for the hand-picked backward cases: bf16 P, dS and
    gradients leave a few 2^-9 of each gradient's size (2e-2 of its largest
    element, 1e-2 of its mean magnitude)."""
    r = np.random.default_rng(seed)
    block = int(r.choice([64, 128]))
    D = int(r.choice([64, 128]))
    B, H = int(r.integers(1, 3)), int(r.integers(1, 3))
    N = int(r.integers(1, 5 * block))
    scale = float(r.uniform(0.05, 0.15)) if r.random() < 0.5 else None
    _log(f"fuzz backward seed={seed} B={B} H={H} N={N} D={D} block={block} scale={scale}")
    q, k, v = synth.random_qkv(B, H, N, D, seed=seed)
    g = synth.random_qkv(B, H, N, D, seed=seed + 50)[0]
    nB = -(-N // block)
    rp, ci = synth.random_block_lists(B, H, nB, seed=seed + 1, density=float(r.uniform(0.2, 1.0)),
                                      empty_rows=min(1, B * H * nB), full_rows=min(1, max(0, B * H * nB - 1)))
    qd, kd, vd, gd = (to_dev_bf16(a) for a in (q, k, v, g))
    rpd, cid = _i32(rp), _i32(ci)
    O, L = bsa.forward(qd, kd, vd, block, rpd, cid, scale=scale)
    dq, dk, dv = bsa.backward(qd, kd, vd, O, gd, block, rpd, cid, L, scale=scale)
    torch.cuda.synchronize()
    wq, wk, wv = oracle.backward(q, k, v, g, block, rp, ci, scale=scale)
    for got, want, name in ((dq, wq, "dQ"), (dk, wk, "dK"), (dv, wv, "dV")):
        if np.abs(want).max() == 0:
            assert torch.all(got == 0), name
        else:
            _rel_close(bf16_to_f64(got), want, 2e-2, 1e-2, f"fuzz {seed} {name}")


@pytest.mark.parametrize("seed", range(1600, 1612))
def test_fuzz_exact_scores(seed):
    """fp32 sums of exp2 against the fp64 oracle: 2e-5 of each row's
    largest score, as for the hand-picked cases."""
    r = np.random.default_rng(seed)
    block = int(r.choice([64, 128]))
    D = int(r.choice([64, 128]))
    B, H = int(r.integers(1, 3)), int(r.integers(1, 3))
    N = int(r.integers(1, 8 * block))
    sigma = float(r.uniform(0.5, 2.0))
    _log(f"fuzz exact scores seed={seed} B={B} H={H} N={N} D={D} block={block} sigma={sigma:.2f}")
    q, k, _ = synth.random_qkv(B, H, N, D, seed=seed, scale=sigma)
    S = bsa.pool_scores(to_dev_bf16(q), to_dev_bf16(k), block, bsa.SCORE_EXACT_AVGPOOL)
    torch.cuda.synchronize()
    So = oracle.scores_exact_avgpool(q, k, block)
    err = np.abs(S.cpu().numpy().astype(np.float64) - So) / np.abs(So).max(axis=-1, keepdims=True)
    assert err.max() <= 2e-5, f"max rel err {err.max():.2e}"


@pytest.mark.parametrize("seed", range(1700, 1712))
def test_fuzz_score_grad(seed):
    """fp32 throughout: 1e-4 of the largest element, 1e-5 of the mean
    magnitude, as for the hand-picked cases."""
    r = np.random.default_rng(seed)
    block = int(r.choice([64, 128]))
    D = int(r.choice([64, 128]))
    B, H = int(r.integers(1, 3)), int(r.integers(1, 3))
    N = int(r.integers(1, 8 * block))
    rr = int(r.integers(1, 65))
    _log(f"fuzz score grad seed={seed} B={B} H={H} N={N} D={D} block={block} r={rr}")
    q, k, _ = synth.random_qkv(B, H, N, D, seed=seed)
    w = (r.standard_normal((D, rr)) / np.sqrt(D)).astype(np.float32)
    nB = -(-N // block)
    dS = r.standard_normal((B, H, nB, nB)).astype(np.float32)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())
    dw, dqp, dkp = bsa.score_grad(to_dev_bf16(q), to_dev_bf16(k), block, t(w), t(dS), pooled=True)
    torch.cuda.synchronize()
    wdw, wdq, wdk = oracle.score_grad(q, k, block, w, dS.astype(np.float64))
    for got, want, name in ((dw, wdw, "dW"), (dqp, wdq, "dQ pooled"), (dkp, wdk, "dK pooled")):
        _rel_close(got.cpu().numpy().astype(np.float64), want, 1e-4, 1e-5, f"fuzz {seed} {name}")


# ---------------------------------------------------------------------------
# the XCD work order (a multiple of 8 heads and more than 16 query blocks:
# the leading blocks query-block-major, the rest head by head per XCD)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,H,nB,block,D,seed", [
    (1, 8, 17, 64, 64, 1800),      # one row per head after the leading blocks
    (2, 4, 40, 64, 128, 1801),
    (1, 16, 21, 128, 64, 1802),
])
def test_work_order_many_heads(B, H, nB, block, D, seed):
    N = nB * block - 5
    _log(f"work order B={B} H={H} nB={nB} block={block} D={D}")
    q, k, v = synth.random_qkv(B, H, N, D, seed=seed)
    g = synth.random_qkv(B, H, N, D, seed=seed + 50)[0]
    rp, ci = synth.random_block_lists(B, H, nB, seed=seed + 1, density=0.4, empty_rows=2, full_rows=2)
    qd, kd, vd, gd = (to_dev_bf16(a) for a in (q, k, v, g))
    rpd, cid = _i32(rp), _i32(ci)
    O, L = bsa.forward(qd, kd, vd, block, rpd, cid)
    dq, dk, dv = bsa.backward(qd, kd, vd, O, gd, block, rpd, cid, L)
    torch.cuda.synchronize()
    Oo, Lo = oracle.forward(q, k, v, block, rp, ci)
    check_forward(bf16_to_f64(O), L.cpu().numpy().astype(np.float64), Oo, Lo, "work order forward")
    wq, wk, wv = oracle.backward(q, k, v, g, block, rp, ci)
    for got, want, name in ((dq, wq, "dQ"), (dk, wk, "dK"), (dv, wv, "dV")):
        _rel_close(bf16_to_f64(got), want, 2e-2, 1e-2, f"work order {name}")
    # FP8 on the exact-weight construction
    q8, k8, v8, scale = _pow2_inputs(B, H, N, D, seed, 0, (0,), 4)
    qkv = bsa.quantize_fp8(to_dev_bf16(q8), to_dev_bf16(k8), to_dev_bf16(v8))
    O8, L8 = bsa.forward_fp8(qkv, block, rpd, cid, scale=scale)
    torch.cuda.synchronize()
    Oo8, Lo8 = oracle.forward_fp8(*oracle.quantize_fp8(q8, k8, v8), block, rp, ci, scale=scale)
    vmax = np.abs(synth.bf16_to_f32(v8)).max(axis=2, keepdims=True)
    assert not (np.abs(bf16_to_f64(O8) - Oo8) > 2.0 ** -8 * np.abs(Oo8) + 1e-4 * vmax).any()
    fin = np.isfinite(Lo8)
    np.testing.assert_allclose(L8.cpu().numpy()[fin], Lo8[fin], rtol=0, atol=3e-5)
