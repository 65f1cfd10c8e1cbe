"""GPU parity of the FP8 (E4M3) path against the fp64 CPU oracle.

* Quantisation: codes and scales bit-exact against oracle.quantize_fp8 (the
  V codes read back through the transposed, key-permuted layout).
* Forward, exact-weight construction: inputs whose logits (log2 units) are
  small integers, so every probability is a power of two that E4M3 holds
  exactly; the kernel's rounding of P is then exact and its output must
  match oracle.forward_fp8 to fp32 / bf16 rounding.  This pins every layout
  (Q, K, permuted V^T), every scale and the row sums.
* Forward, random N(0, 1) inputs: against oracle.forward_fp8 with the
  statistical tolerance of rounding P to E4M3, and against the bf16 oracle
  on the unquantised inputs (quantisation error included).
* The 2K MMDiT arrow workload at full size on sampled rows."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import block_sparse_attention_18_amd as bsa
from helpers import bf16_to_f64, dev, sample_rows, to_dev_bf16

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

# Rounding P to E4M3 (3 mantissa bits, unit roundoff u = 2^-4) perturbs each
# weight by a relative delta_j with RMS about 0.024; the output error of a
# row is then about 0.024 * sigma_v / sqrt(n_eff) (n_eff = effective number
# of keys; >= 24 for the rows below with N(0, 1) logits), i.e. a standard
# deviation <= 5e-3.  Bounds: max 8 sigma, mean 1 sigma, LSE (= ln of the
# relative error of the row sum, same size) 4 sigma.
FP8_O_MAX_ABS = 4e-2
FP8_O_MEAN_ABS = 5e-3
FP8_LSE_MAX_ABS = 2e-2
# Against the bf16 oracle on the unquantised inputs (a sanity check of the
# whole FP8 mode; the kernel's own arithmetic is gated by the FP8 oracle
# above), rounding Q and K adds a logit error of RMS about 0.034 (natural
# units, sqrt(2) * 0.024 * scale * sqrt(sum_d q_d^2 k_d^2)) and rounding V a
# relative 0.024: the output error is about 0.048 / sqrt(n_eff) <= 1e-2
# (mean bound).  The error is a product of rounding terms and has heavy
# tails, so the max bound is a gross-error catch (15 sigma); the LSE of a
# row that one key dominates moves by that key's logit error (3 x 0.034).
E2E_O_MAX_ABS = 0.15
E2E_O_MEAN_ABS = 1e-2
E2E_LSE_MAX_ABS = 0.1


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def _quantize(q, k, v):
    qkv = bsa.quantize_fp8(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v))
    torch.cuda.synchronize()
    return qkv


def _v8_natural(qkv):
    """V codes [B,H,N,D] gathered from the transposed, key-permuted layout, and
    the padding columns."""
    B, H, N, D = qkv.shape
    v8t = qkv.v8t.cpu().numpy()
    cols = np.array([bsa.v8t_key_column(t) for t in range(N)])
    nat = np.ascontiguousarray(v8t[:, :, :, cols].transpose(0, 1, 3, 2))
    pad = np.setdiff1d(np.arange(v8t.shape[3]), cols)
    return nat, v8t[:, :, :, pad]


def _check_quant(qkv, ref):
    q8, qs, k8, ks, v8, vs = ref
    np.testing.assert_array_equal(qkv.q8.cpu().numpy(), q8)
    np.testing.assert_array_equal(qkv.k8.cpu().numpy(), k8)
    nat, pad = _v8_natural(qkv)
    np.testing.assert_array_equal(nat, v8)
    assert np.all(pad == 0)
    for got, want in ((qkv.q_scale, qs), (qkv.k_scale, ks), (qkv.v_scale, vs)):
        np.testing.assert_array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))


# ---------------------------------------------------------------------------
# quantisation
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,H,N,D,seed", [
    (1, 2, 4 * 64, 128, 301),
    (2, 3, 5 * 64 + 37, 64, 302),
    (1, 1, 17, 128, 303),
    (1, 2, 600, 64, 304),        # several 256-key chunks of the V maxima
])
def test_quantize_bit_exact(B, H, N, D, seed):
    _log(f"quantize B={B} H={H} N={N} D={D}")
    rng = np.random.default_rng(seed)
    q, k, v = synth.random_qkv(B, H, N, D, seed=seed)
    # wide dynamic range, plus an all-zero token, K tile and V channel
    amp = np.exp2(rng.integers(-6, 7, size=(B, H, N, 1))).astype(np.float32)
    q = synth.f32_to_bf16(synth.bf16_to_f32(q) * amp)
    q[0, 0, min(3, N - 1)] = 0
    k[0, -1, 0:min(64, N)] = 0
    v[-1, 0, :, 5] = 0
    qkv = _quantize(q, k, v)
    _check_quant(qkv, oracle.quantize_fp8(q, k, v))


# ---------------------------------------------------------------------------
# forward, exact-weight construction
# ---------------------------------------------------------------------------
def _pow2_inputs(B, H, N, D, seed, q_exp, k_exps, nch):
    """Q scales 2^q_exp, K tile scales 2^b (b from k_exps), and codes in
    {-1, 0, 1} on nch channels: the logit of (query, key) in log2 units is
    an integer dot product of codes times 2^b, at most 4 in magnitude with
    scale = ln(2) / 2^q_exp."""
    rng = np.random.default_rng(seed)
    NT = -(-N // 64)
    b = rng.choice(np.array(k_exps), size=(B, H, NT))
    assert nch * 2.0 ** max(k_exps) <= 4
    q = np.zeros((B, H, N, D), np.float32)
    k = np.zeros((B, H, N, D), np.float32)
    q[..., 0] = 448.0 * 2.0 ** q_exp                     # sets the Q scale; k is 0 there
    q[..., 2:2 + nch] = rng.integers(-1, 2, size=(B, H, N, nch)) * 2.0 ** q_exp
    kb = 2.0 ** b[:, :, np.arange(N) // 64]
    k[..., 2:2 + nch] = rng.integers(-1, 2, size=(B, H, N, nch)) * kb[..., None]
    k[:, :, 0::64, 1] = 448.0 * 2.0 ** b                  # sets each tile's K scale; q is 0 there
    vamp = np.exp2(rng.uniform(-3, 3, size=(1, 1, 1, D))).astype(np.float32)
    v = rng.standard_normal((B, H, N, D)).astype(np.float32) * vamp
    scale = float(np.float32(math.log(2.0) / 2.0 ** q_exp))
    return synth.f32_to_bf16(q), synth.f32_to_bf16(k), synth.f32_to_bf16(v), scale


@pytest.mark.parametrize("B,H,N,D,block,q_exp,k_exps,nch,seed", [
    (1, 2, 4 * 128 + 40, 128, 128, 0, (0,), 4, 311),
    (2, 2, 6 * 64 + 9, 64, 64, 3, (0, 1), 2, 312),
    (1, 3, 3 * 128, 64, 128, -2, (0, 1), 2, 313),
    (1, 2, 5 * 64, 128, 64, 1, (0,), 4, 314),
    (1, 1, 40, 128, 128, 0, (0, 1), 2, 315),
])
def test_forward_fp8_exact_weights(B, H, N, D, block, q_exp, k_exps, nch, seed):
    _log(f"fp8 exact weights B={B} H={H} N={N} D={D} block={block}")
    q, k, v, scale = _pow2_inputs(B, H, N, D, seed, q_exp, k_exps, nch)
    nB = -(-N // block)
    rp, ci = synth.random_block_lists(B, H, nB, seed=seed + 1, density=0.6, empty_rows=1, full_rows=2)
    qkv = _quantize(q, k, v)
    ref = oracle.quantize_fp8(q, k, v)
    _check_quant(qkv, ref)
    assert np.all(ref[1] == 2.0 ** q_exp)
    O, L = bsa.forward_fp8(qkv, block, _i32(rp), _i32(ci), scale=scale)
    torch.cuda.synchronize()
    Oo, Lo = oracle.forward_fp8(*ref, block, rp, ci, scale=scale)
    Og, Lg = bf16_to_f64(O), L.cpu().numpy().astype(np.float64)
    # bf16 rounding of O (2^-9 relative) and fp32 sums of exact products
    # (relative 2^-24 per term, at most N terms, scaled by the channel's range)
    vmax = np.abs(synth.bf16_to_f32(v)).max(axis=2, keepdims=True)
    tol = 2.0 ** -8 * np.abs(Oo) + 1e-4 * vmax
    bad = np.abs(Og - Oo) > tol
    assert not bad.any(), f"{bad.sum()} outputs off; worst {np.abs(Og - Oo).max():.3e}"
    fin = np.isfinite(Lo)
    np.testing.assert_array_equal(np.isfinite(Lg), fin)
    assert np.all(Lg[~fin] == Lo[~fin])
    assert np.all(Og.reshape(-1, D)[~fin.reshape(-1)] == 0)
    np.testing.assert_allclose(Lg[fin], Lo[fin], rtol=0, atol=3e-5)


@pytest.mark.parametrize("B,H,N,D,block,cb,mc,msr,seed", [
    (1, 4, 6 * 128 + 40, 128, 128, 1, 4, 100, 316),      # every multi-block row split
    (2, 3, 9 * 64, 64, 64, 2, 3, 4, 317),                # fewer split slots than long rows
])
def test_forward_fp8_split_and_skip_heads_exact(B, H, N, D, block, cb, mc, msr, seed):
    """SKIP heads copied bit for bit from the caches, and long rows cut into
    chunks and merged, on the exact-weight inputs: the computed heads must
    match the FP8 oracle as tightly as the unsplit forward."""
    _log(f"fp8 split+skip B={B} H={H} N={N} D={D} block={block} chunk={cb}")
    q, k, v, scale = _pow2_inputs(B, H, N, D, seed, 0, (0, 1), 2)
    nB = -(-N // block)
    rp, ci = synth.random_block_lists(B, H, nB, seed=seed + 1, density=0.7, empty_rows=1, full_rows=3)
    modes = np.array([bsa.HEAD_FULL, bsa.HEAD_SKIP] + [bsa.HEAD_ARROW] * (H - 2), np.int8)
    cache = synth.random_qkv(B, H, N, D, seed=seed + 2)[0]
    lse_c = np.random.default_rng(seed + 3).standard_normal((B, H, N)).astype(np.float32)
    qkv = _quantize(q, k, v)
    ref = oracle.quantize_fp8(q, k, v)
    split = {"chunk_blocks": cb, "max_chunks": mc, "max_split_rows": msr}
    O, L = bsa.forward_fp8(qkv, block, _i32(rp), _i32(ci), scale=scale, head_modes=modes,
                           o_cache=to_dev_bf16(cache), lse_cache=torch.from_numpy(lse_c).to(dev()), split=split)
    torch.cuda.synchronize()
    comp = modes != bsa.HEAD_SKIP
    Oo, Lo = oracle.forward_fp8(*ref, block, rp, ci, scale=scale)
    Og, Lg = bf16_to_f64(O), L.cpu().numpy().astype(np.float64)
    vmax = np.abs(synth.bf16_to_f32(v)).max(axis=2, keepdims=True)
    tol = 2.0 ** -8 * np.abs(Oo) + 1e-4 * vmax
    bad = (np.abs(Og - Oo) > tol)[:, comp]
    assert not bad.any(), f"{bad.sum()} outputs off; worst {np.abs(Og - Oo)[:, comp].max():.3e}"
    fin = np.isfinite(Lo[:, comp])
    np.testing.assert_array_equal(np.isfinite(Lg[:, comp]), fin)
    np.testing.assert_allclose(Lg[:, comp][fin], Lo[:, comp][fin], rtol=0, atol=3e-5)
    Ob = O.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(Ob[:, ~comp], cache[:, ~comp])
    np.testing.assert_array_equal(L.cpu().numpy()[:, ~comp], lse_c[:, ~comp])
    # the same without splitting: bit-identical SKIP heads, computed heads within rounding
    O1, L1 = bsa.forward_fp8(qkv, block, _i32(rp), _i32(ci), scale=scale, head_modes=modes,
                             o_cache=to_dev_bf16(cache))
    torch.cuda.synchronize()
    assert float((O1.float() - O.float()).abs().max()) <= 2e-2
    assert torch.isnan(L1[:, torch.from_numpy(~comp)]).all()   # no LSE cache: NaN for SKIP heads


# ---------------------------------------------------------------------------
# forward, random inputs
# ---------------------------------------------------------------------------
def _stats(Og, Lg, Oo, Lo):
    d = np.abs(Og - Oo)
    fin = np.isfinite(Lo)
    np.testing.assert_array_equal(np.isfinite(Lg), fin)
    dl = float(np.abs(Lg[fin] - Lo[fin]).max()) if fin.any() else 0.0
    return float(d.max()), float(d.mean()), dl


@pytest.mark.parametrize("B,H,N,D,block,seed", [
    (2, 3, 4 * 64 + 17, 64, 64, 321),
    (1, 2, 5 * 128 + 3, 128, 128, 322),
    (2, 2, 3 * 128, 64, 128, 323),
    (1, 3, 6 * 64, 128, 64, 324),
])
def test_forward_fp8_random(B, H, N, D, block, seed):
    _log(f"fp8 random B={B} H={H} N={N} D={D} block={block}")
    q, k, v = synth.random_qkv(B, H, N, D, seed=seed)
    nB = -(-N // block)
    rp, ci = synth.random_block_lists(B, H, nB, seed=seed + 1, density=0.5, empty_rows=1, full_rows=2)
    qkv = _quantize(q, k, v)
    ref = oracle.quantize_fp8(q, k, v)
    _check_quant(qkv, ref)
    O, L = bsa.forward_fp8(qkv, block, _i32(rp), _i32(ci))
    torch.cuda.synchronize()
    Og, Lg = bf16_to_f64(O), L.cpu().numpy().astype(np.float64)
    mx, mean, dl = _stats(Og, Lg, *oracle.forward_fp8(*ref, block, rp, ci))
    _log(f"  vs fp8 oracle: max {mx:.2e} mean {mean:.2e} lse {dl:.2e}")
    assert mx <= FP8_O_MAX_ABS and mean <= FP8_O_MEAN_ABS and dl <= FP8_LSE_MAX_ABS
    mx, mean, dl = _stats(Og, Lg, *oracle.forward(q, k, v, block, rp, ci))
    _log(f"  vs bf16 oracle: max {mx:.2e} mean {mean:.2e} lse {dl:.2e}")
    assert mx <= E2E_O_MAX_ABS and mean <= E2E_O_MEAN_ABS and dl <= E2E_LSE_MAX_ABS


def test_forward_fp8_is_deterministic_and_validates():
    B, H, N, D, block = 1, 2, 3 * 128, 128, 128
    q, k, v = synth.random_qkv(B, H, N, D, seed=330)
    rp, ci = synth.random_block_lists(B, H, 3, seed=331, density=0.7)
    qkv = _quantize(q, k, v)
    O1, L1 = bsa.forward_fp8(qkv, block, _i32(rp), _i32(ci))
    O2, L2 = bsa.forward_fp8(qkv, block, _i32(rp), _i32(ci))
    torch.cuda.synchronize()
    assert torch.equal(O1.view(torch.int16), O2.view(torch.int16)) and torch.equal(L1, L2)
    with pytest.raises(bsa.BsaError):
        bsa.forward_fp8(qkv, 96, _i32(rp), _i32(ci))


# ---------------------------------------------------------------------------
# the 2K MMDiT arrow workload at full size
# ---------------------------------------------------------------------------
@pytest.mark.slow
def test_workload_c4_fp8():
    wl = synth.WORKLOADS["C4"]
    x = synth.make_inputs(wl)
    B, H, N, D, block, nB = wl.B, wl.H, wl.N, wl.D, wl.block, wl.n_blocks
    modes, wins = x["head_modes"], x["head_windows"]
    assert np.all(modes == bsa.HEAD_ARROW)
    rp, ci = bsa.build_arrow_layout(B, H, N, block, wl.text_len, modes, wins, device=dev())
    qkv = _quantize(x["q"], x["k"], x["v"])
    O, L = bsa.forward_fp8(qkv, block, rp, ci)
    torch.cuda.synchronize()
    rpo, cio = oracle.arrow(B, H, nB, wl.text_blocks, modes, wins)
    np.testing.assert_array_equal(rp.cpu().numpy(), rpo)
    ref = oracle.quantize_fp8(x["q"], x["k"], x["v"])
    _check_quant(qkv, ref)
    must = [((0 * H + h) * N + t) for h in (0, H - 1) for t in (0, N - 1, 600, N // 2)]
    rows = sample_rows(B, H, N, 256, 340, must)
    Og = bf16_to_f64(O).reshape(-1, D)[rows]
    Lg = L.cpu().numpy().reshape(-1)[rows].astype(np.float64)
    mx, mean, dl = _stats(Og, Lg, *oracle.forward_fp8(*ref, block, rpo, cio, rows=rows))
    _log(f"C4 fp8 vs fp8 oracle: max {mx:.2e} mean {mean:.2e} lse {dl:.2e}")
    assert mx <= FP8_O_MAX_ABS and mean <= FP8_O_MEAN_ABS and dl <= FP8_LSE_MAX_ABS
    mx, mean, dl = _stats(Og, Lg, *oracle.forward(x["q"], x["k"], x["v"], block, rpo, cio, rows=rows))
    _log(f"C4 fp8 vs bf16 oracle: max {mx:.2e} mean {mean:.2e} lse {dl:.2e}")
    assert mx <= E2E_O_MAX_ABS and mean <= E2E_O_MEAN_ABS and dl <= E2E_LSE_MAX_ABS


@pytest.mark.slow
def test_workload_c2_fp8_heads_and_split():
    """The FLUX 1024^2 mix in FP8: 12 arrow, 8 full and 4 SKIP heads, long
    rows split as the bf16 forward splits them."""
    wl = synth.WORKLOADS["C2"]
    x = synth.make_inputs(wl)
    B, H, N, D, block, nB = wl.B, wl.H, wl.N, wl.D, wl.block, wl.n_blocks
    modes, wins = x["head_modes"], x["head_windows"]
    assert (modes == bsa.HEAD_SKIP).sum() == 4
    rp, ci = bsa.build_arrow_layout(B, H, N, block, wl.text_len, modes, wins, device=dev())
    qkv = _quantize(x["q"], x["k"], x["v"])
    split = bsa.arrow_split_policy(B, H, N, block, wl.text_len, modes, wins) or \
        {"chunk_blocks": 9, "max_chunks": 4, "max_split_rows": 1000}
    O, L = bsa.forward_fp8(qkv, block, rp, ci, head_modes=modes, o_cache=to_dev_bf16(x["o_cache"]),
                           lse_cache=torch.from_numpy(x["lse_cache"]).to(dev()), split=split)
    torch.cuda.synchronize()
    rpo, cio = oracle.arrow(B, H, nB, wl.text_blocks, modes, wins)
    np.testing.assert_array_equal(rp.cpu().numpy(), rpo)
    ref = oracle.quantize_fp8(x["q"], x["k"], x["v"])
    skip = modes == bsa.HEAD_SKIP
    Ob = O.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(Ob[:, skip], x["o_cache"][:, skip])
    np.testing.assert_array_equal(L.cpu().numpy()[:, skip], x["lse_cache"][:, skip])
    rows = sample_rows(B, H, N, 4096, 341)
    rows = rows[~skip[(rows // N) % H]]
    Og = bf16_to_f64(O).reshape(-1, D)[rows]
    Lg = L.cpu().numpy().reshape(-1)[rows].astype(np.float64)
    mx, mean, dl = _stats(Og, Lg, *oracle.forward_fp8(*ref, block, rpo, cio, rows=rows))
    _log(f"C2 fp8 vs fp8 oracle ({len(rows)} rows): max {mx:.2e} mean {mean:.2e} lse {dl:.2e}")
    assert mx <= FP8_O_MAX_ABS and mean <= FP8_O_MEAN_ABS and dl <= FP8_LSE_MAX_ABS
