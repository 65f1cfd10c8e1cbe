"""Pins of the oracle's FP8 (OCP E4M3) codec, scaled quantisation and
forward on quantised inputs, against the format's definition and against
the bf16 forward.

E4M3 (OCP 8-bit floating point specification): sign, 4 exponent bits with
bias 7, 3 mantissa bits; exponent field 0 encodes subnormals m * 2^-9; the
all-ones pattern S.1111.111 is NaN and there are no infinities; the largest
finite magnitude is 1.75 * 2^8 = 448."""
import math

import numpy as np
import pytest

import oracle
import synth


def _values_by_definition():
    """Value of every code from the bit fields, written out independently."""
    vals = np.empty(256)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            v = float("nan")
        elif e == 0:
            v = m * 2.0 ** -9
        else:
            v = (1 + m / 8) * 2.0 ** (e - 7)
        vals[c] = -v if s else v
    return vals


def test_e4m3_decode_matches_bit_fields():
    want = _values_by_definition()
    got = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    np.testing.assert_array_equal(got[ok], want[ok])
    # landmarks of the format
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9
    assert got[0x08] == 2.0 ** -6 and got[0x44] == 3.0 and got[0xC4] == -3.0
    assert np.all(np.diff(got[:0x7F]) > 0)     # codes 0x00..0x7E increase


@pytest.mark.parametrize("x,code", [
    (1.0, 0x38), (448.0, 0x7E), (-448.0, 0xFE), (2.0 ** -9, 0x01), (2.0 ** -6, 0x08),
    (1.0625, 0x38),           # tie between 1.0 and 1.125 -> even mantissa
    (1.1875, 0x3A),           # tie between 1.125 and 1.25 -> even mantissa
    (1.5 * 2.0 ** -9, 0x02),  # subnormal tie -> even
    (0.5 * 2.0 ** -9, 0x00),  # tie with zero -> zero
    (460.0, 0x7E),            # inside the rounding range of 448
    (470.0, 0x7F),            # beyond it: NaN (no saturation)
    (0.0, 0x00), (-0.0, 0x80),
])
def test_e4m3_encode_landmarks(x, code):
    assert int(oracle.e4m3_encode(np.array([x], np.float32))[0]) == code


def test_e4m3_encode_is_nearest_ties_to_even():
    """Brute force: nearest of the 127 finite magnitudes, ties to the code
    with an even mantissa, sign carried over."""
    vals = _values_by_definition()[:0x7F]
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 40, rng.standard_normal(5000) * 0.01,
                        (vals[:-1] + vals[1:]) / 2,                      # every midpoint
                        rng.uniform(-448, 448, 5000)]).astype(np.float32)
    a = np.abs(x.astype(np.float64))
    d = np.abs(a[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = (d == best)
    even = cand & ((np.arange(0x7F) & 1) == 0)[None, :]
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    want = pick | np.where(np.signbit(x), 0x80, 0)
    np.testing.assert_array_equal(oracle.e4m3_encode(x), want.astype(np.uint8))


def test_e4m3_roundtrip_every_finite_code():
    c = np.arange(256, dtype=np.uint8)
    v = oracle.e4m3_decode(c)
    fin = ~np.isnan(v)
    np.testing.assert_array_equal(oracle.e4m3_encode(v[fin].astype(np.float32)), c[fin])


def _bf16_vals(u16):
    return synth.bf16_to_f32(u16).astype(np.float64)


def test_quantize_fp8_groups_and_error_bound():
    B, H, N, D = 1, 2, 150, 64            # a partial last K tile (150 = 2*64 + 22)
    q, k, v = synth.random_qkv(B, H, N, D, seed=7)
    q8, qs, k8, ks, v8, vs = oracle.quantize_fp8(q, k, v)
    dec = lambda c: oracle.e4m3_decode(c)
    Q, K, V = _bf16_vals(q), _bf16_vals(k), _bf16_vals(v)
    # scales: amax / 448 per token (Q), per 64-key tile (K), per channel (V), in fp32
    np.testing.assert_array_equal(qs, (np.abs(Q).max(axis=-1).astype(np.float32) / np.float32(448)))
    tiles = [np.abs(K[:, :, t:t + 64]).max(axis=(-1, -2)) for t in range(0, N, 64)]
    np.testing.assert_array_equal(ks, (np.stack(tiles, -1).astype(np.float32) / np.float32(448)))
    np.testing.assert_array_equal(vs, (np.abs(V).max(axis=2).astype(np.float32) / np.float32(448)))
    # every group's largest magnitude maps to +-448 exactly, all codes finite
    for codes in (q8, k8, v8):
        assert not np.isnan(dec(codes)).any()
    assert np.all(np.abs(dec(q8)).max(axis=-1) == 448.0)
    assert np.all(np.abs(dec(v8)).max(axis=2) == 448.0)
    # dequantised error: half an ulp (2^-4 relative) or half a subnormal step
    for X, c, sc in ((Q, q8, qs[..., None]), (V, v8, vs[:, :, None, :])):
        err = np.abs(dec(c) * sc - X)
        assert np.all(err <= 2.0 ** -4 * np.abs(X) * (1 + 1e-6) + sc * 2.0 ** -10 + 1e-30)
    ksc = np.repeat(ks, 64, axis=-1)[:, :, :N, None]
    err = np.abs(dec(k8) * ksc - K)
    assert np.all(err <= 2.0 ** -4 * np.abs(K) * (1 + 1e-6) + ksc * 2.0 ** -10 + 1e-30)


def test_quantize_fp8_zero_group():
    B, H, N, D = 1, 1, 64, 64
    z = np.zeros((B, H, N, D), np.uint16)
    q8, qs, k8, ks, v8, vs = oracle.quantize_fp8(z, z, z)
    assert not q8.any() and not k8.any() and not v8.any()
    assert not qs.any() and not ks.any() and not vs.any()


def test_forward_fp8_reduces_to_bf16_forward_when_exact():
    """Inputs that are E4M3 values whose group maxima are exactly 448 quantise
    with scale 1 and no rounding, so the FP8 forward must equal the bf16 one."""
    B, H, N, D, block = 1, 2, 160, 64, 64
    rng = np.random.default_rng(3)
    fin = _values_by_definition()[:0x7E]         # finite magnitudes below 448
    pick = lambda shape: (fin[rng.integers(0, len(fin), shape)] * rng.choice([-1, 1], shape))
    Q, K, V = pick((B, H, N, D)), pick((B, H, N, D)), pick((B, H, N, D))
    Q[..., 0] = 448.0                            # per-token maxima
    for t in range(0, N, 64):
        K[:, :, t, 0] = 448.0                    # per-tile maxima
    V[:, :, 0, :] = -448.0                       # per-channel maxima
    to_bf16 = lambda X: synth.f32_to_bf16(X.astype(np.float32))
    q, k, v = to_bf16(Q), to_bf16(K), to_bf16(V)
    q8, qs, k8, ks, v8, vs = oracle.quantize_fp8(q, k, v)
    assert np.all(qs == 1.0) and np.all(ks == 1.0) and np.all(vs == 1.0)
    nB = -(-N // block)
    rp, ci = synth.random_block_lists(B, H, nB, seed=4, density=0.6, empty_rows=1)
    scale = 2e-6                                 # keeps the logits of order one
    O8, L8 = oracle.forward_fp8(q8, qs, k8, ks, v8, vs, block, rp, ci, scale=scale)
    O, L = oracle.forward(q, k, v, block, rp, ci, scale=scale)
    np.testing.assert_allclose(O8, O, rtol=1e-12, atol=1e-9)
    np.testing.assert_allclose(L8, L, rtol=1e-12, atol=1e-12)
