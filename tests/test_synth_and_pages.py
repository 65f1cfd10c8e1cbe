"""Generator determinism / bf16 rounding, and the workload shapes against
the values the pages print (tests/golden/page_workloads.json)."""
import json
import math
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_workloads.json")


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0, -0.0, 1e-40, 3.0e38],
                 dtype=np.float32)
    b = synth.f32_to_bf16(x)
    y = synth.bf16_to_f32(b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3*2^-8 ties between 1 + 2^-7 and 1 + 2^-6: 1 + 2^-6 is even
    np.testing.assert_array_equal(y[:4], [1.0, 1.0, 1.0 + 2 ** -6, -2.5])
    assert b[4] == 0x0000 and b[5] == 0x8000
    # widening is exact and round-tripping is idempotent
    np.testing.assert_array_equal(synth.f32_to_bf16(y), b)


def test_workload_generation_is_deterministic():
    wl = synth.WORKLOADS["C1"]
    a = synth.make_inputs(wl)
    b = synth.make_inputs(wl)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])
    c = synth.make_inputs(wl, seed=99)
    assert not np.array_equal(a["q"], c["q"])
    assert a["q"].shape == (1, 2, 512, 64) and a["w"].shape == (64, 32)


def test_arrow_modes_counts_and_caches():
    # a reduced copy of C2 (square image grid) keeps the head-mode recipe
    wl = synth.WORKLOADS["C2"].replace(N=256 + 1024, text_len=256, H=24)
    x = synth.make_inputs(wl)
    m = x["head_modes"]
    assert (m == synth.HEAD_ARROW).sum() == 12 and (m == synth.HEAD_FULL).sum() == 8
    assert (m == synth.HEAD_SKIP).sum() == 4
    assert x["o_cache"].shape == x["q"].shape and x["lse_cache"].shape == x["q"].shape[:3]


def test_positional_structure_raises_neighbour_logits():
    wl = synth.WORKLOADS["C2"].replace(N=256 + 1024, text_len=256, H=2, arrow_counts=(2, 0, 0))
    x = synth.make_inputs(wl)
    q = synth.bf16_to_f32(x["q"][0, 0, 256:]).astype(np.float64)
    k = synth.bf16_to_f32(x["k"][0, 0, 256:]).astype(np.float64)
    z = (q * k).sum(-1)                       # co-located query/key pairs
    zf = (q * np.roll(k, 16 * 32, axis=0)).sum(-1)   # 16 grid rows away
    # co-located pairs gain amp^2 * D / 2 = 36 on average; 16 grid rows away
    # only the column half (about 18) survives
    assert abs(z.mean() - 36.0) < 3.0
    assert z.mean() > zf.mean() + 12


def test_workload_shapes_match_page_token_counts():
    g = json.load(open(GOLDEN))
    tc = g["token_counts"]
    c2, c4 = synth.WORKLOADS["C2"], synth.WORKLOADS["C4"]
    assert c2.N == tc["FLUX.1 1024^2"]["sequence"] and c2.text_len == tc["FLUX.1 1024^2"]["text_tokens"]
    assert c4.N == tc["FLUX.1 2048^2"]["sequence"] and c4.text_len == tc["FLUX.1 2048^2"]["text_tokens"]
    for key in tc:
        if key.startswith("_"):
            continue
        e = tc[key]
        lat = e["latent"]
        # patch size 2 on the latent grid
        assert (lat[1] // 2) * (lat[2] // 2) == e["image_tokens"]
        assert e["image_tokens"] + e["text_tokens"] == e["sequence"]
    # the image part of C2 / C4 is a square grid of exactly those tokens
    assert math.isqrt(c2.N - c2.text_len) ** 2 == tc["FLUX.1 1024^2"]["image_tokens"]
    assert math.isqrt(c4.N - c4.text_len) ** 2 == tc["FLUX.1 2048^2"]["image_tokens"]
    d = g["dit_latent_example"]
    assert d["image_tokens"] ** 2 * 2 == d["attn_map_bytes_fp16"]


def test_sparsed_budgets_follow_rho():
    g = json.load(open(GOLDEN))["sparsed_long_context"]
    c5 = synth.WORKLOADS["C5"]
    assert c5.block == g["block_size"]
    for (c0, c1, kk) in c5.groups:
        assert kk == math.ceil(g["rho"] * (c1 - c0) - 1e-9)
    # 61440 prefill + 4096 generation tokens -> 480 + 32 blocks
    assert c5.groups[0][1] * c5.block == 61440 and (c5.groups[1][1] - c5.groups[1][0]) * c5.block == 4096
