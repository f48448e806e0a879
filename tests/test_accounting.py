"""The FLOP/byte accounting and workload shapes against figures the pages print."""
import json
import os

import numpy as np
import pytest

from exact_attention_25_amd import accounting as acc
from exact_attention_25_amd import inputs

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def _close(x, ref, rel):
    assert abs(x - ref) <= rel * abs(ref) + 1e-30, (x, ref)


def test_forward_flops_figure():
    g = GOLD["fwd_flops_n4096_d128_one_head"]
    _close(acc.fwd_flops(1, 1, 4096, 4096, 128), g["value"], g["rel_tol"])
    assert acc.fwd_flops(1, 1, 4096, 4096, 128) == 4 * 4096 ** 2 * 128
    assert acc.fwd_flops(2, 3, 8, 8, 4, causal=True) == acc.fwd_flops(2, 3, 8, 8, 4) / 2
    g = GOLD["fused_time_a100_ms"]
    _close(acc.fwd_flops(1, 1, 4096, 4096, 128) / (g["peak_tflops"] * 1e12) * 1e3, g["value"], g["rel_tol"])


def test_unfused_io_figure():
    g = GOLD["unfused_io_bytes_n4096_d128_fp16"]
    _close(acc.unfused_io_elements(4096, 128) * g["elem_bytes"], g["value"], g["rel_tol"])
    g = GOLD["unfused_time_a100_ms"]
    _close(g["bytes"] / (g["hbm_gbs"] * 1e9) * 1e3, g["value"], g["rel_tol"])


def test_score_matrix_figure():
    g = GOLD["score_matrix_b8_h32_n4096_fp32_bytes"]
    assert acc.score_matrix_bytes(8, 32, 4096) == g["value_gib"] * 2 ** 30


def test_workload_shapes_from_pages():
    g = GOLD["vit_tokens"]
    assert (g["img"] // g["patch"]) ** 2 == g["value"]
    assert inputs.WORKLOADS["vit_bf16_b128_h16_n196_d64"].Nq == g["value"]
    g = GOLD["unet_latent_tokens_512px"]
    assert g["latent_side"] ** 2 == g["value"]
    assert inputs.WORKLOADS["unet_self_fp16_b2_h8_n4096_d40"].Nq == g["value"]


def test_useful_pairs_brute_force():
    rng = np.random.default_rng(3)
    for causal in (False, True):
        N = 13
        lens = rng.integers(0, N + 1, size=4)
        brute = 0
        for L in lens:
            for i in range(N):
                for j in range(N):
                    if j < L and (not causal or j <= i):
                        brute += 1
        assert acc.useful_pairs(N, N, lens, causal, B=4) == brute


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38, 1e-40], dtype=np.float32)
    v = inputs.bf16_value(inputs.bf16_bits(x))
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3*2^-8 ties between 1+2^-7 and 1+2^-6 -> 1 + 2^-6 (even)
    assert list(v[:4]) == [1.0, 1.0, 1.0 + 2 ** -6, -2.5]
    assert np.isfinite(v[4])


def test_generators_are_seeded_and_exact():
    w = inputs.WORKLOADS["tiny_fp32_b1_h2_n128_d64"]
    a, b = inputs.make_inputs(w), inputs.make_inputs(w)
    assert np.array_equal(a["q"], b["q"]) and not np.array_equal(a["q"], a["k"])
    w16 = w.with_(dtype="fp16")
    c = inputs.make_inputs(w16)
    assert np.array_equal(c["q"], c["q_raw"].astype(np.float32))
    wb = w.with_(dtype="bf16")
    d = inputs.make_inputs(wb)
    assert np.array_equal(d["q"], inputs.bf16_value(d["q_raw"]))
    lens = inputs.draw_lens(31, 1000, 20, 77)
    assert lens.min() >= 20 and lens.max() <= 77
