"""Pins of the FP8 oracle (oracle/fp8_ref.py) against things other than itself.

CPU only.
* The E4M3FN code table against values the format's definition fixes
  (1.0, 448, the smallest normal and subnormal, NaN patterns) and its
  invariants (254 finite codes, monotone positive half, exact round trip).
* The encoder against torch's float8_e4m3fn cast (a library routine) on
  values across every binade, ties included, bit for bit.
* Block quantisation: each block's largest magnitude maps to +-448, the
  dequantised error stays within half a unit in the last place, all-zero
  blocks, ragged last blocks, blocks never mix heads or rows of other blocks.
* ref_fwd_fp8 against ref_fwd on the dequantised values, and on inputs whose
  values are exactly representable (quantisation then changes nothing).
"""
import math

import numpy as np
import pytest

from oracle import ref_fwd
from oracle.fp8_ref import (BLOCK, E4M3_MAX, dequantize_blocks, e4m3_decode, e4m3_encode,
                            quantize_blocks, ref_fwd_fp8)

RNG = np.random.default_rng(808)


def test_code_table_fixed_values():
    d = e4m3_decode(np.arange(256, dtype=np.uint8))
    assert d[0x38] == 1.0 and d[0xB8] == -1.0
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0          # largest finite
    assert d[0x08] == 2.0 ** -6                             # smallest normal
    assert d[0x01] == 2.0 ** -9                             # smallest subnormal
    assert d[0x07] == 7 * 2.0 ** -9                         # largest subnormal
    assert d[0x40] == 2.0 and d[0xC4] == -3.0 and d[0x30] == 0.5
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert d[0x00] == 0.0 and d[0x80] == 0.0 and math.copysign(1, d[0x80]) == -1
    fin = np.isfinite(d)
    assert fin.sum() == 254
    pos = d[:0x7F]
    assert np.all(np.diff(pos) > 0)                          # 0x00..0x7E increasing


def test_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def test_encoder_equals_torch_float8_cast():
    torch = pytest.importorskip("torch")
    x = np.concatenate([
        RNG.standard_normal(60000) * np.exp2(RNG.uniform(-14, 9, 60000)),
        np.arange(-448, 448.25, 0.25),
        np.exp2(np.arange(-12, 9, 0.125)),
        # midpoints between neighbouring codes (ties) and their neighbours
        (e4m3_decode(np.arange(0, 0x7E)) + e4m3_decode(np.arange(1, 0x7F))) / 2,
        [0.0, -0.0, 2 ** -10, 3 * 2 ** -11, 447.9, 463.9, 464.0, 470.0],
    ]).astype(np.float32)
    x = x[np.abs(x) <= 470]
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(x), want)


def test_ties_go_to_even_and_overflow_is_nan():
    assert e4m3_encode(np.float32(1.0625)) == 0x38          # between 1 and 1.125: even (1)
    assert e4m3_encode(np.float32(1.1875)) == 0x3A          # between 1.125 and 1.25: even (1.25)
    assert e4m3_encode(np.float32(2.0 ** -10)) == 0x00      # half the smallest subnormal
    assert e4m3_encode(np.float32(460.0)) == 0x7E
    assert e4m3_encode(np.float32(470.0)) == 0x7F


@pytest.mark.parametrize("N", [64, 130, 1])
def test_block_quantisation(N):
    B, H, d = 2, 3, 24
    x = RNG.standard_normal((B, H, N, d)) * np.exp2(RNG.uniform(-3, 3, (B, H, 1, 1)))
    x[1, 2] = 0.0                                            # an all-zero head
    codes, scales = quantize_blocks(x)
    nb = -(-N // BLOCK)
    assert codes.shape == x.shape and scales.shape == (B, H, nb)
    v = e4m3_decode(codes)
    x32 = x.astype(np.float32)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                blk = x32[b, h, i * BLOCK:(i + 1) * BLOCK]
                vb = v[b, h, i * BLOCK:(i + 1) * BLOCK]
                amax = float(np.abs(blk).max())
                if amax == 0:
                    assert scales[b, h, i] == 1.0 and np.all(vb == 0)
                    continue
                assert scales[b, h, i] == np.float32(amax) / np.float32(448)
                # the block's largest magnitude lands on +-448
                j = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
                assert abs(vb[j]) == E4M3_MAX
                # half an ulp: 2^-4 relative in the normal range, 2^-10 below it
                y = blk.astype(np.float64) / float(scales[b, h, i])
                tol = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) * 1.0001
                assert np.all(np.abs(vb - y) <= tol)
    deq = dequantize_blocks(codes, scales)
    rel = np.abs(deq - x) / np.maximum(np.abs(x), 1e-30)
    assert np.median(rel[np.abs(x) > 0.5]) < 2.0 ** -5


def test_attention_on_dequantised_values():
    B, Hq, Hkv, N, d = 1, 4, 2, 100, 32
    q, k, v = (RNG.standard_normal((B, h, N, d)) for h in (Hq, Hkv, Hkv))
    (qc, qs), (kc, ks), (vc, vs) = (quantize_blocks(t) for t in (q, k, v))
    O, L = ref_fwd_fp8(qc, kc, vc, qs, ks, vs, causal=True)
    O2, L2 = ref_fwd(dequantize_blocks(qc, qs), dequantize_blocks(kc, ks),
                     dequantize_blocks(vc, vs), causal=True)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(L, L2)
    # the inputs' quantisation moves O by a few percent: causal row 0 is v_0
    # itself, off by at most half an ulp (2^-4 relative)
    O3, _ = ref_fwd(q, k, v, causal=True)
    assert np.all(np.abs(O[:, :, 0] - O3[:, :, 0]) <= 2.0 ** -4 * np.abs(O3[:, :, 0]) + 1e-12)
    assert np.abs(O - O3).max() < 0.25 and np.sqrt(np.mean((O - O3) ** 2)) < 0.03


def test_representable_inputs_are_unchanged():
    """Values that are E4M3 codes times a power of two, with one 448-sized
    entry per block, quantise exactly: the FP8 reference equals ref_fwd."""
    B, H, N, d = 1, 2, 64, 16
    pool = e4m3_decode(np.array([0x30, 0x38, 0x3C, 0x40, 0x44, 0xB8, 0xC0, 0x00], np.uint8))
    x = [RNG.choice(pool, size=(B, H, N, d)) for _ in range(3)]
    for t in x:
        t[:, :, 0, 0] = 448.0                                # block amax 448 -> scale 1
    codes = [quantize_blocks(t) for t in x]
    for (c, s), t in zip(codes, x):
        assert np.all(s == 1.0) and np.array_equal(e4m3_decode(c), t)
    O, L = ref_fwd_fp8(*(c for c, _ in codes), *(s for _, s in codes), scale=0.01)
    O2, L2 = ref_fwd(*x, scale=0.01)
    np.testing.assert_allclose(O, O2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, L2, rtol=0, atol=1e-12)
