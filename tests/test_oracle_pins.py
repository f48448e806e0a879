"""Pins of the fp64 oracle against things other than itself.

Brute force (pure-Python loops), closed forms, invariants of exact attention,
and the tiled online-softmax model.  CPU only.
"""
import math

import numpy as np
import pytest

from oracle import ref_fwd, ref_probs, ref_fwd_rows, resolve_scale, tiled_fwd
from tests import brute_force

RNG = np.random.default_rng(20261203)


def _rand(*shape, std=1.0):
    return RNG.standard_normal(shape) * std


# ---------------------------------------------------------------- brute force
CASES = [
    # B, Hq, Hkv, Nq, Nk, d, causal, use_mask, use_lens, layout, scale
    (1, 1, 1, 4, 4, 3, False, False, False, "bhnd", None),
    (2, 2, 2, 5, 7, 4, False, False, False, "bhnd", 0.37),
    (1, 2, 1, 6, 6, 3, True, False, False, "bhnd", None),
    (2, 4, 2, 3, 9, 2, False, True, False, "bnhd", None),
    (2, 2, 1, 6, 6, 5, True, True, True, "bnhd", 1.3),
    (3, 2, 2, 4, 8, 3, False, False, True, "bhnd", None),
    (1, 3, 1, 2, 1, 4, False, False, False, "bnhd", None),
]


@pytest.mark.parametrize("case", CASES)
def test_oracle_matches_brute_force(case):
    B, Hq, Hkv, Nq, Nk, d, causal, use_mask, use_lens, layout, scale = case
    q = _rand(B, Hq, Nq, d)
    k = _rand(B, Hkv, Nk, d)
    v = _rand(B, Hkv, Nk, d)
    mask = _rand(B, 1, Nq, Nk) * 2.0 if use_mask else None
    if use_mask:
        mask[0, 0, 0, -1] = -np.inf  # a user -inf entry
    lens = RNG.integers(0, Nk + 1, size=B) if use_lens else None
    if use_lens:
        lens[0] = Nk + 3  # beyond Nk: clamped
    tr = (lambda x: x) if layout == "bhnd" else (lambda x: x.transpose(0, 2, 1, 3).copy())
    O, LSE = ref_fwd(tr(q), tr(k), tr(v), scale=scale, causal=causal,
                     mask=mask, kv_lens=lens, layout=layout)
    O = O if layout == "bhnd" else O.transpose(0, 2, 1, 3)
    s = (1.0 / math.sqrt(d)) if scale is None else scale
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            mb = None if mask is None else mask[b, 0].tolist()
            L = None if lens is None else min(int(lens[b]), Nk)
            o, lse = brute_force.attention(q[b, h].tolist(), k[b, h // G].tolist(),
                                           v[b, h // G].tolist(), s, causal=causal,
                                           mask=mb, kv_len=L)
            np.testing.assert_allclose(O[b, h], np.array(o), rtol=0, atol=1e-12)
            np.testing.assert_array_equal(np.isinf(LSE[b, h]), np.isinf(np.array(lse)))
            fin = np.isfinite(np.array(lse))
            np.testing.assert_allclose(LSE[b, h][fin], np.array(lse)[fin], rtol=0, atol=1e-12)


# --------------------------------------------------------------- closed forms
def test_zero_query_gives_mean_of_visible_values():
    B, H, N, d = 2, 2, 9, 4
    q = np.zeros((B, H, N, d))
    k, v = _rand(B, H, N, d), _rand(B, H, N, d)
    lens = np.array([9, 4])
    O, LSE = ref_fwd(q, k, v, kv_lens=lens)
    for b in range(B):
        L = lens[b]
        np.testing.assert_allclose(O[b], np.broadcast_to(v[b, :, :L].mean(axis=1, keepdims=True), O[b].shape), atol=1e-14)
        np.testing.assert_allclose(LSE[b], math.log(L), atol=1e-14)


def test_causal_zero_query_gives_prefix_mean():
    N, d = 8, 3
    q = np.zeros((1, 1, N, d))
    k, v = _rand(1, 1, N, d), _rand(1, 1, N, d)
    O, LSE = ref_fwd(q, k, v, causal=True)
    for i in range(N):
        np.testing.assert_allclose(O[0, 0, i], v[0, 0, :i + 1].mean(axis=0), atol=1e-14)
        assert abs(LSE[0, 0, i] - math.log(i + 1)) < 1e-14


def test_causal_row0_is_v0():
    N, d = 6, 5
    q, k, v = _rand(1, 2, N, d), _rand(1, 2, N, d), _rand(1, 2, N, d)
    O, LSE = ref_fwd(q, k, v, causal=True, scale=0.7)
    np.testing.assert_allclose(O[0, :, 0], v[0, :, 0], atol=1e-15)
    np.testing.assert_allclose(LSE[0, :, 0], 0.7 * np.einsum("hd,hd->h", q[0, :, 0], k[0, :, 0]), atol=1e-14)


def test_single_key_gives_v0():
    q, k, v = _rand(1, 1, 5, 4), _rand(1, 1, 1, 4), _rand(1, 1, 1, 4)
    O, LSE = ref_fwd(q, k, v)
    np.testing.assert_allclose(O[0, 0], np.repeat(v[0, 0], 5, axis=0), atol=1e-15)
    np.testing.assert_allclose(LSE[0, 0], (q[0, 0] @ k[0, 0, 0]) / 2.0, atol=1e-14)


def test_constant_values_give_constant_output():
    q, k = _rand(2, 3, 7, 4), _rand(2, 3, 11, 4)
    c = _rand(4)
    v = np.broadcast_to(c, (2, 3, 11, 4)).copy()
    O, _ = ref_fwd(q, k, v, causal=False)
    np.testing.assert_allclose(O, np.broadcast_to(c, O.shape), atol=1e-14)


def test_two_keys_closed_form():
    # s_0 - s_1 = x  =>  p_0 = 1 / (1 + e^{-x}),  LSE = s_1 + ln(1 + e^{x})
    q = np.array([[[[1.0, 2.0]]]])
    k = np.array([[[[0.5, 0.25], [-1.0, 0.5]]]])
    v = np.array([[[[3.0, -1.0], [1.0, 5.0]]]])
    s = 0.8
    s0, s1 = s * (0.5 + 0.5), s * (-1.0 + 1.0)
    p0 = 1.0 / (1.0 + math.exp(-(s0 - s1)))
    O, LSE = ref_fwd(q, k, v, scale=s)
    np.testing.assert_allclose(O[0, 0, 0], p0 * v[0, 0, 0] + (1 - p0) * v[0, 0, 1], atol=1e-15)
    assert abs(LSE[0, 0, 0] - (s1 + math.log1p(math.exp(s0 - s1)))) < 1e-15


def test_dominant_key_selects_its_value():
    d = 8
    k = _rand(1, 1, 10, d)
    k[..., 0] = 0.0
    k[0, 0, 6] = 0.0
    k[0, 0, 6, 0] = 10.0          # q . k_6 = 100, q . k_j = 0 otherwise
    q = np.zeros((1, 1, 1, d))
    q[..., 0] = 10.0
    v = _rand(1, 1, 10, d)
    O, LSE = ref_fwd(q, k, v, scale=1.0)
    np.testing.assert_allclose(O[0, 0, 0], v[0, 0, 6], atol=1e-40 + 1e-12)
    assert abs(LSE[0, 0, 0] - 100.0) < 1e-12


def test_default_scale_readings():
    assert resolve_scale(None, 40) == 1.0 / math.sqrt(40)
    assert resolve_scale(0.0, 64) == 0.125
    assert resolve_scale(-2.0, 64) == 0.125
    assert resolve_scale(float("nan"), 16) == 0.25
    assert resolve_scale(0.3, 64) == 0.3


def test_fully_masked_row_is_zero_with_minus_inf_lse():
    q, k, v = _rand(2, 1, 3, 4), _rand(2, 1, 5, 4), _rand(2, 1, 5, 4)
    O, LSE = ref_fwd(q, k, v, kv_lens=[0, 5])
    assert np.all(O[0] == 0.0) and np.all(np.isneginf(LSE[0]))
    assert np.all(np.isfinite(LSE[1]))
    mask = np.zeros((1, 1, 3, 5))
    mask[..., 1, :] = -np.inf
    O, LSE = ref_fwd(q, k, v, mask=mask)
    assert np.all(O[:, 0, 1] == 0.0) and np.all(np.isneginf(LSE[:, 0, 1]))


# ---------------------------------------------------------------- invariants
def test_probability_rows_sum_to_one():
    q, k = _rand(2, 4, 6, 5), _rand(2, 2, 9, 5)
    lens = np.array([9, 3])
    for causal in (False,):
        P = ref_probs(q, k, causal=causal, kv_lens=lens)
        np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-14)
        assert np.all(P[1, :, :, 3:] == 0.0)
    qc, kc = _rand(1, 2, 7, 3), _rand(1, 2, 7, 3)
    P = ref_probs(qc, kc, causal=True)
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-14)
    assert np.all(np.triu(P[0, 0], 1) == 0.0)


# ref_probs against the pure-Python weights: GQA head mapping (q-head h reads
# kv-head h // G), a non-default scale, an additive mask with a -inf entry,
# key lengths, causal rows and the BNHD layout; then P V equals ref_fwd's O.
PROB_CASES = [
    # B, Hq, Hkv, Nq, Nk, d, causal, use_mask, use_lens, layout, scale
    (2, 4, 2, 5, 7, 3, False, True, True, "bhnd", 0.61),
    (1, 6, 2, 6, 6, 4, True, False, False, "bnhd", None),
    (2, 4, 1, 4, 9, 2, False, False, True, "bnhd", 1.7),
]


@pytest.mark.parametrize("case", PROB_CASES)
def test_ref_probs_matches_brute_force(case):
    B, Hq, Hkv, Nq, Nk, d, causal, use_mask, use_lens, layout, scale = case
    q = _rand(B, Hq, Nq, d)
    k = _rand(B, Hkv, Nk, d)
    v = _rand(B, Hkv, Nk, d)
    mask = _rand(B, Hq, Nq, Nk) if use_mask else None
    if use_mask:
        mask[1, 2, 1, 0] = -np.inf
    lens = np.array([Nk - 2, 3][:B]) if use_lens else None
    tr = (lambda x: x) if layout == "bhnd" else (lambda x: x.transpose(0, 2, 1, 3).copy())
    P = ref_probs(tr(q), tr(k), scale=scale, causal=causal, mask=mask, kv_lens=lens,
                  layout=layout)
    assert P.shape == (B, Hq, Nq, Nk)
    s = (1.0 / math.sqrt(d)) if scale is None else scale
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            _, _, pb = brute_force.attention(
                q[b, h].tolist(), k[b, h // G].tolist(), v[b, h // G].tolist(), s,
                causal=causal, mask=None if mask is None else mask[b, h].tolist(),
                kv_len=None if lens is None else int(lens[b]), with_probs=True)
            np.testing.assert_allclose(P[b, h], np.array(pb), rtol=0, atol=1e-13)
    O, _ = ref_fwd(tr(q), tr(k), tr(v), scale=scale, causal=causal, mask=mask, kv_lens=lens,
                   layout=layout)
    O = O if layout == "bhnd" else O.transpose(0, 2, 1, 3)
    vg = np.repeat(v, G, axis=1)
    np.testing.assert_allclose(P @ vg, O, rtol=0, atol=1e-13)


def test_permuting_keys_and_values_together():
    q, k, v = _rand(1, 2, 5, 4), _rand(1, 2, 8, 4), _rand(1, 2, 8, 4)
    perm = RNG.permutation(8)
    O1, L1 = ref_fwd(q, k, v)
    O2, L2 = ref_fwd(q, k[:, :, perm], v[:, :, perm])
    np.testing.assert_allclose(O1, O2, atol=1e-14)
    np.testing.assert_allclose(L1, L2, atol=1e-14)


def test_mask_row_constant_shifts_lse_only():
    q, k, v = _rand(1, 1, 4, 3), _rand(1, 1, 6, 3), _rand(1, 1, 6, 3)
    base = _rand(1, 1, 4, 6)
    shift = np.array([0.0, 2.5, -7.0, 11.0]).reshape(1, 1, 4, 1)
    O1, L1 = ref_fwd(q, k, v, mask=base)
    O2, L2 = ref_fwd(q, k, v, mask=base + shift)
    np.testing.assert_allclose(O1, O2, atol=1e-13)
    np.testing.assert_allclose(L2 - L1, shift[..., 0], atol=1e-13)


def test_affine_values():
    q, k, v = _rand(2, 2, 5, 4), _rand(2, 2, 6, 4), _rand(2, 2, 6, 4)
    O1, _ = ref_fwd(q, k, v, causal=False)
    O2, _ = ref_fwd(q, k, -1.75 * v + 0.5)
    np.testing.assert_allclose(O2, -1.75 * O1 + 0.5, atol=1e-13)


def test_appended_masked_keys_change_nothing():
    q, k, v = _rand(2, 2, 5, 4), _rand(2, 2, 6, 4), _rand(2, 2, 6, 4)
    k2 = np.concatenate([k, _rand(2, 2, 10, 4) * 50], axis=2)
    v2 = np.concatenate([v, _rand(2, 2, 10, 4) * 50], axis=2)
    mask = np.zeros((1, 1, 5, 16))
    mask[..., 6:] = -np.inf
    O1, L1 = ref_fwd(q, k, v)
    O2, L2 = ref_fwd(q, k2, v2, mask=mask)
    O3, L3 = ref_fwd(q, k2, v2, kv_lens=[6, 6])
    for O, L in ((O2, L2), (O3, L3)):
        np.testing.assert_allclose(O, O1, atol=1e-13)
        np.testing.assert_allclose(L, L1, atol=1e-13)


def test_kv_lens_equals_truncation():
    q, k, v = _rand(3, 2, 5, 4), _rand(3, 2, 12, 4), _rand(3, 2, 12, 4)
    lens = np.array([12, 7, 1])
    O, L = ref_fwd(q, k, v, kv_lens=lens)
    for b in range(3):
        Ob, Lb = ref_fwd(q[b:b + 1], k[b:b + 1, :, :lens[b]], v[b:b + 1, :, :lens[b]])
        np.testing.assert_allclose(O[b:b + 1], Ob, atol=1e-14)
        np.testing.assert_allclose(L[b:b + 1], Lb, atol=1e-14)


def test_gqa_equals_repeated_kv_heads():
    q, k, v = _rand(2, 6, 5, 4), _rand(2, 2, 7, 4), _rand(2, 2, 7, 4)
    O1, L1 = ref_fwd(q, k, v, kv_lens=[7, 3])
    O2, L2 = ref_fwd(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), kv_lens=[7, 3])
    np.testing.assert_allclose(O1, O2, atol=0)
    np.testing.assert_allclose(L1, L2, atol=0)


def test_layouts_agree():
    q, k, v = _rand(2, 4, 5, 3), _rand(2, 2, 6, 3), _rand(2, 2, 6, 3)
    O1, L1 = ref_fwd(q, k, v, causal=False)
    t = lambda x: np.ascontiguousarray(x.transpose(0, 2, 1, 3))
    O2, L2 = ref_fwd(t(q), t(k), t(v), layout="bnhd")
    np.testing.assert_allclose(O1, O2.transpose(0, 2, 1, 3), atol=0)
    np.testing.assert_allclose(L1, L2, atol=0)


def test_causal_equals_upper_minus_inf_mask():
    q, k, v = _rand(1, 2, 6, 3), _rand(1, 2, 6, 3), _rand(1, 2, 6, 3)
    mask = np.triu(np.full((6, 6), -np.inf), 1)[None, None]
    O1, L1 = ref_fwd(q, k, v, causal=True)
    O2, L2 = ref_fwd(q, k, v, mask=mask)
    np.testing.assert_allclose(O1, O2, atol=0)
    np.testing.assert_allclose(L1, L2, atol=0)


def test_zero_mask_equals_no_mask():
    q, k, v = _rand(1, 2, 6, 3), _rand(1, 2, 9, 3), _rand(1, 2, 9, 3)
    O1, L1 = ref_fwd(q, k, v)
    O2, L2 = ref_fwd(q, k, v, mask=np.zeros((1, 1, 1, 1)))
    np.testing.assert_allclose(O1, O2, atol=0)
    np.testing.assert_allclose(L1, L2, atol=0)


def test_rows_helper_matches_full():
    q, k, v = _rand(2, 4, 10, 3), _rand(2, 2, 10, 3), _rand(2, 2, 10, 3)
    lens = [10, 6]
    O, L = ref_fwd(q, k, v, causal=True, kv_lens=lens)
    rows = [0, 3, 9]
    o, l = ref_fwd_rows(q, k, v, 1, 3, rows, causal=True, kv_lens=lens)
    np.testing.assert_allclose(o, O[1, 3, rows], atol=1e-15)
    np.testing.assert_allclose(l, L[1, 3, rows], atol=1e-15)


# ------------------------------------------------------------ tiled = full
@pytest.mark.parametrize("trial", range(12))
def test_tiled_online_softmax_equals_full_softmax(trial):
    rng = np.random.default_rng(1000 + trial)
    B, Hkv = 2, int(rng.integers(1, 3))
    Hq = Hkv * int(rng.integers(1, 3))
    causal = bool(trial % 3 == 0)
    Nq = int(rng.integers(1, 40))
    Nk = Nq if causal else int(rng.integers(1, 40))
    d = int(rng.integers(1, 9))
    q = rng.standard_normal((B, Hq, Nq, d)) * 2
    k = rng.standard_normal((B, Hkv, Nk, d)) * 2
    v = rng.standard_normal((B, Hkv, Nk, d))
    lens = rng.integers(0, Nk + 1, size=B) if trial % 2 else None
    mask = rng.standard_normal((1, Hq, Nq, Nk)) * 3 if trial % 4 == 1 else None
    O, L = ref_fwd(q, k, v, causal=causal, kv_lens=lens, mask=mask)
    for br in (1, 3, 7, 16):
        for bc in (1, 3, 7, 16):
            thr = None if (br + bc) % 2 else math.log(2.0) * 8
            Ot, Lt = tiled_fwd(q, k, v, block_r=br, block_c=bc, causal=causal,
                               kv_lens=lens, mask=mask, rescale_threshold=thr)
            np.testing.assert_allclose(Ot, O, atol=1e-12, rtol=0)
            np.testing.assert_array_equal(np.isneginf(Lt), np.isneginf(L))
            fin = np.isfinite(L)
            np.testing.assert_allclose(Lt[fin], L[fin], atol=1e-12, rtol=0)


def test_decode_causal_rule_is_last_rows_of_causal_attention():
    """Decode's causal rule (query i of the last Nq sees keys j <= L - Nq + i)
    applied through an additive mask equals the last Nq rows of ordinary causal
    attention over the whole sequence; with key lengths, equals the same over
    the first L keys."""
    from tests.gpu_util import decode_causal_mask
    rng = np.random.default_rng(21)
    B, H, N, d, Nq = 2, 3, 37, 16, 5
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    O_full, L_full = ref_fwd(q, k, v, causal=True)
    m = decode_causal_mask(B, Nq, N)
    O_dec, L_dec = ref_fwd(q[:, :, N - Nq:], k, v, mask=m)
    np.testing.assert_allclose(O_dec, O_full[:, :, N - Nq:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(L_dec, L_full[:, :, N - Nq:], rtol=0, atol=1e-12)
    # key lengths: batch b has only its first L_b keys; its decode queries are
    # its positions L_b - Nq .. L_b - 1
    lens = np.array([20, 37], dtype=np.int32)
    m = decode_causal_mask(B, Nq, N, lens)
    qd = np.stack([q[b, :, lens[b] - Nq:lens[b]] for b in range(B)])
    O_dec, L_dec = ref_fwd(qd, k, v, mask=m, kv_lens=lens)
    for b in range(B):
        Lb = int(lens[b])
        O_b, L_b = ref_fwd(q[b:b + 1, :, :Lb], k[b:b + 1, :, :Lb], v[b:b + 1, :, :Lb], causal=True)
        np.testing.assert_allclose(O_dec[b], O_b[0, :, Lb - Nq:], rtol=0, atol=1e-12)
        np.testing.assert_allclose(L_dec[b], L_b[0, :, Lb - Nq:], rtol=0, atol=1e-12)
