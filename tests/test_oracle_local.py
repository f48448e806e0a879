"""Pins of the oracle's local masks and soft cap against things other than itself.

CPU only.  Covers the sliding window (flash_attn_func's window_size, the
ChatGLM2-6B page §3 step 3), the 2-D neighbourhood mask and the tanh soft cap
(the FlexAttention mask_mod / score_mod examples of the PyTorch
attention-options article, atyun.com/61003), and decode's last-positions rule
(``bottom_right``):

* pure-Python loops (tests/brute_force.py) on tiny inputs;
* closed forms: with Q = 0 every visible logit is 0, so LSE = ln(count of
  visible keys), and the count has a closed form for a window or a grid;
  window (0, 0) leaves only the diagonal; two keys with a huge logit gap give
  p = 1 / (1 + e^-cap) under a soft cap;
* limits and special cases: no-op windows and grids, window (-1, 0) =
  causal, cap -> infinity = no cap, cap -> 0 = uniform attention;
* the backward against central differences of the forward.
"""
import math

import numpy as np
import pytest

from oracle import local_visible, ref_bwd, ref_fwd, ref_fwd_rows
from tests import brute_force

RNG = np.random.default_rng(4)


def _r(*shape):
    return RNG.standard_normal(shape)


# ---------------------------------------------------------------- brute force
BF = [
    # B, Hq, Hkv, Nq, Nk, d, kw (oracle keywords), lens
    (1, 2, 1, 7, 7, 3, dict(window=(2, 1)), None),
    (2, 2, 2, 9, 9, 4, dict(window=(3, 0), softcap=1.5), None),
    (1, 2, 1, 12, 12, 3, dict(grid=(4, 2, 2)), None),
    (1, 1, 1, 15, 15, 2, dict(grid=(5, 1, 3), causal=True), None),
    (2, 2, 1, 8, 8, 3, dict(softcap=0.7, causal=True), [8, 5]),
    (2, 2, 2, 3, 10, 3, dict(window=(4, -1), bottom_right=True, causal=True), [10, 6]),
    (1, 2, 2, 4, 9, 3, dict(softcap=2.0, bottom_right=True), [7]),
    (1, 1, 1, 10, 10, 3, dict(window=(-1, 2), grid=(3, 2, 5), softcap=3.0), None),
]


@pytest.mark.parametrize("case", BF)
def test_local_options_match_brute_force(case):
    B, Hq, Hkv, Nq, Nk, d, kw, lens = case
    q, k, v = _r(B, Hq, Nq, d) * 2, _r(B, Hkv, Nk, d), _r(B, Hkv, Nk, d)
    mask = _r(B, 1, Nq, Nk)
    O, LSE = ref_fwd(q, k, v, scale=0.8, mask=mask, kv_lens=lens, **kw)
    G = Hq // Hkv
    for b in range(B):
        L = None if lens is None else lens[b]
        for h in range(Hq):
            o, lse = brute_force.attention(
                q[b, h].tolist(), k[b, h // G].tolist(), v[b, h // G].tolist(), 0.8,
                causal=kw.get("causal", False), mask=mask[b, 0].tolist(), kv_len=L,
                softcap=kw.get("softcap"), window=kw.get("window"), grid=kw.get("grid"),
                last_positions=kw.get("bottom_right", False))
            np.testing.assert_allclose(O[b, h], np.array(o), rtol=0, atol=1e-12)
            lse = np.array(lse)
            np.testing.assert_array_equal(np.isneginf(LSE[b, h]), np.isneginf(lse))
            fin = np.isfinite(lse)
            np.testing.assert_allclose(LSE[b, h][fin], lse[fin], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("wl,wr", [(0, 0), (3, 0), (0, 4), (2, 5), (-1, 3), (6, -1)])
def test_window_visible_count(wl, wr):
    """Q = 0: LSE_i = ln(number of visible keys) = ln(lo + 1 + hi) with
    lo = min(i, wl) keys before and hi = min(N - 1 - i, wr) after (an open
    side takes all)."""
    N, d = 23, 4
    q = np.zeros((1, 1, N, d))
    k, v = _r(1, 1, N, d), _r(1, 1, N, d)
    _, LSE = ref_fwd(q, k, v, window=(wl, wr))
    for i in range(N):
        lo = i if wl < 0 else min(i, wl)
        hi = N - 1 - i if wr < 0 else min(N - 1 - i, wr)
        assert LSE[0, 0, i] == pytest.approx(math.log(lo + 1 + hi), abs=1e-12)


def test_grid_visible_count_and_page_sizes():
    """Q = 0 on an R x C grid: the count is a product of a row count and a
    column count.  On the page's 56 x 56 patch grid with both differences
    < 5, an interior token sees 9 x 9 = 81 tokens and a corner token 5 x 5."""
    R, C, nr, nc, d = 7, 6, 3, 2, 2
    N = R * C
    q = np.zeros((1, 1, N, d))
    k, v = _r(1, 1, N, d), _r(1, 1, N, d)
    _, LSE = ref_fwd(q, k, v, grid=(C, nr, nc))

    def span(x, n, rad):
        return min(x, rad - 1) + 1 + min(n - 1 - x, rad - 1)

    for t in range(N):
        r, c = divmod(t, C)
        assert LSE[0, 0, t] == pytest.approx(math.log(span(r, R, nr) * span(c, C, nc)), abs=1e-12)
    vis = local_visible(np.arange(56 * 56), 56 * 56, grid=(56, 5, 5))
    counts = vis.sum(axis=1)
    assert counts[28 * 56 + 28] == 81 and counts[0] == 25 and counts[56 * 56 - 1] == 25
    assert counts[28] == 45  # top edge, middle column: 5 rows x 9 columns


def test_zero_window_is_the_diagonal():
    """window (0, 0): each query sees only its own position: O_i = V_i and
    LSE_i = the capped logit of (i, i)."""
    N, d, cap = 9, 5, 1.25
    q, k, v = _r(1, 2, N, d), _r(1, 2, N, d), _r(1, 2, N, d)
    O, LSE = ref_fwd(q, k, v, scale=0.6, window=(0, 0), softcap=cap)
    np.testing.assert_allclose(O, v, rtol=0, atol=1e-14)
    z = 0.6 * np.einsum("bhnd,bhnd->bhn", q, k)
    np.testing.assert_allclose(LSE, cap * np.tanh(z / cap), rtol=0, atol=1e-14)


def test_softcap_two_keys_saturated():
    """Two keys whose scaled logits are 1e6 and 0: the cap maps them to
    exactly cap and 0, so p = 1 / (1 + e^-cap) on the first key (not 1)."""
    d, cap = 4, 2.0
    q = np.zeros((1, 1, 1, d)); q[..., 0] = 1.0
    k = np.zeros((1, 1, 2, d)); k[0, 0, 0, 0] = 1e6
    v = _r(1, 1, 2, d)
    O, LSE = ref_fwd(q, k, v, scale=1.0, softcap=cap)
    p0 = 1.0 / (1.0 + math.exp(-cap))
    np.testing.assert_allclose(O[0, 0, 0], p0 * v[0, 0, 0] + (1 - p0) * v[0, 0, 1], rtol=0,
                               atol=1e-14)
    assert LSE[0, 0, 0] == pytest.approx(math.log(math.exp(cap) + 1.0), abs=1e-13)


def test_softcap_limits():
    """cap -> infinity: plain attention; cap -> 0: every logit -> 0, so O is
    the mean of the visible values."""
    B, H, N, d = 2, 2, 11, 6
    q, k, v = _r(B, H, N, d), _r(B, H, N, d), _r(B, H, N, d)
    O0, L0 = ref_fwd(q, k, v, causal=True)
    O1, L1 = ref_fwd(q, k, v, causal=True, softcap=1e7)
    np.testing.assert_allclose(O1, O0, rtol=0, atol=1e-10)
    np.testing.assert_allclose(L1, L0, rtol=0, atol=1e-10)
    O2, _ = ref_fwd(q, k, v, causal=True, softcap=1e-9)
    prefix_mean = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    np.testing.assert_allclose(O2, prefix_mean, rtol=0, atol=1e-7)


# ---------------------------------------------------------------- special cases
def test_open_windows_and_wide_grids_change_nothing():
    B, H, N, d = 1, 2, 14, 3
    q, k, v = _r(B, H, N, d), _r(B, H, N, d), _r(B, H, N, d)
    O, L = ref_fwd(q, k, v)
    for kw in (dict(window=(-1, -1)), dict(window=(N, N)), dict(grid=(7, 2, 7)),
               dict(grid=(1, N, 1))):
        O1, L1 = ref_fwd(q, k, v, **kw)
        np.testing.assert_allclose(O1, O, rtol=0, atol=1e-14)
        np.testing.assert_allclose(L1, L, rtol=0, atol=1e-14)


def test_left_window_is_causal():
    B, H, N, d = 2, 2, 13, 4
    q, k, v = _r(B, H, N, d), _r(B, H, N, d), _r(B, H, N, d)
    O, L = ref_fwd(q, k, v, causal=True)
    O1, L1 = ref_fwd(q, k, v, window=(-1, 0))
    np.testing.assert_allclose(O1, O, rtol=0, atol=1e-14)
    np.testing.assert_allclose(L1, L, rtol=0, atol=1e-14)


def test_bottom_right_rows_are_the_last_rows_of_self_attention():
    """Decode's rule with a window: Nq queries at the last positions of the
    batch's L keys equal the last Nq rows of windowed causal self-attention
    over those L keys."""
    B, H, N, d, Nq = 2, 2, 30, 8, 4
    q, k, v = _r(B, H, N, d), _r(B, H, N, d), _r(B, H, N, d)
    lens = np.array([17, 30])
    qd = np.stack([q[b, :, lens[b] - Nq:lens[b]] for b in range(B)])
    O, L = ref_fwd(qd, k, v, kv_lens=lens, causal=True, window=(5, -1), softcap=3.0,
                   bottom_right=True)
    for b in range(B):
        Lb = int(lens[b])
        Of, Lf = ref_fwd(q[b:b + 1, :, :Lb], k[b:b + 1, :, :Lb], v[b:b + 1, :, :Lb],
                         causal=True, window=(5, -1), softcap=3.0)
        np.testing.assert_allclose(O[b], Of[0, :, Lb - Nq:], rtol=0, atol=1e-13)
        np.testing.assert_allclose(L[b], Lf[0, :, Lb - Nq:], rtol=0, atol=1e-13)


def test_rows_helper_with_local_options():
    B, H, N, d = 1, 2, 20, 4
    q, k, v = _r(B, H, N, d), _r(B, H, N, d), _r(B, H, N, d)
    kw = dict(window=(3, 2), grid=(5, 2, 3), softcap=1.0)
    O, L = ref_fwd(q, k, v, **kw)
    rows = np.array([0, 7, 19])
    o, l = ref_fwd_rows(q, k, v, 0, 1, rows, **kw)
    np.testing.assert_allclose(o, O[0, 1, rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(l, L[0, 1, rows], rtol=0, atol=1e-14)


def test_unknown_keyword_is_rejected():
    q = np.zeros((1, 1, 2, 2))
    with pytest.raises(TypeError):
        ref_fwd(q, q, q, windw=(1, 1))


# ---------------------------------------------------------------- backward
def _loss(q, k, v, do, **kw):
    O, _ = ref_fwd(q, k, v, **kw)
    return float(np.sum(O * do))


BWD = [
    dict(softcap=0.9, causal=True),
    dict(window=(2, 1), softcap=2.5),
    dict(grid=(3, 2, 2), mask=True),
]


@pytest.mark.parametrize("kw", BWD)
def test_local_backward_matches_central_differences(kw):
    """The soft cap's derivative factor 1 - tanh^2 and the local masks in the
    backward against central differences of the forward."""
    kw = dict(kw)
    B, Hq, Hkv, N, d = 1, 2, 1, 6, 3
    q, k, v, do = _r(B, Hq, N, d) * 2, _r(B, Hkv, N, d), _r(B, Hkv, N, d), _r(B, Hq, N, d)
    if kw.pop("mask", False):
        kw["mask"] = _r(B, 1, N, N)
    kw["scale"] = 1.1
    dq, dk, dv, _, _ = ref_bwd(q, k, v, do, **kw)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args = {"q": q, "k": k, "v": v}
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args[name] = xp
            fp = _loss(args["q"], args["k"], args["v"], do, **kw)
            args[name] = xm
            fm = _loss(args["q"], args["k"], args["v"], do, **kw)
            num[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(g, num, atol=2e-8, rtol=1e-6, err_msg=name)
