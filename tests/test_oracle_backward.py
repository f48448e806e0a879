"""Pins of the oracle's backward pass: finite differences and identities.

CPU only.  The loss is <dO, O(q, k, v)>, whose gradients are exactly what the
recompute backward produces (dQ, dK, dV).
"""
import numpy as np
import pytest

from oracle import ref_bwd, ref_fwd

RNG = np.random.default_rng(777)


def _loss(q, k, v, do, **kw):
    O, _ = ref_fwd(q, k, v, **kw)
    return float(np.sum(O * do))


CASES = [
    dict(B=1, Hq=2, Hkv=1, Nq=5, Nk=5, d=3, causal=True, lens=None, mask=False, layout="bhnd"),
    dict(B=2, Hq=2, Hkv=2, Nq=4, Nk=6, d=3, causal=False, lens=[6, 2], mask=True, layout="bhnd"),
    dict(B=1, Hq=4, Hkv=2, Nq=6, Nk=6, d=2, causal=True, lens=[4], mask=False, layout="bnhd"),
]


@pytest.mark.parametrize("c", CASES)
def test_backward_matches_central_differences(c):
    B, Hq, Hkv, Nq, Nk, d = c["B"], c["Hq"], c["Hkv"], c["Nq"], c["Nk"], c["d"]
    q = RNG.standard_normal((B, Hq, Nq, d))
    k = RNG.standard_normal((B, Hkv, Nk, d))
    v = RNG.standard_normal((B, Hkv, Nk, d))
    do = RNG.standard_normal((B, Hq, Nq, d))
    mask = RNG.standard_normal((B, 1, Nq, Nk)) if c["mask"] else None
    t = (lambda x: x) if c["layout"] == "bhnd" else (lambda x: np.ascontiguousarray(x.transpose(0, 2, 1, 3)))
    kw = dict(causal=c["causal"], kv_lens=c["lens"], mask=mask, scale=0.9, layout=c["layout"])
    q, k, v, do = t(q), t(k), t(v), t(do)
    dq, dk, dv, _, _ = ref_bwd(q, k, v, do, **kw)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = _loss(args["q"], args["k"], args["v"], do, **kw)
            args[name] = xm
            fm = _loss(args["q"], args["k"], args["v"], do, **kw)
            num[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(g, num, atol=2e-8, rtol=1e-6, err_msg=name)


def test_backward_identities():
    B, Hq, Hkv, N, d = 2, 4, 2, 9, 4
    q = RNG.standard_normal((B, Hq, N, d))
    k = RNG.standard_normal((B, Hkv, N, d))
    v = RNG.standard_normal((B, Hkv, N, d))
    do = RNG.standard_normal((B, Hq, N, d))
    lens = [9, 5]
    dq, dk, dv, O, LSE = ref_bwd(q, k, v, do, causal=True, kv_lens=lens)
    # rows of dS sum to zero, so sum_j dK_j = 0 for every (b, kv-head)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # rows of P sum to one, so sum_j dV_j = sum over the group's rows of dO
    for g in range(Hkv):
        np.testing.assert_allclose(dv[:, g].sum(axis=1),
                                   do[:, 2 * g:2 * g + 2].sum(axis=(1, 2)), atol=1e-12)
    # the backward's own forward is the forward
    O2, L2 = ref_fwd(q, k, v, causal=True, kv_lens=lens)
    np.testing.assert_allclose(O, O2, atol=0)
    np.testing.assert_allclose(LSE, L2, atol=0)


def test_zero_query_gives_zero_dk():
    q = np.zeros((1, 2, 5, 3))
    k, v, do = (RNG.standard_normal((1, 2, 5, 3)) for _ in range(3))
    _, dk, _, _, _ = ref_bwd(q, k, v, do)
    assert np.all(dk == 0.0)


def test_equal_keys_give_zero_dq():
    q = RNG.standard_normal((1, 2, 5, 3))
    k = np.broadcast_to(RNG.standard_normal(3), (1, 2, 7, 3)).copy()
    v, do = RNG.standard_normal((1, 2, 7, 3)), RNG.standard_normal((1, 2, 5, 3))
    dq, _, _, _, _ = ref_bwd(q, k, v, do)
    np.testing.assert_allclose(dq, 0.0, atol=1e-14)


def test_gqa_backward_equals_summed_repeated_heads():
    q = RNG.standard_normal((1, 6, 5, 3))
    k, v = RNG.standard_normal((1, 2, 7, 3)), RNG.standard_normal((1, 2, 7, 3))
    do = RNG.standard_normal((1, 6, 5, 3))
    dq1, dk1, dv1, _, _ = ref_bwd(q, k, v, do, kv_lens=[6])
    dq2, dk2, dv2, _, _ = ref_bwd(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), do, kv_lens=[6])
    np.testing.assert_allclose(dq1, dq2, atol=1e-14)
    np.testing.assert_allclose(dk1, dk2.reshape(1, 2, 3, 7, 3).sum(axis=2), atol=1e-13)
    np.testing.assert_allclose(dv1, dv2.reshape(1, 2, 3, 7, 3).sum(axis=2), atol=1e-13)


def test_fully_masked_rows_have_no_gradient():
    q, k, v, do = (RNG.standard_normal((2, 1, 4, 3)) for _ in range(4))
    dq, dk, dv, O, L = ref_bwd(q, k, v, do, kv_lens=[0, 4])
    assert np.all(dq[0] == 0) and np.all(dk[0] == 0) and np.all(dv[0] == 0)
    assert np.all(np.isneginf(L[0]))
