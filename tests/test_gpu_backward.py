"""GPU backward parity: attn_bwd (recompute from LSE) against the fp64 oracle.

The backward consumes the forward's own (O, LSE) from the GPU path, as a
caller would.  Gradients are fp32 (the default); the bar is max-abs 2e-2 on
dQ, dK and dV, plus a relative-RMS bound.
"""
import sys
import zlib

import numpy as np
import pytest

from exact_attention_25_amd import inputs
from oracle import ref_bwd
from tests.gpu_util import from_layout, host, make_case, to_device, to_layout

pytestmark = pytest.mark.gpu

TOL = 2e-2
TOL_REL_RMS = 1e-2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(w, x, *, layout="bhnd", causal=False, scale=None, grad_dtype="fp32", mask=None):
    import torch
    from exact_attention_25_amd import binding as bd
    t = {n: to_device(to_layout(x[n + "_raw"], layout), w.dtype) for n in ("q", "k", "v", "do")}
    lens = None if x["kv_lens"] is None else torch.from_numpy(x["kv_lens"]).cuda()
    m = None if mask is None else torch.from_numpy(mask.astype(np.float32)).cuda()
    o, lse = bd.attn_fwd(t["q"], t["k"], t["v"], layout=layout, causal=causal, scale=scale,
                         attn_mask=m, kv_lens=lens)
    dq, dk, dv = bd.attn_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], layout=layout,
                             causal=causal, scale=scale, attn_mask=m, kv_lens=lens,
                             grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return dq, dk, dv


def _check(name, got, ref, tol=TOL, rel=TOL_REL_RMS):
    g = host(got)
    assert g.shape == ref.shape, (name, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite"
    err = np.abs(g - ref)
    mx = float(err.max()) if err.size else 0.0
    assert mx <= tol, f"{name}: max-abs {mx:.3e} > {tol}"
    rr = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    if rr > 0:
        rel_rms = float(np.sqrt(np.mean(err ** 2))) / rr
        assert rel_rms <= rel, f"{name}: rel-rms {rel_rms:.3e}"
    return mx


SMALL = [
    # id, B, Hq, Hkv, Nq, Nk, d, dtype, causal, lens, layout, scale
    ("bf16_causal_gqa_lens", 2, 8, 2, 200, 200, 128, "bf16", True, (90, 200), "bhnd", None),
    ("fp16_noncausal_ragged", 2, 2, 2, 150, 90, 64, "fp16", False, None, "bhnd", None),
    ("bf16_bnhd_gqa", 1, 4, 1, 130, 130, 128, "bf16", False, None, "bnhd", 0.2),
    ("fp16_d40_cross_lens", 2, 2, 2, 257, 77, 40, "fp16", False, (20, 77), "bhnd", None),
    ("bf16_lens_zero", 3, 2, 2, 70, 90, 64, "bf16", False, (0, 2), "bhnd", None),
    ("bf16_d96_causal", 1, 2, 2, 300, 300, 96, "bf16", True, None, "bhnd", None),
    ("fp16_many_heads_chunks", 1, 16, 1, 96, 96, 128, "fp16", True, None, "bhnd", None),
]


# Additive masks in the backward (logit units, after scaling; -inf entries
# exclude a key; strides 0 broadcast), alone and with causal and key lengths.
MASKED = [
    # id, B, Hq, Hkv, Nq, Nk, d, dtype, causal, lens, mask kind, layout
    ("bf16_mask_full_gqa", 2, 4, 2, 200, 170, 128, "bf16", False, None, "full", "bhnd"),
    ("fp16_mask_keys_bcast_lens", 2, 2, 2, 150, 260, 64, "fp16", False, (100, 260), "keys", "bhnd"),
    ("bf16_mask_causal_bnhd", 1, 4, 1, 300, 300, 128, "bf16", True, None, "rows11", "bnhd"),
    ("fp16_mask_d40_dead_rows", 1, 2, 2, 96, 96, 40, "fp16", False, None, "dead_rows", "bhnd"),
]


def _bwd_mask(kind, B, Hq, Nq, Nk, rng):
    if kind == "full":
        m = rng.standard_normal((B, Hq, Nq, Nk)) * 2
        m[:, :, :, ::9] = -np.inf
    elif kind == "keys":                       # [B,1,1,Nk]: per-batch key bias, broadcast
        m = np.zeros((B, 1, 1, Nk))
        m[..., Nk // 2:] = -1e9
        m[..., : Nk // 5] += rng.standard_normal(Nk // 5)
    elif kind == "rows11":                     # [1,1,Nq,Nk]: one mask for every (b, h)
        m = rng.standard_normal((1, 1, Nq, Nk))
        m[0, 0, :, 5::11] = -np.inf
    elif kind == "dead_rows":                  # rows whose every key is masked
        m = np.zeros((1, 1, Nq, Nk))
        m[0, 0, 3] = -np.inf
        m[0, 0, 40] = -np.inf
    else:
        raise ValueError(kind)
    return m.astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("case", MASKED, ids=[c[0] for c in MASKED])
def test_backward_additive_mask(gpu_lib, case):
    name, B, Hq, Hkv, Nq, Nk, d, dtype, causal, lens, mkind, layout = case
    _say(f"[bwd-mask] {name}")
    w, x = make_case(B, Hq, Hkv, Nq, Nk, d, dtype, seed=zlib.crc32(name.encode()) % 10000,
                     lens=lens, with_do=True)
    mask = _bwd_mask(mkind, B, Hq, Nq, Nk, np.random.default_rng(11))
    dq, dk, dv = _run(w, x, layout=layout, causal=causal, mask=mask)
    dQ, dK, dV, _, _ = ref_bwd(x["q"], x["k"], x["v"], x["do"], causal=causal, mask=mask,
                               kv_lens=x["kv_lens"])
    _check(name + " dq", from_layout(host(dq), layout), dQ)
    _check(name + " dk", from_layout(host(dk), layout), dK)
    _check(name + " dv", from_layout(host(dv), layout), dV)


# fp32 inputs: every product in fp32 (fp32 MFMA), held to the fp32 bar of
# 1e-5, taken relative to the gradient's own scale: max-abs error
# <= 1e-5 * max(1, max |ref|).  Gradients reach |dQ| ~ 10 where the logits
# are sharp (scale * |q||k| large), and there 1e-5 absolute is ~10 fp32 ulps
# of the largest element, below what any fp32 order of summation reaches.
# The relative-RMS bound is 3e-6: S itself is an fp32 sum of d products of
# size up to ~40 (about 2e-5 absolute), i.e. up to ~6e-6 relative in P at
# scale 0.3 and d = 128.
TOL_F32 = 1e-5
REL_RMS_F32 = 3e-6
FP32 = [
    # id, B, Hq, Hkv, Nq, Nk, d, dtype, causal, lens, mask kind, layout, scale
    ("fp32_tiny_workload_shape", 1, 2, 2, 128, 128, 64, "fp32", False, None, None, "bhnd", 0.125),
    ("fp32_causal_gqa_lens", 2, 4, 2, 150, 150, 64, "fp32", True, (60, 150), None, "bhnd", None),
    ("fp32_d128_bnhd_ragged", 1, 2, 2, 130, 97, 128, "fp32", False, None, None, "bnhd", 0.3),
    ("fp32_d40_mask", 1, 2, 1, 100, 120, 40, "fp32", False, None, "full", "bhnd", None),
    ("fp32_causal_mask_dead_rows", 1, 2, 2, 96, 96, 96, "fp32", True, None, "dead_rows", "bhnd", None),
]


@pytest.mark.parametrize("case", FP32, ids=[c[0] for c in FP32])
def test_backward_fp32(gpu_lib, case):
    name, B, Hq, Hkv, Nq, Nk, d, dtype, causal, lens, mkind, layout, scale = case
    _say(f"[bwd-fp32] {name}")
    w, x = make_case(B, Hq, Hkv, Nq, Nk, d, dtype, seed=zlib.crc32(name.encode()) % 10000,
                     lens=lens, with_do=True)
    mask = None if mkind is None else _bwd_mask(mkind, B, Hq, Nq, Nk, np.random.default_rng(12))
    dq, dk, dv = _run(w, x, layout=layout, causal=causal, scale=scale, mask=mask)
    dQ, dK, dV, _, _ = ref_bwd(x["q"], x["k"], x["v"], x["do"], causal=causal, scale=scale,
                               mask=mask, kv_lens=x["kv_lens"])
    for lbl, got, ref in ((" dq", dq, dQ), (" dk", dk, dK), (" dv", dv, dV)):
        scale_ref = max(1.0, float(np.abs(ref).max()) if ref.size else 0.0)
        mx = _check(name + lbl, from_layout(host(got), layout), ref, tol=TOL_F32 * scale_ref,
                    rel=REL_RMS_F32)
        _say(f"  {lbl.strip()}: max-abs {mx:.2e}, max|ref| {scale_ref:.2f}")


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_backward_small(gpu_lib, case):
    name, B, Hq, Hkv, Nq, Nk, d, dtype, causal, lens, layout, scale = case
    _say(f"[bwd-small] {name}")
    w, x = make_case(B, Hq, Hkv, Nq, Nk, d, dtype, seed=zlib.crc32(name.encode()) % 10000,
                     lens=lens, with_do=True)
    dq, dk, dv = _run(w, x, layout=layout, causal=causal, scale=scale)
    dQ, dK, dV, _, _ = ref_bwd(x["q"], x["k"], x["v"], x["do"], causal=causal, scale=scale,
                               kv_lens=x["kv_lens"])
    _check(name + " dq", from_layout(host(dq), layout), dQ)
    _check(name + " dk", from_layout(host(dk), layout), dK)
    _check(name + " dv", from_layout(host(dv), layout), dV)


def test_backward_16bit_gradients(gpu_lib):
    _say("[bwd] 16-bit gradient outputs")
    w, x = make_case(1, 4, 2, 160, 160, 64, "bf16", seed=11, with_do=True)
    dq, dk, dv = _run(w, x, causal=True, grad_dtype="bf16")
    import torch
    assert dq.dtype == torch.bfloat16
    dQ, dK, dV, _, _ = ref_bwd(x["q"], x["k"], x["v"], x["do"], causal=True)
    # bf16 outputs: the output rounding alone is up to half an ulp of |x|
    for nm, g, r in (("dq", dq, dQ), ("dk", dk, dK), ("dv", dv, dV)):
        _check(nm, g, r, tol=2e-2 + 2 ** -8 * float(np.abs(r).max()), rel=2e-2)


def test_backward_is_deterministic(gpu_lib):
    import torch
    _say("[bwd] determinism")
    w, x = make_case(1, 16, 1, 200, 200, 128, "bf16", seed=12, with_do=True)
    a = _run(w, x, causal=True)
    b = _run(w, x, causal=True)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_workload_causal_gqa_backward(gpu_lib):
    """Full-size causal GQA backward: dQ, dK and dV of every (batch, kv-head)
    group (all 16 q-heads, all rows and keys) against the oracle's exact
    backward, element by element."""
    from tests.full_size import backward_all_groups
    w = inputs.WORKLOADS["causal_gqa_bf16_b4_h32_kv2_n8192_d128"]
    _say("[bwd-workload] generating inputs")
    x = inputs.make_inputs(w)
    _say("[bwd-workload] GPU forward + backward")
    dq, dk, dv = _run(w, x, causal=True)
    dq, dk, dv = (t.float().cpu().numpy() for t in (dq, dk, dv))
    _say(f"[bwd-workload] oracle over all {w.B * w.Hkv} (batch, kv-head) groups")
    tot, secs = backward_all_groups(w, x, dq, dk, dv)
    for n, st in tot.items():
        _say(f"[bwd-workload] {n}: max-abs {st.max_abs:.3e} rel-rms {st.rel_rms:.3e}")
    _say(f"[bwd-workload] oracle {secs:.1f} s")
    assert tot["dq"].n == dq.size and tot["dk"].n == dk.size and tot["dv"].n == dv.size
    for n, st in tot.items():
        assert st.finite, f"{n}: non-finite"
        assert st.max_abs <= TOL, f"{n}: max-abs {st.max_abs:.3e} > {TOL}"
        assert st.rel_rms <= TOL_REL_RMS, f"{n}: rel-rms {st.rel_rms:.3e}"


# bf16 inputs outside the fp16 range of the backward's operand copies: above
# 65504, below 2^-14, or with dP = dO V^T beyond 65504.  Each tensor t is the
# seeded draw times 2^e_t (exact in bf16); the oracle runs on the same scaled
# values.  Gradients scale with the inputs (dV with dO; dQ with K V dO; dK
# with Q V dO), so the bars are relative: max-abs <= 1e-2 max|ref| and
# relative RMS <= 1e-2.
RANGE = [
    # id, exponents (q, k, v, do), causal, lens
    ("q_above_k_below", (17, -17, 0, 0), True, (90, 200)),
    ("v_below_do_above", (0, 0, -20, 18), False, None),
    ("all_below_fp16_normal", (-20, -20, -20, -20), True, None),
    ("dp_above_fp16_range", (0, 0, 7, 7), False, (120, 200)),
]


@pytest.mark.parametrize("case", RANGE, ids=[c[0] for c in RANGE])
def test_backward_bf16_beyond_fp16_range(gpu_lib, case):
    import torch
    from exact_attention_25_amd import binding as bd
    name, ex, causal, lens = case
    _say(f"[bwd-range] {name}")
    w, x = make_case(2, 4, 2, 200, 200, 64, "bf16", seed=zlib.crc32(name.encode()) % 10000,
                     lens=lens, with_do=True)
    t = {}
    for n, e in zip(("q", "k", "v", "do"), ex):
        t[n] = to_device(x[n + "_raw"], "bf16") * (2.0 ** e)   # exact in bf16
        x[n] = x[n] * (2.0 ** e)
    lens_d = None if x["kv_lens"] is None else torch.from_numpy(x["kv_lens"]).cuda()
    o, lse = bd.attn_fwd(t["q"], t["k"], t["v"], causal=causal, kv_lens=lens_d)
    dq, dk, dv = bd.attn_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=causal,
                             kv_lens=lens_d)
    torch.cuda.synchronize()
    dQ, dK, dV, _, _ = ref_bwd(x["q"], x["k"], x["v"], x["do"], causal=causal,
                               kv_lens=x["kv_lens"])
    for lbl, got, ref in (("dq", dq, dQ), ("dk", dk, dK), ("dv", dv, dV)):
        top = float(np.abs(ref).max())
        mx = _check(f"{name} {lbl}", got, ref, tol=1e-2 * top, rel=1e-2)
        _say(f"  {lbl}: max|ref| {top:.3e}, max-abs {mx:.3e}")
