"""GPU parity of the FP8 path: attn_quantize_fp8 and attn_fwd_fp8.

* The quantiser is byte work decided in fp32 (amax, 448 / amax, x * inv,
  round to E4M3): its codes and scales must equal the oracle's
  (oracle/fp8_ref.py) bit for bit, V transposed with zero padding.
* The forward takes the oracle's own codes and scales and is compared with
  attention on the dequantised inputs (ref_fwd_fp8).  Its one approximation
  is the rounding of the probabilities to E4M3 for the product with V; each
  rounding errs by at most 2^-4 of the probability, or 2^-10 in the kernel's
  scaled units where it falls below E4M3's normal range.  The kernel scales p
  by 2^6 sv / svmax relative to a reference no larger than the row's
  maximum, so the row's largest weight is at least 2^6 ratio (ratio = the
  tile's V scale over the head's largest) and a subnormal rounding is at
  most 2^-16 / ratio of the row's total weight.  O is
  divided by the sum of the rounded weights, so
  O - O_ref = sum_j (p~_j - p_j)(v_j - O_ref) / sum_j p~_j, and per element
      |O - O_ref|_ic <= c sum_j P_ij |v_jc - O_ref_ic|
                        + 2^-16 / ratio_min sum_j |v_jc - O_ref_ic| / (1 - 2^-4)
                        + 2^-8 |O_ref_ic| + 1e-6,   c = 2^-4 / (1 - 2^-4)
  (the third term covers the 16-bit output rounding and fp32 sums), with P
  and v the oracle's probabilities and dequantised values.  LSE comes from
  the fp32 sum of the unrounded p and is held to 2e-4.
* The relative RMS error is statistical: rounding to 3 mantissa bits (RNE)
  errs by ulp/2 uniformly, so for values spread log-uniformly over a binade
  its RMS relative error is 2^-3 / (2 sqrt 3) * sqrt(E[1/m^2]) with
  E[1/m^2] = (1/2 - 1/8) / ln 2 over m in [1, 2): 0.0265.  For O, a
  p-weighted mean of v whose weights carry that error independently, the
  RMS error relative to rms(O) is the same 0.0265 when the attention is
  spread over many keys; the bar is 1.5 times that, 0.04.
"""
import sys
import zlib

import numpy as np
import pytest

from exact_attention_25_amd import inputs
from oracle import ref_probs
from oracle.fp8_ref import dequantize_blocks, quantize_blocks, ref_fwd_fp8
from tests.gpu_util import from_layout, host, make_case, to_device, to_layout

pytestmark = pytest.mark.gpu

REL_RMS = 0.04


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _vt(codes, nk_pad):
    """[B, H, N, d] codes -> [B, H, d, nk_pad] with zero columns past N."""
    B, H, N, d = codes.shape
    out = np.zeros((B, H, d, nk_pad), dtype=np.uint8)
    out[..., :N] = codes.transpose(0, 1, 3, 2)
    return out


def _up(a):
    """numpy array (codes or scales) -> device tensor of the same dtype."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


QUANT = [
    # id, B, Hq, Hkv, Nq, Nk, d, dtype, layout
    ("bf16_ragged", 2, 4, 2, 130, 200, 128, "bf16", "bhnd"),
    ("fp16_bnhd", 1, 2, 1, 64, 77, 64, "fp16", "bnhd"),
    ("fp32_d48", 1, 2, 2, 65, 63, 48, "fp32", "bhnd"),
    ("bf16_one_row", 2, 2, 2, 1, 1, 16, "bf16", "bnhd"),
]


@pytest.mark.parametrize("case", QUANT, ids=[c[0] for c in QUANT])
def test_quantiser_is_bit_exact(gpu_lib, case):
    import torch
    from exact_attention_25_amd import binding as bd
    name, B, Hq, Hkv, Nq, Nk, d, dtype, layout = case
    _say(f"[fp8-quant] {name}")
    w, x = make_case(B, Hq, Hkv, Nq, Nk, d, dtype, seed=zlib.crc32(name.encode()) % 10000,
                     std=1.7)
    # an all-zero head (scale 1, zero codes)
    for n in ("q", "k", "v"):
        x[n][0, 0] = 0.0
        x[n + "_raw"][0, 0] = 0
    t = {n: to_device(to_layout(x[n + "_raw"], layout), dtype) for n in ("q", "k", "v")}
    q8, k8, vt8, qs, ks, vs = bd.attn_quantize_fp8(t["q"], t["k"], t["v"], layout=layout)
    torch.cuda.synchronize()
    (qc, qsc), (kc, ksc), (vc, vsc) = (quantize_blocks(x[n]) for n in ("q", "k", "v"))
    assert np.array_equal(from_layout(q8.cpu().numpy(), layout), qc)
    assert np.array_equal(from_layout(k8.cpu().numpy(), layout), kc)
    assert np.array_equal(vt8.cpu().numpy(), _vt(vc, vt8.shape[-1]))
    for got, want in ((qs, qsc), (ks, ksc), (vs, vsc)):
        assert np.array_equal(got.cpu().numpy(), want)


def _check_fp8(o, lse, O_ref, L_ref, P, Vd, vsc, G, label, out_dtype):
    """Element bound of the module docstring; P [B,Hq,Nq,Nk], Vd [B,Hkv,Nk,d]."""
    O = host(o)
    L = host(lse)
    assert np.all(np.isfinite(O)), label
    err = np.abs(O - O_ref)
    c = 2.0 ** -4 / (1 - 2.0 ** -4)
    ratio_min = vsc.min(axis=2) / vsc.max(axis=2)       # [B, Hkv]
    bound = np.empty_like(O_ref)
    for bb in range(O_ref.shape[0]):
        for hh in range(O_ref.shape[1]):
            v = Vd[bb, hh // G]                          # [Nk, d]
            for i in range(O_ref.shape[2]):
                dev = np.abs(v - O_ref[bb, hh, i])       # |v_j - O_i| per key and column
                bound[bb, hh, i] = (c * (P[bb, hh, i] @ dev)
                                    + 2.0 ** -16 / (1 - 2.0 ** -4) / ratio_min[bb, hh // G]
                                    * dev.sum(axis=0))
    bound += 2.0 ** -8 * np.abs(O_ref) + 1e-6
    worst = float((err / bound).max()) if err.size else 0.0
    rms_ref = float(np.sqrt(np.mean(O_ref ** 2))) if O_ref.size else 0.0
    rel = float(np.sqrt(np.mean(err ** 2))) / rms_ref if rms_ref > 0 else 0.0
    _say(f"  {label}: max-abs {err.max():.3e}, max err/bound {worst:.3f}, rel-rms {rel:.3e}")
    assert worst <= 1.0, f"{label}: error above the FP8 bound (x{worst:.2f})"
    assert rel <= REL_RMS, f"{label}: rel-rms {rel:.3e}"
    dead = np.isneginf(L_ref)
    assert np.array_equal(np.isneginf(L), dead), label
    if (~dead).any():
        lerr = float(np.abs(L[~dead] - L_ref[~dead]).max())
        assert lerr <= 2e-4 + 1e-6 * float(np.abs(L_ref[~dead]).max()), f"{label}: LSE {lerr:.3e}"


FWD = [
    # id, B, Hq, Hkv, Nq, Nk, d, out, layout, causal, lens, std
    ("gqa_d128_bf16", 2, 8, 2, 300, 300, 128, "bf16", "bhnd", False, None, 1.0),
    ("causal_d64_fp16_bnhd_lens", 2, 4, 4, 257, 257, 64, "fp16", "bnhd", True, (100, 257), 1.0),
    ("d48_ragged_lens_zero", 2, 2, 1, 130, 77, 48, "bf16", "bhnd", False, (0, 77), 1.0),
    ("cross_nq_ne_nk_d128", 1, 4, 1, 70, 1000, 128, "bf16", "bnhd", False, None, 1.0),
    ("sharp_logits_d128", 1, 2, 2, 256, 512, 128, "bf16", "bhnd", False, None, 2.0),
    ("causal_gqa16_d128", 1, 16, 1, 200, 200, 128, "fp16", "bhnd", True, None, 1.0),
]


@pytest.mark.parametrize("case", FWD, ids=[c[0] for c in FWD])
def test_fp8_forward(gpu_lib, case):
    import torch
    from exact_attention_25_amd import binding as bd
    name, B, Hq, Hkv, Nq, Nk, d, out, layout, causal, lens, std = case
    _say(f"[fp8-fwd] {name}")
    w, x = make_case(B, Hq, Hkv, Nq, Nk, d, "fp32", seed=zlib.crc32(name.encode()) % 10000,
                     lens=lens, qk_std=std)
    (qc, qs), (kc, ks), (vc, vs) = (quantize_blocks(x[n]) for n in ("q", "k", "v"))
    nkp = (Nk + 63) // 64 * 64
    lens_t = None if x["kv_lens"] is None else torch.from_numpy(x["kv_lens"]).cuda()
    o, lse = bd.attn_fwd_fp8(_up(to_layout(qc, layout)), _up(to_layout(kc, layout)),
                             _up(_vt(vc, nkp)), _up(qs), _up(ks), _up(vs), layout=layout,
                             causal=causal, kv_lens=lens_t,
                             out_dtype=torch.bfloat16 if out == "bf16" else torch.float16)
    torch.cuda.synchronize()
    O_ref, L_ref = ref_fwd_fp8(qc, kc, vc, qs, ks, vs, causal=causal, kv_lens=x["kv_lens"])
    Qd, Kd, Vd = dequantize_blocks(qc, qs), dequantize_blocks(kc, ks), dequantize_blocks(vc, vs)
    P = ref_probs(Qd, Kd, causal=causal, kv_lens=x["kv_lens"])
    _check_fp8(from_layout(host(o), layout), lse, O_ref, L_ref, P, Vd, vs, Hq // Hkv, name, out)


def test_fp8_workload_sampled_heads(gpu_lib):
    """B8 H32 N4096 d128 from the bf16 benchmark inputs: the GPU quantiser's
    codes of sampled heads equal the oracle's, and the FP8 forward's rows of
    those heads meet the bound against attention on the dequantised inputs."""
    import torch
    from exact_attention_25_amd import binding as bd
    w = inputs.WORKLOADS["long_bf16_b8_h32_n4096_d128"]
    _say("[fp8-workload] inputs")
    x = inputs.make_inputs(w, with_do=False)
    t = {n: to_device(x[n + "_raw"], w.dtype) for n in ("q", "k", "v")}
    _say("[fp8-workload] GPU quantise + forward")
    q8, k8, vt8, qs, ks, vs = bd.attn_quantize_fp8(t["q"], t["k"], t["v"])
    o, lse = bd.attn_fwd_fp8(q8, k8, vt8, qs, ks, vs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    for (b, h) in [(0, 0), (7, 31), (int(rng.integers(8)), int(rng.integers(32)))]:
        _say(f"[fp8-workload] head ({b}, {h})")
        sl = (slice(b, b + 1), slice(h, h + 1))
        (qc, qsc), (kc, ksc), (vc, vsc) = (quantize_blocks(x[n][sl]) for n in ("q", "k", "v"))
        assert np.array_equal(q8[sl].cpu().numpy(), qc)
        assert np.array_equal(k8[sl].cpu().numpy(), kc)
        assert np.array_equal(vt8[sl].cpu().numpy(), _vt(vc, vt8.shape[-1]))
        assert np.array_equal(qs[sl].cpu().numpy(), qsc) and np.array_equal(vs[sl].cpu().numpy(), vsc)
        rows = np.sort(rng.choice(w.Nq, size=48, replace=False))
        Qd = dequantize_blocks(qc, qsc)[:, :, rows]
        Kd, Vd = dequantize_blocks(kc, ksc), dequantize_blocks(vc, vsc)
        from oracle import ref_fwd
        O_ref, L_ref = ref_fwd(Qd, Kd, Vd)
        P = ref_probs(Qd, Kd)
        _check_fp8(host(o)[b:b + 1, h:h + 1][:, :, rows], host(lse)[b:b + 1, h:h + 1][:, :, rows],
                   O_ref, L_ref, P, Vd, vsc, 1, f"head ({b}, {h})", "bf16")
