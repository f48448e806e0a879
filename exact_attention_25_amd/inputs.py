"""Seeded synthetic inputs, shared by the tests, the benchmark and the oracle.

This module holds no attention arithmetic: it draws Gaussian tensors and
integer lengths from numpy's PCG64 generator and rounds them to the storage
type the GPU reads (round-to-nearest-even).  The oracle is fed exactly the
rounded values (as float32 arrays, which hold every fp16/bf16 value exactly).

Seeding: tensor t of workload w is drawn from
``numpy.random.default_rng([w.seed, t])`` with t = 0 (q), 1 (k), 2 (v),
3 (dO), 4 (key lengths).  Values are N(0, 1) * std in float64, then cast to
float32, then to the storage type.

The workloads stand in for the pages' cases (no dataset is used): a tiny fp32
case; a ViT at 224x224 with 16x16 patches (196 tokens, 16 heads of 64); a
Stable-Diffusion-1.5 UNet latent of 64x64 (4096 tokens, 8 heads of 40) with a
77-token text cross-attention whose valid lengths vary per sample; the
B8 H32 N4096 d128 benchmark shape; a causal grouped-query decoder at 8192
tokens with per-sequence valid lengths; decode steps against a 32K cache; and
the FlexAttention cases of the PyTorch attention-options article (a ViT with
3136 tokens under the tanh soft cap or the 2-D neighbourhood mask).  A
workload may draw q and k with their own std (``qk_std``), so that the
logits reach a soft cap while v keeps unit scale.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3, "lens": 4}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    dtype: str            # "fp32" | "fp16" | "bf16"
    seed: int
    std: float = 1.0
    causal: bool = False
    lens: tuple | None = None   # inclusive uniform range of valid key counts
    backward: bool = False
    # local attention / soft cap of the call (see attn_params in include/attn.h)
    window: tuple | None = None  # (left, right), -1 = open side
    grid: tuple | None = None    # (cols, nbr_rows, nbr_cols)
    softcap: float = 0.0
    qk_std: float | None = None  # std of q and k when it differs from std (v, dO)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_fp32_b1_h2_n128_d64", 1, 2, 2, 128, 128, 64, "fp32", 1),
        Workload("vit_bf16_b128_h16_n196_d64", 128, 16, 16, 196, 196, 64, "bf16", 2, std=0.5),
        Workload("unet_self_fp16_b2_h8_n4096_d40", 2, 8, 8, 4096, 4096, 40, "fp16", 3),
        Workload("unet_cross_fp16_b2_h8_q4096_k77_d40", 2, 8, 8, 4096, 77, 40, "fp16", 31,
                 lens=(20, 77)),
        Workload("long_bf16_b8_h32_n4096_d128", 8, 32, 32, 4096, 4096, 128, "bf16", 4),
        Workload("causal_gqa_bf16_b4_h32_kv2_n8192_d128", 4, 32, 2, 8192, 8192, 128, "bf16", 5,
                 causal=True, lens=(4096, 8192), backward=True),
        # decode: one new token per sequence against a 32K key/value cache whose
        # valid lengths vary over the batch (served with attn_decode)
        Workload("decode_bf16_b8_hq32_kv8_q1_nk32768_d128", 8, 32, 8, 1, 32768, 128, "bf16", 6,
                 lens=(16384, 32768)),
        # the FlexAttention examples of the PyTorch attention-options article:
        # a ViT at 224x224 with 4x4 patches (56 x 56 = 3136 tokens, 12 heads of
        # 64, batch 8), once with the tanh soft cap 30 (inputs scaled so that
        # the logits reach the cap) and once with the neighbourhood mask (row
        # and column differences < 5 on the 56 x 56 grid)
        Workload("vit_softcap_bf16_b8_h12_n3136_d64", 8, 12, 12, 3136, 3136, 64, "bf16", 7,
                 qk_std=2.5, softcap=30.0),
        Workload("vit_nbr_bf16_b8_h12_n3136_d64", 8, 12, 12, 3136, 3136, 64, "bf16", 8,
                 grid=(56, 5, 5)),
        # a sliding-window decode step: one new token, window of 4096 keys
        # behind it, against the same 32K cache
        Workload("decode_window_bf16_b8_hq32_kv8_q1_nk32768_d128", 8, 32, 8, 1, 32768, 128,
                 "bf16", 9, causal=True, lens=(16384, 32768), window=(4095, 0)),
    ]
}


def sweep_workload(n: int) -> Workload:
    """Long-context sweep point: B*N held at 32768, H=32, d=128, bf16."""
    if n not in (1024, 2048, 4096, 8192, 16384):
        raise ValueError("sweep N must be one of 1024..16384 (powers of two)")
    return Workload(f"long_bf16_sweep_b{32768 // n}_h32_n{n}_d128", 32768 // n, 32, 32, n, n,
                    128, "bf16", 40 + int(math.log2(n)))


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 values (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def storage(x64: np.ndarray, dtype: str):
    """Round fp64 draws to the storage dtype.

    Returns (exact_values_f32, storage_array) where storage_array is float32,
    float16, or uint16 bfloat16 bits.
    """
    x32 = x64.astype(np.float32)
    if dtype == "fp32":
        return x32, x32
    if dtype == "fp16":
        h = x32.astype(np.float16)
        return h.astype(np.float32), h
    if dtype == "bf16":
        bits = bf16_bits(x32)
        return bf16_value(bits), bits
    raise ValueError(f"unknown dtype {dtype!r}")


def draw(seed: int, tensor: str, shape, std: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng([seed, TENSOR_IDS[tensor]])
    x = rng.standard_normal(size=shape)
    if std != 1.0:
        x *= std
    return x


def draw_lens(seed: int, B: int, lo: int, hi: int) -> np.ndarray:
    rng = np.random.default_rng([seed, TENSOR_IDS["lens"]])
    return rng.integers(lo, hi + 1, size=B).astype(np.int32)


def make_inputs(w: Workload, with_do: bool | None = None) -> dict:
    """All inputs of a workload in [B, H, N, d] order.

    Keys: q, k, v (exact float32 values), q_raw, k_raw, v_raw (storage
    arrays), kv_lens (int32 [B] or None), and do / do_raw when the workload
    has a backward (or ``with_do``).
    """
    out = {}
    shapes = {"q": (w.B, w.Hq, w.Nq, w.d), "k": (w.B, w.Hkv, w.Nk, w.d),
              "v": (w.B, w.Hkv, w.Nk, w.d), "do": (w.B, w.Hq, w.Nq, w.d)}
    names = ["q", "k", "v"]
    if with_do or (with_do is None and w.backward):
        names.append("do")
    for t in names:
        std = w.qk_std if (w.qk_std is not None and t in ("q", "k")) else w.std
        exact, raw = storage(draw(w.seed, t, shapes[t], std), w.dtype)
        out[t] = exact
        out[t + "_raw"] = raw
    out["kv_lens"] = None if w.lens is None else draw_lens(w.seed, w.B, *w.lens)
    return out
