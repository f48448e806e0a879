"""FP8 block quantisation and attention on quantised inputs (fp64 reference).

TEST INFRASTRUCTURE ONLY (see the package docstring): the GPU library never
imports or calls this module.

The pages describe FP8 attention as block quantisation: the matrix products
run on FP8 operands, every block keeps its own scale factor, and the score /
softmax arithmetic stays at higher precision -- page
"FlashAttention技术解析：优化Transformer注意力计算效率" (jsqmd.com/news/722897),
§4.2 item 3 (FP8 support) and §6.3 item 2 (each block keeps an independent
scale; the critical path stays at 16-bit precision; m and l in fp32, §6.3
item 1).  The pages fix neither the FP8 format nor the block size; the
readings taken here (listed in the design notes) are:

* format: OCP FP8 E4M3 "fn" (1 sign, 4 exponent bits with bias 7, 3 mantissa
  bits; no infinities; the all-ones exponent and mantissa pattern is NaN;
  largest finite value 448 = 1.75 * 2^8; subnormals m * 2^-9), rounded to
  nearest with ties to even; a result beyond 448 after rounding is NaN;
* blocks: 64 consecutive rows (query rows of Q, key rows of K and V) of one
  (batch, head), all d columns; scale = amax / 448 of the block (1 for an
  all-zero block), so the block's largest magnitude maps to 448;
* the codes are computed as in single precision: s = fp32(amax) / 448 and
  inv = 448 / fp32(amax) are correctly rounded fp32 divisions, the scaled
  value fp32(x * inv) is one correctly rounded fp32 product, and that value
  is rounded to E4M3; a value is code * s.

``ref_fwd_fp8`` is attention (``ref_fwd``) on the dequantised inputs: the
exact result the quantised operands define.  How a kernel rounds its
probabilities for the second FP8 product is its own approximation and is
bounded in the tests, not modelled here.
"""
from __future__ import annotations

import numpy as np

from .attention_ref import ref_fwd

E4M3_MAX = 448.0
BLOCK = 64


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3FN code (uint8 array) as float64; NaN for 0x7F/0xFF."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = m * 2.0 ** -9
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, v)


def e4m3_encode(x) -> np.ndarray:
    """Round float values to E4M3FN codes (nearest, ties to even).

    Values whose rounded magnitude exceeds 448 become NaN (0x7F with the
    sign bit of x), as do NaN inputs.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    neg = np.signbit(x)
    # exponent of the binade (normal range starts at 2^-6); below it the
    # spacing is that of the subnormals, 2^-9
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)
    spacing = np.exp2(e - 3)
    q = a / spacing
    n = np.floor(q)
    frac = q - n
    n = n + ((frac > 0.5) | ((frac == 0.5) & (np.fmod(n, 2) == 1)))
    v = n * spacing                       # the rounded magnitude
    out = np.zeros(x.shape, dtype=np.int64)
    sub = v < 2.0 ** -6
    out = np.where(sub, np.round(v / 2.0 ** -9), 0)
    with np.errstate(divide="ignore"):
        ev = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    mant = np.round((v / np.exp2(ev) - 1.0) * 8.0)
    norm_code = ((ev + 7).astype(np.int64) << 3) | mant.astype(np.int64)
    out = np.where(sub, out, norm_code).astype(np.int64)
    bad = (v > E4M3_MAX) | np.isnan(x)
    out = np.where(bad, 0x7F, out)
    out = out | np.where(neg, 0x80, 0)
    return out.astype(np.uint8)


def quantize_blocks(x, block: int = BLOCK):
    """Block quantisation of a [B, H, N, d] array along N.

    Returns (codes uint8 [B, H, N, d], scales float32 [B, H, ceil(N/block)]),
    following the single-precision recipe of the module docstring.
    """
    x32 = np.asarray(x, dtype=np.float32)
    B, H, N, d = x32.shape
    nb = -(-N // block)
    codes = np.zeros(x32.shape, dtype=np.uint8)
    scales = np.ones((B, H, nb), dtype=np.float32)
    for i in range(nb):
        blk = x32[:, :, i * block:(i + 1) * block, :]
        amax = np.abs(blk).max(axis=(2, 3)) if blk.size else np.zeros((B, H), np.float32)
        amax = amax.astype(np.float32)
        pos = amax > 0
        s = np.where(pos, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        inv = np.where(pos, np.float32(E4M3_MAX) / np.where(pos, amax, np.float32(1.0)),
                       np.float32(1.0)).astype(np.float32)
        y = (blk * inv[:, :, None, None]).astype(np.float32)
        codes[:, :, i * block:(i + 1) * block, :] = e4m3_encode(y)
        scales[:, :, i] = s
    return codes, scales


def dequantize_blocks(codes, scales, block: int = BLOCK) -> np.ndarray:
    """codes [B, H, N, d] with scales [B, H, ceil(N/block)] -> float64 values."""
    v = e4m3_decode(codes)
    s = np.repeat(np.asarray(scales, dtype=np.float64), block, axis=2)[:, :, :v.shape[2]]
    return v * s[..., None]


def ref_fwd_fp8(q_codes, k_codes, v_codes, q_scale, k_scale, v_scale, *, block: int = BLOCK,
                **kw):
    """Attention on the dequantised FP8 inputs ([B, H, N, d] codes, 'bhnd'):
    ``ref_fwd(dequantize(q), dequantize(k), dequantize(v), **kw)``."""
    q = dequantize_blocks(q_codes, q_scale, block)
    k = dequantize_blocks(k_codes, k_scale, block)
    v = dequantize_blocks(v_codes, v_scale, block)
    return ref_fwd(q, k, v, **kw)
