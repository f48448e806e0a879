"""CPU model of the tiled double loop with an online softmax (fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

This follows the algorithm as page "FlashAttention技术解析：优化Transformer
注意力计算效率" (jsqmd.com/news/722897) states it in §2.2: Q is cut into
blocks of B_r rows (outer loop) and K/V into blocks of B_c rows (inner loop);
for each query row a running maximum m and a running exponential sum l are
kept and rescaled whenever a new block raises the maximum, so that the final
result equals the full softmax.  §4.1 of the same page adds the deferred
rescaling of FlashAttention-2: the division by l happens once, at the end.

Two options model choices a GPU implementation may make, without changing the
exact result:

* ``skip_masked_tiles``: a key block in which every key is masked for every
  row of the query block (beyond ``kv_len``, or wholly above the causal
  diagonal) is not visited at all;
* ``rescale_threshold``: when not None, the running maximum used as the
  exponent's reference point is only moved when a block's maximum exceeds it
  by more than this many natural-log units; in exact arithmetic the final
  O = sum(p v) / sum(p) does not depend on the reference point.

The model exists to show, on small inputs, that the recurrence reaches the
plain definition in ``attention_ref``; it is never used as the reference for
GPU results.
"""
from __future__ import annotations

import math

import numpy as np


def tiled_fwd(q, k, v, *, block_r: int, block_c: int, scale=None,
              causal=False, mask=None, kv_lens=None, skip_masked_tiles=True,
              rescale_threshold=None):
    """Tiled online-softmax forward on [B,Hq,Nq,d] / [B,Hkv,Nk,d] arrays.

    Returns (O, LSE) in fp64; O is [B,Hq,Nq,d] and LSE [B,Hq,Nq].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    grp = Hq // Hkv
    if scale is None or not (float(scale) > 0.0):
        s = 1.0 / math.sqrt(d)
    else:
        s = float(scale)
    if causal and Nq != Nk:
        raise ValueError("causal attention needs Nq == Nk")
    mask_full = None if mask is None else np.broadcast_to(
        np.asarray(mask, dtype=np.float64), (B, Hq, Nq, Nk))

    O = np.zeros((B, Hq, Nq, d))
    LSE = np.zeros((B, Hq, Nq))
    for b in range(B):
        L = Nk if kv_lens is None else int(min(max(int(kv_lens[b]), 0), Nk))
        for h in range(Hq):
            Kh, Vh = k[b, h // grp], v[b, h // grp]
            for r0 in range(0, Nq, block_r):          # outer loop: query blocks
                r1 = min(r0 + block_r, Nq)
                Qi = q[b, h, r0:r1]
                nr = r1 - r0
                m = np.full(nr, -np.inf)              # running max
                l = np.zeros(nr)                      # running exp-sum
                acc = np.zeros((nr, d))               # unnormalised output
                for c0 in range(0, Nk, block_c):      # inner loop: key blocks
                    c1 = min(c0 + block_c, Nk)
                    if skip_masked_tiles:
                        if c0 >= L:
                            continue                  # all keys padded out
                        if causal and c0 > r1 - 1:
                            continue                  # block above the diagonal
                    Sij = (Qi @ Kh[c0:c1].T) * s
                    if mask_full is not None:
                        Sij = Sij + mask_full[b, h, r0:r1, c0:c1]
                    cols = np.arange(c0, c1)
                    Sij[:, cols >= L] = -np.inf
                    if causal:
                        rows = np.arange(r0, r1)
                        Sij[cols[None, :] > rows[:, None]] = -np.inf
                    bmax = Sij.max(axis=1)
                    m_new = np.maximum(m, bmax)
                    if rescale_threshold is not None:
                        # keep the old reference point unless the block's
                        # maximum overtakes it by more than the threshold
                        keep = np.isfinite(m) & (bmax <= m + rescale_threshold)
                        m_new = np.where(keep, m, m_new)
                    # reference point for the exponentials: a row that has
                    # seen no visible key yet keeps 0 so exp(-inf - 0) = 0
                    ref = np.where(np.isfinite(m_new), m_new, 0.0)
                    alpha = np.where(np.isfinite(m), np.exp(m - ref), 0.0)
                    p = np.exp(Sij - ref[:, None])
                    l = alpha * l + p.sum(axis=1)
                    acc = alpha[:, None] * acc + p @ Vh[c0:c1]
                    m = m_new
                dead = l == 0.0
                O[b, h, r0:r1] = np.where(dead[:, None], 0.0,
                                          acc / np.where(dead, 1.0, l)[:, None])
                with np.errstate(divide="ignore"):
                    LSE[b, h, r0:r1] = np.where(
                        dead, -np.inf,
                        np.where(np.isfinite(m), m, 0.0) + np.log(np.where(dead, 1.0, l)))
    return O, LSE
