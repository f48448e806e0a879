"""Algorithmic work and traffic of attention, for throughput and rooflines.

FLOPs count what the method must compute, with the real head dimension d:

* forward: 4 * B * Hq * Nq * Nk * d (two matrix products of 2*N*N*d each),
  halved for causal attention -- the 4N^2 d count of page
  "FlashAttention技术解析：优化Transformer注意力计算效率"
  (jsqmd.com/news/722897) §3.1;
* backward: 10 * B * Hq * Nq * Nk * d (recompute of S plus dV, dP, dQ, dK),
  halved for causal.

Bytes are the minimum traffic: Q, K, V (and the optional lengths) read once,
O and LSE written once.  K/V re-reads, padding and recompute are not counted.
"""
from __future__ import annotations

ELEM_BYTES = {"fp32": 4, "fp16": 2, "bf16": 2}

# MI355X published peaks
PEAK_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6, "fp32": 157.3, "fp8": 5033.2}
PEAK_HBM_GBS = 8000.0


def fwd_flops(B, Hq, Nq, Nk, d, causal=False) -> float:
    f = 4.0 * B * Hq * Nq * Nk * d
    return f / 2 if causal else f


def bwd_flops(B, Hq, Nq, Nk, d, causal=False) -> float:
    f = 10.0 * B * Hq * Nq * Nk * d
    return f / 2 if causal else f


def useful_pairs(Nq, Nk, kv_lens=None, causal=False, B=1) -> int:
    """Number of visible (query, key) pairs summed over the batch."""
    lens = [Nk] * B if kv_lens is None else [min(max(int(x), 0), Nk) for x in kv_lens]
    tot = 0
    for L in lens:
        if causal:
            # query i sees keys 0..min(i, L-1)
            full = min(L, Nq)
            tot += full * (full + 1) // 2 + max(Nq - L, 0) * L
        else:
            tot += Nq * L
    return tot


def local_pairs(N, kv_lens=None, B=1, causal=False, window=None, grid=None) -> int:
    """Visible (query, key) pairs of a self-attention of N positions summed
    over the batch, under key padding, causal masking, a sliding window
    (left, right; -1 = open) and a 2-D neighbourhood (cols, nbr_rows,
    nbr_cols): the work a local forward must do, 4 d FLOPs per pair and head.
    """
    import numpy as np
    lens = [N] * B if kv_lens is None else [min(max(int(x), 0), N) for x in kv_lens]
    wl, wr = (-1, -1) if window is None else (int(window[0]), int(window[1]))
    if causal:
        wr = 0 if wr < 0 else min(wr, 0)
    tot = 0
    j = np.arange(N, dtype=np.int64)[None, :]
    for L in lens:
        for i0 in range(0, N, 512):
            i = np.arange(i0, min(i0 + 512, N), dtype=np.int64)[:, None]
            ok = j < L
            if wl >= 0:
                ok = ok & (j >= i - wl)
            if wr >= 0:
                ok = ok & (j <= i + wr)
            if grid is not None:
                c, nr, nc = (int(x) for x in grid)
                ok = ok & (np.abs(i // c - j // c) < nr) & (np.abs(i % c - j % c) < nc)
            tot += int(ok.sum())
    return tot


def decode_pairs(Nq, Nk, kv_lens=None, B=1, causal=False, window=None) -> int:
    """Visible (query, key) pairs of a decode call summed over the batch: the
    Nq queries sit at positions L - Nq + i of each batch's L keys."""
    lens = [Nk] * B if kv_lens is None else [min(max(int(x), 0), Nk) for x in kv_lens]
    wl, wr = (-1, -1) if window is None else (int(window[0]), int(window[1]))
    if causal:
        wr = 0 if wr < 0 else min(wr, 0)
    tot = 0
    for L in lens:
        for i in range(Nq):
            p = L - Nq + i
            lo = 0 if wl < 0 else max(p - wl, 0)
            hi = L - 1 if wr < 0 else min(p + wr, L - 1)
            tot += max(hi - lo + 1, 0)
    return tot


def fwd_min_bytes(B, Hq, Hkv, Nq, Nk, d, dtype, with_lens=False) -> int:
    e = ELEM_BYTES[dtype]
    return (B * Hq * Nq * d * e * 2          # Q in, O out
            + B * Hkv * Nk * d * e * 2       # K, V in
            + B * Hq * Nq * 4                # LSE out
            + (B * 4 if with_lens else 0))


def bwd_min_bytes(B, Hq, Hkv, Nq, Nk, d, dtype, grad_bytes=4) -> int:
    e = ELEM_BYTES[dtype]
    return (B * Hq * Nq * d * e * 3          # Q, O, dO in
            + B * Hkv * Nk * d * e * 2       # K, V in
            + B * Hq * Nq * 4 * 2            # LSE in, D out/in
            + B * Hq * Nq * d * grad_bytes   # dQ out
            + B * Hkv * Nk * d * grad_bytes * 2)  # dK, dV out


def decode_min_bytes(B, Hq, Hkv, Nq, Nk, d, dtype, kv_lens=None, window_left=-1) -> int:
    """Minimum traffic of a decode call: the visible part of the K/V cache
    read once (kv_lens[b] entries of batch b, or Nk; with a bounded left
    window only the last Nq + window_left of them), Q read, O and LSE
    written."""
    e = ELEM_BYTES[dtype]
    lens = [Nk] * B if kv_lens is None else [min(max(int(x), 0), Nk) for x in kv_lens]
    if window_left is not None and window_left >= 0:
        lens = [min(L, Nq + int(window_left)) for L in lens]
    return (sum(lens) * Hkv * d * e * 2      # K, V in (valid entries)
            + B * Hq * Nq * d * e * 2        # Q in, O out
            + B * Hq * Nq * 4                # LSE out
            + (B * 4 if kv_lens is not None else 0))


def score_matrix_bytes(B, H, N, elem_bytes=4) -> int:
    """Size of a materialised [B, H, N, N] score matrix."""
    return B * H * N * N * elem_bytes


def unfused_io_elements(N, d) -> int:
    """HBM elements moved by the unfused three-step chain for one head.

    Step 1 reads Q, K (2Nd) and writes S (N^2); step 2 reads S and writes P
    (2N^2); step 3 reads P and V (N^2 + Nd) and writes O (Nd): 4N^2 + 4Nd.
    """
    return 4 * N * N + 4 * N * d
