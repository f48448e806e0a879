"""fp64 reference for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): the GPU library never
imports or calls this module.

This is the plain, unfused definition of attention written out with numpy in
float64.  The score matrix S and the probabilities P of every (batch, head)
are materialised in full, exactly as the "standard" implementation that the
pages replace does it.  Sources for each step:

* the unfused chain S = Q K^T, S / sqrt(d_k), S + attn_mask, softmax over the
  key axis, S V -- page "Step 3.7 Flash 的表现有点意外" (xxmr.cn/news/81028),
  §2.3, and the ``CoreAttention.forward`` original of page
  "如何在ChatGLM2-6B中集成Flash-Attention2？实测性能提升与显存优化"
  (jsqmd.com/news/348824), §3 step 2;
* the two-pass safe softmax (row max m, then l = sum exp(x - m), then
  exp(x - m) / l) -- page "FlashAttention技术解析：优化Transformer注意力计算效率"
  (jsqmd.com/news/722897), §6.2 item 3;
* the per-row statistics kept for the backward pass and the recompute of P
  there -- the same page, §3.3;
* causal masking (``causal=True`` for a decoder) and the [b, s, h, d] /
  [b, h, s, d] layouts -- the ChatGLM2-6B page, §3 step 3 and step 4.

Readings taken where the pages leave a step open (each is listed in the
design notes of the repository):

* scale: ``scale <= 0`` or NaN or None means 1/sqrt(d) with the real head
  dimension d;
* the additive mask is in logit units and is added after scaling;
* key padding (``kv_lens``) and causal masking exclude keys exactly (-inf);
  causal keeps the diagonal (key j visible to query i iff j <= i) and needs
  Nq == Nk;
* a fully masked row gives O = 0 and LSE = -inf;
* LSE is the natural-log log-sum-exp of the scaled, masked logits;
* grouped-query attention: q-head h reads kv-head h // (Hq / Hkv);
* dropout is absent (p = 0).

Local masks and the score modification (all optional, off by default):

* ``softcap``: the scaled logit s becomes cap * tanh(s / cap), before the
  additive mask -- the tanh soft cap of the FlexAttention score_mod example
  in the PyTorch attention-options article (atyun.com/61003), section
  "Score Mod示例：使用Tanh进行软上限" (cap 30 there);
* ``window=(left, right)``: key j is visible to the query at position p iff
  p - left <= j <= p + right, a negative bound leaving its side open -- the
  ``window_size`` argument of flash_attn_func on the ChatGLM2-6B page, §3
  step 3 (whose default (-1, -1) is no window);
* ``grid=(cols, nbr_rows, nbr_cols)``: positions are cells of a row-major
  grid with ``cols`` columns (p -> (p // cols, p % cols)), and key j is
  visible iff its row and column differ from the query's by less than
  nbr_rows and nbr_cols -- the neighbourhood mask_mod example of the same
  PyTorch article, section "Mask Mod示例：邻域屏蔽" (56 x 56 patches, both
  differences < 5);
* positions: query row i sits at position p = i; with ``bottom_right`` the
  Nq queries are the last Nq positions of the batch's L keys (L = kv_len or
  Nk), p = L - Nq + i, the rule of a decode step.  Causal attention then
  means j <= p, and does not need Nq == Nk.
"""
from __future__ import annotations

import math

import numpy as np

_LAYOUTS = ("bhnd", "bnhd")


def resolve_scale(scale, d: int) -> float:
    """Softmax scale: 1/sqrt(d_k) unless a positive scale is given.

    The default follows the S / sqrt(d_k) step of the unfused chain (Step 3.7
    page, §2.3) and ``softmax_scale=None`` meaning "computed inside" on the
    ChatGLM2-6B page, §3 step 3.
    """
    if scale is None:
        return 1.0 / math.sqrt(d)
    s = float(scale)
    if not (s > 0.0):  # also catches NaN
        return 1.0 / math.sqrt(d)
    return s


def _to_bhnd(x: np.ndarray, layout: str) -> np.ndarray:
    if layout not in _LAYOUTS:
        raise ValueError(f"layout must be one of {_LAYOUTS}, got {layout!r}")
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 4:
        raise ValueError("tensors are 4-D")
    return x if layout == "bhnd" else x.transpose(0, 2, 1, 3)


def _from_bhnd(x: np.ndarray, layout: str) -> np.ndarray:
    return x if layout == "bhnd" else x.transpose(0, 2, 1, 3)


def _group(hq: int, hkv: int) -> int:
    if hkv <= 0 or hq % hkv != 0:
        raise ValueError(f"Hq={hq} must be a multiple of Hkv={hkv}")
    return hq // hkv


def query_positions(nq, nk, *, kv_len=None, bottom_right=False, rows=None):
    """Sequence positions of the query rows ``rows`` (default all Nq rows).

    p = i, or with ``bottom_right`` p = L - Nq + i where L is the number of
    valid keys (kv_len clamped to [0, Nk], else Nk).
    """
    ridx = np.arange(nq) if rows is None else np.asarray(rows, dtype=np.int64)
    if not bottom_right:
        return ridx
    L = nk if kv_len is None else int(min(max(int(kv_len), 0), nk))
    return L - nq + ridx


def local_visible(pos, nk, *, window=None, grid=None):
    """[len(pos), Nk] boolean: which keys the sliding window and the 2-D
    neighbourhood leave visible to queries at positions ``pos``.

    window = (left, right): p - left <= j <= p + right; a negative bound is
    open.  grid = (cols, nbr_rows, nbr_cols): |p//cols - j//cols| < nbr_rows
    and |p%cols - j%cols| < nbr_cols.
    """
    pos = np.asarray(pos, dtype=np.int64)[:, None]
    j = np.arange(nk, dtype=np.int64)[None, :]
    vis = np.ones((pos.shape[0], nk), dtype=bool)
    if window is not None:
        left, right = (int(x) for x in window)
        if left >= 0:
            vis &= j >= pos - left
        if right >= 0:
            vis &= j <= pos + right
    if grid is not None:
        cols, nr, nc = (int(x) for x in grid)
        if cols <= 0 or nr <= 0 or nc <= 0:
            raise ValueError("grid needs cols, nbr_rows, nbr_cols > 0")
        if np.any(pos < 0):
            raise ValueError("grid positions must be >= 0")
        vis &= np.abs(pos // cols - j // cols) < nr
        vis &= np.abs(pos % cols - j % cols) < nc
    return vis


def softcap_logits(S, cap):
    """cap * tanh(S / cap): the tanh soft cap (PyTorch attention-options
    article, "Score Mod示例：使用Tanh进行软上限").  cap None or 0: S unchanged."""
    if not cap:
        return S
    return cap * np.tanh(S / cap)


def ref_scores(q_bh, k_bg, *, scale, mask_bh=None, kv_len=None, causal=False,
               rows=None, softcap=None, window=None, grid=None, bottom_right=False):
    """Scaled, masked logits S for one (batch, head): an [Nq, Nk] fp64 array.

    S = (Q K^T) * scale, soft-capped if ``softcap``, then + mask, then keys
    j >= kv_len, (causal) keys j > p and keys outside the window or the
    neighbourhood set to -inf, p being the query's position (p = i unless
    ``bottom_right``).  ``rows`` selects query rows (global indices), so a
    slab of S can be formed without the rest.
    """
    q_bh = np.asarray(q_bh, dtype=np.float64)
    k_bg = np.asarray(k_bg, dtype=np.float64)
    nq, nk = q_bh.shape[0], k_bg.shape[0]
    ridx = np.arange(nq) if rows is None else np.asarray(rows, dtype=np.int64)
    pos = query_positions(nq, nk, kv_len=kv_len, bottom_right=bottom_right, rows=ridx)
    S = softcap_logits((q_bh[ridx] @ k_bg.T) * scale, softcap)
    if mask_bh is not None:
        S = S + np.asarray(mask_bh, dtype=np.float64)[ridx]
    if kv_len is not None:
        L = int(min(max(int(kv_len), 0), nk))
        S[:, L:] = -np.inf
    if causal:
        if nq != nk and not bottom_right:
            raise ValueError("causal attention needs Nq == Nk")
        S[np.arange(nk)[None, :] > pos[:, None]] = -np.inf
    if window is not None or grid is not None:
        S[~local_visible(pos, nk, window=window, grid=grid)] = -np.inf
    return S


def _softmax_rows(S):
    """Two-pass safe softmax over the last axis (FlashAttention技术解析 §6.2).

    Returns (P, LSE).  A row whose max is -inf (every key masked) gets P = 0
    and LSE = -inf.
    """
    m = S.max(axis=-1, keepdims=True)
    dead = ~np.isfinite(m)  # -inf max: fully masked row
    m_safe = np.where(dead, 0.0, m)
    e = np.exp(S - m_safe)
    e[np.broadcast_to(dead, e.shape)] = 0.0
    l = e.sum(axis=-1, keepdims=True)
    P = e / np.where(dead, 1.0, l)
    with np.errstate(divide="ignore"):
        lse = np.where(dead, -np.inf, m_safe + np.log(np.where(dead, 1.0, l)))
    return P, lse[..., 0]


def _mask_for(mask, B, Hq, Nq, Nk):
    if mask is None:
        return None
    mask = np.asarray(mask)
    if mask.ndim != 4:
        raise ValueError("mask must be 4-D and broadcastable to [B,Hq,Nq,Nk]")
    return np.broadcast_to(mask, (B, Hq, Nq, Nk))


def _lens_for(kv_lens, B):
    if kv_lens is None:
        return None
    kv_lens = np.asarray(kv_lens).reshape(-1)
    if kv_lens.shape[0] != B:
        raise ValueError("kv_lens must have B entries")
    return kv_lens


def _shapes(q, k, v):
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if v.shape != k.shape or Bk != B or dk != d:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    return B, Hq, Hkv, Nq, Nk, d


_MODS = ("softcap", "window", "grid", "bottom_right")


def _mods(mods):
    """The local-mask / score-mod keywords (see the module docstring)."""
    bad = set(mods) - set(_MODS)
    if bad:
        raise TypeError(f"unknown keyword(s) {sorted(bad)}")
    return mods


def ref_probs(q, k, *, scale=None, causal=False, mask=None, kv_lens=None,
              layout="bhnd", **mods):
    """P = softmax(S) for every (b, h): [B, Hq, Nq, Nk] fp64 (small shapes)."""
    q = _to_bhnd(q, layout)
    k = _to_bhnd(k, layout)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = _group(Hq, Hkv)
    s = resolve_scale(scale, d)
    M = _mask_for(mask, B, Hq, Nq, Nk)
    L = _lens_for(kv_lens, B)
    P = np.empty((B, Hq, Nq, Nk))
    for b in range(B):
        for h in range(Hq):
            S = ref_scores(q[b, h], k[b, h // G], scale=s,
                           mask_bh=None if M is None else M[b, h],
                           kv_len=None if L is None else L[b], causal=causal,
                           **_mods(mods))
            P[b, h], _ = _softmax_rows(S)
    return P


def ref_fwd(q, k, v, *, scale=None, causal=False, mask=None, kv_lens=None,
            layout="bhnd", **mods):
    """Attention forward: returns (O, LSE) in fp64.

    q: [B,Hq,Nq,d] (layout "bhnd") or [B,Nq,Hq,d] ("bnhd"); k, v likewise
    with Hkv heads and Nk keys.  mask: optional additive array broadcastable
    to [B,Hq,Nq,Nk].  kv_lens: optional [B] valid key counts.  ``mods``:
    softcap, window, grid, bottom_right (module docstring).
    O has q's layout; LSE is [B,Hq,Nq].

    Per (b, h): S from :func:`ref_scores`, P by the two-pass softmax, O = P V,
    LSE = m + ln l (the unfused chain of the Step 3.7 page §2.3 with the safe
    softmax of FlashAttention技术解析 §6.2).
    """
    q = _to_bhnd(q, layout)
    k = _to_bhnd(k, layout)
    v = _to_bhnd(v, layout)
    B, Hq, Hkv, Nq, Nk, d = _shapes(q, k, v)
    G = _group(Hq, Hkv)
    s = resolve_scale(scale, d)
    M = _mask_for(mask, B, Hq, Nq, Nk)
    L = _lens_for(kv_lens, B)
    O = np.empty((B, Hq, Nq, d))
    LSE = np.empty((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            S = ref_scores(q[b, h], k[b, g], scale=s,
                           mask_bh=None if M is None else M[b, h],
                           kv_len=None if L is None else L[b], causal=causal,
                           **_mods(mods))
            P, lse = _softmax_rows(S)
            O[b, h] = P @ v[b, g]
            LSE[b, h] = lse
    return _from_bhnd(O, layout), LSE


def ref_fwd_rows(q, k, v, b, h, rows, *, scale=None, causal=False, mask=None,
                 kv_lens=None, layout="bhnd", **mods):
    """(O rows, LSE rows) of one head (b, h) for the query indices ``rows``.

    Rows of attention are independent, so a sample of rows of a large problem
    is computed exactly without forming the rest.
    """
    q = _to_bhnd(q, layout)
    k = _to_bhnd(k, layout)
    v = _to_bhnd(v, layout)
    B, Hq, Hkv, Nq, Nk, d = _shapes(q, k, v)
    G = _group(Hq, Hkv)
    s = resolve_scale(scale, d)
    M = _mask_for(mask, B, Hq, Nq, Nk)
    L = _lens_for(kv_lens, B)
    S = ref_scores(q[b, h], k[b, h // G], scale=s,
                   mask_bh=None if M is None else M[b, h],
                   kv_len=None if L is None else L[b], causal=causal, rows=rows,
                   **_mods(mods))
    P, lse = _softmax_rows(S)
    return P @ v[b, h // G], lse


def ref_bwd_group(q, k, v, do, b, g, *, scale=None, causal=False, mask=None,
                  kv_lens=None, layout="bhnd", **mods):
    """Exact backward for one batch b and one kv-head g (all its q-heads).

    Returns (dQ [G,Nq,d] for q-heads g*G..g*G+G-1, dK [Nk,d], dV [Nk,d],
    O [G,Nq,d], LSE [G,Nq]) in fp64, with G = Hq / Hkv.

    The gradient of O = softmax(S) V, S = s Q K^T + mask, given dO
    (FlashAttention技术解析 §3.3: only O(N) statistics are kept and P is
    formed again in the backward; here P is simply formed in full):
        D_i  = sum_c dO_ic O_ic
        dP   = dO V^T
        dS   = P * (dP - D)
        dQ   = s dS K,   dK += s dS^T Q,   dV += P^T dO
    summed over the q-heads that share kv-head g.  No gradient reaches the
    mask.  With a soft cap the logit is cap * tanh(z / cap) of z = s q.k, so
    dS is multiplied by its derivative 1 - tanh(z / cap)^2 before the
    products with K and Q (chain rule).
    """
    q = _to_bhnd(q, layout)
    k = _to_bhnd(k, layout)
    v = _to_bhnd(v, layout)
    do = _to_bhnd(do, layout)
    B, Hq, Hkv, Nq, Nk, d = _shapes(q, k, v)
    if do.shape != q.shape:
        raise ValueError("dO must have q's shape")
    G = _group(Hq, Hkv)
    s = resolve_scale(scale, d)
    M = _mask_for(mask, B, Hq, Nq, Nk)
    L = _lens_for(kv_lens, B)
    dQ = np.empty((G, Nq, d))
    O = np.empty((G, Nq, d))
    LSE = np.empty((G, Nq))
    dK = np.zeros((Nk, d))
    dV = np.zeros((Nk, d))
    Kg, Vg = k[b, g], v[b, g]
    for r in range(G):
        h = g * G + r
        S = ref_scores(q[b, h], Kg, scale=s,
                       mask_bh=None if M is None else M[b, h],
                       kv_len=None if L is None else L[b], causal=causal,
                           **_mods(mods))
        P, lse = _softmax_rows(S)
        Oh = P @ Vg
        dOh = do[b, h]
        D = np.sum(dOh * Oh, axis=1, keepdims=True)
        dP = dOh @ Vg.T
        dS = P * (dP - D)
        cap = mods.get("softcap")
        if cap:
            # d/dz [cap tanh(z / cap)] = 1 - tanh(z / cap)^2 at z = s q.k
            dS = dS * (1.0 - np.tanh((q[b, h] @ Kg.T) * s / cap) ** 2)
        dQ[r] = s * (dS @ Kg)
        dK += s * (dS.T @ q[b, h])
        dV += P.T @ dOh
        O[r] = Oh
        LSE[r] = lse
    return dQ, dK, dV, O, LSE


def ref_bwd(q, k, v, do, *, scale=None, causal=False, mask=None, kv_lens=None,
            layout="bhnd", **mods):
    """Exact backward for the whole problem: returns (dQ, dK, dV, O, LSE).

    dQ/dK/dV/O come back in the input layout; LSE is [B,Hq,Nq].
    """
    qb = _to_bhnd(q, layout)
    kb = _to_bhnd(k, layout)
    B, Hq, Nq, d = qb.shape
    Hkv, Nk = kb.shape[1], kb.shape[2]
    G = _group(Hq, Hkv)
    dQ = np.empty((B, Hq, Nq, d))
    O = np.empty((B, Hq, Nq, d))
    LSE = np.empty((B, Hq, Nq))
    dK = np.empty((B, Hkv, Nk, d))
    dV = np.empty((B, Hkv, Nk, d))
    for b in range(B):
        for g in range(Hkv):
            dq, dk, dv, o, lse = ref_bwd_group(
                q, k, v, do, b, g, scale=scale, causal=causal, mask=mask,
                kv_lens=kv_lens, layout=layout, **mods)
            dQ[b, g * G:(g + 1) * G] = dq
            O[b, g * G:(g + 1) * G] = o
            LSE[b, g * G:(g + 1) * G] = lse
            dK[b, g] = dk
            dV[b, g] = dv
    return (_from_bhnd(dQ, layout), _from_bhnd(dK, layout),
            _from_bhnd(dV, layout), _from_bhnd(O, layout), LSE)
