"""Full-size parity helpers: every (batch, head, row) of a workload against the oracle.

Rows of attention are independent, so the oracle's row function computes a
workload slab by slab (at most ``SLAB`` query rows of one head at a time,
which bounds the materialised score block) in a pool of threads (numpy's
matrix products and element-wise loops release the interpreter lock).  Every
element of the GPU output is compared; the statistics of the comparison are
returned and printed so that a test log carries the table of errors.
"""
from __future__ import annotations

import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import ref_bwd_group, ref_fwd_rows

SLAB = 4096
WORKERS = 8


def _pool_map(fn, items, workers=WORKERS, blas_threads=1):
    from threadpoolctl import threadpool_limits
    # few BLAS threads per worker: the pool supplies the parallelism
    with threadpool_limits(blas_threads), ThreadPoolExecutor(workers) as ex:
        return list(ex.map(fn, items))


class ErrStats:
    """Running max-abs and relative-RMS of one compared tensor."""

    def __init__(self):
        self.max_abs = 0.0
        self.sq_err = 0.0
        self.sq_ref = 0.0
        self.n = 0
        self.finite = True

    def add(self, got, ref):
        got = np.asarray(got, dtype=np.float64)
        if got.size == 0:
            return
        self.finite &= bool(np.all(np.isfinite(got)))
        err = np.abs(got - ref)
        self.max_abs = max(self.max_abs, float(err.max()))
        self.sq_err += float(np.sum(err * err))
        self.sq_ref += float(np.sum(ref * ref))
        self.n += got.size

    def merge(self, o):
        self.max_abs = max(self.max_abs, o.max_abs)
        self.sq_err += o.sq_err
        self.sq_ref += o.sq_ref
        self.n += o.n
        self.finite &= o.finite

    @property
    def rel_rms(self):
        return float(np.sqrt(self.sq_err / self.sq_ref)) if self.sq_ref > 0 else 0.0


def forward_all_rows(w, x, o_host, lse_host, *, mods=None, batches=None, workers=WORKERS):
    """Compare O [B,Hq,Nq,d] and LSE [B,Hq,Nq] (host arrays, "bhnd" order)
    with the oracle on every row of every head of the batches ``batches``
    (default all).  Returns (O stats, LSE max-abs over finite rows, largest
    |LSE|, count of rows whose -inf LSE disagrees, oracle seconds)."""
    mods = mods or {}
    bs = range(w.B) if batches is None else batches
    items = [(b, h, r0) for b in bs for h in range(w.Hq) for r0 in range(0, w.Nq, SLAB)]

    def one(it):
        b, h, r0 = it
        rows = np.arange(r0, min(r0 + SLAB, w.Nq))
        O_ref, L_ref = ref_fwd_rows(x["q"], x["k"], x["v"], b, h, rows, causal=w.causal,
                                    kv_lens=x["kv_lens"], **mods)
        st = ErrStats()
        st.add(o_host[b, h, r0:r0 + len(rows)], O_ref)
        L = np.asarray(lse_host[b, h, r0:r0 + len(rows)], dtype=np.float64)
        dead = np.isneginf(L_ref)
        mism = int(np.sum(np.isneginf(L) != dead))
        lerr = float(np.abs(L[~dead] - L_ref[~dead]).max()) if (~dead).any() else 0.0
        lmax = float(np.abs(L_ref[~dead]).max()) if (~dead).any() else 0.0
        return st, lerr, lmax, mism

    t0 = time.perf_counter()
    res = _pool_map(one, items, workers)
    secs = time.perf_counter() - t0
    st = ErrStats()
    lerr = lmax = 0.0
    mism = 0
    for s, le, lm, mi in res:
        st.merge(s)
        lerr = max(lerr, le)
        lmax = max(lmax, lm)
        mism += mi
    return st, lerr, lmax, mism, secs


def backward_all_groups(w, x, dq, dk, dv, *, mods=None, workers=4, blas_threads=4):
    """Compare dQ [B,Hq,Nq,d], dK/dV [B,Hkv,Nk,d] (host arrays) with the
    oracle's exact backward of every (batch, kv-head) group.  Returns
    ({"dq", "dk", "dv"}: stats, oracle seconds)."""
    G = w.Hq // w.Hkv
    items = [(b, g) for b in range(w.B) for g in range(w.Hkv)]

    def one(it):
        b, g = it
        dQ, dK, dV, _, _ = ref_bwd_group(x["q"], x["k"], x["v"], x["do"], b, g, causal=w.causal,
                                         kv_lens=x["kv_lens"], **(mods or {}))
        out = {n: ErrStats() for n in ("dq", "dk", "dv")}
        out["dq"].add(dq[b, g * G:(g + 1) * G], dQ)
        out["dk"].add(dk[b, g], dK)
        out["dv"].add(dv[b, g], dV)
        return out

    t0 = time.perf_counter()
    res = _pool_map(one, items, workers, blas_threads)
    secs = time.perf_counter() - t0
    tot = {n: ErrStats() for n in ("dq", "dk", "dv")}
    for r in res:
        for n in tot:
            tot[n].merge(r[n])
    return tot, secs
