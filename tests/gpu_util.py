"""Helpers for the GPU parity tests: upload seeded inputs, compare with the oracle."""
import numpy as np

from exact_attention_25_amd import inputs

TOL_O = {"fp32": 1e-5, "fp16": 2e-2, "bf16": 2e-2}      # max-abs on O
TOL_O_REL_RMS = {"fp32": 1e-6, "fp16": 5e-3, "bf16": 1e-2}


def torch_dtype(name):
    import torch
    return {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[name]


def to_device(raw: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(raw)).cuda()


def to_layout(x: np.ndarray, layout: str) -> np.ndarray:
    return x if layout == "bhnd" else np.ascontiguousarray(x.transpose(0, 2, 1, 3))


def from_layout(x: np.ndarray, layout: str) -> np.ndarray:
    return x if layout == "bhnd" else x.transpose(0, 2, 1, 3)


def host(t) -> np.ndarray:
    """Device tensor (any float dtype) or array -> float64 numpy array."""
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().float().cpu().numpy().astype(np.float64)


def make_case(B, Hq, Hkv, Nq, Nk, d, dtype, seed, std=1.0, lens=None, with_do=False,
              qk_std=None):
    w = inputs.Workload("case", B, Hq, Hkv, Nq, Nk, d, dtype, seed, std=std, lens=lens,
                        qk_std=qk_std)
    return w, inputs.make_inputs(w, with_do=with_do)


def check_out(o_gpu, lse_gpu, O_ref, L_ref, dtype, label=""):
    """Element-wise comparison of O and LSE with the oracle (max-abs bar of the tolerance table)."""
    O = host(o_gpu)
    L = host(lse_gpu)
    assert O.shape == O_ref.shape, (O.shape, O_ref.shape)
    assert np.all(np.isfinite(O)), f"{label}: non-finite output"
    err = np.abs(O - O_ref)
    max_abs = float(err.max()) if err.size else 0.0
    assert max_abs <= TOL_O[dtype], f"{label}: O max-abs {max_abs:.3e} > {TOL_O[dtype]}"
    rms_ref = float(np.sqrt(np.mean(O_ref ** 2))) if O_ref.size else 0.0
    if rms_ref > 0:
        rel = float(np.sqrt(np.mean(err ** 2))) / rms_ref
        assert rel <= TOL_O_REL_RMS[dtype], f"{label}: O rel-rms {rel:.3e}"
    dead = np.isneginf(L_ref)
    assert np.array_equal(np.isneginf(L), dead), f"{label}: -inf LSE rows differ"
    if (~dead).any():
        lerr = np.abs(L[~dead] - L_ref[~dead])
        ltol = (1e-5 if dtype == "fp32" else 1e-4) + 1e-6 * float(np.abs(L_ref[~dead]).max())
        assert float(lerr.max()) <= ltol, f"{label}: LSE max-abs {lerr.max():.3e}"
    return max_abs


def decode_causal_mask(B, Nq, Nk, kv_lens=None):
    """Additive [B,1,Nq,Nk] mask of decode's causal rule: the Nq queries are the
    last Nq positions of a sequence of L = kv_lens[b] (or Nk) keys, so query i
    sees keys j <= L - Nq + i.  Keys at or past L are left to kv_lens."""
    m = np.zeros((B, 1, Nq, Nk))
    j = np.arange(Nk)[None, :]
    for b in range(B):
        L = Nk if kv_lens is None else int(min(max(kv_lens[b], 0), Nk))
        lim = L - Nq + np.arange(Nq)[:, None]
        m[b, 0][j > lim] = -np.inf
    return m
