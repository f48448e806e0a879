"""Thin ctypes binding over the C ABI of ``libattn.so`` (``include/attn.h``).

Argument marshalling only: the functions here check tensor shapes, allocate
outputs with torch (the library itself never allocates), pass raw device
pointers and the current HIP stream, and turn a non-OK status into an
exception.  Every step of the computation runs in the library's kernels;
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EALIGN, ATTN_EWORKSPACE, ATTN_EHIP, \
    ATTN_ESCRATCH = range(7)
ATTN_DECODE_SCRATCH_BYTES = 16 << 20   # include/attn.h
ATTN_FP32, ATTN_FP16, ATTN_BF16 = 0, 1, 2
ATTN_BHND, ATTN_BNHD = 0, 1

EXPORTS = ("attn_validate", "attn_fwd", "attn_bwd_workspace_bytes", "attn_bwd",
           "attn_decode_workspace_bytes", "attn_decode", "attn_decode_static",
           "attn_quantize_fp8", "attn_fwd_fp8", "attn_status_string")


class AttnParams(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Nq", ctypes.c_int32), ("Nk", ctypes.c_int32), ("d", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("layout", ctypes.c_int32),
        ("scale", ctypes.c_float), ("causal", ctypes.c_int32),
        ("mask", ctypes.c_void_p),
        ("mask_sb", ctypes.c_int64), ("mask_sh", ctypes.c_int64), ("mask_sq", ctypes.c_int64),
        ("kv_lens", ctypes.c_void_p),
        ("window", ctypes.c_int32), ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
        ("grid_cols", ctypes.c_int32), ("nbr_rows", ctypes.c_int32), ("nbr_cols", ctypes.c_int32),
        ("softcap", ctypes.c_float),
    ]


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {attn_status_string(status)} (status {status})")
        self.status = status


_lib = None


def load():
    """Load the library once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(AttnParams)
    vp = ctypes.c_void_p
    lib.attn_validate.argtypes = [P, ctypes.c_int]
    lib.attn_validate.restype = ctypes.c_int
    lib.attn_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_bwd_workspace_bytes.argtypes = [P]
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp,
                             ctypes.c_size_t, vp]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_decode_workspace_bytes.argtypes = [P]
    lib.attn_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_decode.argtypes = [P, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.attn_decode.restype = ctypes.c_int
    lib.attn_decode_static.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.attn_decode_static.restype = ctypes.c_int
    lib.attn_quantize_fp8.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.attn_quantize_fp8.restype = ctypes.c_int
    lib.attn_fwd_fp8.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.attn_fwd_fp8.restype = ctypes.c_int
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def attn_status_string(status: int) -> str:
    return load().attn_status_string(int(status)).decode()


def make_params(B, Hq, Hkv, Nq, Nk, d, dtype=ATTN_BF16, layout=ATTN_BHND, scale=None,
                causal=False, mask_ptr=None, mask_strides=(0, 0, 0), kv_lens_ptr=None,
                window_size=(-1, -1), grid=None, softcap=0.0) -> AttnParams:
    """attn_params for the C calls.  window_size = (left, right) as in
    flash_attn_func (-1 = open side); grid = (cols, nbr_rows, nbr_cols) or
    None; softcap 0 = off."""
    p = AttnParams()
    p.B, p.Hq, p.Hkv, p.Nq, p.Nk, p.d = B, Hq, Hkv, Nq, Nk, d
    p.dtype, p.layout = dtype, layout
    p.scale = 0.0 if scale is None else float(scale)
    p.causal = 1 if causal else 0
    p.mask = mask_ptr
    p.mask_sb, p.mask_sh, p.mask_sq = (int(x) for x in mask_strides)
    p.kv_lens = kv_lens_ptr
    wl, wr = (int(x) for x in window_size)
    p.window = 1 if (wl >= 0 or wr >= 0) else 0
    p.window_left, p.window_right = wl, wr
    if grid is not None:
        p.grid_cols, p.nbr_rows, p.nbr_cols = (int(x) for x in grid)
    p.softcap = float(softcap or 0.0)
    return p


def attn_validate(params: AttnParams, for_backward: bool = False) -> int:
    return load().attn_validate(ctypes.byref(params), 1 if for_backward else 0)


def attn_bwd_workspace_bytes(params: AttnParams) -> int:
    return int(load().attn_bwd_workspace_bytes(ctypes.byref(params)))


def attn_decode_workspace_bytes(params: AttnParams) -> int:
    return int(load().attn_decode_workspace_bytes(ctypes.byref(params)))


# ----------------------------------------------------------------- torch side
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    return {torch.float32: ATTN_FP32, torch.float16: ATTN_FP16, torch.bfloat16: ATTN_BF16}[t]


def _layout_code(layout: str) -> int:
    if layout not in ("bhnd", "bnhd"):
        raise ValueError("layout must be 'bhnd' or 'bnhd'")
    return ATTN_BHND if layout == "bhnd" else ATTN_BNHD


def _dims(q, k, v, layout):
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q, k, v must be 4-D and k, v must have the same shape")
    if layout == "bhnd":
        B, Hq, Nq, d = q.shape
        Bk, Hkv, Nk, dk = k.shape
    else:
        B, Nq, Hq, d = q.shape
        Bk, Nk, Hkv, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)}")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError("q, k, v must be contiguous device tensors of one dtype")
    return B, Hq, Hkv, Nq, Nk, d


def _stream_ptr(device):
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def attn_fwd(q, k, v, *, layout="bhnd", causal=False, scale=None, attn_mask=None,
             kv_lens=None, window_size=(-1, -1), grid=None, softcap=0.0, out=None, lse=None):
    """Forward attention.  Returns (o, lse).

    q: [B,Hq,Nq,d] ("bhnd") or [B,Nq,Hq,d] ("bnhd"); k, v likewise with Hkv
    heads.  attn_mask: optional float32 tensor broadcastable to [B,Hq,Nq,Nk]
    (additive, logit units).  kv_lens: optional int32 [B] device tensor.
    window_size: (left, right) sliding window, -1 = open side.  grid:
    (cols, nbr_rows, nbr_cols) 2-D neighbourhood.  softcap: tanh soft cap of
    the scaled logits (0 = off).
    """
    torch = _torch()
    lib = load()
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v, layout)
    attn_mask, mask_ptr, mstr = _mask_arg(attn_mask, B, Hq, Nq, Nk)
    lens_ptr = None
    if kv_lens is not None:
        if kv_lens.dtype != torch.int32 or not kv_lens.is_cuda or kv_lens.numel() != B:
            raise ValueError("kv_lens must be an int32 device tensor with B entries")
        kv_lens = kv_lens.contiguous()
        lens_ptr = kv_lens.data_ptr()
    p = make_params(B, Hq, Hkv, Nq, Nk, d, _dtype_code(q.dtype), _layout_code(layout), scale,
                    causal, mask_ptr, mstr, lens_ptr, window_size, grid, softcap)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    st = lib.attn_fwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                      lse.data_ptr(), _stream_ptr(q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd")
    return out, lse


def _mask_arg(attn_mask, B, Hq, Nq, Nk):
    """(tensor, pointer, strides) for an additive float32 mask broadcastable to
    [B,Hq,Nq,Nk], or (None, None, (0, 0, 0))."""
    torch = _torch()
    if attn_mask is None:
        return None, None, (0, 0, 0)
    if attn_mask.dtype != torch.float32 or not attn_mask.is_cuda:
        raise ValueError("attn_mask must be a float32 device tensor")
    m = attn_mask.expand(B, Hq, Nq, Nk)
    if m.stride(3) != 1:
        m = m.contiguous()
    return m, m.data_ptr(), (m.stride(0), m.stride(1), m.stride(2))


def attn_bwd(q, k, v, o, lse, dout, *, layout="bhnd", causal=False, scale=None, attn_mask=None,
             kv_lens=None, window_size=(-1, -1), grid=None, softcap=0.0, grad_dtype="fp32",
             workspace=None):
    """Backward attention from the forward's (o, lse).  Returns (dq, dk, dv).

    attn_mask, window_size, grid, softcap: the same ones the forward took.
    """
    torch = _torch()
    lib = load()
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v, layout)
    if dout.shape != q.shape or o.shape != q.shape:
        raise ValueError("o and dout must have q's shape")
    attn_mask, mask_ptr, mstr = _mask_arg(attn_mask, B, Hq, Nq, Nk)
    lens_ptr = None
    if kv_lens is not None:
        if kv_lens.dtype != torch.int32 or not kv_lens.is_cuda or kv_lens.numel() != B:
            raise ValueError("kv_lens must be an int32 device tensor with B entries")
        kv_lens = kv_lens.contiguous()
        lens_ptr = kv_lens.data_ptr()
    p = make_params(B, Hq, Hkv, Nq, Nk, d, _dtype_code(q.dtype), _layout_code(layout), scale,
                    causal, mask_ptr, mstr, lens_ptr, window_size, grid, softcap)
    gcode = ATTN_FP32 if grad_dtype == "fp32" else _dtype_code(q.dtype)
    gdt = torch.float32 if gcode == ATTN_FP32 else q.dtype
    dq = torch.empty(q.shape, dtype=gdt, device=q.device)
    dk = torch.empty(k.shape, dtype=gdt, device=q.device)
    dv = torch.empty(v.shape, dtype=gdt, device=q.device)
    need = attn_bwd_workspace_bytes(p)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = lib.attn_bwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                      lse.data_ptr(), dout.contiguous().data_ptr(), dq.data_ptr(), dk.data_ptr(),
                      dv.data_ptr(), gcode, workspace.data_ptr(), workspace.numel(),
                      _stream_ptr(q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd")
    return dq, dk, dv


def attn_decode(q, k, v, *, layout="bhnd", causal=False, scale=None, kv_lens=None,
                window_size=(-1, -1), softcap=0.0, workspace=None, out=None, lse=None):
    """Split-KV decode: Nq new queries against the k/v cache.  Returns (o, lse).

    q: [B,Hq,Nq,d] ("bhnd") or [B,Nq,Hq,d] ("bnhd"); k, v: the cache with Hkv
    heads and Nk entries.  kv_lens: optional int32 [B] device tensor of valid
    cache entries.  Query i sits at position p = L - Nq + i: causal means
    keys j <= p, window_size = (left, right) keys p - left .. p + right.
    softcap: tanh soft cap of the scaled logits (0 = off).
    """
    torch = _torch()
    lib = load()
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v, layout)
    lens_ptr = None
    if kv_lens is not None:
        if kv_lens.dtype != torch.int32 or not kv_lens.is_cuda or kv_lens.numel() != B:
            raise ValueError("kv_lens must be an int32 device tensor with B entries")
        kv_lens = kv_lens.contiguous()
        lens_ptr = kv_lens.data_ptr()
    p = make_params(B, Hq, Hkv, Nq, Nk, d, _dtype_code(q.dtype), _layout_code(layout), scale,
                    causal, None, (0, 0, 0), lens_ptr, window_size, None, softcap)
    need = attn_decode_workspace_bytes(p)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    st = lib.attn_decode(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                         out.data_ptr(), lse.data_ptr(), workspace.data_ptr(), workspace.numel(),
                         _stream_ptr(q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode")
    return out, lse


def attn_decode_static(q, k, v, *, layout="bhnd", causal=False, scale=None, kv_lens=None,
                       window_size=(-1, -1), softcap=0.0, out=None, lse=None):
    """attn_decode with the library's fixed per-GPU scratch instead of a
    workspace (no device allocation by the library; out / lse are allocated
    here unless given).  Arguments and result as for attn_decode."""
    torch = _torch()
    lib = load()
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v, layout)
    kv_lens, lens_ptr = _lens_arg(kv_lens, B)
    p = make_params(B, Hq, Hkv, Nq, Nk, d, _dtype_code(q.dtype), _layout_code(layout), scale,
                    causal, None, (0, 0, 0), lens_ptr, window_size, None, softcap)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    st = lib.attn_decode_static(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                out.data_ptr(), lse.data_ptr(), _stream_ptr(q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_static")
    return out, lse


def _lens_arg(kv_lens, B):
    torch = _torch()
    if kv_lens is None:
        return None, None
    if kv_lens.dtype != torch.int32 or not kv_lens.is_cuda or kv_lens.numel() != B:
        raise ValueError("kv_lens must be an int32 device tensor with B entries")
    kv_lens = kv_lens.contiguous()
    return kv_lens, kv_lens.data_ptr()


def attn_quantize_fp8(q, k, v, *, layout="bhnd"):
    """FP8 (E4M3FN) block quantisation of q, k, v (64-row blocks, one fp32
    scale per block).  Returns (q8, k8, vt8, q_scale, k_scale, v_scale):
    q8 / k8 uint8 codes in q's / k's shape and layout, vt8 uint8
    [B, Hkv, d, Nk rounded up to 64] (v transposed), scales float32
    [B, H, ceil(N / 64)]."""
    torch = _torch()
    lib = load()
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v, layout)
    p = make_params(B, Hq, Hkv, Nq, Nk, d, _dtype_code(q.dtype), _layout_code(layout))
    dev = q.device
    q8 = torch.empty(q.shape, dtype=torch.uint8, device=dev)
    k8 = torch.empty(k.shape, dtype=torch.uint8, device=dev)
    vt8 = torch.empty((B, Hkv, d, (Nk + 63) // 64 * 64), dtype=torch.uint8, device=dev)
    qs = torch.empty((B, Hq, (Nq + 63) // 64), dtype=torch.float32, device=dev)
    ks = torch.empty((B, Hkv, (Nk + 63) // 64), dtype=torch.float32, device=dev)
    vs = torch.empty((B, Hkv, (Nk + 63) // 64), dtype=torch.float32, device=dev)
    st = lib.attn_quantize_fp8(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                               q8.data_ptr(), k8.data_ptr(), vt8.data_ptr(), qs.data_ptr(),
                               ks.data_ptr(), vs.data_ptr(), _stream_ptr(dev))
    if st != ATTN_OK:
        raise AttnError(st, "attn_quantize_fp8")
    return q8, k8, vt8, qs, ks, vs


def attn_fwd_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, *, layout="bhnd", causal=False,
                 scale=None, kv_lens=None, out_dtype=None, out=None, lse=None):
    """FP8 forward on attn_quantize_fp8's outputs.  Returns (o, lse); o is
    bf16 (default) or fp16 in q's shape and layout."""
    torch = _torch()
    lib = load()
    if q8.dim() != 4 or k8.dim() != 4 or q8.dtype != torch.uint8 or k8.dtype != torch.uint8:
        raise ValueError("q8, k8 must be 4-D uint8 tensors")
    if layout == "bhnd":
        B, Hq, Nq, d = q8.shape
        _, Hkv, Nk, _ = k8.shape
    else:
        B, Nq, Hq, d = q8.shape
        _, Nk, Hkv, _ = k8.shape
    if tuple(vt8.shape) != (B, Hkv, d, (Nk + 63) // 64 * 64):
        raise ValueError("vt8 must be [B, Hkv, d, Nk rounded up to 64]")
    for t in (q8, k8, vt8, q_scale, k_scale, v_scale):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("fp8 inputs must be contiguous device tensors")
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    kv_lens, lens_ptr = _lens_arg(kv_lens, B)
    p = make_params(B, Hq, Hkv, Nq, Nk, d, _dtype_code(out_dtype), _layout_code(layout), scale,
                    causal, None, (0, 0, 0), lens_ptr)
    if out is None:
        out = torch.empty(q8.shape, dtype=out_dtype, device=q8.device)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q8.device)
    st = lib.attn_fwd_fp8(ctypes.byref(p), q8.data_ptr(), k8.data_ptr(), vt8.data_ptr(),
                          q_scale.data_ptr(), k_scale.data_ptr(), v_scale.data_ptr(),
                          out.data_ptr(), lse.data_ptr(), _stream_ptr(q8.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_fp8")
    return out, lse
