"""attn_decode_static (no allocation: the split partials go to the library's
fixed per-GPU scratch) against attn_decode (caller workspace) through the C
ABI: bit-identical O and LSE on two calls in a row, the second smaller than
the first (the scratch keeps the first call's contents)."""
import sys
import zlib

import pytest

from tests.gpu_util import make_case, to_device

pytestmark = pytest.mark.gpu

CALLS = [
    # id, B, Hq, Hkv, Nq, Nk, d, dtype, causal, lens, window, softcap
    ("gqa_cache_bf16", 8, 32, 8, 1, 32768, 128, "bf16", True, (16384, 32768), (-1, -1), 0.0),
    ("small_fp16_window", 2, 8, 2, 3, 2000, 64, "fp16", True, (500, 2000), (300, 0), 20.0),
]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_decode_static_equals_decode_on_two_calls(gpu_lib):
    import torch
    from exact_attention_25_amd import binding as bd
    for case in CALLS:
        name, B, Hq, Hkv, Nq, Nk, d, dtype, causal, lens, window, cap = case
        _say(f"[decode-static] {name}")
        w, x = make_case(B, Hq, Hkv, Nq, Nk, d, dtype, seed=zlib.crc32(name.encode()) % 10000,
                         lens=lens)
        q, k, v = (to_device(x[n + "_raw"], dtype) for n in ("q", "k", "v"))
        lens_d = torch.from_numpy(x["kv_lens"]).cuda()
        kw = dict(causal=causal, kv_lens=lens_d, window_size=window, softcap=cap)
        p = bd.make_params(B, Hq, Hkv, Nq, Nk, d, bd._dtype_code(q.dtype), causal=causal,
                           window_size=window, softcap=cap)
        assert bd.attn_decode_workspace_bytes(p) <= bd.ATTN_DECODE_SCRATCH_BYTES
        o1, l1 = bd.attn_decode(q, k, v, **kw)
        o2, l2 = bd.attn_decode_static(q, k, v, **kw)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(o1).all())
        assert torch.equal(o1, o2) and torch.equal(l1, l2), name
