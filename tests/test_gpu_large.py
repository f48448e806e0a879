"""Tensors past 2^31 elements: every offset of the kernels is 64-bit.

B = 260, H = 128, N = 512, d = 128 in bf16 gives 2.18e9 elements per tensor
(4.4 GB), so the last heads start more than 2^31 elements (and 2^32 bytes)
into Q, K, V, O and the gradients.  The forward (non-causal and
causal, both on the pipelined kernel: 512 keys = 8 tiles), the split-KV
decode (K / V as the cache) and the causal backward run on the whole tensors; the heads at the start, the middle and the
very end are checked against the oracle (each head is its own problem:
Hq = Hkv), to the same bars as the other parity tests.

The inputs are N(0, 1) draws of a seeded torch generator on the device,
rounded to bf16 there; the checked heads are copied back, so the oracle sees
exactly the values the kernels read.  The sizes are the only reason for
drawing on the device (2^31 normal draws on the host take minutes).
"""
import sys

import numpy as np
import pytest

from tests.gpu_util import TOL_O, TOL_O_REL_RMS, host

pytestmark = pytest.mark.gpu

B, H, N, D = 260, 128, 512, 128
HEADS = [(0, 0), (B // 2, 7), (B - 1, H - 1)]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _draw(gen, shape):
    import torch
    x = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32)
    return x.to(torch.bfloat16)


def _head(t, b, h):
    return host(t[b:b + 1, h:h + 1].float()).astype(np.float64)


def _rel_rms(err, ref):
    return float(np.sqrt(np.mean(err ** 2)) / max(np.sqrt(np.mean(ref ** 2)), 1e-30))


@pytest.fixture(scope="module")
def big():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    assert B * H * N * D > 2 ** 31
    gen = torch.Generator(device="cuda")
    gen.manual_seed(12345)
    t = {n: _draw(gen, (B, H, N, D)) for n in ("q", "k", "v", "do")}
    yield t
    del t
    torch.cuda.empty_cache()


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
def test_forward_past_2_31_elements(gpu_lib, big, causal):
    import torch
    from exact_attention_25_amd import binding as bd
    from oracle import ref_fwd
    _say(f"[large] forward causal={causal}: B{B} H{H} N{N} d{D} bf16, "
         f"{B * H * N * D} elements per tensor")
    o, lse = bd.attn_fwd(big["q"], big["k"], big["v"], causal=causal)
    torch.cuda.synchronize()
    for b, h in HEADS:
        q, k, v = (_head(big[n], b, h) for n in ("q", "k", "v"))
        O, L = ref_fwd(q, k, v, causal=causal)
        got = _head(o, b, h)
        err = np.abs(got - O)
        lerr = float(np.abs(host(lse[b, h]).astype(np.float64) - L[0, 0]).max())
        _say(f"[large]   head ({b}, {h}): O max-abs {err.max():.3e} rel-rms "
             f"{_rel_rms(got - O, O):.3e}, LSE max-abs {lerr:.3e}")
        assert np.all(np.isfinite(got))
        assert err.max() <= TOL_O["bf16"]
        assert _rel_rms(got - O, O) <= TOL_O_REL_RMS["bf16"]
        assert lerr <= 1e-4 + 1e-6 * float(np.abs(L).max())
    del o, lse
    torch.cuda.empty_cache()


def test_decode_past_2_31_elements(gpu_lib, big):
    # the 4.4 GB K / V as a decode cache of 512 entries per (batch, head), two
    # new queries per head (the last two positions, causal): their rows equal
    # the last two rows of causal attention over the whole sequence
    import torch
    from exact_attention_25_amd import binding as bd
    from oracle import ref_fwd_rows
    _say(f"[large] decode: 2 queries against a B{B} H{H} {N}-entry d{D} bf16 cache")
    q2 = big["q"][:, :, N - 2:].contiguous()
    o, lse = bd.attn_decode(q2, big["k"], big["v"], causal=True)
    torch.cuda.synchronize()
    for b, h in HEADS:
        q, k, v = (_head(big[n], b, h) for n in ("q", "k", "v"))
        O, L = ref_fwd_rows(q, k, v, 0, 0, np.array([N - 2, N - 1]), causal=True)
        got = _head(o, b, h)[0, 0]
        err = np.abs(got - O)
        lerr = float(np.abs(host(lse[b, h]).astype(np.float64) - L).max())
        _say(f"[large]   head ({b}, {h}): O max-abs {err.max():.3e}, LSE max-abs {lerr:.3e}")
        assert np.all(np.isfinite(got))
        assert err.max() <= TOL_O["bf16"]
        assert lerr <= 1e-4 + 1e-6 * float(np.abs(L).max())
    del o, lse, q2
    torch.cuda.empty_cache()


def test_backward_past_2_31_elements(gpu_lib, big):
    import torch
    from exact_attention_25_amd import binding as bd
    from oracle import ref_bwd
    _say(f"[large] causal backward: B{B} H{H} N{N} d{D} bf16, fp32 gradients")
    o, lse = bd.attn_fwd(big["q"], big["k"], big["v"], causal=True)
    dq, dk, dv = bd.attn_bwd(big["q"], big["k"], big["v"], o, lse, big["do"], causal=True)
    torch.cuda.synchronize()
    for b, h in HEADS:
        q, k, v, do = (_head(big[n], b, h) for n in ("q", "k", "v", "do"))
        ref = dict(zip(("dq", "dk", "dv"), ref_bwd(q, k, v, do, causal=True)[:3]))
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            got = host(t[b:b + 1, h:h + 1]).astype(np.float64)
            r = ref[name]
            err = np.abs(got - r)
            _say(f"[large]   head ({b}, {h}) {name}: max-abs {err.max():.3e} "
                 f"rel-rms {_rel_rms(got - r, r):.3e}")
            assert np.all(np.isfinite(got))
            assert err.max() <= 2e-2
            assert _rel_rms(got - r, r) <= 1e-2
    del o, lse, dq, dk, dv
    torch.cuda.empty_cache()
