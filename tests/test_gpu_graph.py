"""HIP graph capture of the C-ABI calls.

attn_fwd (pipelined, resident and staged forward kernels) and
attn_decode_static (which allocates nothing, for callers that capture their
launches) are captured once and the graph is replayed several times, with
eager work and synchronisations between the replays and the outputs cleared
before each; every replay must equal the eager call bit for bit.  The
library's launches put no memset or allocation into the stream.
"""
import sys
import zlib

import pytest

from tests.gpu_util import make_case, to_device

pytestmark = pytest.mark.gpu

FWD = [
    # id, B, Hq, Hkv, Nq, Nk, d, dtype, causal, lens
    ("pipelined_bf16_gqa", 1, 4, 2, 600, 600, 128, "bf16", False, None),
    ("pipelined_causal_fp16", 1, 2, 2, 700, 700, 64, "fp16", True, None),
    ("resident_bf16_lens", 2, 3, 3, 196, 196, 64, "bf16", False, (100, 196)),
    ("staged_fp16_d128", 2, 2, 1, 200, 300, 128, "fp16", False, None),
]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _replay_and_check(fn, outs, refs, replays=3):
    """Capture fn() (which writes outs), then replay with eager work between."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()   # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    junk = torch.randn(1 << 16, device="cuda")
    for i in range(replays):
        for o in outs:
            o.zero_()
        junk.mul_(1.0001).add_(0.5)   # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o, r), f"replay {i} differs from the eager call"


@pytest.mark.parametrize("case", FWD, ids=[c[0] for c in FWD])
def test_forward_graph_replays_match_eager(gpu_lib, case):
    import torch
    from exact_attention_25_amd import binding as bd
    name, B, Hq, Hkv, Nq, Nk, d, dtype, causal, lens = case
    _say(f"[graph-fwd] {name}")
    w, x = make_case(B, Hq, Hkv, Nq, Nk, d, dtype, seed=zlib.crc32(name.encode()) % 10000,
                     lens=lens)
    q, k, v = (to_device(x[n + "_raw"], dtype) for n in ("q", "k", "v"))
    lens_d = None if x["kv_lens"] is None else torch.from_numpy(x["kv_lens"]).cuda()
    o_ref, l_ref = bd.attn_fwd(q, k, v, causal=causal, kv_lens=lens_d)
    torch.cuda.synchronize()
    o = torch.empty_like(q)
    lse = torch.empty_like(l_ref)
    _replay_and_check(lambda: bd.attn_fwd(q, k, v, causal=causal, kv_lens=lens_d, out=o, lse=lse),
                      [o, lse], [o_ref, l_ref])


def test_decode_static_graph_replays_match_eager(gpu_lib):
    import torch
    from exact_attention_25_amd import binding as bd
    name = "decode_static_gqa_bf16"
    _say(f"[graph-decode] {name}")
    B, Hq, Hkv, Nq, Nk, d = 2, 16, 4, 2, 5000, 128
    w, x = make_case(B, Hq, Hkv, Nq, Nk, d, "bf16", seed=zlib.crc32(name.encode()) % 10000,
                     lens=(3000, 5000))
    q, k, v = (to_device(x[n + "_raw"], "bf16") for n in ("q", "k", "v"))
    lens_d = torch.from_numpy(x["kv_lens"]).cuda()
    o_ref, l_ref = bd.attn_decode(q, k, v, causal=True, kv_lens=lens_d)
    torch.cuda.synchronize()
    o = torch.empty_like(q)
    lse = torch.empty_like(l_ref)
    _replay_and_check(lambda: bd.attn_decode_static(q, k, v, causal=True, kv_lens=lens_d, out=o,
                                                    lse=lse),
                      [o, lse], [o_ref, l_ref])
