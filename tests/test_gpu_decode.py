"""GPU parity of the split-KV decode (attn_decode) against the fp64 oracle.

Decode computes the same O and LSE as the forward for a few new queries
against a key/value cache; with ``causal`` the queries are the last Nq
positions, so query i sees keys j <= L - Nq + i.  The oracle is the plain
definition (ref_fwd) with that rule as an additive -inf mask (the rule itself
is pinned against ordinary causal attention in test_oracle_pins.py).
"""
import sys
import zlib

import numpy as np
import pytest

from exact_attention_25_amd import inputs
from oracle import ref_fwd
from tests.gpu_util import check_out, decode_causal_mask, from_layout, host, make_case, \
    to_device, to_layout

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _decode(w, x, *, layout="bhnd", causal=False):
    import torch
    from exact_attention_25_amd import binding as bd
    t = {n: to_device(to_layout(x[n + "_raw"], layout), w.dtype) for n in ("q", "k", "v")}
    lens = None if x["kv_lens"] is None else torch.from_numpy(x["kv_lens"]).cuda()
    o, lse = bd.attn_decode(t["q"], t["k"], t["v"], layout=layout, causal=causal, kv_lens=lens)
    torch.cuda.synchronize()
    return o, lse


def _reference(w, x, causal):
    mask = decode_causal_mask(w.B, w.Nq, w.Nk, x["kv_lens"]) if causal else None
    return ref_fwd(x["q"], x["k"], x["v"], mask=mask, kv_lens=x["kv_lens"])


CASES = [
    # id, B, Hq, Hkv, Nq, Nk, d, dtype, causal, lens, layout
    ("bf16_mqa_nq1", 2, 8, 1, 1, 1000, 128, "bf16", False, None, "bhnd"),
    ("fp16_gqa4_nq3_causal_lens", 3, 8, 2, 3, 777, 64, "fp16", True, (0, 777), "bhnd"),
    ("bf16_gqa16_nq2_bnhd_causal", 1, 32, 2, 2, 5000, 128, "bf16", True, (100, 5000), "bnhd"),
    ("fp16_nq16_d40_causal", 1, 2, 2, 16, 300, 40, "fp16", True, None, "bhnd"),
    ("bf16_one_key", 2, 4, 4, 1, 1, 128, "bf16", False, None, "bhnd"),
    ("bf16_80_rows_three_blocks", 1, 16, 1, 5, 2000, 128, "bf16", True, None, "bhnd"),
    ("fp16_lens_below_nq", 2, 4, 2, 8, 64, 64, "fp16", True, (3, 5), "bhnd"),
    ("bf16_d96_many_splits", 1, 4, 4, 1, 70000, 96, "bf16", False, None, "bnhd"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_small(gpu_lib, case):
    name, B, Hq, Hkv, Nq, Nk, d, dtype, causal, lens, layout = case
    _say(f"[decode] {name}")
    w, x = make_case(B, Hq, Hkv, Nq, Nk, d, dtype, seed=zlib.crc32(name.encode()) % 10000,
                     lens=lens)
    o, lse = _decode(w, x, layout=layout, causal=causal)
    O_ref, L_ref = _reference(w, x, causal)
    check_out(from_layout(host(o), layout), lse, O_ref, L_ref, dtype, name)


def test_decode_no_keys(gpu_lib):
    _say("[decode] no keys")
    w, x = make_case(2, 4, 2, 1, 0, 64, "bf16", seed=3)
    o, lse = _decode(w, x)
    assert np.all(host(o) == 0) and np.all(np.isneginf(host(lse)))


def test_decode_matches_forward_and_is_deterministic(gpu_lib):
    """Decode and the forward compute the same function; repeated calls are bitwise equal."""
    import torch
    from exact_attention_25_amd import binding as bd
    _say("[decode] vs forward")
    w, x = make_case(2, 8, 2, 4, 3000, 128, "bf16", seed=17, lens=(1000, 3000))
    o1, l1 = _decode(w, x)
    o2, l2 = _decode(w, x)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    t = {n: to_device(x[n + "_raw"], w.dtype) for n in ("q", "k", "v")}
    lens = torch.from_numpy(x["kv_lens"]).cuda()
    of, lf = bd.attn_fwd(t["q"], t["k"], t["v"], kv_lens=lens)
    torch.cuda.synchronize()
    assert float((o1.float() - of.float()).abs().max()) <= 2e-2
    assert float((l1 - lf).abs().max()) <= 1e-4


def test_workload_decode(gpu_lib):
    """The full decode workload (B8 Hq32 Hkv8, one new token, 32K cache with
    lengths U{16384..32768}): every row against the oracle."""
    w = inputs.WORKLOADS["decode_bf16_b8_hq32_kv8_q1_nk32768_d128"]
    _say(f"[decode] {w.name}")
    x = inputs.make_inputs(w)
    o, lse = _decode(w, x)
    O_ref, L_ref = ref_fwd(x["q"], x["k"], x["v"], kv_lens=x["kv_lens"])
    check_out(host(o), lse, O_ref, L_ref, w.dtype, w.name)
