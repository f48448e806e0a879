"""GPU forward parity: the HIP path through the C ABI against the fp64 oracle.

Small cases span several tiles with ragged tails in both sequence axes and
cover every feature (dtypes, head dims incl. padded ones, layouts, causal,
key padding, additive masks, GQA, empty and fully masked rows).  The
full-size workloads are checked on every row of every head (the oracle
computes rows independently, in slabs, on a pool of threads).
"""
import sys
import zlib

import numpy as np
import pytest

from exact_attention_25_amd import inputs
from oracle import ref_fwd
from tests.gpu_util import (TOL_O, TOL_O_REL_RMS, check_out, from_layout, host, make_case,
                            to_device, to_layout)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(w, x, *, layout="bhnd", causal=False, scale=None, mask=None):
    import torch
    from exact_attention_25_amd import binding as bd
    q = to_device(to_layout(x["q_raw"], layout), w.dtype)
    k = to_device(to_layout(x["k_raw"], layout), w.dtype)
    v = to_device(to_layout(x["v_raw"], layout), w.dtype)
    lens = None if x["kv_lens"] is None else torch.from_numpy(x["kv_lens"]).cuda()
    m = None if mask is None else torch.from_numpy(mask.astype(np.float32)).cuda()
    o, lse = bd.attn_fwd(q, k, v, layout=layout, causal=causal, scale=scale, attn_mask=m,
                         kv_lens=lens)
    torch.cuda.synchronize()
    return o, lse


SMALL = [
    # id, B, Hq, Hkv, Nq, Nk, d, dtype, causal, lens, mask, layout, scale, std
    ("bf16_d128_tiles", 1, 2, 2, 256, 256, 128, "bf16", False, None, None, "bhnd", None, 1.0),
    ("bf16_d128_ragged", 2, 2, 1, 300, 333, 128, "bf16", False, None, None, "bhnd", None, 1.0),
    ("fp16_d64_vit_tail", 2, 3, 3, 196, 196, 64, "fp16", False, None, None, "bhnd", None, 0.5),
    ("fp16_d40_cross_lens", 2, 2, 2, 257, 77, 40, "fp16", False, (20, 77), None, "bhnd", None, 1.0),
    ("bf16_d128_causal_gqa_lens", 2, 8, 2, 320, 320, 128, "bf16", True, (100, 320), None, "bhnd", None, 1.0),
    ("bf16_d128_bnhd_gqa", 2, 4, 2, 200, 190, 128, "bf16", False, None, None, "bnhd", None, 1.0),
    ("bf16_d64_mask_bcast", 1, 2, 2, 130, 150, 64, "bf16", False, None, "full11", "bhnd", None, 1.0),
    ("fp16_d128_mask_keys_scale", 2, 2, 2, 70, 140, 128, "fp16", False, None, "keys", "bhnd", 0.3, 1.0),
    ("fp32_d64_tiny", 1, 2, 2, 128, 128, 64, "fp32", False, None, None, "bhnd", None, 1.0),
    ("fp32_d128_causal_mask_lens", 2, 2, 1, 150, 150, 128, "fp32", True, (40, 150), "full11", "bhnd", None, 1.0),
    ("fp32_d40_bnhd_ragged", 1, 2, 2, 33, 70, 40, "fp32", False, None, None, "bnhd", None, 1.0),
    ("bf16_d8_min", 1, 1, 1, 5, 9, 8, "bf16", False, None, None, "bhnd", None, 1.0),
    ("bf16_single", 1, 1, 1, 1, 1, 128, "bf16", False, None, None, "bhnd", None, 1.0),
    ("bf16_d96_pad", 1, 2, 2, 100, 180, 96, "bf16", False, None, None, "bhnd", None, 1.0),
    ("fp16_causal_bnhd", 1, 4, 4, 129, 129, 64, "fp16", True, None, None, "bnhd", None, 1.0),
    ("bf16_large_logits", 1, 2, 2, 200, 500, 128, "bf16", False, None, None, "bhnd", 2.0, 1.0),
    ("fp16_dead_rows_mask", 1, 1, 1, 64, 64, 64, "fp16", False, None, "dead_rows", "bhnd", None, 1.0),
    ("bf16_lens_zero", 3, 2, 2, 70, 90, 64, "bf16", False, (0, 2), None, "bhnd", None, 1.0),
    # >= 8 key tiles without masks: the software-pipelined kernel
    ("bf16_d128_pipe_ragged_gqa", 1, 2, 1, 300, 700, 128, "bf16", False, None, None, "bhnd", None, 1.0),
    ("fp16_d64_pipe_lens_mid_tile", 2, 2, 2, 129, 600, 64, "fp16", False, (530, 600), None, "bhnd", None, 1.0),
    ("bf16_d40_pipe_bnhd_tail", 1, 3, 3, 70, 515, 40, "bf16", False, None, None, "bnhd", None, 1.0),
    ("fp16_d128_pipe_large_logits", 1, 2, 2, 64, 1030, 128, "fp16", False, None, None, "bhnd", 2.0, 1.0),
    ("bf16_d128_pipe_one_tile", 2, 1, 1, 40, 520, 128, "bf16", False, (3, 64), None, "bhnd", None, 1.0),
    # d <= 64 beyond 1024 keys: the pipelined kernel with 128-key tiles
    ("fp16_d64_pipe128_causal_lens", 2, 2, 1, 1300, 1300, 64, "fp16", True, (700, 1300), None, "bhnd", None, 1.0),
    ("bf16_d40_pipe128_bnhd_ragged", 1, 3, 3, 150, 1500, 40, "bf16", False, None, None, "bnhd", None, 1.0),
    ("fp16_d64_pipe128_large_logits", 1, 2, 2, 64, 1100, 64, "fp16", False, (1030, 1100), None, "bhnd", None, 3.0),
    # d <= 48: the QK^T contraction of the pipelined kernel stops at column 48
    ("fp16_d48_pipe128_lens", 1, 2, 2, 300, 1200, 48, "fp16", False, (1100, 1200), None, "bhnd", None, 1.0),
    ("bf16_d32_pipe_gqa", 1, 4, 2, 130, 600, 32, "bf16", False, None, None, "bhnd", None, 1.0),
]


def _mask(kind, B, Hq, Nq, Nk, rng):
    if kind is None:
        return None
    if kind == "full11":
        m = rng.standard_normal((1, 1, Nq, Nk)) * 2
        m[0, 0, :, ::7] = -np.inf
        return m.astype(np.float32).astype(np.float64)
    if kind == "keys":
        m = np.zeros((B, 1, 1, Nk))
        m[..., Nk // 2:] = -1e9
        m[..., : Nk // 5] += rng.standard_normal(Nk // 5)
        return m.astype(np.float32).astype(np.float64)
    if kind == "dead_rows":
        m = np.zeros((1, 1, Nq, Nk))
        m[0, 0, 3] = -np.inf
        m[0, 0, 40] = -np.inf
        return m
    raise ValueError(kind)


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_forward_small(gpu_lib, case):
    name, B, Hq, Hkv, Nq, Nk, d, dtype, causal, lens, mkind, layout, scale, std = case
    _say(f"[fwd-small] {name}")
    w, x = make_case(B, Hq, Hkv, Nq, Nk, d, dtype, seed=zlib.crc32(name.encode()) % 10000,
                     std=std, lens=lens)
    mask = _mask(mkind, B, Hq, Nq, Nk, np.random.default_rng(5))
    o, lse = _run(w, x, layout=layout, causal=causal, scale=scale, mask=mask)
    O_ref, L_ref = ref_fwd(x["q"], x["k"], x["v"], scale=scale, causal=causal, mask=mask,
                           kv_lens=x["kv_lens"])
    check_out(from_layout(host(o), layout), lse, O_ref, L_ref, dtype, name)


# At d <= 64 the forward streams key tiles through three LDS stages whose
# roles rotate with the tile index (loads run two tiles ahead): every key-tile
# count from 1 to 7, so each count modulo 3 ends the loop at each stage, with
# causal rows (per-wave tile counts), key lengths, an additive mask, GQA,
# BNHD and ragged last tiles.  224 < Nk < 512 keeps these on that kernel
# (shorter key ranges without a mask take the resident kernel below); the
# one- to three-tile counts come from key lengths (drawn in 1..64, 65..128
# and 129..192).
STAGES = [
    # id, B, Hq, Hkv, Nq, Nk, d, dtype, causal, lens, mask, layout
    ("tiles1_d64", 2, 2, 1, 40, 300, 64, "bf16", False, (20, 64), None, "bhnd"),
    ("tiles2_d64_fp16", 1, 2, 2, 70, 260, 64, "fp16", False, (65, 128), None, "bhnd"),
    ("tiles3_d40", 2, 2, 2, 100, 300, 40, "bf16", False, (129, 192), None, "bhnd"),
    ("tiles4_causal_d64", 1, 2, 1, 256, 256, 64, "bf16", True, None, None, "bhnd"),
    ("tiles4_5_lens_d64", 2, 2, 2, 130, 320, 64, "fp16", False, (200, 320), None, "bhnd"),
    ("tiles5_mask_d64", 1, 2, 2, 90, 300, 64, "bf16", False, None, "full11", "bhnd"),
    ("tiles6_d32", 2, 2, 1, 64, 383, 32, "bf16", False, None, None, "bhnd"),
    ("tiles7_causal_gqa_d64", 1, 4, 2, 448, 448, 64, "bf16", True, None, None, "bhnd"),
    ("tiles7_d48_bnhd", 1, 3, 3, 100, 447, 48, "fp16", False, None, None, "bnhd"),
]


@pytest.mark.parametrize("case", STAGES, ids=[c[0] for c in STAGES])
def test_forward_stage_rotation(gpu_lib, case):
    name, B, Hq, Hkv, Nq, Nk, d, dtype, causal, lens, mkind, layout = case
    _say(f"[fwd-stages] {name}")
    w, x = make_case(B, Hq, Hkv, Nq, Nk, d, dtype, seed=zlib.crc32(name.encode()) % 10000,
                     lens=lens)
    mask = _mask(mkind, B, Hq, Nq, Nk, np.random.default_rng(11))
    o, lse = _run(w, x, layout=layout, causal=causal, mask=mask)
    O_ref, L_ref = ref_fwd(x["q"], x["k"], x["v"], causal=causal, mask=mask,
                           kv_lens=x["kv_lens"])
    check_out(from_layout(host(o), layout), lse, O_ref, L_ref, dtype, name)


# Short key ranges (Nk <= 224) at d <= 64 without a mask: every key tile of
# the head resident in LDS (32-key tiles; 16-key chunks past the key range
# skipped).  Key counts at the chunk and tile edges (16, 17, 32, 33, 48, 65,
# 224), key lengths that end mid-chunk, causal (with key lengths), GQA, BNHD,
# d = 8/32/40/64, query blocks past the first work-group, and 225 keys (the
# first count the staged kernel takes) beside 224.
RESIDENT = [
    # id, B, Hq, Hkv, Nq, Nk, d, dtype, causal, lens, layout
    ("res_k16_d64", 1, 2, 2, 50, 16, 64, "bf16", False, None, "bhnd"),
    ("res_k17_fp16", 2, 2, 1, 33, 17, 64, "fp16", False, None, "bhnd"),
    ("res_k32_d32", 1, 3, 3, 64, 32, 32, "bf16", False, None, "bnhd"),
    ("res_k33_lens", 2, 2, 2, 70, 33, 40, "fp16", False, (1, 33), "bhnd"),
    ("res_k48_causal", 1, 2, 1, 48, 48, 64, "bf16", True, None, "bhnd"),
    ("res_k65_causal", 1, 2, 2, 65, 65, 64, "fp16", True, None, "bhnd"),
    ("res_k130_causal_gqa_lens", 2, 4, 2, 130, 130, 64, "bf16", True, (75, 130), "bhnd"),
    ("res_k196_vit", 2, 3, 3, 196, 196, 64, "bf16", False, None, "bhnd"),
    ("res_k224_rows600", 1, 2, 1, 600, 224, 40, "fp16", False, (150, 209), "bnhd"),
    ("res_k224_d8", 1, 2, 2, 300, 224, 8, "bf16", False, None, "bhnd"),
    ("staged_k225", 1, 2, 2, 300, 225, 64, "bf16", False, None, "bhnd"),
]


@pytest.mark.parametrize("case", RESIDENT, ids=[c[0] for c in RESIDENT])
def test_forward_resident(gpu_lib, case):
    name, B, Hq, Hkv, Nq, Nk, d, dtype, causal, lens, layout = case
    _say(f"[fwd-resident] {name}")
    w, x = make_case(B, Hq, Hkv, Nq, Nk, d, dtype, seed=zlib.crc32(name.encode()) % 10000,
                     lens=lens)
    o, lse = _run(w, x, layout=layout, causal=causal)
    O_ref, L_ref = ref_fwd(x["q"], x["k"], x["v"], causal=causal, kv_lens=x["kv_lens"])
    check_out(from_layout(host(o), layout), lse, O_ref, L_ref, dtype, name)


# Causal calls whose work-groups see >= 8 key tiles (min(Nq, Nk) >= 512) take
# the software-pipelined kernel: diagonal tiles masked per row, the tile
# count capped at each block's last row, ragged last blocks, key lengths
# below and above the diagonal, GQA, both layouts, a padded head dimension
# (query i sees keys <= i; causal calls have Nq = Nk).
PIPE_CAUSAL = [
    # id, B, Hq, Hkv, Nq, Nk, d, dtype, lens, layout
    ("pipe_causal_d128", 1, 4, 4, 600, 600, 128, "bf16", None, "bhnd"),
    ("pipe_causal_gqa_lens_d128", 2, 8, 2, 700, 700, 128, "bf16", (100, 700), "bhnd"),
    ("pipe_causal_fp16_d64_bnhd", 1, 2, 1, 520, 520, 64, "fp16", None, "bnhd"),
    ("pipe_causal_lens_d96", 2, 2, 2, 900, 900, 96, "bf16", (530, 900), "bhnd"),
    ("pipe_causal_fp16_d128_bnhd", 1, 2, 1, 1000, 1000, 128, "fp16", None, "bnhd"),
    ("pipe_causal_d48_lens", 1, 2, 1, 1100, 1100, 48, "bf16", (600, 1100), "bhnd"),
]


@pytest.mark.parametrize("case", PIPE_CAUSAL, ids=[c[0] for c in PIPE_CAUSAL])
def test_forward_pipelined_causal(gpu_lib, case):
    name, B, Hq, Hkv, Nq, Nk, d, dtype, lens, layout = case
    _say(f"[fwd-pipe-causal] {name}")
    w, x = make_case(B, Hq, Hkv, Nq, Nk, d, dtype, seed=zlib.crc32(name.encode()) % 10000,
                     lens=lens)
    o, lse = _run(w, x, layout=layout, causal=True)
    O_ref, L_ref = ref_fwd(x["q"], x["k"], x["v"], causal=True, kv_lens=x["kv_lens"])
    check_out(from_layout(host(o), layout), lse, O_ref, L_ref, dtype, name)


def test_forward_empty_and_no_keys(gpu_lib):
    import torch
    from exact_attention_25_amd import binding as bd
    _say("[fwd] empty / Nk=0")
    q = torch.randn(2, 3, 0, 64, device="cuda", dtype=torch.bfloat16)
    k = torch.randn(2, 3, 5, 64, device="cuda", dtype=torch.bfloat16)
    o, lse = bd.attn_fwd(q, k, k)
    assert o.shape == q.shape and lse.shape == (2, 3, 0)
    q = torch.randn(2, 3, 7, 64, device="cuda", dtype=torch.bfloat16)
    k = torch.randn(2, 3, 0, 64, device="cuda", dtype=torch.bfloat16)
    o, lse = bd.attn_fwd(q, k, k)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("nk", [333, 600])
def test_forward_is_deterministic_and_layout_invariant(gpu_lib, nk):
    import torch
    _say(f"[fwd] determinism / layouts nk={nk}")
    w, x = make_case(2, 4, 2, 333, nk, 128, "bf16", seed=77)
    o1, l1 = _run(w, x)
    o2, l2 = _run(w, x)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o3, l3 = _run(w, x, layout="bnhd")
    assert torch.equal(o1, o3.transpose(1, 2)) and torch.equal(l1, l3)


def test_forward_causal_row0_is_v0(gpu_lib):
    import torch
    _say("[fwd] causal row 0")
    w, x = make_case(2, 4, 2, 130, 130, 128, "bf16", seed=8)
    o, _ = _run(w, x, causal=True)
    v = to_device(x["v_raw"], "bf16")
    assert torch.equal(o[:, :, 0], v[:, [0, 0, 1, 1], 0])


# ------------------------------------------------------- full-size workloads
# Every row of every head of each workload is compared with the oracle
# (tests/full_size.py), element by element, with the same bars as the small
# cases; the error statistics are printed for the design notes' table.
def _full_check(w, batches=None):
    from tests.full_size import forward_all_rows
    _say(f"[fwd-workload] {w.name}: generating inputs")
    x = inputs.make_inputs(w, with_do=False)
    _say(f"[fwd-workload] {w.name}: running GPU")
    o, lse = _run(w, x, causal=w.causal)
    oh = o.float().cpu().numpy()
    lh = lse.cpu().numpy()
    _say(f"[fwd-workload] {w.name}: oracle over every row"
         + ("" if batches is None else f" of batches {list(batches)}"))
    st, lerr, lmax, mism, secs = forward_all_rows(w, x, oh, lh, batches=batches)
    _say(f"[fwd-workload] {w.name}: O max-abs {st.max_abs:.3e} rel-rms {st.rel_rms:.3e}, "
         f"LSE max-abs {lerr:.3e}, rows {st.n // w.d}, oracle {secs:.1f} s")
    assert st.finite, f"{w.name}: non-finite output"
    assert st.n == len(batches or range(w.B)) * w.Hq * w.Nq * w.d
    assert st.max_abs <= TOL_O[w.dtype], f"{w.name}: O max-abs {st.max_abs:.3e}"
    assert st.rel_rms <= TOL_O_REL_RMS[w.dtype], f"{w.name}: O rel-rms {st.rel_rms:.3e}"
    assert mism == 0, f"{w.name}: {mism} rows disagree on a fully masked (-inf) LSE"
    ltol = (1e-5 if w.dtype == "fp32" else 1e-4) + 1e-6 * lmax
    assert lerr <= ltol, f"{w.name}: LSE max-abs {lerr:.3e}"
    return w, x, o, lse


def test_workload_tiny_fp32(gpu_lib):
    _full_check(inputs.WORKLOADS["tiny_fp32_b1_h2_n128_d64"])


def test_workload_vit_bf16(gpu_lib):
    _full_check(inputs.WORKLOADS["vit_bf16_b128_h16_n196_d64"])


def test_workload_unet_cross_fp16(gpu_lib):
    _full_check(inputs.WORKLOADS["unet_cross_fp16_b2_h8_q4096_k77_d40"])


def test_workload_unet_self_fp16(gpu_lib):
    _full_check(inputs.WORKLOADS["unet_self_fp16_b2_h8_n4096_d40"])


def test_workload_long_bf16(gpu_lib):
    _full_check(inputs.WORKLOADS["long_bf16_b8_h32_n4096_d128"])


@pytest.mark.parametrize("part", [0, 1])
def test_workload_causal_gqa_forward(gpu_lib, part):
    import torch
    w = inputs.WORKLOADS["causal_gqa_bf16_b4_h32_kv2_n8192_d128"]
    w, x, o, lse = _full_check(w, batches=range(2 * part, 2 * part + 2))
    v = to_device(x["v_raw"], w.dtype)
    G = w.Hq // w.Hkv
    assert torch.equal(o[:, :, 0], v[:, :, 0].repeat_interleave(G, dim=1))


# The pipelined kernel (8-wave work-groups, more than 16 key tiles) on every
# row of a mid-size call with ragged Nq / Nk tails, 8 q-heads per kv-head and
# key lengths that end mid-tile (4 * 64 * 8 = 2048 work-groups).
def test_forward_pipelined_ragged_gqa_lens(gpu_lib):
    _full_check(inputs.Workload("pipe_bf16_b4_h64_kv8_n2000_d128", 4, 64, 8, 2000, 2000, 128,
                                "bf16", 41, lens=(1100, 2000)))


# the long-context sweep (B * N = 32768); N = 16384 in two halves of the batch
SWEEP = [(1024, None), (2048, None), (8192, None), (16384, (0,)), (16384, (1,))]


@pytest.mark.parametrize("n,batches", SWEEP,
                         ids=[f"n{n}" + ("" if b is None else f"_b{b[0]}") for n, b in SWEEP])
def test_workload_long_sweep(gpu_lib, n, batches):
    _full_check(inputs.sweep_workload(n), batches=batches)
