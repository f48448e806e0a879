"""Benchmark of the exact-attention forward on one MI355X.

A step is one forward call (attn_fwd through the C ABI) on the
B=8, H=32, N=4096, d=128 bf16 workload (non-causal, no mask), inputs already
resident in HBM.  The script prints ONE JSON line with the throughput in
TFLOP/s (4*B*H*N^2*d per call), the roofline position of the forward kernel
(launch duration from HIP events on the launch stream), and the fp64 CPU
oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--pass fwd|bwd] [--extras] [--no-cpu-baseline]
                    [--copy-calibration]

--pass bwd times attn_bwd instead (from the forward's O and LSE), e.g. on
--workload causal_gqa_bf16_b4_h32_kv2_n8192_d128; its CPU baseline is the
oracle's backward on one (batch, kv-head) group.

--extras also times the other workloads (the ViT, UNet self/cross, causal
GQA forward and backward, and the long-context sweep) and adds them to the
JSON line under "extras", with the unfused torch chain (Q K^T, scale,
softmax, P V) at the B8 H32 N4096 d128 shape timed beside the fused call as
context.

Workloads with a sliding window, a 2-D neighbourhood or a soft cap (the
FlexAttention cases, e.g. vit_nbr_bf16_b8_h12_n3136_d64) pass them to the
call; their FLOPs count 4*d per visible (query, key) pair and head.  --copy-calibration runs a plain device copy of a
known size (for scaling HBM byte counters under rocprofv3).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOPS & % of bf16 MFMA peak at B8 H32 N4096 d128"
DEFAULT_WORKLOAD = "long_bf16_b8_h32_n4096_d128"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_long_bf16_b8_h32_n4096_d128_traffic.txt")
# Workloads whose floor is HBM bandwidth (or launch latency) rather than MFMA
HBM_BOUND = ("vit_bf16_b128_h16_n196_d64", "unet_cross_fp16_b2_h8_q4096_k77_d40")
# The sources the measured forward kernel (fwd_pipe_kernel) and its launch are
# built from: its counters stay valid while these are unchanged.
KERNEL_SOURCES = [os.path.join(ROOT, "exact_attention_25_amd", "csrc", f)
                  for f in ("attn_fwd.hip", "attn_fwd_pipe_kernel.h", "device_common.h",
                            "attn_kernels.h", "local_mask.h")]


def is_local(w) -> bool:
    return bool(w.window or w.grid)


def local_kw(w) -> dict:
    """The window / grid / soft cap keywords of a workload's calls."""
    return {"window_size": w.window or (-1, -1), "grid": w.grid, "softcap": w.softcap}


def fwd_flops_of(w, kv_lens):
    from exact_attention_25_amd import accounting as acc
    if is_local(w):
        return 4.0 * w.d * w.Hq * acc.local_pairs(w.Nq, kv_lens, w.B, w.causal, w.window, w.grid)
    return acc.fwd_flops(w.B, w.Hq, w.Nq, w.Nk, w.d, w.causal)


def fwd_kernel_name(w) -> str:
    """The forward kernel instance attn_fwd dispatches to for workload w
    (mirrors the dispatch in attn_fwd.hip and attn_fwd_local.hip)."""
    D = 128 if w.d > 64 else 64
    if w.dtype == "fp32":
        return f"attn::fwd32_kernel<{D},...>"
    e = "BF16" if w.dtype == "bf16" else "FP16"
    if is_local(w) or w.softcap:
        return (f"attn::fwd_kernel<{e},{D},8,64,causal={str(w.causal and not is_local(w)).lower()},"
                f"mask=false,local={str(is_local(w)).lower()},softcap={str(bool(w.softcap)).lower()}>")
    if w.d <= 64 and w.Nk <= 224:
        return f"attn::fwd_resident_kernel<{e},causal={str(w.causal).lower()}>"
    span = min(w.Nq, w.Nk) if w.causal else w.Nk
    if span >= 8 * 64:
        nw = 4 if span <= 16 * 64 else 8
        bc = 128 if (D == 64 and nw == 8) else 64
        dk = ",DK=48" if (D == 64 and w.d <= 48) else ""
        return f"attn::fwd_pipe_kernel<{e},{D},{bc},causal={str(w.causal).lower()},NW={nw}{dk}>"
    return f"attn::fwd_kernel<{e},{D},8,64,causal={str(w.causal).lower()},mask=false>"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source (else None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    txt = open(TRAFFIC_FILE).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    m_val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_hash or not m_val or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_val.group(1))


def upload(raw, dtype, device):
    import numpy as np
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(raw)).to(device)


def time_calls(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def time_graph(fn, steps, warmup, outs):
    """Per-call time of `steps` calls captured in one HIP graph and replayed:
    the calls then run back to back on the GPU, without the host's per-call
    launch time between them (which exceeds the kernel time of the smallest
    workloads).  outs: the output tensors the calls write; every replay's
    outputs are checked against an eager run's, bit for bit."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps):
            fn()
    torch.cuda.synchronize()
    for _ in range(2):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        if not all(torch.equal(o, r) for o, r in zip(outs, ref)):
            raise RuntimeError("graph replay differs from the eager calls")
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del g
    return ms


def sample_sclk(fn, ms_per_call, n_samples=3, max_s=15.0):
    """Engine clock (MHz, mean over the XCDs) read with amd-smi while fn()
    runs back to back: n_samples readings from a second thread, the first
    half a second into the calls.  The calls go in batches of ~20 ms with a
    synchronisation after each, so the GPU stays loaded until the last
    reading and the queue never runs far ahead.  Returns the list of
    readings ([] if amd-smi is missing or prints no clock).  The clock moves
    within milliseconds under power management, so each reading is one
    sample of it."""
    import shutil
    import subprocess
    import threading
    import torch
    exe = "/opt/rocm/bin/amd-smi" if os.path.exists("/opt/rocm/bin/amd-smi") else shutil.which("amd-smi")
    if not exe:
        return []
    cmd = [exe]
    try:
        # amd-smi is a Python script: run it with this interpreter, so that no
        # launcher (`env` in its first line) has to replace itself
        real = os.path.realpath(exe)
        with open(real, "rb") as fh:
            if b"python" in fh.readline():
                cmd = [sys.executable, real]
    except OSError:
        pass
    got = []

    def probe():
        time.sleep(0.5)
        for _ in range(n_samples):
            try:
                r = subprocess.run(cmd + ["metric", "-c", "--json"], capture_output=True, text=True,
                                   timeout=20)
                d = json.loads(r.stdout)
                clocks = (d["gpu_data"] if isinstance(d, dict) else d)[0]["clock"]
                vals = [float(v["clk"]["value"]) for k, v in clocks.items()
                        if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
                if vals:
                    got.append(sum(vals) / len(vals))
            except Exception:
                return

    batch = max(1, int(20.0 / max(ms_per_call, 1e-3)))
    th = threading.Thread(target=probe, daemon=True)
    t0 = time.perf_counter()
    th.start()
    while th.is_alive() and time.perf_counter() - t0 < max_s:
        for _ in range(batch):
            fn()
        torch.cuda.synchronize()
    th.join(timeout=1.0)
    return got


def clock_fields(samples, value, peak) -> dict:
    """The engine clock under load (median of the readings, and the
    readings) and the %-of-peak at that clock (the published peaks assume
    2400 MHz)."""
    if not samples:
        return {"sclk_mhz_under_load": None}
    mhz = sorted(samples)[len(samples) // 2]
    return {"sclk_mhz_under_load": round(mhz),
            "sclk_mhz_samples": [round(v) for v in samples],
            "pct_of_peak_at_measured_clock": round(value / (peak * mhz / 2400.0) * 100, 2)}


def call_percentiles(fn, n, stream):
    """Per-call durations (ms) of n further calls, each bracketed by its own
    HIP events on the launch stream: p10, p50, p90."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for e0, e1 in evs:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    ts = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    q = lambda f: ts[min(len(ts) - 1, int(round(f * (len(ts) - 1))))]
    return {"p10": round(q(0.1), 4), "p50": round(q(0.5), 4), "p90": round(q(0.9), 4), "calls": n}


def rotating_sets(t, w, min_bytes):
    """Copies of the inputs (and the outputs' room) so that cycling through
    them touches at least min_bytes of HBM: with a working set above the
    256 MB last-level cache every call reads its inputs from HBM."""
    # q, k, v read and o (the size of q) written per call
    per_set = sum(t[n].numel() * t[n].element_size() for n in ("q", "k", "v", "q"))
    n = max(2, min(256, -(-min_bytes // per_set)))
    return [{k: (v.clone() if v is not None else None) for k, v in t.items()} for _ in range(n)]


def workload_inputs(w, device, with_do=False):
    from exact_attention_25_amd import inputs
    x = inputs.make_inputs(w, with_do=with_do)
    t = {n: upload(x[n + "_raw"], w.dtype, device) for n in ("q", "k", "v")}
    if with_do:
        t["do"] = upload(x["do_raw"], w.dtype, device)
    import torch
    t["kv_lens"] = None if x["kv_lens"] is None else torch.from_numpy(x["kv_lens"]).to(device)
    return x, t


def local_config(w) -> dict:
    out = {}
    if w.window:
        out["window_size"] = list(w.window)
    if w.grid:
        out["grid"] = {"cols": w.grid[0], "nbr_rows": w.grid[1], "nbr_cols": w.grid[2]}
    if w.softcap:
        out["softcap"] = w.softcap
    return out


def cpu_baseline(w, x, budget_s=15.0, backward=False, decode=False, fp8=False):
    """The fp64 oracle on (batch, head) pairs in order, until ~budget_s of CPU
    time; returns a dict in the metric's unit (TFLOP/s).  decode: the queries
    are the last positions of each batch's keys (the decode rule)."""
    from threadpoolctl import threadpool_info
    from exact_attention_25_amd import accounting as acc
    from oracle import ref_bwd_group, ref_fwd
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    G = w.Hq // w.Hkv
    done = 0
    t0 = time.perf_counter()
    mods = {k: v for k, v in (("window", w.window), ("grid", w.grid),
                              ("softcap", w.softcap or None)) if v}
    if backward:
        # one (batch, kv-head) group per oracle call: G heads
        flops = 0.0
        for b in range(w.B):
            lens = None if x["kv_lens"] is None else x["kv_lens"][b:b + 1]
            per_head = (10.0 * w.d * acc.local_pairs(w.Nq, lens, 1, w.causal, w.window, w.grid)
                        if is_local(w) else acc.bwd_flops(1, 1, w.Nq, w.Nk, w.d, w.causal))
            for g in range(w.Hkv):
                ref_bwd_group(x["q"], x["k"], x["v"], x["do"], b, g, causal=w.causal,
                              kv_lens=x["kv_lens"], **mods)
                done += G
                flops += G * per_head
                if time.perf_counter() - t0 >= budget_s:
                    break
            if time.perf_counter() - t0 >= budget_s:
                break
        what = "fp64 numpy oracle backward (incl. its forward)"
    else:
        if decode:
            mods["bottom_right"] = True
        flops = 0.0
        for b in range(w.B):
            lens = None if x["kv_lens"] is None else x["kv_lens"][b:b + 1]
            if decode:
                per_head = 4.0 * w.d * acc.decode_pairs(w.Nq, w.Nk, lens, 1, w.causal, w.window)
            elif is_local(w):
                per_head = 4.0 * w.d * acc.local_pairs(w.Nq, lens, 1, w.causal, w.window, w.grid)
            else:
                per_head = acc.fwd_flops(1, 1, w.Nq, w.Nk, w.d, w.causal)
            for h in range(w.Hq):
                g = h // G
                sl = (slice(b, b + 1), slice(h, h + 1))
                sk = (slice(b, b + 1), slice(g, g + 1))
                if fp8:
                    # the oracle's block quantisation and attention on the dequantised values
                    from oracle.fp8_ref import quantize_blocks, ref_fwd_fp8
                    (qc, qs), (kc, ks), (vc, vs) = (quantize_blocks(x[n][s]) for n, s in
                                                    (("q", sl), ("k", sk), ("v", sk)))
                    ref_fwd_fp8(qc, kc, vc, qs, ks, vs, causal=w.causal, kv_lens=lens)
                else:
                    ref_fwd(x["q"][sl], x["k"][sk], x["v"][sk], causal=w.causal, kv_lens=lens,
                            **mods)
                done += 1
                flops += per_head
                if time.perf_counter() - t0 >= budget_s:
                    break
            if time.perf_counter() - t0 >= budget_s:
                break
        what = "fp64 numpy oracle FP8 forward (quantisation + attention)" if fp8 else \
            "fp64 numpy oracle forward"
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{what} on the first {done} of {w.B * w.Hq} (batch, head) pairs of "
                      f"{w.name}, {dt:.1f} s; TFLOP/s counted like the GPU value",
            "tiny_fp32_one_core": tiny_one_core()}


def cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def tiny_one_core(reps=20):
    """The oracle forward on the whole tiny fp32 workload (B1 H2 N128 d64) on
    one BLAS thread: seconds per call (median of reps) and TFLOP/s."""
    from threadpoolctl import threadpool_limits
    from exact_attention_25_amd import accounting as acc
    from exact_attention_25_amd import inputs
    from oracle import ref_fwd
    w = inputs.WORKLOADS["tiny_fp32_b1_h2_n128_d64"]
    x = inputs.make_inputs(w, with_do=False)
    ts = []
    with threadpool_limits(1):
        for _ in range(reps):
            t0 = time.perf_counter()
            ref_fwd(x["q"], x["k"], x["v"])
            ts.append(time.perf_counter() - t0)
    t = sorted(ts)[len(ts) // 2]
    return {"seconds": round(t, 6), "cores": 1,
            "tflops": round(acc.fwd_flops(w.B, w.Hq, w.Nq, w.Nk, w.d, False) / t / 1e12, 6)}


def run_extras(device, steps, warmup):
    import torch
    from exact_attention_25_amd import accounting as acc
    from exact_attention_25_amd import binding as bd
    from exact_attention_25_amd import inputs
    stream = torch.cuda.current_stream(device)
    out = {}
    names = ["vit_bf16_b128_h16_n196_d64", "unet_self_fp16_b2_h8_n4096_d40",
             "unet_cross_fp16_b2_h8_q4096_k77_d40", "causal_gqa_bf16_b4_h32_kv2_n8192_d128"]
    # the sweep first: the long backward at the end heats the chip, which
    # lowers the clock the others would run at
    ws = [inputs.sweep_workload(n) for n in (1024, 2048, 8192, 16384)] + \
        [inputs.WORKLOADS[n] for n in names]
    for w in ws:
        x, t = workload_inputs(w, device, with_do=w.backward)
        o_b = torch.empty_like(t["q"])
        l_b = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=device)
        fn = lambda: bd.attn_fwd(t["q"], t["k"], t["v"], causal=w.causal, kv_lens=t["kv_lens"],
                                 out=o_b, lse=l_b)
        ms, _ = time_calls(fn, steps, warmup, stream)
        fl = acc.fwd_flops(w.B, w.Hq, w.Nq, w.Nk, w.d, w.causal)
        by = acc.fwd_min_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.dtype, x["kv_lens"] is not None)
        rec = {"fwd_ms": round(ms, 4), "fwd_tflops": round(fl / ms / 1e9, 1),
               "fwd_pct_peak": round(fl / ms / 1e9 / acc.PEAK_TFLOPS[w.dtype] * 100, 2),
               "fwd_min_bytes_gbs": round(by / ms / 1e6, 1),
               "tokens_per_s": round(w.B * w.Nq / ms * 1e3, 1)}
        if w.name in HBM_BOUND:
            # inputs rotated through >= 768 MB so that they come from HBM, not
            # from the last-level cache
            sets = rotating_sets(t, w, 768 << 20)
            for u in sets:
                u["o"] = torch.empty_like(u["q"])
                u["lse"] = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=device)
            it = [0]

            def rfn():
                u = sets[it[0] % len(sets)]
                it[0] += 1
                return bd.attn_fwd(u["q"], u["k"], u["v"], causal=w.causal, kv_lens=u["kv_lens"],
                                   out=u["o"], lse=u["lse"])
            rms, _ = time_calls(rfn, max(steps, 2 * len(sets)), len(sets), stream)
            # the same calls replayed from one HIP graph: kernel time without
            # the host's launch time between calls
            gms = time_graph(rfn, 2 * len(sets), len(sets),
                             [x for u in sets for x in (u["o"], u["lse"])])
            rec.update({"fwd_ms_rotated": round(rms, 4),
                        "fwd_min_bytes_gbs_rotated": round(by / rms / 1e6, 1),
                        "rotated_sets": len(sets),
                        "fwd_pct_hbm_peak_rotated": round(by / rms / 1e6 / acc.PEAK_HBM_GBS * 100, 1),
                        "fwd_ms_rotated_graph": round(gms, 4),
                        "fwd_pct_hbm_peak_rotated_graph":
                            round(by / gms / 1e6 / acc.PEAK_HBM_GBS * 100, 1)})
            del sets
        if w.backward:
            o, lse = fn()
            bfn = lambda: bd.attn_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=w.causal,
                                      kv_lens=t["kv_lens"])
            try:
                bms, _ = time_calls(bfn, max(steps // 2, 2), 2, stream)
                bfl = acc.bwd_flops(w.B, w.Hq, w.Nq, w.Nk, w.d, w.causal)
                rec.update({"bwd_ms": round(bms, 4), "bwd_tflops": round(bfl / bms / 1e9, 1),
                            "bwd_pct_peak": round(bfl / bms / 1e9 / acc.PEAK_TFLOPS[w.dtype] * 100, 2)})
            except bd.AttnError as e:
                rec["bwd_error"] = str(e)
        out[w.name] = rec
        del t
        torch.cuda.empty_cache()
    return out


def unfused_chain(device, steps, warmup):
    """The unfused chain the pages compare against (S = Q K^T, scaled,
    softmax, S V, each a separate torch op in bf16 with the N x N scores in
    HBM) at the B8 H32 N4096 d128 shape, beside the fused kernel on the same
    inputs: context for the pages' fused-over-unfused speed-up, not a
    target.  K^T is made contiguous once, outside the timed calls (torch's
    batched bf16 products are not given a transposed right operand)."""
    import torch
    from exact_attention_25_amd import accounting as acc
    from exact_attention_25_amd import binding as bd
    from exact_attention_25_amd import inputs
    stream = torch.cuda.current_stream(device)
    w = inputs.WORKLOADS[DEFAULT_WORKLOAD]
    _, t = workload_inputs(w, device)
    q, k, v = t["q"], t["k"], t["v"]
    kt = k.transpose(-1, -2).contiguous()
    scale = w.d ** -0.5

    def chain():
        s = torch.matmul(q, kt)
        return torch.matmul(torch.softmax(s * scale, dim=-1), v)

    ums, _ = time_calls(chain, steps, warmup, stream)
    o_u = chain()
    o_f, _ = bd.attn_fwd(q, k, v)
    fms, _ = time_calls(lambda: bd.attn_fwd(q, k, v), steps, warmup, stream)
    torch.cuda.synchronize()
    diff = float((o_u.float() - o_f.float()).abs().max())
    fl = acc.fwd_flops(w.B, w.Hq, w.Nq, w.Nk, w.d, False)
    del kt, o_u
    torch.cuda.empty_cache()
    return {"workload": w.name, "unfused_ms": round(ums, 4),
            "unfused_tflops": round(fl / ums / 1e9, 1), "fused_ms": round(fms, 4),
            "fused_speedup": round(ums / fms, 2), "max_abs_diff_unfused_vs_fused": diff,
            "scores_bytes_per_call": 2 * w.B * w.Hq * w.Nq * w.Nk}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--extras", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the engine-clock reading (amd-smi, ~1 s of extra calls)")
    ap.add_argument("--rotate", action="store_true",
                    help="forward: cycle through copies of the inputs totalling >= 768 MB, so that "
                         "they come from HBM (for the memory-bound workloads)")
    ap.add_argument("--graph", action="store_true",
                    help="forward: time the steps as one captured HIP graph (back-to-back kernels, "
                         "no host launch time between calls; for the microsecond-scale workloads)")
    ap.add_argument("--batch", type=int, default=0,
                    help="override the workload's batch size (counter runs whose per-dispatch "
                         "cycle counts must stay below 2^31); the JSON line then names the new B")
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd", "decode", "fp8"), default="fwd",
                    help="time the forward (default), the backward from the forward's O/LSE, "
                         "the split-KV decode (attn_decode; --workload a decode workload), or "
                         "the FP8 forward (attn_fwd_fp8 on attn_quantize_fp8's output)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the attention of every (batch, head) is "
              f"independent and the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from exact_attention_25_amd import accounting as acc
    from exact_attention_25_amd import binding as bd
    from exact_attention_25_amd import inputs
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    bd.load()
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    stream = torch.cuda.current_stream(device)

    w = inputs.WORKLOADS.get(args.workload)
    if w is None:
        m = re.match(r"long_bf16_sweep_b\d+_h32_n(\d+)_d128", args.workload)
        if not m:
            raise SystemExit(f"unknown workload {args.workload}")
        w = inputs.sweep_workload(int(m.group(1)))
    if args.batch > 0 and args.batch != w.B:
        import dataclasses
        w = dataclasses.replace(w, B=args.batch, name=re.sub(r"_b\d+_", f"_b{args.batch}_", w.name, 1))
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    bwd = args.which == "bwd"
    x, t = workload_inputs(w, device, with_do=bwd)

    if args.copy_calibration:
        # a plain copy of known size: 1 GiB read + 1 GiB written per launch
        src = torch.empty(1 << 28, dtype=torch.float32, device=device).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] copy calibration: 3 x 1 GiB device copies", file=sys.stderr, flush=True)
        del src, dst

    lkw = local_kw(w)
    # outputs allocated once, outside the timed calls
    o_buf = torch.empty_like(t["q"])
    l_buf = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=device)
    outs = [o_buf, l_buf]
    fwd = lambda: bd.attn_fwd(t["q"], t["k"], t["v"], causal=w.causal, kv_lens=t["kv_lens"],
                              out=o_buf, lse=l_buf, **lkw)
    n_sets = 0
    if args.rotate and args.which == "fwd":
        # inputs (and outputs) rotated through >= 768 MB, so that every call
        # reads its inputs from HBM rather than from the 256 MB last-level cache
        sets = rotating_sets(t, w, 768 << 20)
        for u in sets:
            u["o"] = torch.empty_like(u["q"])
            u["lse"] = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=device)
        n_sets = len(sets)
        rot = [0]
        outs = [x for u in sets for x in (u["o"], u["lse"])]

        def fwd():
            u = sets[rot[0] % n_sets]
            rot[0] += 1
            return bd.attn_fwd(u["q"], u["k"], u["v"], causal=w.causal, kv_lens=u["kv_lens"],
                               out=u["o"], lse=u["lse"], **lkw)
    dec = args.which == "decode"
    fp8 = args.which == "fp8"
    if fp8:
        q8, k8, vt8, qs, ks, vs = bd.attn_quantize_fp8(t["q"], t["k"], t["v"])
        qfn = lambda: bd.attn_quantize_fp8(t["q"], t["k"], t["v"])
        q_ms, _ = time_calls(qfn, 10, 2, stream)
        out_dt = torch.bfloat16 if w.dtype == "bf16" else torch.float16
        o8 = torch.empty(t["q"].shape, dtype=out_dt, device=device)
        l8 = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=device)
        fn = lambda: bd.attn_fwd_fp8(q8, k8, vt8, qs, ks, vs, causal=w.causal, kv_lens=t["kv_lens"],
                                     out_dtype=out_dt, out=o8, lse=l8)
        flops = acc.fwd_flops(w.B, w.Hq, w.Nq, w.Nk, w.d, w.causal)
    elif dec:
        dws = torch.empty(bd.attn_decode_workspace_bytes(bd.make_params(
            w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, bd.ATTN_BF16 if w.dtype == "bf16" else bd.ATTN_FP16,
            causal=w.causal, window_size=lkw["window_size"], softcap=w.softcap)),
            dtype=torch.uint8, device=device)
        fn = lambda: bd.attn_decode(t["q"], t["k"], t["v"], causal=w.causal,
                                    kv_lens=t["kv_lens"], window_size=lkw["window_size"],
                                    softcap=w.softcap, workspace=dws)
        flops = 4.0 * w.d * w.Hq * acc.decode_pairs(w.Nq, w.Nk, x["kv_lens"], w.B, w.causal,
                                                    w.window)
        dec_bytes = acc.decode_min_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.dtype, x["kv_lens"],
                                         w.window[0] if w.window else -1)
    elif bwd:
        o, lse = fwd()
        ws = torch.empty(bd.attn_bwd_workspace_bytes(bd.make_params(
            w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, bd.ATTN_BF16 if w.dtype == "bf16" else bd.ATTN_FP16,
            causal=w.causal)), dtype=torch.uint8, device=device)
        fn = lambda: bd.attn_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=w.causal,
                                 kv_lens=t["kv_lens"], workspace=ws, **lkw)
        # 10 d FLOPs per pair and head against the forward's 4 d
        flops = (2.5 * fwd_flops_of(w, x["kv_lens"]) if is_local(w)
                 else acc.bwd_flops(w.B, w.Hq, w.Nq, w.Nk, w.d, w.causal))
    else:
        fn = fwd
        flops = fwd_flops_of(w, x["kv_lens"])
    print(f"[bench] timing {args.steps} steps after {args.warmup} warm-up", file=sys.stderr, flush=True)
    graph = args.graph and args.which == "fwd"
    if graph:
        steps = args.steps if n_sets == 0 else -(-args.steps // n_sets) * n_sets
        ms = time_graph(fn, steps, max(args.warmup, n_sets), outs)
    else:
        ms, _ = time_calls(fn, args.steps, args.warmup, stream)

    pct = call_percentiles(fn, min(args.steps, 50), stream)
    clk = [] if args.no_clock else sample_sclk(fn, ms)

    tflops = flops / ms / 1e9
    peak = acc.PEAK_TFLOPS["fp8" if fp8 else w.dtype]
    if dec:
        gbs = dec_bytes / ms / 1e6
        rec = {
            "metric": "attention decode HBM GB/s (visible K/V cache read once, plus Q/O/LSE)",
            "value": round(gbs, 1),
            "unit": "GB/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(ms, 4),
            "ms_per_call_percentiles": pct,
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": w.dtype,
            "data": f"synthetic (seeded N(0,1) inputs, numpy PCG64, rounded to {w.dtype})",
            "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq,
                       "Nk": w.Nk, "d": w.d, "causal": w.causal,
                       "key_padding": w.lens is not None, "pass": "decode",
                       **local_config(w)},
            "pct_of_hbm_peak": round(gbs / acc.PEAK_HBM_GBS * 100, 2),
            "sclk_mhz_under_load": clock_fields(clk, 1.0, 1.0)["sclk_mhz_under_load"],
            "tokens_per_s": round(w.B * w.Nq / ms * 1e3, 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": acc.PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / acc.PEAK_HBM_GBS, 4),
                         "traffic": None,
                         "kernel": "attn::decode_split_kernel + attn::decode_merge_kernel, "
                                   "one call per step"},
        }
        if not args.no_cpu_baseline:
            print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
            cb = cpu_baseline(w, x, decode=True)
            # the oracle's time in the same unit: bytes of the sampled heads over its time
            frac = cb["value"] / max(tflops, 1e-30)
            cb = {"value": round(gbs * frac, 4), "unit": "GB/s", "cores": cb["cores"],
                  "kind": "oracle", "sample": cb["sample"] + "; converted to GB/s at the decode's "
                  "bytes per FLOP"}
            rec["cpu_baseline"] = cb
        print(json.dumps(rec), flush=True)
        return
    metric = METRIC
    if fp8:
        metric = ("attention fwd FP8 TFLOPS (4*B*H*N^2*d; E4M3 operands with 64-row block scales) "
                  "& % of the FP8 MFMA peak")
    elif bwd and is_local(w):
        metric = "attention bwd TFLOPS (10*d FLOPs per visible (query, key) pair and head)"
    elif bwd:
        metric = "attention bwd TFLOPS (10*B*H*N^2*d, halved for causal)"
    elif is_local(w):
        metric = "attention fwd TFLOPS (4*d FLOPs per visible (query, key) pair and head)"
    elif w.name != DEFAULT_WORKLOAD:
        metric = "attention fwd TFLOPS (4*B*H*N^2*d, halved for causal)"
    rec = {
        "metric": metric,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_call_percentiles": pct,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if fp8 else w.dtype,
        "data": f"synthetic (seeded N(0,1) inputs, numpy PCG64, rounded to {w.dtype}"
                + (", then block-quantised to E4M3 by attn_quantize_fp8)" if fp8 else ")"),
        "config": {"workload": w.name, "B": w.B, "H": w.Hq, "Hkv": w.Hkv, "N": w.Nq,
                   "Nk": w.Nk, "d": w.d, "causal": w.causal, "mask": None,
                   "key_padding": w.lens is not None, "rotated_input_sets": n_sets,
                   "launch": "hip_graph" if graph else "eager",
                   "pass": "fp8 forward" if fp8 else ("backward" if bwd else "forward"),
                   **local_config(w)},
        "pct_of_peak": round(tflops / peak * 100, 2),
        **clock_fields(clk, tflops, peak),
        "tokens_per_s": round(w.B * w.Nq / ms * 1e3, 1),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                     "traffic": None if (bwd or fp8 or w.name != DEFAULT_WORKLOAD) else recorded_traffic(),
                     "kernel": ("attn::bwd_prep_kernel + attn::bwd_q_kernel + attn::bwd_kv_kernel (+ reduce), one call per step"
                                if bwd else ("attn::fwd_fp8_kernel (one launch per step)" if fp8
                                             else fwd_kernel_name(w) + " (one launch per step)"))},
    }
    if not (bwd or fp8) and w.name in HBM_BOUND:
        # memory-bound forward: the roofline is HBM bandwidth over the
        # algorithmic bytes (Q, K, V read once, O and LSE written once)
        by = acc.fwd_min_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.dtype, x["kv_lens"] is not None)
        gbs = by / ms / 1e6
        rec["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": acc.PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": round(gbs / acc.PEAK_HBM_GBS, 4),
                           "traffic": None, "bytes_per_call": by,
                           "kernel": rec["roofline"]["kernel"]}
    if fp8:
        rec["quantize_ms"] = round(q_ms, 4)
    if args.extras:
        print("[bench] extras", file=sys.stderr, flush=True)
        rec["extras"] = run_extras(device, max(args.steps // 2, 10), 5)
        rec["extras"]["unfused_chain"] = unfused_chain(device, 10, 3)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(w, x, backward=bwd, fp8=fp8)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
