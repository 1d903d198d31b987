#!/usr/bin/env python3
"""Forward-attention throughput on one MI355X.

One step = the bf16 exact-attention forward at d = 128 and N = 4096 on the
sequence-length sweep's 16384-token batch (B=4, H=16, bf16 N(0, 1) inputs,
seed 73212, scale 1/sqrt(d)), run once non-causal and once causal, inputs
resident in HBM.  FLOPs are counted as 4 B H N^2 d per forward, halved for
causal.  The JSON line also carries:

* ``roofline`` of the dominant kernel (the non-causal bf16 forward of the
  step), whose average launch duration is measured with HIP events on the
  stream the kernel runs on, against the dense bf16 MFMA peak (2516.6
  TFLOP/s);
* ``config.fp8``: the FP8 workload (B4 H16 N4096 d128, 0.1 % outliers,
  per-128-row amax / 448 block scales, Hadamard-rotated Q and K): forward
  TFLOPS and its fraction of the FP8 peak (5033.2 TFLOP/s), prep GB/s and
  the end-to-end rate, from the ``fp8`` leg;
* ``legs``: per-kernel figures -- the standard block (B4 H16 N2048 d128),
  the sequence-length sweeps at 16384 total tokens for d = 128, 64 and 256
  (TFLOPS and fraction of peak vs N, both causal flags, plus the
  algorithmic HBM rate for N <= 1024), the long causal context (B1 H16
  N65536 d128), the FP8 workload (also with power-of-two V scales), the
  backward, decode and packed-batch shapes.  Legs time 30 launches after 10
  warm-ups (5 after 1 for the long context) and give the mean plus the rates
  at the p90/median/p10 durations; N = 512 and the prep kernels are also
  timed with cold caches (a 1 GiB write before each launch);
* ``cpu_baseline``: the CPU fp64 oracle timed on a bounded sample of the
  same step on this host (core count and CPU model recorded).

``roofline.traffic`` is the kernel's HBM bytes per launch read by two
rocprofv3 counter passes (FETCH_SIZE, WRITE_SIZE, each scaled by what the
counter reads for a 256 MiB device copy), recorded in
profiles/fwd_bf16_N4096_noncausal_traffic.md together with the SHA-256 of
the kernel's sources; it is null when those sources changed since.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--quick]
                       [--legs std,sweep,sweep64,sweep256,long,fp8,bwd,decode,varlen,mfma_loop] [--copy-calibration]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

PEAK_BF16 = 2516.6  # TFLOP/s, dense bf16 MFMA, MI355X public spec
PEAK_FP8 = 5033.2
PEAK_HBM = 8000.0  # GB/s
METRIC = "attention fwd TFLOPS (bf16, fp8) at d=128 vs N, and % of MFMA peak"
GPU_HOLD_CYCLES = 20_000_000  # a short device-side spin before each timed region
ROOT = os.path.dirname(os.path.abspath(__file__))
# HBM traffic of the dominant kernel, from rocprofv3 FETCH_SIZE / WRITE_SIZE
# passes; valid only while the kernel sources hash to what was profiled
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "fwd_bf16_N4096_noncausal_traffic.md")
TRAFFIC_SOURCES = ("exact_attention_73_amd/csrc/fa_fwd_bf16.hip", "exact_attention_73_amd/csrc/fa_device.h")
COPY_CALIBRATION_BYTES = 256 << 20


ALL_LEGS = ("std", "sweep", "sweep64", "sweep256", "long", "fp8", "bwd", "decode", "varlen", "mfma_loop")


def fwd_bytes(B, H, N, d):
    """Algorithmic HBM bytes of one forward: bf16 Q, K, V read once, fp32 O and lse written once."""
    return B * H * N * (3 * d * 2 + d * 4 + 4)


def decode_bytes(B, Hq, Hkv, Nq, Nk, d):
    """Algorithmic HBM bytes of one decode forward: bf16 K and V read once
    per KV head, bf16 Q read once, fp32 O and lse written once."""
    return B * Hkv * Nk * d * 2 * 2 + B * Hq * Nq * (d * 2 + d * 4 + 4)


def fwd_flops(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def _stats(ts):
    """mean, median, p10 and p90 (seconds) of per-launch durations."""
    ts = sorted(ts)
    n = len(ts)
    return {"mean": sum(ts) / n, "median": ts[n // 2], "p10": ts[int(round(0.1 * (n - 1)))],
            "p90": ts[int(round(0.9 * (n - 1)))]}


def _time_launches(fn, reps, warmup):
    """Per-launch durations of fn() (hot caches): HIP events recorded between
    consecutive launches on the current stream, after a device-side spin that
    lets the host queue every launch first."""
    import torch

    for _ in range(warmup):
        fn()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    torch.cuda._sleep(GPU_HOLD_CYCLES)
    ev[0].record()
    for i in range(reps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    return _stats([ev[i].elapsed_time(ev[i + 1]) / 1e3 for i in range(reps)])


def _time_cold(fn, reps, warmup, flush):
    """Per-launch durations with cold caches: flush() (a 1 GiB write, larger
    than the L2s and the MALL together) runs before each launch, outside the
    event pair that brackets the launch."""
    import torch

    for _ in range(warmup):
        fn()
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for e0, e1 in pairs:
        flush()
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return _stats([e0.elapsed_time(e1) / 1e3 for e0, e1 in pairs])


def _rates(work, st, scale):
    """Rates at the p90, median and p10 durations (ascending), rounded."""
    return [round(work / st[k] / scale, 1) for k in ("p90", "median", "p10")]


def kernel_sources_sha256():
    """SHA-256 over the code of the traffic kernel's sources: comments and
    blank lines removed (neither source holds a string with a comment
    marker), so an edit of the prose alone keeps the counters valid."""
    import hashlib
    import re

    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        h.update(("\n".join(ln.rstrip() for ln in src.splitlines() if ln.strip()) + "\n").encode())
    return h.hexdigest()


def profiled_traffic():
    """Bytes per launch (FETCH + WRITE, calibrated) from the committed counter
    summary, or None when it is missing or the kernel changed since."""
    try:
        fields = {}
        with open(TRAFFIC_SUMMARY) as f:
            for ln in f:
                if ln.startswith("- `") and "`: " in ln:
                    key, val = ln[3:].split("`: ", 1)
                    fields[key] = val.strip().strip("`")
        if fields.get("kernel_sources_sha256") != kernel_sources_sha256():
            return None
        return int(fields["fetch_bytes_per_launch"]) + int(fields["write_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="run only the timed step, no legs (for profiling runs)")
    ap.add_argument("--legs", default=None,
                    help=f"comma-separated legs to run after the step (default: all of {','.join(ALL_LEGS)})")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, copy 256 MiB device-to-device once, untimed, so that a "
                         "counter pass sees a kernel of known traffic beside the attention kernels")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (every (batch, head) pair is "
              "independent, so more GPUs would each run this same kernel on their own share)", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_attention_73_amd as fa
    from exact_attention_73_amd.inputs import (WORKLOADS, make_do, make_qkv, make_signs, packed_batch_lengths,
                                              softmax_scale, sweep_workloads)

    HEADLINE = next(x for x in sweep_workloads() if x.d == 128 and x.N == 4096)

    fa.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = HEADLINE
    B, H, N, d = w.B, w.H, w.N, w.d
    q, k, v = (x.to(dev) for x in make_qkv(B, H, N, d, w.seed))
    sc = softmax_scale(d)
    o = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)

    def step():
        fa.fwd_bf16(q, k, v, causal=False, softmax_scale=sc, out=o, lse=lse)
        fa.fwd_bf16(q, k, v, causal=True, softmax_scale=sc, out=o, lse=lse)

    for _ in range(args.warmup):
        step()
    # per-launch durations inside the timed region, on the kernels' stream
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    torch.cuda._sleep(GPU_HOLD_CYCLES)
    ev[0].record()
    for i in range(args.steps):
        fa.fwd_bf16(q, k, v, causal=False, softmax_scale=sc, out=o, lse=lse)
        ev[2 * i + 1].record()
        fa.fwd_bf16(q, k, v, causal=True, softmax_scale=sc, out=o, lse=lse)
        ev[2 * i + 2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    nc = [ev[2 * i].elapsed_time(ev[2 * i + 1]) / 1e3 for i in range(args.steps)]
    ca = [ev[2 * i + 1].elapsed_time(ev[2 * i + 2]) / 1e3 for i in range(args.steps)]
    gpu_total = ev[0].elapsed_time(ev[-1]) / 1e3
    step_flops = fwd_flops(B, H, N, d, False) + fwd_flops(B, H, N, d, True)
    ms_per_step = 1e3 * gpu_total / args.steps
    value = step_flops / (gpu_total / args.steps) / 1e12
    t_nc = sum(nc) / len(nc)
    t_ca = sum(ca) / len(ca)
    achieved = fwd_flops(B, H, N, d, False) / t_nc / 1e12

    legs = {
        "step_noncausal_tflops": round(achieved, 2),
        "step_causal_tflops": round(fwd_flops(B, H, N, d, True) / t_ca / 1e12, 2),
        "step_noncausal_us": round(t_nc * 1e6, 2),
        "step_causal_us": round(t_ca * 1e6, 2),
    }
    del q, k, v

    legs_on = set() if args.quick else set(ALL_LEGS)
    if args.legs is not None:
        legs_on = {x for x in args.legs.split(",") if x}
        bad = legs_on - set(ALL_LEGS)
        if bad:
            raise SystemExit(f"unknown legs {sorted(bad)}; choose from {ALL_LEGS}")

    scratch = None

    def flush():
        nonlocal scratch
        if scratch is None:
            scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        scratch.fill_(1.0)

    if "std" in legs_on:
        ws_ = WORKLOADS["std"]
        qs, ks, vs = (x.to(dev) for x in make_qkv(ws_.B, ws_.H, ws_.N, ws_.d, ws_.seed))
        row = {"workload": f"B{ws_.B} H{ws_.H} N{ws_.N} d{ws_.d}"}
        for causal in (False, True):
            st = _time_launches(lambda: fa.fwd_bf16(qs, ks, vs, causal=causal), 30, 10)
            fl = fwd_flops(ws_.B, ws_.H, ws_.N, ws_.d, causal)
            key = "causal" if causal else "noncausal"
            row[key + "_tflops"] = round(fl / st["mean"] / 1e12, 1)
            row[key + "_frac"] = round(fl / st["mean"] / 1e12 / PEAK_BF16, 4)
            row[key + "_us"] = round(st["mean"] * 1e6, 2)
        legs["bf16_std"] = row
        del qs, ks, vs

    for dd, name in ((128, "sweep"), (64, "sweep64"), (256, "sweep256")):
        if name not in legs_on:
            continue
        sweep = {}
        for sw in sweep_workloads():
            if sw.d != dd:
                continue
            qs, ks, vs = (x.to(dev) for x in make_qkv(sw.B, sw.H, sw.N, sw.d, sw.seed))
            row = {}
            for causal in (False, True):
                call = lambda: fa.fwd_bf16(qs, ks, vs, causal=causal)
                st = _time_launches(call, 30, 10)
                fl = fwd_flops(sw.B, sw.H, sw.N, sw.d, causal)
                tf = fl / st["mean"] / 1e12
                key = "causal" if causal else "noncausal"
                row[key] = round(tf, 1)
                row[key + "_frac"] = round(tf / PEAK_BF16, 4)
                row[key + "_p10_p50_p90"] = _rates(fl, st, 1e12)
                if sw.N <= 1024:  # short sequences: algorithmic HBM rate, hot and cold caches
                    by = fwd_bytes(sw.B, sw.H, sw.N, sw.d)
                    row[key + "_gbps"] = round(by / st["mean"] / 1e9, 1)
                    if sw.N == 512:
                        sc = _time_cold(call, 30, 3, flush)
                        row[key + "_cold_gbps"] = round(by / sc["mean"] / 1e9, 1)
                        row[key + "_cold_tflops"] = round(fl / sc["mean"] / 1e12, 1)
            sweep[str(sw.N)] = row
            del qs, ks, vs
        legs[f"bf16_d{dd}_sweep_tflops"] = sweep

    if "long" in legs_on:
        wl = WORKLOADS["long"]
        ql, kl, vl = (x.to(dev) for x in make_qkv(wl.B, wl.H, wl.N, wl.d, wl.seed))
        st = _time_launches(lambda: fa.fwd_bf16(ql, kl, vl, causal=True), 5, 1)
        fl = fwd_flops(wl.B, wl.H, wl.N, wl.d, True)
        tf = fl / st["mean"] / 1e12
        legs["bf16_long"] = {"workload": f"B{wl.B} H{wl.H} N{wl.N} d{wl.d} causal", "tflops": round(tf, 1),
                             "frac": round(tf / PEAK_BF16, 4), "ms": round(st["mean"] * 1e3, 3),
                             "tflops_p10_p50_p90": _rates(fl, st, 1e12)}
        del ql, kl, vl

    if "fp8" in legs_on:
        w8 = WORKLOADS["fp8"]
        q, k, v = (x.to(dev) for x in make_qkv(w8.B, w8.H, w8.N, w8.d, w8.seed, outliers=True))
        signs = make_signs(w8.H, w8.d, w8.seed + 1).to(dev)
        q8, qs_ = fa.fp8_prep(q, signs=signs)
        k8, ks_ = fa.fp8_prep(k, signs=signs)
        v8t, vs_ = fa.fp8_prep_v(v)
        prep_q = lambda: fa.fp8_prep(q, signs=signs, out=q8, scale_out=qs_)
        prep_v = lambda: fa.fp8_prep_v(v, out=v8t, scale_out=vs_)
        t_prep = _time_launches(prep_q, 30, 10)
        t_prep_v = _time_launches(prep_v, 30, 10)
        c_prep = _time_cold(prep_q, 30, 3, flush)
        c_prep_v = _time_cold(prep_v, 30, 3, flush)
        fa.fp8_prep(k, signs=signs, out=k8, scale_out=ks_)
        o8 = torch.empty((w8.B, w8.H, w8.N, w8.d), dtype=torch.float32, device=dev)
        l8 = torch.empty((w8.B, w8.H, w8.N), dtype=torch.float32, device=dev)
        t8 = _time_launches(lambda: fa.fwd_fp8(q8, k8, v8t, qs_, ks_, vs_, out=o8, lse=l8), 30, 10)
        t8c = _time_launches(lambda: fa.fwd_fp8(q8, k8, v8t, qs_, ks_, vs_, causal=True, out=o8, lse=l8), 30, 10)
        v8p, vsp = fa.fp8_prep_v(v, pow2_scale=True)
        t8p = _time_launches(lambda: fa.fwd_fp8(q8, k8, v8p, qs_, ks_, vsp, out=o8, lse=l8), 30, 10)
        elems = w8.B * w8.H * w8.N * w8.d
        prep_bytes = elems * 2 + elems + w8.B * w8.H * ((w8.N + 127) // 128) * 4
        f8 = fwd_flops(w8.B, w8.H, w8.N, w8.d, False)
        tb = _time_launches(lambda: fa.fwd_bf16(q, k, v, out=o8, lse=l8), 30, 10)
        legs["fp8"] = {
            "workload": "B4 H16 N4096 d128 non-causal, 0.1% N(0,10^2) outliers, per-128-row amax/448 block scales, "
                        "Hadamard-rotated Q and K",
            "fwd_fp8_tflops": round(f8 / t8["mean"] / 1e12, 1),
            "fwd_fp8_frac_of_fp8_peak": round(f8 / t8["mean"] / 1e12 / PEAK_FP8, 4),
            "fwd_fp8_tflops_p10_p50_p90": _rates(f8, t8, 1e12),
            "fwd_fp8_causal_tflops": round(f8 / 2 / t8c["mean"] / 1e12, 1),
            "fwd_fp8_vpow2_tflops": round(f8 / t8p["mean"] / 1e12, 1),
            "fwd_bf16_same_shape_tflops": round(f8 / tb["mean"] / 1e12, 1),
            "prep_qk_rotated_gbps": round(prep_bytes / t_prep["mean"] / 1e9, 1),
            "prep_qk_rotated_frac_of_hbm": round(prep_bytes / t_prep["mean"] / 1e9 / PEAK_HBM, 4),
            "prep_qk_rotated_cold_gbps": round(prep_bytes / c_prep["mean"] / 1e9, 1),
            "prep_v_transposed_gbps": round(prep_bytes / t_prep_v["mean"] / 1e9, 1),
            "prep_v_transposed_cold_gbps": round(prep_bytes / c_prep_v["mean"] / 1e9, 1),
            "end_to_end_tflops": round(f8 / (t8["mean"] + 2 * t_prep["mean"] + t_prep_v["mean"]) / 1e12, 1),
        }
        del q, k, v, q8, k8, v8t, v8p, o8, l8
    scratch = None

    if "bwd" in legs_on:
        # backward: 2.5 x the forward's FLOPs (dQ, dK, dV and the recomputed
        # S), halved for causal; the delta, dK/dV and dQ kernels in one call
        bw = {}
        for (Bb, Hb, Nb, db) in ((4, 16, 2048, 128), (4, 16, 4096, 128), (4, 16, 2048, 64), (4, 8, 2048, 256)):
            qb_, kb_, vb_ = (x.to(dev) for x in make_qkv(Bb, Hb, Nb, db, 73002))
            gb_ = make_do(Bb, Hb, Nb, db, 73002).to(dev)
            for causal in (False, True):
                ob_, lb_ = fa.fwd_bf16(qb_, kb_, vb_, causal=causal)
                outs = [torch.empty_like(ob_) for _ in range(3)]
                ws = torch.empty_like(lb_)
                st = _time_launches(lambda: fa.bwd_bf16(qb_, kb_, vb_, ob_, lb_, gb_, causal=causal, dq=outs[0],
                                                        dk=outs[1], dv=outs[2], delta=ws), 20, 5)
                fl = 2.5 * fwd_flops(Bb, Hb, Nb, db, causal)
                bw[f"B{Bb} H{Hb} N{Nb} d{db} {'causal' if causal else 'non-causal'}"] = {
                    "tflops": round(fl / st["mean"] / 1e12, 1), "frac": round(fl / st["mean"] / 1e12 / PEAK_BF16, 4),
                    "us": round(st["mean"] * 1e6, 1), "tflops_p10_p50_p90": _rates(fl, st, 1e12)}
            del qb_, kb_, vb_, gb_, ob_, lb_, outs, ws
        legs["bf16_bwd"] = bw

    if "decode" in legs_on:
        # few queries against long keys: HBM-bound on the K/V read.  The split
        # count is the library's choice; the prefill-shaped kernel on the same
        # shape is timed beside it.
        dec = {}
        for (Bd, Hq, Hkv, Nq, Nk, dd) in ((16, 32, 8, 1, 8192, 128), (1, 32, 8, 1, 131072, 128),
                                           (8, 32, 32, 1, 8192, 128), (16, 32, 8, 4, 8192, 128),
                                           (32, 16, 2, 1, 8192, 64), (16, 16, 4, 1, 8192, 256)):
            qd_, _, _ = make_qkv(Bd, Hq, Nq, dd, 73600)
            _, kd_, vd_ = make_qkv(Bd, Hkv, Nk, dd, 73601)
            qd_, kd_, vd_ = qd_.to(dev), kd_.to(dev), vd_.to(dev)
            od_ = torch.empty((Bd, Hq, Nq, dd), dtype=torch.float32, device=dev)
            ld_ = torch.empty((Bd, Hq, Nq), dtype=torch.float32, device=dev)
            splits = fa.decode_splits(Bd, Hq, Hkv, Nq, Nk, dd)
            need = fa.decode_workspace_bytes(Bd, Hq, Nq, dd, splits)
            wsd = torch.empty(max(need // 4, 1), dtype=torch.float32, device=dev)
            call = lambda: fa.fwd_bf16_decode(qd_, kd_, vd_, causal=True, num_splits=splits, out=od_, lse=ld_,
                                              workspace=wsd)
            st = _time_launches(call, 30, 10)
            sc = _time_cold(call, 30, 3, flush)
            sp = _time_launches(lambda: fa.fwd_bf16_gqa(qd_, kd_, vd_, causal=True, out=od_, lse=ld_), 10, 3)
            by = decode_bytes(Bd, Hq, Hkv, Nq, Nk, dd)
            dec[f"B{Bd} Hq{Hq} Hkv{Hkv} Nq{Nq} Nk{Nk} d{dd} causal"] = {
                "splits": splits, "us": round(st["mean"] * 1e6, 1), "gbps": round(by / st["mean"] / 1e9, 1),
                "frac_of_hbm": round(by / st["mean"] / 1e9 / PEAK_HBM, 4),
                "cold_us": round(sc["mean"] * 1e6, 1), "cold_gbps": round(by / sc["mean"] / 1e9, 1),
                "cold_frac_of_hbm": round(by / sc["mean"] / 1e9 / PEAK_HBM, 4),
                "gbps_p10_p50_p90": _rates(by, st, 1e9),
                "prefill_kernel_same_shape_us": round(sp["mean"] * 1e6, 1)}
            del qd_, kd_, vd_, od_, ld_, wsd
        legs["bf16_decode"] = dec

    if "varlen" in legs_on:
        # 16 causal sequences of mixed lengths (seeded, 256..4096 keys) packed
        # end to end; FLOPs count each sequence's own work only.  The same
        # batch padded to its longest sequence is timed beside it.
        lens = packed_batch_lengths()
        Hv, dv_ = 16, 128
        tot = sum(lens)
        qv_, _, _ = make_qkv(1, Hv, tot, dv_, 73801)
        _, kv_, vv_ = make_qkv(1, Hv, tot, dv_, 73802)
        qv_, kv_, vv_ = (x[0].transpose(0, 1).contiguous().to(dev) for x in (qv_, kv_, vv_))
        cu = torch.tensor([0] + lens, dtype=torch.int32).cumsum(0).to(torch.int32).to(dev)
        ov_ = torch.empty((tot, Hv, dv_), dtype=torch.float32, device=dev)
        lv_ = torch.empty((Hv, tot), dtype=torch.float32, device=dev)
        st = _time_launches(lambda: fa.fwd_bf16_varlen(qv_, kv_, vv_, cu, cu, max(lens), causal=True, out=ov_,
                                                       lse=lv_), 20, 5)
        fl = sum(4.0 * Hv * n * n * dv_ / 2 for n in lens)
        Np = max(lens)
        qp, kp, vp = (torch.zeros((16, Hv, Np, dv_), dtype=torch.bfloat16, device=dev) for _ in range(3))
        sp = _time_launches(lambda: fa.fwd_bf16(qp, kp, vp, causal=True), 10, 3)
        legs["bf16_varlen"] = {
            "workload": f"16 sequences, {tot} tokens (lengths 256..4096, seeded), H16 d128 causal",
            "tflops": round(fl / st["mean"] / 1e12, 1), "frac": round(fl / st["mean"] / 1e12 / PEAK_BF16, 4),
            "us": round(st["mean"] * 1e6, 1), "padded_to_longest_us": round(sp["mean"] * 1e6, 1)}
        del qv_, kv_, vv_, ov_, lv_, qp, kp, vp

    if "mfma_loop" in legs_on:
        legs["mfma_loop"] = mfma_loop_rates(torch, dev)

    if args.copy_calibration:
        src = torch.ones(COPY_CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(B, H, N, d, w.seed)

    props = torch.cuda.get_device_properties(0)
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "sequence-length sweep point B4 H16 N4096 d128 (16384 tokens), bf16 forward, "
                        "non-causal + causal per step",
            "B": B, "H": H, "N": N, "d": d, "causal": [False, True], "seed": w.seed,
            "flop_convention": "4*B*H*N^2*d per forward, halved for causal",
            "device": props.name, "arch": getattr(props, "gcnArchName", ""), "cus": props.multi_processor_count,
            "torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
            "host_wall_s": round(wall, 4),
            "mfma_loop_tflops": ({k_: legs["mfma_loop"][k_] for k_ in ("bf16", "fp8")}
                                 if legs.get("mfma_loop") else None),
            "fp8": ({k_: legs["fp8"][k_] for k_ in ("workload", "fwd_fp8_tflops", "fwd_fp8_frac_of_fp8_peak",
                                                    "fwd_fp8_causal_tflops", "fwd_fp8_vpow2_tflops",
                                                    "prep_qk_rotated_gbps", "prep_v_transposed_gbps",
                                                    "end_to_end_tflops")} if "fp8" in legs else None),
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "fwd_bf16_pp_kernel<128, non-causal> at B4 H16 N4096 d128",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16, 4),
            "traffic": profiled_traffic(),
            "traffic_unit": "bytes per launch",
            "frac_of_mfma_loop": (round(achieved / legs["mfma_loop"]["bf16"], 4) if legs.get("mfma_loop") else None),
        },
        "legs": legs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def mfma_loop_rates(torch, dev):
    """Sustained matrix-core rate of this GPU in this run: one workgroup of 8
    waves per CU, each wave issuing independent 32x32 products on register
    operands (8 chains of bf16 32x32x16, 4 of FP8 32x32x64), timed with HIP
    events; a reference point beside the published peaks.  Uses the test
    probe library (tests/hip/libprobes.so) when it is built."""
    import ctypes

    path = os.path.join(ROOT, "tests", "hip", "libprobes.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.probe_mfma_rate.restype = ctypes.c_int
    lib.probe_mfma_rate.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p]
    grid = torch.cuda.get_device_properties(0).multi_processor_count
    src = torch.full((512,), 0x3C003C00, dtype=torch.int32, device=dev)  # bf16 pairs of 1.0; E4M3 1.5 and 0
    out = torch.empty(grid * 512, dtype=torch.float32, device=dev)
    iters = 40000
    res = {"workgroups": grid, "waves_per_simd": 2, "iters": iters}
    for fp8, name, chains, flop in ((0, "bf16", 8, 2 * 32 * 32 * 16), (1, "fp8", 4, 2 * 32 * 32 * 64)):
        st_ = torch.cuda.current_stream().cuda_stream
        call = lambda: lib.probe_mfma_rate(fp8, src.data_ptr(), out.data_ptr(), iters, grid, st_)
        ts = []
        for i in range(7):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            if call() != 0:
                return None
            e1.record()
            torch.cuda.synchronize()
            if i >= 2:
                ts.append(e0.elapsed_time(e1) / 1e3)
        t = sorted(ts)[len(ts) // 2]
        res[name] = round(grid * 8 * iters * chains * flop / t / 1e12, 1)
    # LDS read rate per CU (bytes per ns): ds_read_b128 and the transposed
    # ds_read_b64_tr_b16 of the forward's V operand
    lib.probe_lds_rate.restype = ctypes.c_int
    lib.probe_lds_rate.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    for tr, name, by in ((0, "lds_read_b128_bytes_per_ns_per_cu", 1024), (1, "lds_read_tr_b16_bytes_per_ns_per_cu", 512)):
        st_ = torch.cuda.current_stream().cuda_stream
        ts = []
        for i in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            if lib.probe_lds_rate(tr, out.data_ptr(), 20000, grid, st_) != 0:
                return None
            e1.record()
            torch.cuda.synchronize()
            if i >= 1:
                ts.append(e0.elapsed_time(e1) / 1e3)
        t = sorted(ts)[len(ts) // 2]
        res[name] = round(8 * 20000 * 16 * by / t / 1e9, 1)
    res["bf16_frac_of_published"] = round(res["bf16"] / PEAK_BF16, 4)
    res["fp8_frac_of_published"] = round(res["fp8"] / PEAK_FP8, 4)
    return res


def cpu_baseline(B, H, N, d, seed):
    """The oracle, as it stands, on a bounded sample of heads of the step."""
    import numpy as np

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = os.cpu_count() or 1
    from exact_attention_73_amd.inputs import make_qkv, softmax_scale
    from oracle import attention_ref

    q, k, v = make_qkv(B, H, N, d, seed)
    sc = softmax_scale(d)
    qn, kn, vn = (x.float().numpy().astype(np.float64) for x in (q, k, v))

    def run_heads(nh):
        """Non-causal + causal forward of the first nh (batch, head) pairs."""
        t0 = time.perf_counter()
        for i in range(nh):
            b, h = divmod(i, H)
            sl = (slice(b, b + 1), slice(h, h + 1))
            for causal in (False, True):
                attention_ref(qn[sl], kn[sl], vn[sl], causal=causal, scale=sc)
        return time.perf_counter() - t0

    # bounded sample: whole steps (all B*H heads) repeated until >= 10 s, at
    # most 30 s; on a slow host, a prefix of the heads
    run_heads(1)  # warm-up (thread pools, first-touch)
    t1 = run_heads(1)
    per_step = t1 * B * H
    if per_step <= 10.0:
        reps = max(1, min(int(10.0 // per_step) + 1, int(30.0 // per_step)))
        t = sum(run_heads(B * H) for _ in range(reps))
        nh, desc = reps * B * H, f"{reps} whole step(s), all {B * H} heads"
    else:
        nh = int(max(1, min(B * H, 15.0 // max(t1, 1e-3))))
        t = run_heads(nh)
        desc = f"{nh} of {B * H} heads of one step"
    flops = (fwd_flops(1, nh, N, d, False) + fwd_flops(1, nh, N, d, True))
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(flops / t / 1e12, 6),
        "unit": "TFLOPS",
        "cores": int(threads),
        "cpu_model": model,
        "host_logical_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": f"{desc} (non-causal + causal), fp64 NumPy, {t:.2f} s; the oracle evaluates full score rows, "
                  f"so causal does twice the counted work",
    }


if __name__ == "__main__":
    main()
