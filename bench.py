#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
the forward (O and LSE) and the backward (delta pre-pass, dK/dV, dQ), each
kernel launched through the C ABI on the current stream.  The default
workload is B=8, H=16, N=2048, d=128, causal, bf16 (the forward+backward
problem); ``--workload`` picks another from fa_inputs.WORKLOADS (forward-only
workloads time the forward alone).

FLOPs: forward 4*B*H*N^2*d, backward 10*B*H*N^2*d (the five N^2*d products
of the recomputing backward), each halved for causal.  The value printed is
the whole step's FLOPs over its wall time between two synchronisations.

Each kernel is also bracketed by HIP events on the launch stream; the kernel
with the largest average duration is reported with its roofline:
achieved = its algorithmic FLOPs per launch / its average duration, against
the MI355X dense bf16 matrix-core peak.

cpu_baseline: the fp64 oracle (materialising S and P) timed on the host on
the first whole heads of the same workload, forward+backward, for about
``--cpu-seconds`` seconds.

One JSON line on stdout.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, 8 TB/s
PEAK_FP8_TFLOPS = 5033.2   # dense FP8 matrix cores, twice the bf16 rate
DEFAULT_WORKLOAD = "bf16_b8h16n2048d128_causal_fwdbwd"
CLOCK_WARMUP_S = 1.0   # untimed work before the timed steps (clock ramp-up)
CLOCK_REWARM_S = 0.3   # untimed burst before each secondary measurement
HEADLINE_FWD = ["bf16_b4h16n4096d128_causal_x0.5", "bf16_b1h16n16384d128_causal", "bf16_b1h16n16384d128"]


def _products(w, n):
    """FLOPs of n N^2*d products (2*N^2*d each) over all heads, halved if causal."""
    f = 2.0 * n * w.B * w.H * w.N * w.N * w.d
    return f / 2 if w.causal else f


def kernel_source_digest() -> str:
    """sha256 over the HIP sources and headers the library is built from."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_attention_18_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    with open(os.path.join(ROOT, "include", "fa.h"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    counter summary, or None if there is none for the current sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    if fields.get("source_digest") != kernel_source_digest():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(dev, mib: int, reps: int):
    """Plain device-to-device copies of a known size, for scaling the HBM
    byte counters: each copy reads and writes exactly `mib` MiB."""
    import torch

    src = torch.empty(mib * 2**20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()


def cpu_baseline(w, budget_s: float):
    import numpy as np
    from threadpoolctl import threadpool_info

    import fa_inputs as fi
    import oracle

    x = fi.make_inputs(w, with_grad=True)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done = 0
    t0 = time.perf_counter()
    for (b, h) in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        args = [fi.exact_f64(x[n][sl]) for n in ("q", "k", "v")]
        oracle.attention_forward(*args, w.causal, w.scale)
        if w.backward:
            oracle.attention_backward(*args, fi.exact_f64(x["do"][sl]), w.causal, w.scale)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    per_head = (w.fwd_flops() + (w.bwd_flops() if w.backward else 0.0)) / (w.B * w.H)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {
        "value": per_head * done / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} of {w.B * w.H} (batch, head) pairs, forward{'+backward' if w.backward else ''}, "
                  f"fp64 numpy, {dt:.1f} s, host nproc {os.cpu_count()}",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-headline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run 3 plain copies of MIB MiB (for counter calibration)")
    ap.add_argument("--print-digest", action="store_true", help="print the kernel source digest and exit")
    args = ap.parse_args()
    if args.print_digest:
        print(kernel_source_digest())
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build runs the attention kernels on a single "
              "MI355X and has no multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import exact_attention_18_amd as fa
    import fa_inputs as fi

    fa._lib.load()  # raises if the HIP library is missing
    w = fi.WORKLOADS[args.workload]
    if w.dtype != "bf16":
        raise SystemExit("bench.py times the bf16 path")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    x = fi.make_inputs(w, with_grad=True)
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    B, H, N, d, causal, scale = w.B, w.H, w.N, w.d, int(w.causal), w.scale
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = fa.fa_backward_workspace_size(B, H, N, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    P = {n: t.data_ptr() for n, t in dict(q=q, k=k, v=v, do=do, o=o, lse=lse, dq=dq, dk=dk, dv=dv, ws=ws).items()}

    kernels = [
        ("fwd", lambda: fa.fa_forward(P["q"], P["k"], P["v"], P["o"], P["lse"], B, H, N, d, causal, scale, sp),
         _products(w, 2)),
    ]
    if w.backward:
        # The backward as fa_backward runs it at this size: dQ (computing
        # -delta of its queries on the way), then dK/dV.
        kernels += [
            ("bwd_dq", lambda: fa.fa_backward_dq_delta(P["q"], P["k"], P["v"], P["o"], P["lse"], P["do"], P["dq"],
                                                       B, H, N, d, causal, scale, P["ws"], ws_bytes, sp),
             _products(w, 1)),
            ("bwd_dkdv", lambda: fa.fa_backward_dkdv(P["q"], P["k"], P["v"], P["lse"], P["do"], P["dk"], P["dv"],
                                                     B, H, N, d, causal, scale, P["ws"], ws_bytes, sp),
             _products(w, 4)),
        ]
    step_flops = w.fwd_flops() + (w.bwd_flops() if w.backward else 0.0)

    def clock_warm(fn, seconds=CLOCK_WARMUP_S):
        """Run ``fn`` untimed, back to back, for about ``seconds``."""
        torch.cuda.synchronize()
        t_end = time.perf_counter() + seconds
        while time.perf_counter() < t_end:
            for _ in range(8):
                fn()
            torch.cuda.synchronize()

    def run_step(evs=None):
        for i, (name, fn, _) in enumerate(kernels):
            if evs is not None:
                evs[i][0].record(stream)
            st = fn()
            if st != 0:
                raise RuntimeError(f"{name}: {fa.fa_status_string(st)}")
            if evs is not None:
                evs[i][1].record(stream)

    # The GPU runs at lower clocks for roughly its first second of work, so
    # the step runs untimed for CLOCK_WARMUP_S before the W warm-up steps.
    clock_warm(run_step)
    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in kernels]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        run_step(evs[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    per_kernel_ms = {}
    for i, (name, _, _) in enumerate(kernels):
        per_kernel_ms[name] = float(np.mean([evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(args.steps)]))
    dom = max(kernels, key=lambda kk: per_kernel_ms[kk[0]])
    dom_ms = per_kernel_ms[dom[0]]
    achieved = dom[2] / (dom_ms * 1e-3) / 1e12

    kernel_table = {n: {"ms": round(per_kernel_ms[n], 4),
                        "tflops": round(f / (per_kernel_ms[n] * 1e-3) / 1e12, 1) if f else None}
                    for n, _, f in kernels}

    def time_launches(fn, n=10, warm=3):
        """Mean HIP-event time (ms) of ``fn`` launched ``n`` times on ``stream``,
        after a short untimed burst that brings the clocks back up."""
        clock_warm(fn, CLOCK_REWARM_S)
        for _ in range(warm):
            fn()
        evs_ = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b_ in evs_:
            a.record(stream)
            fn()
            b_.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b_) for a, b_ in evs_]))

    def checked(st, what):
        if st != 0:
            raise RuntimeError(f"{what}: {fa.fa_status_string(st)}")

    headline = []
    block_sparse = []
    if not args.no_headline:
        for name in HEADLINE_FWD:
            hw = fi.WORKLOADS[name]
            hx = fi.make_inputs(hw, with_grad=False)
            hq, hk, hv = (to_dev(hx[n]) for n in ("q", "k", "v"))
            ho = torch.empty_like(hq)
            hl = torch.empty((hw.B, hw.H, hw.N), dtype=torch.float32, device=dev)
            hms = time_launches(lambda: checked(fa.fa_forward(
                hq.data_ptr(), hk.data_ptr(), hv.data_ptr(), ho.data_ptr(), hl.data_ptr(),
                hw.B, hw.H, hw.N, hw.d, int(hw.causal), hw.scale, sp), "fwd"))
            tf = hw.fwd_flops() / (hms * 1e-3) / 1e12
            headline.append({"workload": name, "kernel": "fwd", "ms": round(hms, 4), "tflops": round(tf, 1),
                             "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
            del hq, hk, hv, ho, hl

        # Block-sparse forward: FLOPs counted on the visible (query, key)
        # pairs only; the dense forward at the same shape is timed beside it.
        for name, sw in fi.BLOCK_SPARSE_WORKLOADS.items():
            bw = sw.base
            bx = fi.make_inputs(bw, with_grad=False)
            bq, bk, bv = (to_dev(bx[n]) for n in ("q", "k", "v"))
            bm = torch.from_numpy(sw.mask()).to(dev)
            bo = torch.empty_like(bq)
            bl = torch.empty((bw.B, bw.H, bw.N), dtype=torch.float32, device=dev)
            args_ = (bq.data_ptr(), bk.data_ptr(), bv.data_ptr(), bo.data_ptr(), bl.data_ptr())
            bsw = fa.fa_block_sparse_workspace_size(bw.B, bw.H, bw.N, bw.d)
            bws = torch.empty(bsw, dtype=torch.uint8, device=dev)
            sms = time_launches(lambda: checked(fa.fa_forward_block_sparse(
                *args_, bm.data_ptr(), bw.B, bw.H, bw.N, bw.d, int(bw.causal), bw.scale, bws.data_ptr(), bsw, sp),
                "block_sparse"))
            sms_one = time_launches(lambda: checked(fa.fa_forward_block_sparse(
                *args_, bm.data_ptr(), bw.B, bw.H, bw.N, bw.d, int(bw.causal), bw.scale, 0, 0, sp),
                "block_sparse_one_pass"))
            dms = time_launches(lambda: checked(fa.fa_forward(
                *args_, bw.B, bw.H, bw.N, bw.d, int(bw.causal), bw.scale, sp), "fwd"))
            tf = sw.fwd_flops() / (sms * 1e-3) / 1e12
            block_sparse.append({"workload": name, "kernel": "fwd_block_sparse",
                                 "density": round(float(sw.mask().mean()), 4), "ms": round(sms, 4),
                                 "tflops_visible": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                                 "dense_ms": round(dms, 4), "speedup_vs_dense": round(dms / sms, 2),
                                 "one_pass_ms": round(sms_one, 4)})
            del bq, bk, bv, bm, bo, bl, bws

    # FP8 forward with incoherent processing on the headline shapes: the
    # quantisation pass and the attention are timed apart; the attention's
    # rate is set against the dense FP8 matrix-core peak.
    fp8 = []
    if not args.no_headline:
        signs = torch.from_numpy(fi.random_signs(0, 128)).to(dev)
        for name in HEADLINE_FWD:
            hw = fi.WORKLOADS[name]
            hx = fi.make_inputs(hw, with_grad=False)
            hq, hk, hv = (to_dev(hx[n]) for n in ("q", "k", "v"))
            ho = torch.empty_like(hq)
            hl = torch.empty((hw.B, hw.H, hw.N), dtype=torch.float32, device=dev)
            nb = fa.fa_fp8_buffer_size(hw.B, hw.H, hw.N, hw.d)
            hb = torch.empty(nb, dtype=torch.uint8, device=dev)
            pms = time_launches(lambda: checked(fa.fa_fp8_prepare(
                hq.data_ptr(), hk.data_ptr(), hv.data_ptr(), signs.data_ptr(), hw.B, hw.H, hw.N, hw.d,
                hb.data_ptr(), nb, sp), "fp8_prepare"))
            fms = time_launches(lambda: checked(fa.fa_forward_fp8_prepared(
                hb.data_ptr(), nb, ho.data_ptr(), hl.data_ptr(), hw.B, hw.H, hw.N, hw.d, int(hw.causal), hw.scale,
                1, sp), "fp8_forward"))
            tf = hw.fwd_flops() / (fms * 1e-3) / 1e12
            fp8.append({"workload": name, "kernel": "fwd_fp8", "prepare_ms": round(pms, 4), "ms": round(fms, 4),
                        "tflops": round(tf, 1), "peak_fp8": PEAK_FP8_TFLOPS,
                        "frac_of_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
                        "tflops_incl_prepare": round(hw.fwd_flops() / ((fms + pms) * 1e-3) / 1e12, 1)})
            del hq, hk, hv, ho, hl, hb

    # Decode (split-KV): HBM-bound, so reported against the HBM peak with the
    # algorithmic bytes (Q, K, V read once; O, LSE written once).
    decode = []
    if not args.no_headline:
        for name, dw in fi.DECODE_WORKLOADS.items():
            dx = fi.make_decode_inputs(dw)
            dq_, dk_, dv_ = (to_dev(dx[n]) for n in ("q", "k", "v"))
            do_ = torch.empty_like(dq_)
            dl_ = torch.empty((dw.B, dw.H, dw.Nq), dtype=torch.float32, device=dev)
            dws_bytes = fa.fa_decode_workspace_size(dw.B, dw.H, dw.Nq, dw.Nk, dw.d)
            dws = torch.empty(dws_bytes, dtype=torch.uint8, device=dev)
            dms = time_launches(lambda: checked(fa.fa_decode(
                dq_.data_ptr(), dk_.data_ptr(), dv_.data_ptr(), do_.data_ptr(), dl_.data_ptr(), dw.B, dw.H,
                dw.Nq, dw.Nk, dw.d, int(dw.causal), dw.scale, dws.data_ptr(), dws_bytes, sp), "decode"), n=20)
            gbs = dw.hbm_bytes() / (dms * 1e-3) / 1e9
            decode.append({"workload": name, "entry": "fa_decode", "ms": round(dms, 4),
                           "algorithmic_bytes": dw.hbm_bytes(), "GB_per_s": round(gbs, 1),
                           "hbm_peak_GB_per_s": PEAK_HBM_GBS, "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                           "tflops": round(dw.flops() / (dms * 1e-3) / 1e12, 2)})
            del dq_, dk_, dv_, do_, dl_, dws

    # Backward with a stored dS (fa_backward_stored_ds, O(N^2) workspace) on
    # the step's own tensors, beside fa_backward on the same tensors: both
    # whole backward passes (row-dot pre-pass included), same FLOP count.
    stored_ds = []
    if w.backward and not args.no_headline:
        sws_bytes = fa.fa_backward_stored_ds_workspace_size(B, H, N, d)
        if sws_bytes:
            sws = torch.empty(sws_bytes, dtype=torch.uint8, device=dev)
            args_b = (P["q"], P["k"], P["v"], P["o"], P["lse"], P["do"], P["dq"], P["dk"], P["dv"], B, H, N, d,
                      causal, scale)
            sms_ = time_launches(lambda: checked(fa.fa_backward_stored_ds(*args_b, sws.data_ptr(), sws_bytes, sp),
                                                 "backward_stored_ds"))
            bms_ = time_launches(lambda: checked(fa.fa_backward(*args_b, P["ws"], ws_bytes, sp), "backward"))
            bf = w.bwd_flops()
            stored_ds.append({"workload": w.name, "entry": "fa_backward_stored_ds", "ms": round(sms_, 4),
                              "tflops": round(bf / (sms_ * 1e-3) / 1e12, 1), "workspace_MiB": round(sws_bytes / 2**20),
                              "fa_backward_ms": round(bms_, 4),
                              "fa_backward_tflops": round(bf / (bms_ * 1e-3) / 1e12, 1)})
            del sws

    if args.copy_calibration:
        copy_calibration(dev, args.copy_calibration, 3)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)

    value = step_flops / (ms_per_step * 1e-3) / 1e12
    out = {
        "metric": "attention fwd/bwd TFLOPs/s (bf16, d=64/128, causal) + % of MFMA bf16 peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "causal": bool(causal),
                   "step": "forward+backward" if w.backward else "forward",
                   "step_gflop": round(step_flops / 1e9, 2), "parallelism": "single GPU",
                   "clock_warmup_s": CLOCK_WARMUP_S,
                   "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4)},
        "roofline": {"bound": "mfma", "kernel": dom[0], "achieved": round(achieved, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(dom[0], w.name),
                     "flop_per_launch": dom[2], "avg_ms": round(dom_ms, 4)},
        "kernels": kernel_table,
        "headline_forward": headline,
        "block_sparse_forward": block_sparse,
        "decode": decode,
        "fp8_forward": fp8,
        "backward_stored_ds": stored_ds,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
