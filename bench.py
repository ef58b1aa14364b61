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
the MI355X dense bf16 matrix-core peak.  Beside it, the vendor bf16 GEMM
(torch.matmul on 8192-square operands) is timed in the same run: under
sustained matrix-core load the chip does not hold its 2.4 GHz clock, and
that GEMM shows what dense bf16 work reaches at the clock it does hold.

Timing series (page "Flash Attention 2で打破するローカルLLMの「メモリの壁」：IO最適化の
実践的エンジニアリング", section 「推論レイテンシとスループットの測定方法」: CUDA events
around repeated launches after warm-up): the step and every secondary
workload are also launched SERIES_N times, each launch bracketed by its own
pair of HIP events, and reported as the median and the minimum; a second
series reads a 512 MiB scratch buffer before every launch, which evicts the
L2 caches and the MALL, so that no input starts out on chip.

The single-pass backward (fa_backward_atomic: dQ added with float32 atomics
in the dK/dV pass) is timed beside fa_backward on the step's inputs
(``series.fa_backward_atomic``); it is not part of the step.

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
HEADLINE_FWD = ["bf16_b16h32n1024d64", "bf16_b16h32n1024d64_causal", "bf16_b4h16n4096d128_causal_x0.5",
                "bf16_b1h16n16384d128_causal", "bf16_b1h16n16384d128"]
FP8_FWD = ["bf16_b4h16n4096d128_causal_x0.5", "bf16_b1h16n16384d128_causal", "bf16_b1h16n16384d128"]
EXTRA_BWD = ["bf16_b16h32n1024d64_causal_fwdbwd"]
SERIES_N = 20          # launches per timing series
FLUSH_MIB = 512        # scratch read before each launch of the flushed series
GEMM_REF_N = 8192      # square bf16 GEMM timed as the dense matrix-core reference


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


def _profile_fields(name: str):
    """Fields of a committed counter summary profiles/<name>.txt, or None if
    there is none or it was taken on other sources."""
    path = os.path.join(ROOT, "profiles", name + ".txt")
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
    return fields


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    FETCH_SIZE / WRITE_SIZE summary, or None."""
    fields = _profile_fields(f"traffic_{kernel}_{workload}")
    try:
        return float(fields["traffic_bytes_per_launch"]) if fields else None
    except (KeyError, ValueError):
        return None


def measured_mfma(kernel: str, workload: str):
    """Matrix-core counters of `kernel` on `workload` from the committed
    summary (SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES against
    SQ_BUSY_CU_CYCLES, GRBM_GUI_ACTIVE), or None."""
    fields = _profile_fields(f"mfma_{kernel}_{workload}")
    if not fields:
        return None
    out = {}
    for key in ("counter_flop_per_launch", "mfma_busy_frac", "gpu_clock_ghz", "kernel_us"):
        try:
            out[key] = float(fields[key])
        except (KeyError, ValueError):
            pass
    return out or None


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
    pools = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in pools] or [1])
    blas = ", ".join(sorted({f"{i.get('internal_api', '?')} {i.get('version', '')}".strip() for i in pools
                             if i.get("user_api") == "blas"})) or "unknown"
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": per_head * done / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} of {w.B * w.H} (batch, head) pairs, forward{'+backward' if w.backward else ''}, "
                  f"fp64 numpy, {dt:.1f} s, host nproc {os.cpu_count()}",
        "cpu_model": cpu_model,
        "blas": blas,
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
    ap.add_argument("--progress", action="store_true", help="print a line to stderr as each part finishes")
    args = ap.parse_args()

    def note(msg):
        if args.progress:
            print(f"bench: {msg}", file=sys.stderr, flush=True)
    if args.print_digest:
        print(kernel_source_digest())
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs the attention kernels on a single "
              "MI355X and has no multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import exact_attention_18_amd as fa
    import fa_inputs as fi

    fa._lib.load()  # raises if the HIP library is missing
    w = fi.WORKLOADS.get(args.workload) or fi.EXTRA_WORKLOADS[args.workload]
    if w.dtype != "bf16":
        raise SystemExit("bench.py times the bf16 path")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    def checked(st, what):
        if st != 0:
            raise RuntimeError(f"{what}: {fa.fa_status_string(st)}")

    def step_kernels(wl, with_backward):
        """Device tensors of a workload and its kernels as the library runs
        them: forward, then (large grids) dQ computing -delta, then dK/dV."""
        x = fi.make_inputs(wl, with_grad=with_backward)
        t = {n: to_dev(a) for n, a in x.items()}
        B_, H_, N_, d_ = wl.B, wl.H, wl.N, wl.d
        c_, s_ = int(wl.causal), wl.scale
        t["o"] = torch.empty_like(t["q"])
        t["lse"] = torch.empty((B_, H_, N_), dtype=torch.float32, device=dev)
        ks = [("fwd", lambda: fa.fa_forward(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(),
                                            t["o"].data_ptr(), t["lse"].data_ptr(), B_, H_, N_, d_, c_, s_, sp),
               _products(wl, 2))]
        if with_backward:
            for n in ("dq", "dk", "dv"):
                t[n] = torch.empty_like(t["q"])
            nb = fa.fa_backward_workspace_size(B_, H_, N_, d_)
            t["ws"] = torch.empty(nb, dtype=torch.uint8, device=dev)
            P_ = {n: v.data_ptr() for n, v in t.items()}
            ks += [
                ("bwd_dq", lambda: fa.fa_backward_dq_delta(P_["q"], P_["k"], P_["v"], P_["o"], P_["lse"], P_["do"],
                                                           P_["dq"], B_, H_, N_, d_, c_, s_, P_["ws"], nb, sp),
                 _products(wl, 1)),
                ("bwd_dkdv", lambda: fa.fa_backward_dkdv(P_["q"], P_["k"], P_["v"], P_["lse"], P_["do"], P_["dk"],
                                                         P_["dv"], B_, H_, N_, d_, c_, s_, P_["ws"], nb, sp),
                 _products(wl, 4)),
            ]
        return t, ks

    tensors, kernels = step_kernels(w, w.backward)
    B, H, N, d, causal, scale = w.B, w.H, w.N, w.d, int(w.causal), w.scale
    step_flops = w.fwd_flops() + (w.bwd_flops() if w.backward else 0.0)

    def clock_warm(fn, seconds=CLOCK_WARMUP_S):
        """Run ``fn`` untimed, back to back, for about ``seconds``."""
        torch.cuda.synchronize()
        t_end = time.perf_counter() + seconds
        while time.perf_counter() < t_end:
            for _ in range(8):
                fn()
            torch.cuda.synchronize()

    def run_kernels(ks, evs=None):
        for i, (name, fn, _) in enumerate(ks):
            if evs is not None:
                evs[i][0].record(stream)
            checked(fn(), name)
            if evs is not None:
                evs[i][1].record(stream)

    def run_step(evs=None):
        run_kernels(kernels, evs)

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

    # The flush reads the scratch buffer (a reduction into one value): a read
    # evicts L2 and MALL lines as a write does, but leaves no dirty lines
    # whose write-back would fall into the timed launch (writing the buffer
    # instead made the decode launch after it 25% slower).
    flush_buf = torch.zeros(FLUSH_MIB * 2**20 // 4, dtype=torch.float32, device=dev)
    flush_out = torch.empty((), dtype=torch.float32, device=dev)

    def flush():
        torch.sum(flush_buf, dim=0, out=flush_out)

    def series(fn, flushed, n=SERIES_N, warm=3):
        """HIP-event times (ms) of ``fn`` launched ``n`` times on ``stream``,
        each launch bracketed by its own events (after a short untimed burst
        that brings the clocks back up); ``flushed`` reads the scratch buffer
        before every launch.  Returns median, minimum and mean."""
        clock_warm(fn, CLOCK_REWARM_S)
        for _ in range(warm):
            fn()
        evs_ = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b_ in evs_:
            if flushed:
                flush()
            a.record(stream)
            fn()
            b_.record(stream)
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b_) for a, b_ in evs_])
        return {"median_ms": round(float(np.median(t)), 4), "min_ms": round(float(t.min()), 4),
                "mean_ms": round(float(t.mean()), 4), "n": n}

    def both_series(fn, flops):
        out = {}
        for key, fl in (("warm", False), ("flushed", True)):
            sr = series(fn, fl)
            sr["tflops_median"] = round(flops / (sr["median_ms"] * 1e-3) / 1e12, 1)
            sr["frac_of_peak_median"] = round(sr["tflops_median"] / PEAK_BF16_TFLOPS, 4)
            out[key] = sr
        return out

    note(f"timed steps done ({ms_per_step:.4f} ms per step)")
    step_series = both_series(run_step, step_flops)
    note("step series done")
    backward_series = None
    atomic_series = None
    if w.backward:
        backward_series = both_series(lambda: checked(fa.fa_backward(
            *(tensors[n].data_ptr() for n in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv")),
            B, H, N, d, causal, scale, tensors["ws"].data_ptr(), tensors["ws"].numel(), sp), "backward"),
            w.bwd_flops())
        # The single-pass form (dQ by float32 atomics in the dK/dV pass),
        # timed on the same inputs; FLOPs counted as for fa_backward.
        nat = fa.fa_backward_atomic_workspace_size(B, H, N, d)
        ws_at = torch.empty(nat, dtype=torch.uint8, device=dev)
        atomic_series = both_series(lambda: checked(fa.fa_backward_atomic(
            *(tensors[n].data_ptr() for n in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv")),
            B, H, N, d, causal, scale, ws_at.data_ptr(), nat, sp), "backward_atomic"), w.bwd_flops())
        del ws_at

    headline = []
    extra_backward = []
    block_sparse = []
    if not args.no_headline:
        for name in HEADLINE_FWD:
            hw = fi.WORKLOADS[name]
            ht, hk = step_kernels(hw, False)
            sr = both_series(lambda: checked(hk[0][1](), "fwd"), hw.fwd_flops())
            tf = sr["warm"]["tflops_median"]
            note(f"forward {name} done")
            headline.append({"workload": name, "kernel": "fwd", "ms": sr["warm"]["median_ms"], "tflops": tf,
                             "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4), "series": sr})
            del ht, hk

        # d = 64 forward + backward: the step's kernels at that shape, and
        # fa_backward as a whole.
        for name in EXTRA_BWD:
            ew = fi.EXTRA_WORKLOADS[name]
            et, ek = step_kernels(ew, True)
            run_kernels(ek)
            torch.cuda.synchronize()
            ebw = both_series(lambda: checked(fa.fa_backward(
                *(et[n].data_ptr() for n in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv")),
                ew.B, ew.H, ew.N, ew.d, int(ew.causal), ew.scale, et["ws"].data_ptr(), et["ws"].numel(), sp),
                "backward"), ew.bwd_flops())
            estep = both_series(lambda: run_kernels(ek), ew.fwd_flops() + ew.bwd_flops())
            note(f"backward {name} done")
            extra_backward.append({"workload": name, "fa_backward": ebw, "step": estep})
            del et, ek

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
            sms = series(lambda: checked(fa.fa_forward_block_sparse(
                *args_, bm.data_ptr(), bw.B, bw.H, bw.N, bw.d, int(bw.causal), bw.scale, bws.data_ptr(), bsw, sp),
                "block_sparse"), False)["median_ms"]
            sms_one = series(lambda: checked(fa.fa_forward_block_sparse(
                *args_, bm.data_ptr(), bw.B, bw.H, bw.N, bw.d, int(bw.causal), bw.scale, 0, 0, sp),
                "block_sparse_one_pass"), False)["median_ms"]
            dms = series(lambda: checked(fa.fa_forward(
                *args_, bw.B, bw.H, bw.N, bw.d, int(bw.causal), bw.scale, sp), "fwd"), False)["median_ms"]
            tf = sw.fwd_flops() / (sms * 1e-3) / 1e12
            note(f"block-sparse {name} done")
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
        for name in FP8_FWD:
            hw = fi.WORKLOADS[name]
            hx = fi.make_inputs(hw, with_grad=False)
            hq, hk, hv = (to_dev(hx[n]) for n in ("q", "k", "v"))
            ho = torch.empty_like(hq)
            hl = torch.empty((hw.B, hw.H, hw.N), dtype=torch.float32, device=dev)
            nb = fa.fa_fp8_buffer_size(hw.B, hw.H, hw.N, hw.d)
            hb = torch.empty(nb, dtype=torch.uint8, device=dev)
            pms = series(lambda: checked(fa.fa_fp8_prepare(
                hq.data_ptr(), hk.data_ptr(), hv.data_ptr(), signs.data_ptr(), hw.B, hw.H, hw.N, hw.d,
                hb.data_ptr(), nb, sp), "fp8_prepare"), False)["median_ms"]
            fms = series(lambda: checked(fa.fa_forward_fp8_prepared(
                hb.data_ptr(), nb, ho.data_ptr(), hl.data_ptr(), hw.B, hw.H, hw.N, hw.d, int(hw.causal), hw.scale,
                1, sp), "fp8_forward"), False)["median_ms"]
            tf = hw.fwd_flops() / (fms * 1e-3) / 1e12
            note(f"FP8 forward {name} done")
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
            dsr = series(lambda: checked(fa.fa_decode(
                dq_.data_ptr(), dk_.data_ptr(), dv_.data_ptr(), do_.data_ptr(), dl_.data_ptr(), dw.B, dw.H,
                dw.Nq, dw.Nk, dw.d, int(dw.causal), dw.scale, dws.data_ptr(), dws_bytes, sp), "decode"), True)
            dms = dsr["median_ms"]
            gbs = dw.hbm_bytes() / (dms * 1e-3) / 1e9
            note(f"decode {name} done")
            decode.append({"workload": name, "entry": "fa_decode", "ms": round(dms, 4), "flushed": True,
                           "algorithmic_bytes": dw.hbm_bytes(), "GB_per_s": round(gbs, 1),
                           "hbm_peak_GB_per_s": PEAK_HBM_GBS, "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                           "tflops": round(dw.flops() / (dms * 1e-3) / 1e12, 2)})
            del dq_, dk_, dv_, do_, dl_, dws

    # Reference for what dense bf16 matrix-core work reaches on this GPU at
    # the clocks it holds under load: the vendor GEMM (torch.matmul, i.e.
    # hipBLASLt) on square 8192 operands, timed the same way.
    ga_ = torch.randn(GEMM_REF_N, GEMM_REF_N, device=dev, dtype=torch.bfloat16)
    gb_ = torch.randn(GEMM_REF_N, GEMM_REF_N, device=dev, dtype=torch.bfloat16)
    gemm_ms = series(lambda: torch.matmul(ga_, gb_), False)["median_ms"]
    gemm_tf = 2.0 * GEMM_REF_N ** 3 / (gemm_ms * 1e-3) / 1e12
    note("vendor bf16 GEMM done")
    gemm_ref = {"op": f"torch.matmul bf16 {GEMM_REF_N}x{GEMM_REF_N}x{GEMM_REF_N} (hipBLASLt)",
                "median_ms": round(gemm_ms, 4), "tflops": round(gemm_tf, 1),
                "frac_of_peak": round(gemm_tf / PEAK_BF16_TFLOPS, 4)}
    del ga_, gb_
    # The same for FP8 (OCP E4M3, the format of the FP8 path), through
    # torch._scaled_mm with unit scales; left out where this torch build has
    # no such kernel.
    gemm_ref_fp8 = None
    try:
        fa_ = torch.randn(GEMM_REF_N, GEMM_REF_N, device=dev).to(torch.float8_e4m3fn)
        fb_ = torch.randn(GEMM_REF_N, GEMM_REF_N, device=dev).to(torch.float8_e4m3fn).t()
        one_ = torch.ones((), device=dev)
        f8ms = series(lambda: torch._scaled_mm(fa_, fb_, scale_a=one_, scale_b=one_, out_dtype=torch.bfloat16),
                      False)["median_ms"]
        f8tf = 2.0 * GEMM_REF_N ** 3 / (f8ms * 1e-3) / 1e12
        gemm_ref_fp8 = {"op": f"torch._scaled_mm fp8 e4m3 {GEMM_REF_N}x{GEMM_REF_N}x{GEMM_REF_N} (hipBLASLt)",
                        "median_ms": round(f8ms, 4), "tflops": round(f8tf, 1),
                        "frac_of_peak": round(f8tf / PEAK_FP8_TFLOPS, 4)}
        del fa_, fb_
    except (RuntimeError, AttributeError, TypeError):
        pass
    if gemm_ref_fp8:
        for e in fp8:
            e["frac_of_library_fp8_gemm"] = round(e["tflops"] / gemm_ref_fp8["tflops"], 4)
    del flush_buf
    if args.copy_calibration:
        copy_calibration(dev, args.copy_calibration, 3)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)

    value = step_flops / (ms_per_step * 1e-3) / 1e12
    mfma = measured_mfma(dom[0], w.name)
    roofline = {"bound": "mfma", "kernel": dom[0], "achieved": round(achieved, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(dom[0], w.name),
                "flop_per_launch": dom[2], "avg_ms": round(dom_ms, 4),
                "library_gemm_tflops": gemm_ref["tflops"],
                "frac_of_library_gemm": round(achieved / gemm_ref["tflops"], 4)}
    if mfma:
        # the matrix-core work the counters saw (recomputed products
        # included) over this run's launch time, and the busy fraction
        if "counter_flop_per_launch" in mfma:
            roofline["counter_tflops"] = round(mfma["counter_flop_per_launch"] / (dom_ms * 1e-3) / 1e12, 1)
            roofline["counter_frac"] = round(roofline["counter_tflops"] / PEAK_BF16_TFLOPS, 4)
        if "mfma_busy_frac" in mfma:
            roofline["mfma_busy_frac"] = mfma["mfma_busy_frac"]
        if "gpu_clock_ghz" in mfma:
            roofline["gpu_clock_ghz"] = mfma["gpu_clock_ghz"]
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
        "roofline": roofline,
        "kernels": kernel_table,
        "series": {"launches": SERIES_N, "flush_MiB": FLUSH_MIB, "step": step_series,
                   "fa_backward": backward_series, "fa_backward_atomic": atomic_series},
        "gemm_reference": gemm_ref,
        "gemm_reference_fp8": gemm_ref_fp8,
        "headline_forward": headline,
        "backward_d64": extra_backward,
        "block_sparse_forward": block_sparse,
        "decode": decode,
        "fp8_forward": fp8,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)

if __name__ == "__main__":
    main()
