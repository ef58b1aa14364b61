"""Helpers for the GPU parity tests: move the seeded inputs to the device,
run the library through its binding, and compare with the oracle."""
from __future__ import annotations

import numpy as np

import fa_inputs as fi


def dev(a: np.ndarray):
    """numpy input (bf16 bits as uint16, or float32) -> torch tensor on cuda:0."""
    import torch

    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to("cuda:0")


def host64(t) -> np.ndarray:
    """torch tensor (bf16 or float32, any device) -> float64 numpy."""
    import torch

    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def max_abs(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    if not (np.all(np.isfinite(a))):
        return float("inf")
    return float(np.max(np.abs(a - b)))


def storage_floor(ref: np.ndarray) -> float:
    """Error that rounding the exact result to bf16 alone would leave."""
    r32 = ref.astype(np.float32)
    return max_abs(fi.bf16_bits_to_f32(fi.f32_to_bf16_bits(r32)).astype(np.float64), ref)


def random_inputs(seed, shape, dtype, count, mult=1.0):
    arrs = fi.draw_f32(seed, shape, count, mult)
    if dtype == "bf16":
        return [fi.f32_to_bf16_bits(a) for a in arrs]
    return arrs


def parallel(fn, tasks):
    """Run fn over tasks on the host cores (numpy releases the GIL inside
    its loops and products), with one BLAS thread per worker."""
    import concurrent.futures as cf
    import os

    from threadpoolctl import threadpool_limits

    workers = max(1, min(16, os.cpu_count() or 1))
    with threadpool_limits(limits=1):
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(fn, tasks))


def report(name, what, err, floor, n):
    print(f"PARITY {name} {what}: max_abs_err {err:.5g} storage_floor {floor:.5g} elements {n}", flush=True)
