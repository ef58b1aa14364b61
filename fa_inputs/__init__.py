"""Seeded synthetic inputs for exact attention, shared by the oracle side and the GPU side.

This module holds no attention arithmetic: it only draws random samples and
converts them between float32 and bfloat16 bit patterns.  Both the oracle and
the HIP path read the same arrays from here, so the two sides see the exact same
numbers while sharing no code that computes attention.

Recipe (one reading of the pages, which print no input distribution):
* ``numpy.random.default_rng(seed)`` (PCG64), ``standard_normal(shape,
  dtype=float32)`` with shape ``[B, H, N, d]`` in C order, drawn in the order
  Q, K, V, dO.
* an optional multiplier on the samples (the 4096-token d=128 workload uses
  0.5; a power of two, so it commutes exactly with bf16 rounding);
* bf16 tensors are the round-to-nearest-even bf16 of those float32 samples.

The shapes follow the FlashAttention-2 kernel benchmark described on the page
"FlashAttention-2を読む：長い文脈のアテンションをGPUで効率化する仕組み", section
「約2倍という数値の対象を確認する」 (sequence 512 to 16k, head dim 64 and 128,
causal and non-causal, batch x sequence fixed at 16k tokens).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "draw_f32",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "make_inputs",
    "random_block_mask",
    "local_global_block_mask",
    "visible_pairs",
    "BlockSparseWorkload",
    "BLOCK_SPARSE_WORKLOADS",
    "DecodeWorkload",
    "DECODE_WORKLOADS",
    "make_decode_inputs",
    "random_signs",
    "with_outliers",
    "with_channel_outliers",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as ``uint16``.  NaN stays a quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), r)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def draw_f32(seed: int, shape, count: int, mult: float = 1.0) -> list[np.ndarray]:
    """Draw ``count`` float32 arrays of ``shape`` from N(0,1) with PCG64(seed),
    each multiplied by ``mult``, in draw order."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        a = rng.standard_normal(tuple(shape), dtype=np.float32)
        if mult != 1.0:
            a = (a * np.float32(mult)).astype(np.float32)
        out.append(a)
    return out


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention problem: shapes, dtype, mask, input distribution."""

    name: str
    dtype: str  # "bf16" or "f32"
    B: int
    H: int
    N: int
    d: int
    causal: bool
    mult: float = 1.0
    seed: int = 0
    backward: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)

    def fwd_flops(self) -> float:
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def bwd_flops(self) -> float:
        f = 10.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f


# The five problem sizes: one fp32 case small enough for a pure-Python check,
# and four bf16 cases with 16k tokens and hidden size 2048.
WORKLOADS = {
    "f32_b1h2n128d64": Workload("f32_b1h2n128d64", "f32", 1, 2, 128, 64, False),
    "bf16_b16h32n1024d64": Workload("bf16_b16h32n1024d64", "bf16", 16, 32, 1024, 64, False),
    "bf16_b16h32n1024d64_causal": Workload("bf16_b16h32n1024d64_causal", "bf16", 16, 32, 1024, 64, True),
    "bf16_b4h16n4096d128_causal_x0.5": Workload(
        "bf16_b4h16n4096d128_causal_x0.5", "bf16", 4, 16, 4096, 128, True, mult=0.5),
    "bf16_b1h16n16384d128_causal": Workload("bf16_b1h16n16384d128_causal", "bf16", 1, 16, 16384, 128, True),
    "bf16_b1h16n16384d128": Workload("bf16_b1h16n16384d128", "bf16", 1, 16, 16384, 128, False),
    "bf16_b8h16n2048d128_causal_fwdbwd": Workload(
        "bf16_b8h16n2048d128_causal_fwdbwd", "bf16", 8, 16, 2048, 128, True, backward=True),
}

# Secondary problems: the d = 64 shape above with a backward pass as well
# (Q, K, V, dO drawn in that order), so that both head dimensions have a
# measured backward.
EXTRA_WORKLOADS = {
    "bf16_b16h32n1024d64_causal_fwdbwd": Workload(
        "bf16_b16h32n1024d64_causal_fwdbwd", "bf16", 16, 32, 1024, 64, True, backward=True),
}
__all__.append("EXTRA_WORKLOADS")


def make_inputs(w: Workload, with_grad: bool | None = None):
    """Inputs of a workload as numpy arrays.

    Returns a dict with ``q, k, v`` (and ``do`` when a backward is wanted):
    for bf16 workloads each entry is a ``uint16`` array of bf16 bits, for f32
    workloads a float32 array.  ``exact_f64(arr)`` gives the exact values.
    """
    if with_grad is None:
        with_grad = w.backward
    names = ["q", "k", "v"] + (["do"] if with_grad else [])
    arrs = draw_f32(w.seed, w.shape, len(names), w.mult)
    out = {}
    for n, a in zip(names, arrs):
        out[n] = f32_to_bf16_bits(a) if w.dtype == "bf16" else a
    return out


def exact_f64(a: np.ndarray) -> np.ndarray:
    """The exact value of an input array (bf16 bits or float32) as float64."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


__all__.append("exact_f64")


# --- block masks (block-sparse attention) ----------------------------------

def random_block_mask(seed: int, nb: int, density: float) -> np.ndarray:
    """[nb, nb] uint8 mask, each block visible with probability ``density``
    (PCG64 seeded with (seed, 1), uniform draws in C order)."""
    rng = np.random.default_rng([seed, 1])
    return (rng.random((nb, nb)) < density).astype(np.uint8)


def local_global_block_mask(nb: int, window: int, n_global: int) -> np.ndarray:
    """[nb, nb] uint8 mask of a local band plus global blocks: query block a
    sees key block b when |a - b| <= window, or b < n_global (global keys), or
    a < n_global (global queries see everything)."""
    a = np.arange(nb)[:, None]
    b = np.arange(nb)[None, :]
    vis = (np.abs(a - b) <= window) | (b < n_global) | (a < n_global)
    return vis.astype(np.uint8)


def visible_pairs(mask: np.ndarray, n: int, block: int, causal: bool) -> int:
    """Number of (query, key) pairs a block mask leaves visible for sequence
    length ``n`` (counted block by block; ragged last block clipped)."""
    nb = mask.shape[0]
    sizes = np.minimum(block, n - block * np.arange(nb))
    total = 0
    for a in range(nb):
        for b in range(nb):
            if not mask[a, b]:
                continue
            if not causal or b < a:
                total += int(sizes[a]) * int(sizes[b])
            elif b == a:
                total += int(sizes[a]) * (int(sizes[a]) + 1) // 2
    return total


@dataclasses.dataclass(frozen=True)
class BlockSparseWorkload:
    """A block-sparse problem: a dense workload's shapes and inputs plus a
    local-band + global-blocks mask of 128 x 128 blocks."""

    base: Workload
    window: int
    n_global: int
    block: int = 128

    @property
    def name(self) -> str:
        return f"{self.base.name}_local{self.window}_global{self.n_global}"

    def mask(self) -> np.ndarray:
        nb = -(-self.base.N // self.block)
        return local_global_block_mask(nb, self.window, self.n_global)

    def fwd_flops(self) -> float:
        w = self.base
        return 4.0 * w.B * w.H * w.d * visible_pairs(self.mask(), w.N, self.block, w.causal)


# 16k tokens (B x N), hidden size 2048, d = 128; 64 x 64 blocks of which a
# band of 5 plus one global row and column are visible (about 11%).
BLOCK_SPARSE_WORKLOADS = {
    "bf16_b2h16n8192d128_local2_global1": BlockSparseWorkload(
        Workload("bf16_b2h16n8192d128", "bf16", 2, 16, 8192, 128, False), window=2, n_global=1),
}



# --- decode (few new queries over a long key/value cache) -------------------

@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """Nq new queries per (batch, head) over Nk cached keys and values."""

    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    causal: bool = True
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def visible_pairs(self) -> int:
        """(query, key) pairs per (batch, head) the mask leaves visible."""
        if not self.causal:
            return self.Nq * self.Nk
        return sum(max(0, min(self.Nk, self.Nk - self.Nq + i + 1)) for i in range(self.Nq))

    def flops(self) -> float:
        return 4.0 * self.B * self.H * self.d * self.visible_pairs()

    def hbm_bytes(self) -> int:
        """Bytes the pass must move at least: Q, K, V read once; O, LSE written."""
        bh = self.B * self.H
        return bh * (2 * self.Nq * self.d * 2 + 2 * self.Nk * self.d * 2 + self.Nq * 4)


def make_decode_inputs(w: DecodeWorkload):
    """bf16 bits of q [B,H,Nq,d], k and v [B,H,Nk,d]: PCG64(seed) standard
    normals drawn in the order q, k, v, rounded to nearest even."""
    rng = np.random.default_rng(w.seed)
    out = {}
    for n, nn in (("q", w.Nq), ("k", w.Nk), ("v", w.Nk)):
        a = rng.standard_normal((w.B, w.H, nn, w.d), dtype=np.float32)
        out[n] = f32_to_bf16_bits(a)
    return out


# A decode step of a hidden-size-2048 model (16 heads of 128) at batch 8 with
# a 16k-token cache: 1.07 GB of keys and values per step.
DECODE_WORKLOADS = {
    "bf16_b8h16q1k16384d128_decode": DecodeWorkload("bf16_b8h16q1k16384d128_decode", 8, 16, 1, 16384, 128),
}


# --- FP8 forward ----------------------------------------------------------------

def random_signs(seed: int, d: int) -> np.ndarray:
    """Length-d float32 vector of random +-1 (PCG64 seeded with (seed, 2)):
    the random diagonal of the incoherent-processing rotation."""
    rng = np.random.default_rng([seed, 2])
    return (rng.integers(0, 2, size=d) * 2 - 1).astype(np.float32)


def with_outliers(x: np.ndarray, seed: int, frac: float = 0.001, factor: float = 10.0) -> np.ndarray:
    """Copy of float32 samples with a fraction ``frac`` of the entries (chosen
    by PCG64 seeded with (seed, 3)) multiplied by ``factor``: the large-entry
    outliers that incoherent processing is meant to spread."""
    rng = np.random.default_rng([seed, 3])
    out = np.array(x, dtype=np.float32, copy=True)
    hit = rng.random(out.shape) < frac
    out[hit] *= np.float32(factor)
    return out


def with_channel_outliers(arrays, seed: int, n_channels: int = 2, factor: float = 10.0) -> list[np.ndarray]:
    """Copies of float32 samples [..., d] in which the same ``n_channels``
    feature coordinates (chosen by PCG64 seeded with (seed, 4)) are
    multiplied by ``factor`` in every array: outlier feature channels shared
    by Q and K, the large coordinates that incoherent processing spreads."""
    d = arrays[0].shape[-1]
    rng = np.random.default_rng([seed, 4])
    ch = rng.choice(d, n_channels, replace=False)
    out = []
    for a in arrays:
        b = np.array(a, dtype=np.float32, copy=True)
        b[..., ch] *= np.float32(factor)
        out.append(b)
    return out
