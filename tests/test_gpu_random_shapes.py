"""Seeded random shapes through the forward, backward, block-sparse, decode
and FP8 entry points, each against the fp64 oracle: O max-abs 2e-2, LSE
1e-3, the FP8 path within its P-rounding bound.

The shapes are drawn once from fixed PCG64 seeds, so the set is the same on
every run. They mix ragged lengths around the tile sizes (64 and 128) with
longer ones, both head dimensions, causal and not, and batch x heads from 1
to 12.  The forward/backward case also draws the softmax scale (0.05 to 0.2,
up to 2.3 times 1/sqrt(128)), which makes some gradients larger than 1;
the gradient bar is 2e-2 times max(1, their largest magnitude), because the
bf16 rounding of the score gradient ahead of its two products is relative.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.gpu_util import dev, host64, max_abs, random_inputs, storage_floor

pytestmark = pytest.mark.gpu

TOL, TOL_LSE = 2e-2, 1e-3


def _shapes(count, seed):
    r = np.random.default_rng(seed)
    out = []
    for i in range(count):
        B, H = int(r.integers(1, 4)), int(r.integers(1, 5))
        N = int(r.choice([r.integers(1, 200), r.integers(200, 900), 64 * r.integers(1, 12) + r.integers(-1, 2)]))
        out.append((i, B, H, max(1, N), int(r.choice([64, 128])), bool(r.integers(0, 2))))
    return out


@pytest.fixture(scope="module")
def fa():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_18_amd as fa

    fa._lib.load()
    return fa


@pytest.mark.parametrize("i,B,H,N,d,causal", _shapes(24, 2024))
def test_random_forward_backward(fa, i, B, H, N, d, causal):
    import torch

    q, k, v, do = random_inputs(1000 + i, (B, H, N, d), "bf16", 4)
    scale = float(np.random.default_rng(i).uniform(0.05, 0.2))   # not only 1/sqrt(d)
    tq, tk, tv, tdo = dev(q), dev(k), dev(v), dev(do)
    o, lse = fa.forward(tq, tk, tv, causal=causal, scale=scale)
    dq, dk, dv = fa.backward(tq, tk, tv, o, lse, tdo, causal=causal, scale=scale)
    torch.cuda.synchronize()
    qf, kf, vf, gf = (fi.exact_f64(a) for a in (q, k, v, do))
    ro, rl = oracle.attention_forward(qf, kf, vf, causal, scale)
    assert max_abs(host64(o), ro) <= TOL
    assert max_abs(host64(lse), rl) <= TOL_LSE
    for name, x, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), oracle.attention_backward(qf, kf, vf, gf, causal, scale)):
        e, bar = max_abs(host64(x), r), TOL * max(1.0, float(np.abs(r).max()))
        assert e <= bar, f"{name} {e:.3g} > {bar:.3g} (floor {storage_floor(r):.3g})"


@pytest.mark.parametrize("i,B,H,N,d,causal", _shapes(12, 7))
def test_random_block_sparse(fa, i, B, H, N, d, causal):
    import torch

    nb = -(-N // 128)
    mask = fi.random_block_mask(3000 + i, nb, float(np.random.default_rng(i).uniform(0.1, 0.9)))
    q, k, v = random_inputs(2000 + i, (B, H, N, d), "bf16", 3)
    tm = torch.from_numpy(mask).to("cuda:0")
    ro, rl = oracle.attention_forward_block_sparse(fi.exact_f64(q), fi.exact_f64(k), fi.exact_f64(v), mask, 128,
                                                   causal, 1 / math.sqrt(d))
    for balance in (False, True):
        o, lse = fa.forward_block_sparse(dev(q), dev(k), dev(v), tm, causal=causal, balance=balance)
        torch.cuda.synchronize()
        oh, lh = host64(o), host64(lse)
        live = np.isfinite(rl)
        assert np.all(np.isfinite(oh)) and max_abs(oh, ro) <= TOL
        assert np.array_equal(np.isneginf(lh), ~live)
        if live.any():
            assert np.abs(lh[live] - rl[live]).max() <= TOL_LSE


@pytest.mark.parametrize("i,B,H,N,d,causal", _shapes(12, 11))
def test_random_decode(fa, i, B, H, N, d, causal):
    import torch

    nq = int(np.random.default_rng(i).integers(1, 9))
    w = fi.DecodeWorkload("t", B, H, nq, N, d, causal, 4000 + i)
    x = fi.make_decode_inputs(w)
    o, lse = fa.decode(dev(x["q"]), dev(x["k"]), dev(x["v"]), causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward_kv(fi.exact_f64(x["q"]), fi.exact_f64(x["k"]), fi.exact_f64(x["v"]), causal,
                                         w.scale)
    oh, lh = host64(o), host64(lse)
    live = np.isfinite(rl)
    assert np.all(np.isfinite(oh)) and max_abs(oh, ro) <= TOL
    assert np.array_equal(np.isneginf(lh), ~live)
    if live.any():
        assert np.abs(lh[live] - rl[live]).max() <= TOL_LSE


@pytest.mark.parametrize("i,B,H,N,d,causal", [s for s in _shapes(16, 13) if s[4] == 128])
def test_random_fp8(fa, i, B, H, N, d, causal):
    """FP8 forward (d = 128 only) with and without the rotation, within the
    P-rounding bound of the oracle's FP8 attention."""
    import torch

    from oracle import fp8 as ofp8

    q, k, v = random_inputs(5000 + i, (B, H, N, d), "bf16", 3)
    for rotate in (False, True):
        sg = fi.random_signs(i, d) if rotate else None
        o, lse = fa.forward_fp8(dev(q), dev(k), dev(v), None if sg is None else torch.from_numpy(sg).to("cuda:0"),
                                causal=causal)
        torch.cuda.synchronize()
        ro, rl, parts = ofp8.attention_forward_fp8(fi.exact_f64(q), fi.exact_f64(k), fi.exact_f64(v), sg, causal,
                                                   1 / math.sqrt(d), return_parts=True)
        tol = 2.0 ** -4 * parts["p_error_bound"] + 2.0 ** -8 * np.abs(ro) + 1e-4
        oh = host64(o)
        assert np.all(np.isfinite(oh)) and np.all(np.abs(oh - ro) <= tol)
        assert np.abs(host64(lse) - rl).max() <= TOL_LSE
