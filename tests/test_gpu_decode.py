"""GPU parity of the decode (split-KV) forward against the fp64 oracle.

Tolerances as for the forward: O max-abs 2e-2 (bf16 output), LSE 1e-3;
queries that see no key must give O = 0 and LSE = -inf exactly.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.gpu_util import dev, host64, max_abs

pytestmark = pytest.mark.gpu

TOL_O = 2e-2
TOL_LSE = 1e-3


@pytest.fixture(scope="module")
def fa():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_18_amd as fa

    fa._lib.load()
    return fa


def _compare(o, lse, ro, rl):
    oh, lh = host64(o), host64(lse)
    assert np.all(np.isfinite(oh)), "non-finite O"
    eo = max_abs(oh, ro)
    assert eo <= TOL_O, f"O error {eo:.3g}"
    dead = ~np.isfinite(rl)
    assert np.array_equal(np.isneginf(lh), dead), "LSE -inf rows differ"
    assert np.all(oh[dead] == 0.0)
    el = float(np.max(np.abs(lh[~dead] - rl[~dead]))) if (~dead).any() else 0.0
    assert el <= TOL_LSE, f"LSE error {el:.3g}"


def _check(fa, B, H, Nq, Nk, d, causal, seed):
    import torch

    w = fi.DecodeWorkload("t", B, H, Nq, Nk, d, causal, seed)
    x = fi.make_decode_inputs(w)
    tq, tk, tv = dev(x["q"]), dev(x["k"]), dev(x["v"])
    need = fa.fa_decode_workspace_size(B, H, Nq, Nk, d)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=tq.device)  # garbage on entry
    o, lse = fa.decode(tq, tk, tv, causal=causal, scale=w.scale, workspace=ws)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward_kv(fi.exact_f64(x["q"]), fi.exact_f64(x["k"]), fi.exact_f64(x["v"]),
                                         causal, w.scale)
    _compare(o, lse, ro, rl)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Nk", [1, 7, 64, 65, 300, 4097])
@pytest.mark.parametrize("Nq", [1, 3, 4, 8])
def test_decode_small(fa, Nq, Nk, d, causal):
    _check(fa, 2, 3, Nq, Nk, d, causal, seed=Nq * 1000 + Nk)


@pytest.mark.parametrize("Nq", [2, 5, 8])
def test_decode_more_queries_than_keys(fa, Nq):
    _check(fa, 1, 2, Nq, Nq - 1 if Nq > 2 else 1, 128, True, seed=Nq)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_many_chunks(fa, d):
    """B*H*Nk large enough for chunks longer than 64 keys and hundreds of
    chunks per (batch, head): the merge over many partials."""
    _check(fa, 2, 2, 2, 40000, d, True, seed=77)


def test_decode_equals_last_rows_of_forward(fa):
    """Decode of the last query equals the last row of the square causal
    forward to within both kernels' rounding (both against the oracle)."""
    import torch

    B, H, N, d = 2, 4, 1500, 128
    w = fi.DecodeWorkload("t", B, H, N, N, d, True, 3)
    x = fi.make_decode_inputs(w)
    tq, tk, tv = dev(x["q"]), dev(x["k"]), dev(x["v"])
    of, lf = fa.forward(tq, tk, tv, causal=True)
    od, ld = fa.decode(tq[:, :, N - 4:].contiguous(), tk, tv, causal=True)
    torch.cuda.synchronize()
    assert max_abs(host64(od), host64(of[:, :, N - 4:])) <= 2 * TOL_O
    assert max_abs(host64(ld), host64(lf[:, :, N - 4:])) <= 2 * TOL_LSE


@pytest.mark.parametrize("name", sorted(fi.DECODE_WORKLOADS))
def test_full_size_decode(fa, name):
    """The benchmarked decode workload at full size, every output checked,
    and bit-identical on a repeated launch."""
    import torch

    w = fi.DECODE_WORKLOADS[name]
    x = fi.make_decode_inputs(w)
    tq, tk, tv = dev(x["q"]), dev(x["k"]), dev(x["v"])
    o, lse = fa.decode(tq, tk, tv, causal=w.causal, scale=w.scale)
    o2, lse2 = fa.decode(tq, tk, tv, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)
    ro, rl = oracle.attention_forward_kv(fi.exact_f64(x["q"]), fi.exact_f64(x["k"]), fi.exact_f64(x["v"]),
                                         w.causal, w.scale)
    _compare(o, lse, ro, rl)


@pytest.mark.parametrize("Nq", [1, 6])
def test_decode_scale_zero_is_mean(fa, Nq):
    """scale = 0: each query's output is the mean of the values it sees and
    LSE = log(count) (closed form)."""
    import torch

    B, H, Nk, d = 1, 2, 777, 128
    w = fi.DecodeWorkload("t", B, H, Nq, Nk, d, True, 5)
    x = fi.make_decode_inputs(w)
    o, lse = fa.decode(dev(x["q"]), dev(x["k"]), dev(x["v"]), causal=True, scale=0.0)
    torch.cuda.synchronize()
    vf = fi.exact_f64(x["v"])
    for i in range(Nq):
        cnt = Nk - Nq + i + 1
        assert max_abs(host64(o)[:, :, i], vf[:, :, :cnt].mean(axis=2)) <= TOL_O
        assert np.abs(host64(lse)[:, :, i] - np.log(cnt)).max() <= TOL_LSE


def test_decode_rejects_bad_tensors(fa):
    import torch

    q = torch.zeros((1, 2, 9, 128), dtype=torch.bfloat16, device="cuda:0")   # Nq = 9 > 8
    k = torch.zeros((1, 2, 64, 128), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(fa.FaError):
        fa.decode(q, k, k)
    with pytest.raises(ValueError):
        fa.decode(q[:, :, :4], k, k)          # not contiguous
