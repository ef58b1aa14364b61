"""fa_backward_atomic, the single-pass backward (dQ accumulated with float32
atomics in the dK/dV pass), through the C ABI: dK and dV bit-identical to
fa_backward's, dQ within the bf16 tolerance of the oracle, over ragged and
tile-edge sizes, both head dimensions and both mask modes, and on every
element of the forward+backward workloads the benchmark times."""
from __future__ import annotations

import math

import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.gpu_util import dev, host64, max_abs, parallel, random_inputs, report, storage_floor

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2


@pytest.fixture(scope="module")
def fa():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_18_amd as fa

    fa._lib.load()  # raises if the HIP library is missing: no fallback
    return fa


def _call(fa, tq, tk, tv, o, lse, tdo, B, H, N, d, causal, scale, ws=None, fill=float("nan")):
    """fa_backward_atomic on outputs prefilled with `fill` and, unless given,
    a workspace prefilled with garbage (its contents on entry are ignored)."""
    import torch

    need = fa.fa_backward_atomic_workspace_size(B, H, N, d)
    if ws is None:
        ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=tq.device)
    out = [torch.full_like(tq, fill) for _ in range(3)]
    st = fa.fa_backward_atomic(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), lse.data_ptr(),
                               tdo.data_ptr(), out[0].data_ptr(), out[1].data_ptr(), out[2].data_ptr(), B, H, N,
                               d, int(causal), scale, ws.data_ptr(), ws.numel() * ws.element_size(),
                               torch.cuda.current_stream().cuda_stream)
    assert st == 0, fa.fa_status_string(st)
    return out, ws


def _check_small(fa, B, H, N, d, causal, seed):
    import torch

    q, k, v, do = random_inputs(seed, (B, H, N, d), "bf16", 4)
    scale = 1.0 / math.sqrt(d)
    tq, tk, tv, tdo = dev(q), dev(k), dev(v), dev(do)
    o, lse = fa.forward(tq, tk, tv, causal=causal, scale=scale)
    got, _ = _call(fa, tq, tk, tv, o, lse, tdo, B, H, N, d, causal, scale)
    ref2 = fa.backward(tq, tk, tv, o, lse, tdo, causal=causal, scale=scale)
    torch.cuda.synchronize()
    for name, a, b in zip(("dK", "dV"), got[1:], ref2[1:]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name} differs from fa_backward"
    exact = oracle.attention_backward(*(fi.exact_f64(a) for a in (q, k, v, do)), causal, scale)
    for name, a, r in zip(("dQ", "dK", "dV"), got, exact):
        e = max_abs(host64(a), r)
        assert e <= TOL_BF16, f"{name} error {e:.3g} (storage floor {storage_floor(r):.3g})"
    # dQ of the two forms: the same bf16 dS and K, summed in another order
    assert max_abs(host64(got[0]), host64(ref2[0])) <= 1e-2


SMALL_N = [1, 2, 17, 63, 64, 65, 127, 128, 129, 300, 1000]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", SMALL_N)
def test_atomic_backward_small(fa, N, d, causal):
    _check_small(fa, 1, 2, N, d, causal, seed=N + d)


@pytest.mark.parametrize("B,H,N,d,causal", [(2, 3, 777, 128, True), (3, 2, 1500, 64, False),
                                            (1, 16, 2048, 128, False), (2, 5, 4100, 64, True)])
def test_atomic_backward_shapes(fa, B, H, N, d, causal):
    _check_small(fa, B, H, N, d, causal, seed=B * 1000 + N)


def test_atomic_backward_workspace_reuse(fa):
    """A second call with the same workspace (holding the first call's
    accumulator) and a different problem size gives the right dQ: the
    accumulator is cleared on every call."""
    import torch

    shapes = [(2, 4, 700, 128, True), (1, 3, 300, 64, False)]
    big = max(fa.fa_backward_atomic_workspace_size(B, H, N, d) for B, H, N, d, _ in shapes)
    ws = torch.empty(big // 4, dtype=torch.float32, device="cuda:0")
    for i, (B, H, N, d, causal) in enumerate(shapes):
        q, k, v, do = random_inputs(40 + i, (B, H, N, d), "bf16", 4)
        scale = 1.0 / math.sqrt(d)
        tq, tk, tv, tdo = dev(q), dev(k), dev(v), dev(do)
        o, lse = fa.forward(tq, tk, tv, causal=causal, scale=scale)
        got, _ = _call(fa, tq, tk, tv, o, lse, tdo, B, H, N, d, causal, scale, ws=ws)
        torch.cuda.synchronize()
        exact = oracle.attention_backward(*(fi.exact_f64(a) for a in (q, k, v, do)), causal, scale)
        assert max_abs(host64(got[0]), exact[0]) <= TOL_BF16


def test_atomic_backward_argument_checks(fa):
    import torch

    B, H, N, d = 1, 2, 64, 128
    t = [torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda:0") for _ in range(8)]
    lse = torch.zeros((B, H, N), dtype=torch.float32, device="cuda:0")
    need = fa.fa_backward_atomic_workspace_size(B, H, N, d)
    assert need == fa.fa_backward_workspace_size(B, H, N, d) + 4 * B * H * N * d
    assert fa.fa_backward_atomic_workspace_size(0, H, N, d) == 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    p = [t[0].data_ptr(), t[1].data_ptr(), t[2].data_ptr(), t[3].data_ptr(), lse.data_ptr(), t[4].data_ptr(),
         t[5].data_ptr(), t[6].data_ptr(), t[7].data_ptr()]
    sp = torch.cuda.current_stream().cuda_stream
    assert fa.fa_backward_atomic(*p, B, H, N, d, 1, 0.1, ws.data_ptr(), need - 1, sp) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_backward_atomic(*p, B, H, N, 96, 1, 0.1, ws.data_ptr(), need, sp) == fa.FA_ERR_UNSUPPORTED
    # the output dq may not overlap the workspace
    q2 = p.copy()
    q2[6] = ws.data_ptr()
    assert fa.fa_backward_atomic(*q2, B, H, N, d, 1, 0.1, ws.data_ptr(), need, sp) == fa.FA_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        f = [x.float() for x in t[:5]]
        fa.backward_atomic(f[0], f[1], f[2], f[3], lse, f[4], causal=True)


@pytest.mark.parametrize("name", ["bf16_b8h16n2048d128_causal_fwdbwd", "bf16_b16h32n1024d64_causal_fwdbwd"])
def test_atomic_backward_full_size(fa, name):
    """The forward+backward workloads the benchmark times: dK and dV equal
    to fa_backward's on every element, dQ against the oracle on every
    element of every head."""
    import torch

    w = fi.WORKLOADS.get(name) or fi.EXTRA_WORKLOADS[name]
    x = fi.make_inputs(w, with_grad=True)
    tq, tk, tv, tdo = (dev(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(tq, tk, tv, causal=True, scale=w.scale)
    got, _ = _call(fa, tq, tk, tv, o, lse, tdo, w.B, w.H, w.N, w.d, True, w.scale)
    ref2 = fa.backward(tq, tk, tv, o, lse, tdo, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    for nm, a, b in zip(("dK", "dV"), got[1:], ref2[1:]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), nm
    assert bool(torch.isfinite(got[0]).all())
    dq_gap = max_abs(host64(got[0]), host64(ref2[0]))
    dq = host64(got[0])
    del got, ref2

    def one(t):
        b, h = t
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oracle.attention_backward(*(fi.exact_f64(x[n][sl]) for n in ("q", "k", "v", "do")), True, w.scale)
        return max_abs(dq[sl], ref[0]), storage_floor(ref[0])

    res = np.array(parallel(one, [(b, h) for b in range(w.B) for h in range(w.H)]))
    e, f = float(res[:, 0].max()), float(res[:, 1].max())
    report(w.name, "dQ (single pass)", e, f, dq.size)
    print(f"PARITY {w.name} dQ single pass vs fa_backward: max_abs_diff {dq_gap:.5g}", flush=True)
    assert e <= TOL_BF16, f"dQ: {e:.4g} (storage floor {f:.3g})"
