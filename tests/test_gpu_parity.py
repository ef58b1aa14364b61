"""GPU parity: the HIP kernels (through the C ABI binding) against the fp64 oracle.

Tolerances (max over all compared elements of |GPU - oracle|):
  * bf16 I/O, float32 accumulation: O, dQ, dK, dV <= 2e-2;
  * float32 debug path: O, dQ, dK, dV <= 1e-5;
  * LSE <= 1e-3 on both paths.
The oracle is evaluated on the exact values the GPU receives (bf16 bits widened
to float64), so the difference measures only the kernels' own rounding.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.gpu_util import dev, host64, max_abs, random_inputs, storage_floor
from tests.gpu_util import parallel as _parallel
from tests.gpu_util import report as _report

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_F32 = 1e-5
TOL_LSE = 1e-3


@pytest.fixture(scope="module")
def fa():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_18_amd as fa

    fa._lib.load()  # raises if the HIP library is missing: no fallback
    return fa


def _run_fwd(fa, q, k, v, causal, scale):
    import torch

    o, lse = fa.forward(dev(q), dev(k), dev(v), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def _check_fwd(fa, dtype, B, H, N, d, causal, seed=0, mult=1.0):
    q, k, v = random_inputs(seed, (B, H, N, d), dtype, 3, mult)
    scale = 1.0 / math.sqrt(d)
    o, lse = _run_fwd(fa, q, k, v, causal, scale)
    ro, rl = oracle.attention_forward(fi.exact_f64(q), fi.exact_f64(k), fi.exact_f64(v), causal, scale)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    eo, el = max_abs(host64(o), ro), max_abs(host64(lse), rl)
    assert eo <= tol, f"O error {eo:.3g} > {tol} (storage floor {storage_floor(ro):.3g})"
    assert el <= (TOL_LSE if dtype == "bf16" else TOL_F32), f"LSE error {el:.3g}"
    return eo, el


def _check_bwd(fa, dtype, B, H, N, d, causal, seed=0, mult=1.0):
    import torch

    q, k, v, do = random_inputs(seed, (B, H, N, d), dtype, 4, mult)
    scale = 1.0 / math.sqrt(d)
    tq, tk, tv, tdo = dev(q), dev(k), dev(v), dev(do)
    o, lse = fa.forward(tq, tk, tv, causal=causal, scale=scale)
    dq, dk, dv = fa.backward(tq, tk, tv, o, lse, tdo, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(fi.exact_f64(q), fi.exact_f64(k), fi.exact_f64(v), fi.exact_f64(do),
                                    causal, scale)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    errs = [max_abs(host64(x), r) for x, r in zip((dq, dk, dv), ref)]
    for name, e, r in zip(("dQ", "dK", "dV"), errs, ref):
        assert e <= tol, f"{name} error {e:.3g} > {tol} (storage floor {storage_floor(r):.3g})"
    return errs


SMALL_N = [1, 2, 17, 63, 64, 65, 127, 128, 129, 300]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", SMALL_N + [1000])
def test_bf16_forward_small(fa, N, d, causal):
    _check_fwd(fa, "bf16", 2, 3, N, d, causal, seed=N)


@pytest.mark.parametrize("N", [2049, 2113, 2300, 2623, 3000])
def test_bf16_forward_causal_above_2048(fa, N):
    """Causal d = 128 problems longer than 2048 keys take the two-group
    kernel (256-query blocks): ragged ends against its 64-key tiles and
    256-query blocks, and a diagonal that crosses the two groups' slices."""
    _check_fwd(fa, "bf16", 1, 2, N, 128, True, seed=N)


@pytest.mark.parametrize("N", [2305, 2500])
def test_two_group_forward_rows_independent_of_n(fa, N):
    """The two-group kernel computes each query row from the keys it sees, in
    the same tile order whatever N is: the first 2304 rows of a causal
    problem with N > 2304 are bit-identical to the causal N = 2304 problem on
    the same rows (both run the two-group kernel)."""
    import torch

    q, k, v = random_inputs(7, (1, 2, N, 128), "bf16", 3)
    o1, l1 = _run_fwd(fa, q, k, v, True, 128 ** -0.5)
    o2, l2 = _run_fwd(fa, q[:, :, :2304].copy(), k[:, :, :2304].copy(), v[:, :, :2304].copy(), True, 128 ** -0.5)
    assert torch.equal(o1[:, :, :2304].view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1[:, :, :2304], l2)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", SMALL_N)
def test_bf16_backward_small(fa, N, d, causal):
    _check_bwd(fa, "bf16", 2, 2, N, d, causal, seed=100 + N)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [4, 64, 100, 128])
@pytest.mark.parametrize("N", [1, 2, 17, 33, 64, 65, 129, 300])
def test_f32_forward_small(fa, N, d, causal):
    _check_fwd(fa, "f32", 2, 2, N, d, causal, seed=200 + N)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [4, 64, 128])
@pytest.mark.parametrize("N", [1, 2, 17, 65, 129, 300])
def test_f32_backward_small(fa, N, d, causal):
    _check_bwd(fa, "f32", 1, 2, N, d, causal, seed=300 + N)


def test_f32_workload(fa):
    """The float32 problem B=1, H=2, N=128, d=64, non-causal, seed 0, scale 1/8,
    forward and backward at 1e-5."""
    w = fi.WORKLOADS["f32_b1h2n128d64"]
    _check_fwd(fa, "f32", w.B, w.H, w.N, w.d, w.causal, seed=0)
    _check_bwd(fa, "f32", w.B, w.H, w.N, w.d, w.causal, seed=0)


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_invariants_on_gpu_output(fa, dtype, causal):
    """Pins that hold whatever the oracle says: constant V gives O = V; the
    first causal row is V[0]; Q = 0 gives the mean of the visible rows with
    LSE = log(#visible); sum_j exp(scale*q.k_j - LSE) = 1."""
    B, H, N, d = 1, 2, 200, 64
    q, k, v = random_inputs(7, (B, H, N, d), dtype, 3)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    scale = 0.125
    # constant V
    vc = np.broadcast_to(v[:, :, :1], v.shape).copy()
    o, _ = _run_fwd(fa, q, k, vc, causal, scale)
    assert max_abs(host64(o), fi.exact_f64(vc)) <= tol
    # Q = 0
    z = np.zeros_like(q)
    o, lse = _run_fwd(fa, z, k, v, causal, scale)
    vv = fi.exact_f64(v)
    if causal:
        cnt = np.arange(1, N + 1, dtype=np.float64)
        mean = np.cumsum(vv, axis=2) / cnt[None, None, :, None]
    else:
        cnt = np.full(N, float(N))
        mean = np.broadcast_to(vv.mean(axis=2, keepdims=True), vv.shape)
    assert max_abs(host64(o), mean) <= tol
    assert max_abs(host64(lse), np.broadcast_to(np.log(cnt), (B, H, N))) <= TOL_LSE
    # first causal row and LSE normalisation
    o, lse = _run_fwd(fa, q, k, v, causal, scale)
    qq, kk = fi.exact_f64(q), fi.exact_f64(k)
    if causal:
        assert max_abs(host64(o)[:, :, 0], vv[:, :, 0]) <= tol
    s = scale * np.einsum("bhid,bhjd->bhij", qq, kk)
    if causal:
        s = np.where(np.triu(np.ones((N, N), bool), 1), -np.inf, s)
    tot = np.exp(s - host64(lse)[..., None]).sum(-1)
    assert np.max(np.abs(tot - 1.0)) <= 2 * TOL_LSE


# ---------------------------------------------------------------- full sizes

FULL_FWD = [
    "bf16_b16h32n1024d64",
    "bf16_b16h32n1024d64_causal",
    "bf16_b4h16n4096d128_causal_x0.5",
    "bf16_b1h16n16384d128_causal",
    "bf16_b1h16n16384d128",
    "bf16_b8h16n2048d128_causal_fwdbwd",
]


def _sample_rows(N, n, rng):
    rows = {0, 1, N - 1, N - 2, N // 2}
    rows.update(rng.choice(N, size=min(n, N), replace=False).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < N))


@pytest.mark.parametrize("name", FULL_FWD)
def test_full_size_forward(fa, name):
    """Full-size workloads in the benchmark's launch configuration, compared
    with the oracle on EVERY element of O and LSE (the oracle runs per
    (batch, head) in slabs of query rows); every element written (outputs
    prefilled with NaN) and bit-identical on a repeated launch."""
    import torch

    w = fi.WORKLOADS[name]
    x = fi.make_inputs(w, with_grad=False)
    tq, tk, tv = dev(x["q"]), dev(x["k"]), dev(x["v"])
    o = torch.full_like(tq, float("nan"))
    lse = torch.full((w.B, w.H, w.N), float("nan"), dtype=torch.float32, device=tq.device)
    st = fa.fa_forward(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       w.B, w.H, w.N, w.d, w.causal, w.scale, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    o2, lse2 = fa.forward(tq, tk, tv, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)
    oh, lh = host64(o), host64(lse)
    del o2, lse2, tq, tk, tv

    slab = min(w.N, 2048)
    tasks = [(b, h, r0) for b in range(w.B) for h in range(w.H) for r0 in range(0, w.N, slab)]

    def one(t):
        b, h, r0 = t
        rows = np.arange(r0, min(w.N, r0 + slab))
        ro, rl = oracle.attention_forward_rows(fi.exact_f64(x["q"][b, h]), fi.exact_f64(x["k"][b, h]),
                                               fi.exact_f64(x["v"][b, h]), rows, w.causal, w.scale)
        return (max_abs(oh[b, h, rows], ro), max_abs(lh[b, h, rows], rl), storage_floor(ro))

    res = np.array(_parallel(one, tasks))
    eo, el, fl = (float(res[:, i].max()) for i in range(3))
    _report(name, "O", eo, fl, oh.size)
    _report(name, "LSE", el, 0.0, lh.size)
    assert eo <= TOL_BF16, f"O error {eo:.4g} (storage floor {fl:.3g})"
    assert el <= TOL_LSE, f"LSE error {el:.4g}"


@pytest.mark.parametrize("name", ["bf16_b8h16n2048d128_causal_fwdbwd", "bf16_b16h32n1024d64_causal_fwdbwd"])
def test_full_size_backward(fa, name):
    """The forward+backward workloads the benchmark times (B=8 H=16 N=2048
    d=128 causal, and B=16 H=32 N=1024 d=64 causal): dQ, dK and dV compared
    with the oracle on EVERY element of every head; whole outputs written
    (prefilled with NaN), finite and bit-identical on a repeated launch."""
    import torch

    w = fi.WORKLOADS.get(name) or fi.EXTRA_WORKLOADS[name]
    x = fi.make_inputs(w, with_grad=True)
    tq, tk, tv, tdo = (dev(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(tq, tk, tv, causal=True, scale=w.scale)
    grads = [torch.full_like(tq, float("nan")) for _ in range(3)]
    ws = torch.empty(fa.fa_backward_workspace_size(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=tq.device)
    st = fa.fa_backward(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        tdo.data_ptr(), grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(),
                        w.B, w.H, w.N, w.d, 1, w.scale, ws.data_ptr(), ws.numel(),
                        torch.cuda.current_stream().cuda_stream)
    assert st == 0
    again = fa.backward(tq, tk, tv, o, lse, tdo, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    for a, b in zip(grads, again):
        assert bool(torch.isfinite(a).all())
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    got = [host64(t) for t in grads]
    del again, grads

    def one(t):
        b, h = t
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oracle.attention_backward(*(fi.exact_f64(x[n][sl]) for n in ("q", "k", "v", "do")), True, w.scale)
        return [v for g, r in zip(got, ref) for v in (max_abs(g[sl], r), storage_floor(r))]

    res = np.array(_parallel(one, [(b, h) for b in range(w.B) for h in range(w.H)]))
    for i, name in enumerate(("dQ", "dK", "dV")):
        e, f = float(res[:, 2 * i].max()), float(res[:, 2 * i + 1].max())
        _report(w.name, name, e, f, got[i].size)
        assert e <= TOL_BF16, f"{name}: {e:.4g} (storage floor {f:.3g})"


# (B, H, N, d, causal): up to 512 workgroups per grid at d=128 (768 at d=64)
# fa_backward runs dK/dV and dQ in one launch, above that in two.
STAGE_SHAPES = [(1, 16, 2048, 128, True), (2, 16, 2048, 128, True), (2, 16, 2048, 128, False),
                (4, 16, 2048, 128, True), (3, 5, 1000, 128, True), (1, 1, 1, 128, False),
                (6, 16, 1024, 64, True), (7, 16, 1024, 64, False), (4, 16, 2048, 64, True)]


@pytest.mark.parametrize("B,H,N,d,causal", STAGE_SHAPES)
def test_backward_equals_its_stages(fa, B, H, N, d, causal):
    """fa_backward (one launch for both passes on small grids, two on large
    ones) gives the same bits as fa_backward_preprocess, fa_backward_dkdv and
    fa_backward_dq called one by one, and as fa_backward_dq_delta followed by
    fa_backward_dkdv; sampled heads agree with the oracle."""
    import torch

    q, k, v, do = random_inputs(500 + N + B, (B, H, N, d), "bf16", 4)
    scale = 1.0 / math.sqrt(d)
    tq, tk, tv, tdo = dev(q), dev(k), dev(v), dev(do)
    o, lse = fa.forward(tq, tk, tv, causal=causal, scale=scale)
    whole = fa.backward(tq, tk, tv, o, lse, tdo, causal=causal, scale=scale)
    staged = [torch.full_like(tq, float("nan")) for _ in range(3)]
    nb = fa.fa_backward_workspace_size(B, H, N, d)
    ws = torch.empty(nb, dtype=torch.uint8, device=tq.device)
    sp = torch.cuda.current_stream().cuda_stream
    assert fa.fa_backward_preprocess(o.data_ptr(), tdo.data_ptr(), B, H, N, d, ws.data_ptr(), nb, sp) == 0
    assert fa.fa_backward_dq(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), lse.data_ptr(), tdo.data_ptr(),
                             staged[0].data_ptr(), B, H, N, d, causal, scale, ws.data_ptr(), nb, sp) == 0
    assert fa.fa_backward_dkdv(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), lse.data_ptr(), tdo.data_ptr(),
                               staged[1].data_ptr(), staged[2].data_ptr(), B, H, N, d, causal, scale,
                               ws.data_ptr(), nb, sp) == 0
    # the other sequence: dQ computing -delta itself, into a NaN-filled
    # workspace (so dK/dV can only have read what that pass wrote), then dK/dV
    ws2 = torch.full((nb // 4,), float("nan"), dtype=torch.float32, device=tq.device)
    staged2 = [torch.full_like(tq, float("nan")) for _ in range(3)]
    assert fa.fa_backward_dq_delta(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                   tdo.data_ptr(), staged2[0].data_ptr(), B, H, N, d, causal, scale,
                                   ws2.data_ptr(), nb, sp) == 0
    assert fa.fa_backward_dkdv(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), lse.data_ptr(), tdo.data_ptr(),
                               staged2[1].data_ptr(), staged2[2].data_ptr(), B, H, N, d, causal, scale,
                               ws2.data_ptr(), nb, sp) == 0
    torch.cuda.synchronize()
    for name, a, b, c2 in zip(("dQ", "dK", "dV"), whole, staged, staged2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
        assert torch.equal(a.view(torch.int16), c2.view(torch.int16)), name + " (dq_delta order)"
    # both sequences leave the same -delta rows in the workspace
    rows = B * H * N
    assert torch.equal(ws.view(torch.float32)[:rows], ws2[:rows])
    got = [host64(t) for t in whole]
    for (b, h) in sorted({(0, 0), (B - 1, H - 1)}):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oracle.attention_backward(*(fi.exact_f64(a[sl]) for a in (q, k, v, do)), causal, scale)
        for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
            e = max_abs(g[sl], r)
            assert e <= TOL_BF16, f"{name} head {(b, h)}: {e:.4g} (storage floor {storage_floor(r):.3g})"


@pytest.mark.parametrize("N,causal", [(131072, True), (65536, False)])
def test_long_sequence_forward(fa, N, causal):
    """One head of a long sequence (1024-2048 key tiles per row block):
    sampled rows of O and LSE against the oracle."""
    q, k, v = random_inputs(900 + N, (1, 1, N, 128), "bf16", 3)
    scale = 128 ** -0.5
    o, lse = _run_fwd(fa, q, k, v, causal, scale)
    rows = _sample_rows(N, 12, np.random.default_rng(N))
    ro, rl = oracle.attention_forward_rows(fi.exact_f64(q[0, 0]), fi.exact_f64(k[0, 0]), fi.exact_f64(v[0, 0]),
                                           rows, causal, scale)
    assert max_abs(host64(o)[0, 0, rows], ro) <= TOL_BF16
    assert max_abs(host64(lse)[0, 0, rows], rl) <= TOL_LSE


@pytest.mark.parametrize("causal", [True, False])
def test_long_sequence_backward(fa, causal):
    """One head, N = 32768: sampled rows of dQ against the oracle, and two
    identities of the backward over all rows: sum_j dK_j = 0 (every row of dS
    sums to zero) and sum_j dV_j = sum_i dO_i (every row of P sums to one),
    within the rounding of the bf16-stored gradients."""
    import torch

    N, d = 32768, 128
    q, k, v, do = random_inputs(950 + int(causal), (1, 1, N, d), "bf16", 4)
    scale = d ** -0.5
    tq, tk, tv, tdo = dev(q), dev(k), dev(v), dev(do)
    o, lse = fa.forward(tq, tk, tv, causal=causal, scale=scale)
    dq, dk, dv = fa.backward(tq, tk, tv, o, lse, tdo, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rows = _sample_rows(N, 10, np.random.default_rng(N + int(causal)))
    rdq = oracle.attention_backward_dq_rows(*(fi.exact_f64(a[0, 0]) for a in (q, k, v, do)), rows, causal, scale)
    assert max_abs(host64(dq)[0, 0, rows], rdq) <= TOL_BF16
    gk, gv = host64(dk)[0, 0], host64(dv)[0, 0]
    # each stored value is within 2^-9 of its own magnitude of the exact one
    assert np.all(np.abs(gk.sum(0)) <= 2.0 ** -9 * np.abs(gk).sum(0) + 1e-3)
    dsum = fi.exact_f64(do)[0, 0].sum(0)
    assert np.all(np.abs(gv.sum(0) - dsum) <= 2.0 ** -9 * np.abs(gv).sum(0) + 1e-3)

def test_forward_is_deterministic_across_streams(fa):
    import torch

    q, k, v = random_inputs(9, (2, 4, 777, 128), "bf16", 3)
    tq, tk, tv = dev(q), dev(k), dev(v)
    ref, rl = fa.forward(tq, tk, tv, causal=True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        outs = [fa.forward(tq, tk, tv, causal=True) for _ in range(5)]
    torch.cuda.synchronize()
    for o, lse in outs:
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16))
        assert torch.equal(lse, rl)



@pytest.mark.parametrize("N,d,causal", [(2048, 128, False), (2048, 128, True), (3000, 128, True),
                                        (2048, 64, False), (1500, 64, True)])
def test_forward_scores_rising_along_keys(fa, N, d, causal):
    """Scores that grow along the key axis (K_j = K0_j + t_j u, Q_i = Q0_i + u,
    t_j from 0 to 6, |u|^2 = 100): every few tiles some score exceeds the
    reference max by more than the lazy-rescale threshold, so the rescale
    path runs repeatedly, in the middle of rows rather than only at their
    first tile.  O and LSE against the oracle."""
    rng = np.random.default_rng(1234 + N + d)
    q0, k0, v = (rng.standard_normal((1, 2, N, d)).astype(np.float32) for _ in range(3))
    u = rng.standard_normal(d).astype(np.float32)
    u *= 10.0 / np.linalg.norm(u)
    t = np.linspace(0.0, 6.0, N, dtype=np.float32)[None, None, :, None]
    q, k, v = (fi.f32_to_bf16_bits(a) for a in (q0 + u, k0 + t * u, v))
    scale = 1.0 / math.sqrt(d)
    o, lse = _run_fwd(fa, q, k, v, causal, scale)
    ro, rl = oracle.attention_forward(fi.exact_f64(q), fi.exact_f64(k), fi.exact_f64(v), causal, scale)
    eo, el = max_abs(host64(o), ro), max_abs(host64(lse), rl)
    assert eo <= TOL_BF16, f"O error {eo:.3g} (storage floor {storage_floor(ro):.3g})"
    assert el <= TOL_LSE, f"LSE error {el:.3g}"

@pytest.mark.parametrize("causal", [False, True])
def test_large_magnitude_inputs(fa, causal):
    """Inputs x8 (scores up to ~1e3 * scale): the running max jumps by far
    more than the lazy-rescale threshold between tiles and exp() would
    overflow without the max subtraction; forward and backward stay within
    tolerance of the oracle relative to the inputs' scale."""
    import torch

    B, H, N, d = 1, 2, 700, 128
    q, k, v, do = random_inputs(77, (B, H, N, d), "bf16", 4, mult=8.0)
    scale = 1.0 / math.sqrt(d)
    tq, tk, tv, tdo = dev(q), dev(k), dev(v), dev(do)
    o, lse = fa.forward(tq, tk, tv, causal=causal, scale=scale)
    dq, dk, dv = fa.backward(tq, tk, tv, o, lse, tdo, causal=causal, scale=scale)
    torch.cuda.synchronize()
    qf, kf, vf, gf = (fi.exact_f64(a) for a in (q, k, v, do))
    ro, rl = oracle.attention_forward(qf, kf, vf, causal, scale)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    # O (up to ~35) and LSE (up to ~330) are far from unit scale: the bar for
    # O is 1% of its largest magnitude plus its bf16 storage rounding
    assert max_abs(host64(o), ro) <= 0.01 * np.abs(ro).max() + storage_floor(ro)
    assert np.abs(host64(lse) - rl).max() <= TOL_LSE
    ref = oracle.attention_backward(qf, kf, vf, gf, causal, scale)
    # gradients at this scale are large: the bar is 2% of their largest
    # magnitude plus their own bf16 storage rounding
    for name, x, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        e = max_abs(host64(x), r)
        bar = 0.02 * np.abs(r).max() + storage_floor(r)
        assert e <= bar, f"{name}: {e:.3g} > {bar:.3g} (floor {storage_floor(r):.3g})"
