"""GPU parity of the block-sparse forward against the fp64 oracle.

Same tolerances as the dense forward (O max-abs 2e-2, LSE 1e-3 on finite
rows); rows that see no key must give O = 0 and LSE = -inf exactly.  With
every block visible the block-sparse kernel must reproduce the dense forward
bit for bit.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.gpu_util import dev, host64, max_abs, random_inputs

pytestmark = pytest.mark.gpu

TOL_O = 2e-2
TOL_LSE = 1e-3
BLK = 128


@pytest.fixture(scope="module")
def fa():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_18_amd as fa

    fa._lib.load()
    return fa


def _mask_dev(mask):
    import torch

    return torch.from_numpy(np.ascontiguousarray(mask, dtype=np.uint8)).to("cuda:0")


def _compare(o, lse, ro, rl):
    """O everywhere; LSE on finite rows; -inf rows exactly."""
    oh, lh = host64(o), host64(lse)
    assert np.all(np.isfinite(oh)), "non-finite O"
    eo = max_abs(oh, ro)
    assert eo <= TOL_O, f"O error {eo:.3g}"
    dead = ~np.isfinite(rl)
    assert np.array_equal(np.isneginf(lh), dead), "LSE -inf rows differ"
    assert np.all(oh[dead] == 0.0), "rows with no visible key must be zero"
    el = float(np.max(np.abs(lh[~dead] - rl[~dead]))) if (~dead).any() else 0.0
    assert el <= TOL_LSE, f"LSE error {el:.3g}"


def _check(fa, B, H, N, d, causal, mask, seed=0):
    import torch

    q, k, v = random_inputs(seed, (B, H, N, d), "bf16", 3)
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.forward_block_sparse(dev(q), dev(k), dev(v), _mask_dev(mask), causal=causal, scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward_block_sparse(fi.exact_f64(q), fi.exact_f64(k), fi.exact_f64(v),
                                                   mask, BLK, causal, scale)
    _compare(o, lse, ro, rl)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 65, 128, 129, 300, 1000])
@pytest.mark.parametrize("density", [0.3, 0.7])
def test_block_sparse_random_masks(fa, N, d, causal, density):
    nb = -(-N // BLK)
    mask = fi.random_block_mask(N + d, nb, density)
    _check(fa, 2, 2, N, d, causal, mask, seed=N)


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_empty_rows_and_columns(fa, causal):
    N, nb = 700, 6
    mask = fi.random_block_mask(11, nb, 0.6)
    mask[2, :] = 0          # query block 2 sees nothing: O = 0, LSE = -inf
    mask[:, 4] = 0          # key block 4 is never read
    mask[5, 5] = 1
    _check(fa, 1, 3, N, 128, causal, mask, seed=5)


@pytest.mark.parametrize("N", [100, 513])
def test_block_sparse_all_hidden(fa, N):
    import torch

    nb = -(-N // BLK)
    q, k, v = (dev(a) for a in random_inputs(3, (1, 2, N, 64), "bf16", 3))
    o, lse = fa.forward_block_sparse(q, k, v, _mask_dev(np.zeros((nb, nb), np.uint8)))
    torch.cuda.synchronize()
    assert bool((o.float() == 0).all()) and bool(torch.isneginf(lse).all())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_all_visible_equals_dense_bitwise(fa, d, causal):
    """With every block visible the block-sparse kernel does the dense
    kernel's arithmetic tile by tile: bit-identical to fa_forward wherever
    fa_forward runs the same kernel family (d = 64, and causal d = 128 up to
    N = 2048); the d = 128 non-causal forward runs the two-group kernel (its
    lazy rescale decides per 128 keys), so there both are compared with the
    oracle."""
    import torch

    N = 777
    nb = -(-N // BLK)
    qh, kh, vh = random_inputs(4, (2, 3, N, d), "bf16", 3)
    q, k, v = dev(qh), dev(kh), dev(vh)
    od, ld = fa.forward(q, k, v, causal=causal)
    same_kernel = d == 64 or causal
    ref = None if same_kernel else oracle.attention_forward(*(fi.exact_f64(a) for a in (qh, kh, vh)), causal,
                                                            d ** -0.5)
    for balance in (False, True):   # every row has the same count: nothing is split either way
        o, lse = fa.forward_block_sparse(q, k, v, _mask_dev(np.ones((nb, nb), np.uint8)), causal=causal,
                                         balance=balance)
        torch.cuda.synchronize()
        if same_kernel:
            assert torch.equal(o.view(torch.int16), od.view(torch.int16))
            assert torch.equal(lse, ld)
        else:
            for oo, ll in ((o, lse), (od, ld)):
                assert max_abs(host64(oo), ref[0]) <= 2e-2 and max_abs(host64(ll), ref[1]) <= 1e-3


def test_block_diagonal_equals_independent_segments(fa):
    """A block-diagonal mask is independent attention within each 128-key
    segment: compare with the dense kernel run on each segment alone."""
    import torch

    N, nb = 512, 4
    q, k, v = (dev(a) for a in random_inputs(6, (1, 2, N, 128), "bf16", 3))
    o, lse = fa.forward_block_sparse(q, k, v, _mask_dev(np.eye(nb, dtype=np.uint8)), causal=True)
    for s in range(nb):
        sl = slice(BLK * s, BLK * (s + 1))
        os_, ls_ = fa.forward(q[:, :, sl].contiguous(), k[:, :, sl].contiguous(), v[:, :, sl].contiguous(),
                              causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o[:, :, sl].view(torch.int16), os_.view(torch.int16))
        assert torch.equal(lse[:, :, sl], ls_)


@pytest.mark.parametrize("name", sorted(fi.BLOCK_SPARSE_WORKLOADS))
def test_full_size_block_sparse(fa, name):
    """The benchmarked block-sparse workload at full size: sampled rows of
    sampled heads against the oracle (restricted to those rows), whole output
    finite, bit-identical on a repeated launch."""
    import torch

    sw = fi.BLOCK_SPARSE_WORKLOADS[name]
    w = sw.base
    mask = sw.mask()
    x = fi.make_inputs(w, with_grad=False)
    tq, tk, tv = dev(x["q"]), dev(x["k"]), dev(x["v"])
    tm = _mask_dev(mask)
    o, lse = fa.forward_block_sparse(tq, tk, tv, tm, causal=w.causal, scale=w.scale)
    o2, lse2 = fa.forward_block_sparse(tq, tk, tv, tm, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)

    rng = np.random.default_rng(3)
    oh, lh = host64(o), host64(lse)
    for (b, h) in sorted({(0, 0), (w.B - 1, w.H - 1), (int(rng.integers(w.B)), int(rng.integers(w.H)))}):
        rows = np.unique(np.concatenate([[0, 1, 127, 128, w.N // 2, w.N - 1],
                                         rng.choice(w.N, 48, replace=False)]))
        ro, rl = oracle.attention_forward_block_sparse_rows(
            fi.exact_f64(x["q"][b, h]), fi.exact_f64(x["k"][b, h]), fi.exact_f64(x["v"][b, h]), rows,
            mask, BLK, w.causal, w.scale)
        assert max_abs(oh[b, h, rows], ro) <= TOL_O
        assert max_abs(lh[b, h, rows], rl) <= TOL_LSE


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_scale_zero_is_mean_of_visible(fa, causal):
    """scale = 0: uniform weights over the visible keys, so O is the mean of
    the visible V rows and LSE = log(count) (closed form, no oracle call)."""
    import torch

    N, nb = 300, 3
    mask = np.array([[1, 0, 1], [0, 1, 0], [1, 1, 0]], np.uint8)
    q, k, v = random_inputs(31, (1, 2, N, 64), "bf16", 3)
    o, lse = fa.forward_block_sparse(dev(q), dev(k), dev(v), _mask_dev(mask), causal=causal, scale=0.0)
    torch.cuda.synchronize()
    vis = oracle.block_visibility(mask, N, BLK)
    if causal:
        vis &= np.tril(np.ones((N, N), bool))
    vf = fi.exact_f64(v)
    cnt = vis.sum(1)
    mean = (vis[None, None] @ vf) / np.maximum(cnt, 1)[None, None, :, None]
    oh, lh = host64(o), host64(lse)
    live = cnt > 0
    assert max_abs(oh[:, :, live], mean[:, :, live]) <= TOL_O
    assert np.abs(lh[:, :, live] - np.log(cnt[live])).max() <= TOL_LSE
    assert np.all(oh[:, :, ~live] == 0) and np.all(np.isneginf(lh[:, :, ~live]))


def test_block_sparse_mid_size_d64(fa):
    N = 2048
    nb = N // BLK
    mask = fi.local_global_block_mask(nb, 1, 1)
    _check(fa, 1, 4, N, 64, True, mask, seed=8)


def _heavy_mask(nb, seed):
    """A sparse random mask plus one dense query-block row (a "global" row):
    the kind of mask whose rows the balanced path splits."""
    m = fi.random_block_mask(seed, nb, 0.15)
    np.fill_diagonal(m, 1)
    m[nb // 3, :] = 1
    m[nb - 1, :] = 1   # dense also under a causal mask
    return m


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1500, 2048])
def test_balanced_split_rows_vs_oracle(fa, N, d, causal):
    nb = -(-N // BLK)
    mask = _heavy_mask(nb, N + d)
    if not causal:
        mask[0, :] = 1   # a second dense row
    _check(fa, 1, 3, N, d, causal, mask, seed=N)


@pytest.mark.parametrize("causal", [False, True])
def test_balanced_unsplit_rows_bitwise_equal_one_pass(fa, causal):
    """Rows the plan does not split follow the one-pass tile sequence: same
    bits.  The dense row is split; its result stays within tolerance of the
    oracle (checked above)."""
    import torch

    N = 2048
    nb = N // BLK
    mask = _heavy_mask(nb, 5)
    q, k, v = (dev(a) for a in random_inputs(17, (1, 2, N, 128), "bf16", 3))
    tm = _mask_dev(mask)
    o1, l1 = fa.forward_block_sparse(q, k, v, tm, causal=causal, balance=False)
    o2, l2 = fa.forward_block_sparse(q, k, v, tm, causal=causal, balance=True)
    torch.cuda.synchronize()
    cnt = mask.sum(1) if not causal else np.tril(mask).sum(1)
    mean = max(1, -(-int(cnt.sum()) // nb))
    unsplit = np.repeat(cnt <= 2 * mean, BLK)[:N]
    assert (~unsplit).any() and unsplit.any()
    rows = torch.from_numpy(np.nonzero(unsplit)[0]).to(q.device)
    assert torch.equal(o1[:, :, rows].view(torch.int16), o2[:, :, rows].view(torch.int16))
    assert torch.equal(l1[:, :, rows], l2[:, :, rows])


@pytest.mark.parametrize("causal", [False, True])
def test_one_pass_path_random_masks(fa, causal):
    """The path without a workspace (one workgroup per query block)."""
    import torch

    N, d = 700, 128
    nb = -(-N // BLK)
    mask = _heavy_mask(nb, 3)
    q, k, v = random_inputs(23, (2, 2, N, d), "bf16", 3)
    o, lse = fa.forward_block_sparse(dev(q), dev(k), dev(v), _mask_dev(mask), causal=causal, balance=False)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward_block_sparse(fi.exact_f64(q), fi.exact_f64(k), fi.exact_f64(v), mask, BLK,
                                                   causal, 1 / math.sqrt(d))
    _compare(o, lse, ro, rl)
