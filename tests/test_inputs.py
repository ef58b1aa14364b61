"""The seeded input generators (CPU only)."""
import numpy as np
import pytest
import torch

import fa_inputs as fi


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(3)
    x = np.concatenate([
        r.standard_normal(100000).astype(np.float32),
        (r.standard_normal(1000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-40, np.inf, -np.inf], dtype=np.float32),
        # exact ties: the low 16 bits are 0x8000
        (np.array([0x3F808000, 0x3F818000, 0xBF808000], dtype=np.uint32)).view(np.float32),
    ])
    ours = fi.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = fi.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_generator_is_seeded_and_ordered():
    w = fi.WORKLOADS["f32_b1h2n128d64"]
    a = fi.make_inputs(w, with_grad=True)
    b = fi.make_inputs(w, with_grad=True)
    for n in ("q", "k", "v", "do"):
        assert np.array_equal(a[n], b[n])
    rng = np.random.default_rng(0)
    q = rng.standard_normal(w.shape, dtype=np.float32)
    k = rng.standard_normal(w.shape, dtype=np.float32)
    assert np.array_equal(a["q"], q) and np.array_equal(a["k"], k)


def test_half_multiplier_commutes_with_rounding():
    w = fi.WORKLOADS["bf16_b4h16n4096d128_causal_x0.5"]
    small = fi.Workload("t", "bf16", 1, 1, 64, 128, True, mult=0.5)
    full = fi.Workload("t", "bf16", 1, 1, 64, 128, True, mult=1.0)
    a = fi.exact_f64(fi.make_inputs(small)["q"])
    b = fi.exact_f64(fi.make_inputs(full)["q"])
    assert np.array_equal(a, 0.5 * b)
    assert w.mult == 0.5


def test_workload_flop_counts():
    w = fi.WORKLOADS["bf16_b4h16n4096d128_causal_x0.5"]
    assert w.fwd_flops() == 4 * 4 * 16 * 4096 * 4096 * 128 / 2
    assert w.bwd_flops() == 2.5 * w.fwd_flops()


@pytest.mark.parametrize("N", [1, 100, 128, 129, 300, 513])
@pytest.mark.parametrize("causal", [False, True])
def test_visible_pairs_matches_element_count(N, causal):
    nb = -(-N // 128)
    mask = fi.random_block_mask(3, nb, 0.5)
    i = np.arange(N)
    vis = mask[i[:, None] // 128, i[None, :] // 128] != 0
    if causal:
        vis &= i[None, :] <= i[:, None]
    assert int(vis.sum()) == fi.visible_pairs(mask, N, 128, causal)


def test_block_masks():
    m = fi.local_global_block_mask(6, 1, 1)
    assert m.dtype == np.uint8 and m.shape == (6, 6)
    assert m[0].all() and m[:, 0].all() and m[3, 2] and m[3, 4] and not m[3, 5] and not m[5, 2]
    a, b = fi.random_block_mask(4, 16, 0.3), fi.random_block_mask(4, 16, 0.3)
    assert np.array_equal(a, b) and 0.1 < a.mean() < 0.5
    w = fi.BLOCK_SPARSE_WORKLOADS["bf16_b2h16n8192d128_local2_global1"]
    assert w.fwd_flops() == 4.0 * 2 * 16 * 128 * 128 * 128 * int(w.mask().sum())


def test_decode_workload_counts():
    w = fi.DecodeWorkload("t", 2, 3, 4, 10, 64, causal=True)
    assert w.visible_pairs() == 7 + 8 + 9 + 10
    assert fi.DecodeWorkload("t", 2, 3, 12, 10, 64, causal=True).visible_pairs() == sum(range(1, 11))
    assert fi.DecodeWorkload("t", 2, 3, 4, 10, 64, causal=False).visible_pairs() == 40
    x = fi.make_decode_inputs(w)
    assert x["q"].shape == (2, 3, 4, 64) and x["k"].shape == (2, 3, 10, 64) and x["k"].dtype == np.uint16
    assert w.hbm_bytes() == 6 * (2 * 4 * 64 * 2 + 2 * 10 * 64 * 2 + 4 * 4)


def test_signs_and_outliers():
    s = fi.random_signs(3, 128)
    assert s.dtype == np.float32 and set(np.unique(s)) == {-1.0, 1.0} and np.array_equal(s, fi.random_signs(3, 128))
    x = np.ones((4, 1000), np.float32)
    y = fi.with_outliers(x, 1, frac=0.01, factor=10.0)
    assert set(np.unique(y)) == {1.0, 10.0} and 10 < (y == 10).sum() < 80 and np.all(x == 1)
