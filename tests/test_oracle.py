"""The fp64 oracle against facts other than itself (CPU only).

Every pin lives in tests/oracle_pins.py.  Here the battery runs on the real
oracle (all pins must hold) and on copies of the oracle with one planted
mistake each (some pin must fail), which shows the pins would catch that kind
of error.
"""
import inspect
import textwrap

import numpy as np
import pytest

import oracle
from oracle import attention as oa
from tests import oracle_pins as pins


def test_golden_file_parses():
    cases = pins.load_golden()
    assert len(cases) >= 5
    assert any("dq" in c for c in cases)


def test_forward_pins_hold():
    assert pins.forward_pin_failures(oracle.attention_forward) == []


def test_backward_pins_hold():
    assert pins.backward_pin_failures(oracle.attention_backward, oracle.attention_forward) == []


def test_rows_of_p_sum_to_one_and_mask_is_zero():
    r = np.random.default_rng(5)
    q, k, v = (r.standard_normal((2, 3, 17, 8)) for _ in range(3))
    for causal in (False, True):
        _, _, p = oracle.attention_forward(q, k, v, causal, 0.35, return_p=True)
        assert np.allclose(p.sum(-1), 1.0, atol=1e-13, rtol=0)
        assert np.all(p >= 0)
        if causal:
            upper = np.triu(np.ones((17, 17), dtype=bool), 1)
            assert np.all(p[..., upper] == 0.0)


def test_forward_rows_equals_full():
    r = np.random.default_rng(6)
    q, k, v = (r.standard_normal((1, 1, 40, 8)) for _ in range(3))
    rows = np.array([0, 3, 17, 39])
    for causal in (False, True):
        o, lse = oracle.attention_forward(q, k, v, causal, 0.3)
        orow, lrow = oracle.attention_forward_rows(q[0, 0], k[0, 0], v[0, 0], rows, causal, 0.3)
        assert np.array_equal(o[0, 0, rows], orow)
        assert np.array_equal(lse[0, 0, rows], lrow)


def test_backward_dq_rows_equals_full():
    """The row-restricted dQ is the full backward's dQ on those rows (the full
    backward is pinned by finite differences and the softmax identities)."""
    r = np.random.default_rng(16)
    q, k, v, do = (r.standard_normal((1, 1, 40, 8)) for _ in range(4))
    rows = np.array([0, 1, 17, 38, 39])
    for causal in (False, True):
        dq, _, _ = oracle.attention_backward(q, k, v, do, causal, 0.3)
        dqr = oracle.attention_backward_dq_rows(q[0, 0], k[0, 0], v[0, 0], do[0, 0], rows, causal, 0.3)
        assert np.allclose(dq[0, 0, rows], dqr, rtol=1e-12, atol=1e-12)


def test_block_sparse_rows_equals_full():
    r = np.random.default_rng(8)
    q, k, v = (r.standard_normal((1, 1, 40, 8)) for _ in range(3))
    mask = np.array([[1, 0, 0, 1, 0], [0, 0, 0, 0, 0], [1, 1, 0, 0, 1], [0, 1, 1, 1, 0], [1, 1, 1, 1, 1]])
    rows = np.array([0, 3, 9, 17, 30, 39])  # row 9 sits in the empty block row
    for causal in (False, True):
        o, lse = oracle.attention_forward_block_sparse(q, k, v, mask, 8, causal, 0.3)
        orow, lrow = oracle.attention_forward_block_sparse_rows(q[0, 0], k[0, 0], v[0, 0], rows, mask, 8,
                                                                causal, 0.3)
        assert np.array_equal(o[0, 0, rows], orow)
        assert np.array_equal(lse[0, 0, rows], lrow)


def test_large_scores_do_not_overflow():
    # scores near 1e3 would overflow exp() without the max subtraction
    q = np.full((1, 1, 4, 2), 30.0)
    k = np.full((1, 1, 4, 2), 30.0)
    k[0, 0, 2] = 29.0
    v = np.arange(8, dtype=np.float64).reshape(1, 1, 4, 2)
    o, lse = oracle.attention_forward(q, k, v, False, 1.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert np.allclose(lse, 1800.0 + np.log(3 + np.exp(-60.0)), atol=1e-9)


# --- planted mistakes ------------------------------------------------------

def _mutant(func, old, new):
    """Copy of ``func`` from the oracle module with one source substitution."""
    src = textwrap.dedent(inspect.getsource(func))
    assert old in src, (old, func.__name__)
    src = src.replace(old, new, 1)
    ns = dict(vars(oa))
    exec(compile(src, "<mutant>", "exec"), ns)
    return ns[func.__name__], ns


FORWARD_MUTANTS = [
    # (function, original text, planted mistake)
    (oa.scores, "q @ k.T", "k @ q.T"),                                # transposed S
    (oa.scores, "float(scale) * (q @ k.T)", "(q @ k.T)"),             # scale dropped
    (oa.scores, "> pos[:, None]", ">= pos[:, None]"),                 # mask hides the diagonal
    (oa.scores, "> pos[:, None]", "< pos[:, None]"),                  # mask on the wrong side
    (oa.softmax_rows, "np.max(s, axis=-1", "np.max(s, axis=-2"),      # max over the wrong axis
    (oa.softmax_rows, "np.sum(e, axis=-1", "np.sum(e, axis=-2"),      # normalise columns
    (oa.softmax_rows, "(m + np.log(z))", "(np.log(z))"),              # LSE without the max
    (oa.attention_forward, "p @ v[b, h]", "p.T @ v[b, h]"),           # P transposed in PV
    (oa.attention_forward, "s = scores(q[b, h], k[b, h]", "s = scores(k[b, h], q[b, h]"),
]


@pytest.mark.parametrize("func,old,new", FORWARD_MUTANTS, ids=[m[2] for m in FORWARD_MUTANTS])
def test_forward_pins_catch_planted_mistake(func, old, new, monkeypatch):
    mutated, _ = _mutant(func, old, new)
    monkeypatch.setattr(oa, func.__name__, mutated)
    assert pins.forward_pin_failures(oa.attention_forward) != []


BACKWARD_MUTANTS = [
    ("p.T @ g", "p @ g"),                        # dV with P untransposed
    ("g @ v[b, h].T", "g @ v[b, h].T * 0.5"),    # dP scaled wrongly
    ("(dp - rowdot)", "(dp + rowdot)"),          # sign error in the softmax Jacobian
    ("(dp - rowdot)", "(dp)"),                   # dropped term
    ("scale * (ds @ k[b, h])", "(ds @ k[b, h])"),  # dQ without the scale
    ("ds.T @ q[b, h]", "ds @ q[b, h]"),          # dK with dS untransposed
    ("ds @ k[b, h]", "ds.T @ k[b, h]"),          # dQ with dS transposed
    ("np.sum(p * dp, axis=-1", "np.sum(p * dp, axis=-2"),  # row sum over the wrong axis
]


@pytest.mark.parametrize("old,new", BACKWARD_MUTANTS, ids=[m[1] for m in BACKWARD_MUTANTS])
def test_backward_pins_catch_planted_mistake(old, new):
    mutated, _ = _mutant(oa.attention_backward, old, new)
    assert pins.backward_pin_failures(mutated, oracle.attention_forward) != []


def test_block_sparse_pins_hold():
    assert pins.block_sparse_pin_failures(oracle.attention_forward_block_sparse, oracle.attention_forward) == []


BLOCK_SPARSE_MUTANTS = [
    (oa.block_visibility, "bm[idx[:, None], idx[None, :]]", "bm[idx[None, :], idx[:, None]]"),  # transposed mask
    (oa.block_visibility, "np.arange(n) // block", "np.arange(n) // (block + 1)"),             # wrong block size
    (oa.attention_forward_block_sparse, "s = np.where(vis, s, -np.inf)", "s = s"),             # mask ignored
    (oa.attention_forward_block_sparse, "o = np.zeros(", "o = np.ones("),                      # empty rows not zero
]


@pytest.mark.parametrize("func,old,new", BLOCK_SPARSE_MUTANTS, ids=[m[2] for m in BLOCK_SPARSE_MUTANTS])
def test_block_sparse_pins_catch_planted_mistake(func, old, new, monkeypatch):
    mutated, _ = _mutant(func, old, new)
    monkeypatch.setattr(oa, func.__name__, mutated)
    assert pins.block_sparse_pin_failures(oa.attention_forward_block_sparse, oracle.attention_forward) != []


def test_kv_pins_hold():
    assert pins.kv_pin_failures(oracle.attention_forward_kv, oracle.attention_forward) == []


KV_MUTANTS = [
    ("np.arange(nk - nq, nk)", "np.arange(nq)"),            # top-left instead of bottom-right causal
    ("np.arange(nk - nq, nk)", "np.arange(nk - nq + 1, nk + 1)"),  # positions off by one
    ("o = np.zeros(", "o = np.ones("),                       # empty rows not zero
    ("p @ v[b, h]", "p @ v[b, h][::-1]"),                     # values reversed
]


@pytest.mark.parametrize("old,new", KV_MUTANTS, ids=[m[1] for m in KV_MUTANTS])
def test_kv_pins_catch_planted_mistake(old, new):
    mutated, _ = _mutant(oa.attention_forward_kv, old, new)
    assert pins.kv_pin_failures(mutated, oracle.attention_forward) != []


def test_fp8_pins_hold():
    from oracle import fp8
    assert pins.fp8_pin_failures(fp8) == []


FP8_MUTANTS = [
    ("fwht_f32", "np.stack([a + b, a - b]", "np.stack([a + b, b - a]"),              # wrong butterfly sign
    ("block_exponent", "e - 9, e - 8", "e - 8, e - 8"),                              # exponent off by one
    ("e4m3_encode", "(_MAG_CODES[i] & 1) == 0", "(_MAG_CODES[i] & 1) == 1"),          # ties to odd
    ("attention_forward_fp8", "s_scale = float(scale) / d", "s_scale = float(scale)"),  # rotation scale lost
    ("attention_forward_fp8", "kr = fwht_f32(k.astype(np.float32) * sg)",
     "kr = fwht_f32(k.astype(np.float32))"),                                          # K rotated without signs
    ("_dequant_v", "np.swapaxes(_dequant_rows(codes, t), -1, -2)[..., :n, :]",
     "_dequant_rows(codes, t)[..., :n]"),                                              # V used untransposed
    ("e4m3_decode", "(1.0 + m / 8.0)", "(1.0 + m / 16.0)"),                            # wrong mantissa width
    ("p_rounding_bound", "return w @ np.abs(", "return 0.5 * w @ np.abs("),          # bound half as large
    ("p_rounding_bound", "return w @ np.abs(", "return 2.0 * w @ np.abs("),          # bound twice as large
    ("p_rounding_bound", "np.maximum(p, 2.0 ** -6 * p.max", "np.maximum(p, 0.0 * p.max"),  # no subnormal floor
    ("p_rounding_bound", "np.maximum(p, 2.0 ** -6 * p.max", "np.maximum(p, 2.0 ** -5 * p.max"),  # floor too high
    ("p_rounding_bound", "w @ np.abs(np.asarray(vd", "w @ (np.asarray(vd"),          # |v| dropped
]


@pytest.mark.parametrize("func,old,new", FP8_MUTANTS, ids=[m[2] for m in FP8_MUTANTS])
def test_fp8_pins_catch_planted_mistake(func, old, new):
    import types

    from oracle import fp8
    src = inspect.getsource(fp8)
    assert old in src, (func, old)
    mod = types.ModuleType("fp8_mutant")
    mod.__dict__["__name__"] = "oracle.fp8_mutant"
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new, 1), "<fp8 mutant>", "exec"), mod.__dict__)
    try:
        fails = pins.fp8_pin_failures(mod)
    except Exception as e:  # a mutant that breaks a shape or a range also counts as caught
        fails = [repr(e)]
    assert fails != []


def test_fp8_rows_equals_full():
    from oracle import fp8
    r = np.random.default_rng(9)
    q, k, v = (r.standard_normal((1, 1, 150, 128)) for _ in range(3))
    sg = np.where(r.random(128) < 0.5, -1.0, 1.0)
    rows = np.array([0, 5, 63, 64, 149])
    for signs in (None, sg):
        for causal in (False, True):
            o, l, parts = fp8.attention_forward_fp8(q, k, v, signs, causal, 0.09, return_parts=True)
            orow, lrow, brow = fp8.attention_forward_fp8_rows(q[0, 0], k[0, 0], v[0, 0], rows, signs, causal, 0.09)
            assert np.allclose(orow, o[0, 0, rows], rtol=0, atol=1e-13)
            assert np.allclose(lrow, l[0, 0, rows], rtol=0, atol=1e-13)
            assert np.allclose(brow, parts["p_error_bound"][0, 0, rows], rtol=0, atol=1e-13)
