"""fa_backward_noalloc (the backward on the library's static scratch) against
fa_backward on the same inputs, through the C ABI: two calls in a row, the
second on a smaller problem, each bit-identical to fa_backward and within the
bf16 tolerance of the oracle; and the size limit."""
from __future__ import annotations

import math

import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.gpu_util import dev, host64, max_abs, random_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_18_amd as fa

    fa._lib.load()  # raises if the HIP library is missing: no fallback
    return fa


def _run_both(fa, B, H, N, d, causal, seed):
    import torch

    q, k, v, do = random_inputs(seed, (B, H, N, d), "bf16", 4)
    scale = 1.0 / math.sqrt(d)
    tq, tk, tv, tdo = dev(q), dev(k), dev(v), dev(do)
    o, lse = fa.forward(tq, tk, tv, causal=causal, scale=scale)
    ref = fa.backward(tq, tk, tv, o, lse, tdo, causal=causal, scale=scale)
    got = [torch.full_like(tq, float("nan")) for _ in range(3)]
    sp = torch.cuda.current_stream().cuda_stream
    st = fa.fa_backward_noalloc(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                tdo.data_ptr(), got[0].data_ptr(), got[1].data_ptr(), got[2].data_ptr(),
                                B, H, N, d, int(causal), scale, sp)
    assert st == 0, fa.fa_status_string(st)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
    exact = oracle.attention_backward(*(fi.exact_f64(a[:1, :1]) for a in (q, k, v, do)), causal, scale)
    for name, a, r in zip(("dQ", "dK", "dV"), got, exact):
        assert max_abs(host64(a[:1, :1]), r) <= 2e-2, name


def test_noalloc_backward_two_calls(fa):
    # the first call is large enough to take the two-launch backward (dQ
    # computing -delta into the scratch, then dK/dV reading it); the second
    # is smaller and takes the one-launch form after the row-dot pass
    _run_both(fa, 4, 16, 2048, 128, True, 11)
    _run_both(fa, 1, 3, 333, 64, False, 12)


def test_noalloc_backward_size_limit(fa):
    import torch

    t = torch.zeros(16, dtype=torch.bfloat16, device="cuda:0")
    lse = torch.zeros(16, dtype=torch.float32, device="cuda:0")
    p = [t.data_ptr()] * 4 + [lse.data_ptr(), t.data_ptr()]
    outs = [torch.zeros(16, dtype=torch.bfloat16, device="cuda:0").data_ptr() for _ in range(3)]
    rows = fa.NOALLOC_SCRATCH_BYTES // 4
    # one row more than the scratch holds: rejected before any buffer is used
    st = fa.fa_backward_noalloc(*p, *outs, 1, 1, rows + 1, 64, 0, 0.125, 0)
    assert st == fa.FA_ERR_TOO_LARGE
    assert "scratch" in fa.fa_status_string(st)
