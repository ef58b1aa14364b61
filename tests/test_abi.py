"""The C ABI library on the host: it loads, exports every declared symbol, and
rejects bad arguments before any HIP call (so these run with no GPU)."""
import ctypes
import math
import os
import re

import pytest

from exact_attention_18_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

INVALID, UNSUP = _lib.FA_ERR_INVALID_ARG, _lib.FA_ERR_UNSUPPORTED


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(_lib.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_matches_header(lib):
    m = re.search(r"#define\s+FA_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert lib.fa_abi_version() == int(m.group(1))


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4):
        s = lib.fa_status_string(code).decode()
        assert s.startswith("FA_")
    assert lib.fa_status_string(7).decode() == "unknown status"


def test_workspace_size(lib):
    assert lib.fa_backward_workspace_size(8, 16, 2048, 128) == 8 * 16 * 2048 * 4
    assert lib.fa_backward_workspace_size(1, 1, 1, 64) == 256
    assert lib.fa_backward_workspace_size(0, 1, 1, 64) == 0
    assert lib.fa_backward_workspace_size(1, 1, -5, 64) == 0


# Fake device addresses: never dereferenced, because every call below fails
# validation on the host.  Each buffer sits in its own 4 GiB window.
def ptr(i, off=0):
    return (i + 1) << 32 | off


def fwd(lib, B=1, H=1, N=8, d=64, causal=0, scale=0.125, ptrs=None, f32=False):
    p = ptrs or [ptr(i) for i in range(5)]
    fn = lib.fa_forward_f32 if f32 else lib.fa_forward
    return fn(*p, B, H, N, d, causal, scale, None)


def bwd(lib, B=1, H=1, N=8, d=64, causal=0, scale=0.125, ptrs=None, ws_bytes=None, f32=False):
    p = ptrs or [ptr(i) for i in range(10)]
    if ws_bytes is None:
        ws_bytes = lib.fa_backward_workspace_size(B, H, N, d)
    fn = lib.fa_backward_f32 if f32 else lib.fa_backward
    return fn(*p[:9], B, H, N, d, causal, scale, p[9], ws_bytes, None)


@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0), dict(d=0), dict(B=-1), dict(N=-3),
                                dict(causal=2), dict(causal=-1), dict(scale=-0.5),
                                dict(scale=math.inf), dict(scale=math.nan), dict(B=1 << 20, H=1 << 12)])
def test_forward_rejects_bad_sizes(lib, kw, f32):
    assert fwd(lib, f32=f32, **kw) == INVALID
    assert bwd(lib, f32=f32, **kw) == INVALID


@pytest.mark.parametrize("d", [16, 32, 96, 192, 256])
def test_bf16_rejects_unsupported_head_dim(lib, d):
    assert fwd(lib, d=d) == UNSUP
    assert bwd(lib, d=d) == UNSUP


@pytest.mark.parametrize("d", [2, 6, 130, 256])
def test_f32_rejects_unsupported_head_dim(lib, d):
    assert fwd(lib, d=d, f32=True) == UNSUP
    assert bwd(lib, d=d, f32=True) == UNSUP


@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("which", range(5))
def test_forward_rejects_null_and_misaligned(lib, which, f32):
    p = [ptr(i) for i in range(5)]
    p[which] = None
    assert fwd(lib, ptrs=p, f32=f32) == INVALID
    p = [ptr(i) for i in range(5)]
    p[which] = ptr(which, 8)
    assert fwd(lib, ptrs=p, f32=f32) == INVALID


@pytest.mark.parametrize("which", range(10))
def test_backward_rejects_null_and_misaligned(lib, which):
    p = [ptr(i) for i in range(10)]
    p[which] = None
    assert bwd(lib, ptrs=p) == INVALID
    p = [ptr(i) for i in range(10)]
    p[which] = ptr(which, 4)
    assert bwd(lib, ptrs=p) == INVALID


def test_forward_rejects_overlapping_outputs(lib):
    base = [ptr(i) for i in range(5)]
    o_on_q = list(base)
    o_on_q[3] = base[0] + 64  # o starts inside q
    assert fwd(lib, ptrs=o_on_q) == INVALID
    lse_in_o = list(base)
    lse_in_o[4] = base[3] + 16  # lse inside o
    assert fwd(lib, ptrs=lse_in_o) == INVALID


def test_backward_rejects_overlaps_and_small_workspace(lib):
    base = [ptr(i) for i in range(10)]
    p = list(base)
    p[9] = base[6]  # workspace on dq
    assert bwd(lib, ptrs=p) == INVALID
    p = list(base)
    p[7] = base[5]  # dk on dO
    assert bwd(lib, ptrs=p) == INVALID
    need = lib.fa_backward_workspace_size(1, 1, 8, 64)
    assert bwd(lib, ws_bytes=need - 1) == INVALID


def atomic(lib, B=1, H=1, N=8, d=64, causal=0, scale=0.125, ptrs=None, ws_bytes=None):
    p = ptrs or [ptr(i) for i in range(10)]
    if ws_bytes is None:
        ws_bytes = lib.fa_backward_atomic_workspace_size(B, H, N, d)
    return lib.fa_backward_atomic(*p[:9], B, H, N, d, causal, scale, p[9], ws_bytes, None)


def test_backward_atomic_workspace_size(lib):
    # the rows -delta (rounded to 256 bytes), then the float32 dQ accumulator
    assert lib.fa_backward_atomic_workspace_size(8, 16, 2048, 128) == 8 * 16 * 2048 * 4 + 8 * 16 * 2048 * 128 * 4
    assert lib.fa_backward_atomic_workspace_size(1, 1, 1, 64) == 256 + 64 * 4
    assert lib.fa_backward_atomic_workspace_size(0, 1, 1, 64) == 0
    assert lib.fa_backward_atomic_workspace_size(1, 1, -5, 64) == 0


@pytest.mark.parametrize("which", range(10))
def test_backward_atomic_rejects_null_and_misaligned(lib, which):
    p = [ptr(i) for i in range(10)]
    p[which] = None
    assert atomic(lib, ptrs=p) == INVALID
    p = [ptr(i) for i in range(10)]
    p[which] = ptr(which, 4)
    assert atomic(lib, ptrs=p) == INVALID


def test_backward_atomic_rejects_bad_arguments(lib):
    assert atomic(lib, d=96) == UNSUP
    assert atomic(lib, N=0) == INVALID
    assert atomic(lib, causal=2) == INVALID
    need = lib.fa_backward_atomic_workspace_size(1, 1, 8, 64)
    assert atomic(lib, ws_bytes=need - 1) == INVALID
    p = [ptr(i) for i in range(10)]
    p[9] = p[6]  # workspace on dq
    assert atomic(lib, ptrs=p) == INVALID
    p = [ptr(i) for i in range(10)]
    p[8] = p[0] + 64  # dv inside q
    assert atomic(lib, ptrs=p) == INVALID


def test_backward_atomic_too_large_is_refused_before_launch(lib):
    # One head of 2^23 rows of d = 128: 2 GiB per tensor, past the 32-bit
    # buffer offsets of the kernels.  Each tensor fits its own 4 GiB window
    # and the 4 GiB workspace sits apart, so the host checks pass and the
    # launcher refuses the size before any HIP call.
    N, d = 1 << 23, 128
    p = [ptr(2 * i) for i in range(9)] + [ptr(40)]
    assert atomic(lib, N=N, d=d, ptrs=p) == _lib.FA_ERR_HIP


def test_python_binding_names_match_abi():
    import exact_attention_18_amd as fa

    for n in declared_functions():
        assert callable(getattr(fa, n)), n
    assert fa.fa_status_string(-1).startswith("FA_ERR_INVALID_ARG")


def sparse(lib, B=1, H=1, N=300, d=64, causal=0, scale=0.125, ptrs=None, ws=None, ws_bytes=0):
    p = ptrs or [ptr(i) for i in range(6)]
    return lib.fa_forward_block_sparse(*p, B, H, N, d, causal, scale, ws, ws_bytes, None)


@pytest.mark.parametrize("kw", [dict(B=0), dict(N=0), dict(causal=3), dict(scale=-1.0),
                                dict(scale=math.nan), dict(B=1 << 20, H=1 << 12)])
def test_block_sparse_rejects_bad_sizes(lib, kw):
    assert sparse(lib, **kw) == INVALID


@pytest.mark.parametrize("d", [32, 96, 256])
def test_block_sparse_rejects_unsupported_head_dim(lib, d):
    assert sparse(lib, d=d) == UNSUP


@pytest.mark.parametrize("which", range(6))
def test_block_sparse_rejects_null(lib, which):
    p = [ptr(i) for i in range(6)]
    p[which] = None
    assert sparse(lib, ptrs=p) == INVALID


def test_block_sparse_mask_overlap(lib):
    # the byte mask may sit at any address (no case here passes validation:
    # a call that did would launch on these fake addresses), but not inside
    # an output
    p = [ptr(i) for i in range(6)]
    p[5] = p[3] + 1  # mask inside o
    assert sparse(lib, ptrs=p) == INVALID
    p = [ptr(i) for i in range(6)]
    p[5] = p[4] - 2  # mask (3 x 3 bytes for N = 300) runs into lse
    assert sparse(lib, ptrs=p) == INVALID
    p = [ptr(i) for i in range(6)]
    p[3] = p[0] + 16  # o on q
    assert sparse(lib, ptrs=p) == INVALID


def dec(lib, B=1, H=2, Nq=1, Nk=300, d=128, causal=1, scale=0.1, ptrs=None, ws_bytes=None):
    p = ptrs or [ptr(i) for i in range(6)]
    if ws_bytes is None:
        ws_bytes = lib.fa_decode_workspace_size(B, H, Nq, Nk, d)
    return lib.fa_decode(*p[:5], B, H, Nq, Nk, d, causal, scale, p[5], ws_bytes, None)


def test_decode_workspace_size(lib):
    assert lib.fa_decode_workspace_size(1, 1, 1, 1, 64) >= 64 * 4 + 8
    assert lib.fa_decode_workspace_size(8, 16, 1, 16384, 128) > 0
    for bad in [(0, 1, 1, 8, 64), (1, 1, 0, 8, 64), (1, 1, 9, 8, 64), (1, 1, 1, 0, 64), (1, 1, 1, 8, 96)]:
        assert lib.fa_decode_workspace_size(*bad) == 0


@pytest.mark.parametrize("kw", [dict(B=0), dict(Nq=0), dict(Nk=0), dict(causal=2), dict(scale=-1.0),
                                dict(scale=math.inf), dict(Nk=1 << 24)])
def test_decode_rejects_bad_sizes(lib, kw):
    ws = None if "Nk" not in kw or kw["Nk"] > 0 else 1 << 20
    assert dec(lib, ws_bytes=ws, **kw) == INVALID


@pytest.mark.parametrize("kw", [dict(Nq=9), dict(d=96), dict(d=32)])
def test_decode_rejects_unsupported(lib, kw):
    assert dec(lib, ws_bytes=1 << 30, **kw) == UNSUP


@pytest.mark.parametrize("which", range(6))
def test_decode_rejects_null_and_misaligned(lib, which):
    p = [ptr(i) for i in range(6)]
    p[which] = None
    assert dec(lib, ptrs=p) == INVALID
    p = [ptr(i) for i in range(6)]
    p[which] = ptr(which, 8)
    assert dec(lib, ptrs=p) == INVALID


def test_decode_rejects_overlaps_and_small_workspace(lib):
    need = lib.fa_decode_workspace_size(1, 2, 1, 300, 128)
    assert dec(lib, ws_bytes=need - 1) == INVALID
    p = [ptr(i) for i in range(6)]
    p[5] = p[3]  # workspace on o
    assert dec(lib, ptrs=p) == INVALID
    p = [ptr(i) for i in range(6)]
    p[3] = p[1] + 256  # o inside k
    assert dec(lib, ptrs=p) == INVALID


def test_fp8_buffer_size(lib):
    # Np = 128 rows for N = 100: 3 code sections of 128 B per row, 3 scale sections of 4 B per row
    assert lib.fa_fp8_buffer_size(1, 1, 100, 128) == 3 * 128 * 128 + 3 * 128 * 4
    assert lib.fa_fp8_buffer_size(1, 1, 100, 64) == 0
    assert lib.fa_fp8_buffer_size(0, 1, 100, 128) == 0


def fp8_fwd(lib, B=1, H=1, N=100, d=128, causal=0, scale=0.1, ptrs=None, buf_bytes=None):
    p = ptrs or [ptr(i) for i in range(7)]   # q k v signs o lse buf
    if buf_bytes is None:
        buf_bytes = lib.fa_fp8_buffer_size(B, H, N, 128)
    return lib.fa_forward_fp8(*p[:6], B, H, N, d, causal, scale, p[6], buf_bytes, None)


@pytest.mark.parametrize("kw", [dict(B=0), dict(N=0), dict(causal=2), dict(scale=-1.0), dict(buf_bytes=100)])
def test_fp8_rejects_bad_args(lib, kw):
    assert fp8_fwd(lib, **kw) == INVALID


def test_fp8_rejects_d64(lib):
    assert fp8_fwd(lib, d=64) == UNSUP
    assert lib.fa_fp8_prepare(*[ptr(i) for i in range(4)], 1, 1, 100, 64, ptr(6), 1 << 20, None) == UNSUP
    assert lib.fa_forward_fp8_prepared(ptr(6), 1 << 20, ptr(4), ptr(5), 1, 1, 100, 64, 0, 0.1, 1, None) == UNSUP


@pytest.mark.parametrize("which", [0, 1, 2, 4, 5, 6])
def test_fp8_rejects_null_and_misaligned(lib, which):
    p = [ptr(i) for i in range(7)]
    p[which] = None
    assert fp8_fwd(lib, ptrs=p) == INVALID
    p = [ptr(i) for i in range(7)]
    p[which] = ptr(which, 8)
    assert fp8_fwd(lib, ptrs=p) == INVALID


def test_fp8_rejects_overlaps(lib):
    p = [ptr(i) for i in range(7)]
    p[6] = p[4] + 64  # buffer inside o
    assert fp8_fwd(lib, ptrs=p) == INVALID
    p = [ptr(i) for i in range(7)]
    p[6] = p[3]       # buffer on the signs
    assert fp8_fwd(lib, ptrs=p) == INVALID
    need = lib.fa_fp8_buffer_size(1, 1, 100, 128)
    assert lib.fa_forward_fp8_prepared(ptr(6), need, ptr(4), ptr(5), 1, 1, 100, 128, 0, 0.1, 2, None) == INVALID
    assert lib.fa_forward_fp8_prepared(ptr(6), need - 1, ptr(4), ptr(5), 1, 1, 100, 128, 0, 0.1, 1, None) == INVALID
    assert lib.fa_forward_fp8_prepared(ptr(6), need, ptr(6) + 32, ptr(5), 1, 1, 100, 128, 0, 0.1, 1, None) == INVALID


def test_fp8_too_large_is_refused_before_launch(lib):
    # One head of 2^24 rows of d = 128: 4 GiB per bf16 tensor, past the
    # 32-bit offsets of the FP8 attention kernel.  Each buffer gets its own
    # window (q, k, v, o: 4 GiB each; the prepared buffer, ~6.4 GiB, far
    # apart), so the host checks pass and the one-call entry refuses the size
    # before it launches the quantisation.
    N = 1 << 24
    p = [ptr(2 * i) for i in range(6)] + [ptr(60)]
    assert fp8_fwd(lib, N=N, ptrs=p) == _lib.FA_ERR_HIP


def test_block_sparse_workspace(lib):
    need = lib.fa_block_sparse_workspace_size(1, 1, 300, 64)
    assert need > 0 and lib.fa_block_sparse_workspace_size(1, 1, 300, 96) == 0
    assert sparse(lib, ws=ptr(7), ws_bytes=need - 1) == INVALID         # too small
    assert sparse(lib, ws=ptr(7, 8), ws_bytes=need) == INVALID          # misaligned
    assert sparse(lib, ws=ptr(3, 16), ws_bytes=need) == INVALID         # inside o


# ---- fa_backward_noalloc (static scratch): host-side rejections

def bwd_noalloc(lib, B=1, H=1, N=8, d=64, causal=0, scale=0.125, ptrs=None):
    p = ptrs or [ptr(i) for i in range(9)]
    return lib.fa_backward_noalloc(*p, B, H, N, d, causal, scale, None)


@pytest.mark.parametrize("kw", [dict(B=0), dict(N=-1), dict(causal=3), dict(scale=-0.5), dict(scale=math.inf)])
def test_noalloc_rejects_bad_sizes(lib, kw):
    assert bwd_noalloc(lib, **kw) == INVALID


@pytest.mark.parametrize("d", [32, 96, 256])
def test_noalloc_rejects_unsupported_head_dim(lib, d):
    assert bwd_noalloc(lib, d=d) == UNSUP


@pytest.mark.parametrize("which", range(9))
def test_noalloc_rejects_null_misaligned_and_overlap(lib, which):
    p = [ptr(i) for i in range(9)]
    p[which] = None
    assert bwd_noalloc(lib, ptrs=p) == INVALID
    p = [ptr(i) for i in range(9)]
    p[which] = ptr(which, 8)
    assert bwd_noalloc(lib, ptrs=p) == INVALID
    if which >= 6:   # an output starting inside another buffer
        p = [ptr(i) for i in range(9)]
        p[which] = ptr((which + 1) % 9, 16)
        assert bwd_noalloc(lib, ptrs=p) == INVALID


def test_noalloc_size_limit(lib):
    rows = _lib.NOALLOC_SCRATCH_BYTES // 4
    m = re.search(r"#define\s+FA_NOALLOC_SCRATCH_BYTES\s+\((\d+)u << (\d+)\)", open(HEADER).read())
    assert int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES
    assert lib.fa_backward_workspace_size(1, 1, rows, 64) == _lib.NOALLOC_SCRATCH_BYTES
    # the largest problem that fits passes the size check (and then fails on
    # the fake pointers' overlap: every buffer is given the same address)
    same = [ptr(0)] * 9
    assert bwd_noalloc(lib, N=rows, ptrs=same) == INVALID
    assert bwd_noalloc(lib, N=rows + 1) == _lib.FA_ERR_TOO_LARGE
    assert bwd_noalloc(lib, B=2, H=3, N=rows // 6 + 1) == _lib.FA_ERR_TOO_LARGE


# The stages of fa_backward: name -> (number of leading pointer arguments,
# whether causal and scale follow the sizes, indices of the outputs among
# those pointers).  The workspace pointer comes after the sizes.
STAGES = {
    "fa_backward_preprocess": (2, False, ()),
    "fa_backward_dkdv": (7, True, (5, 6)),
    "fa_backward_dq": (6, True, (5,)),
    "fa_backward_dq_delta": (7, True, (6,)),
}


def stage(lib, name, B=1, H=1, N=8, d=64, causal=0, scale=0.125, ptrs=None, ws=None, ws_bytes=None):
    n, has_cs, _ = STAGES[name]
    p = ptrs or [ptr(i) for i in range(n)]
    w = ptr(n) if ws is None else ws
    if ws_bytes is None:
        ws_bytes = lib.fa_backward_workspace_size(B, H, N, d)
    fn = getattr(lib, name)
    if has_cs:
        return fn(*p, B, H, N, d, causal, scale, w, ws_bytes, None)
    return fn(*p, B, H, N, d, w, ws_bytes, None)


@pytest.mark.parametrize("name", sorted(STAGES))
@pytest.mark.parametrize("kw", [dict(B=0), dict(N=-1), dict(d=0), dict(causal=2), dict(scale=math.nan)])
def test_backward_stages_reject_bad_sizes(lib, name, kw):
    if not STAGES[name][1] and ("causal" in kw or "scale" in kw):
        pytest.skip("this stage takes no causal flag or scale")
    assert stage(lib, name, **kw) == INVALID


@pytest.mark.parametrize("name", sorted(STAGES))
def test_backward_stages_reject_null_misaligned_and_small_workspace(lib, name):
    n = STAGES[name][0]
    for which in range(n):
        p = [ptr(i) for i in range(n)]
        p[which] = None
        assert stage(lib, name, ptrs=p) == INVALID, which
        p = [ptr(i) for i in range(n)]
        p[which] = ptr(which, 4)
        assert stage(lib, name, ptrs=p) == INVALID, which
    assert stage(lib, name, ws=0) == INVALID
    need = lib.fa_backward_workspace_size(1, 1, 8, 64)
    assert stage(lib, name, ws_bytes=need - 1) == INVALID


@pytest.mark.parametrize("name", ["fa_backward_dkdv", "fa_backward_dq", "fa_backward_dq_delta"])
def test_backward_stages_reject_outputs_on_inputs_or_workspace(lib, name):
    n, _, outs = STAGES[name]
    for o in outs:
        p = [ptr(i) for i in range(n)]
        p[o] = p[0] + 64  # output starts inside q
        assert stage(lib, name, ptrs=p) == INVALID
        p = [ptr(i) for i in range(n)]
        assert stage(lib, name, ptrs=p, ws=p[o]) == INVALID  # workspace on an output


@pytest.mark.parametrize("name", ["fa_backward_dkdv", "fa_backward_dq", "fa_backward_dq_delta"])
def test_backward_stages_reject_unsupported_head_dim(lib, name):
    assert stage(lib, name, d=100) == UNSUP
