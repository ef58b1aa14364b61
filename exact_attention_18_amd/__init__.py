"""Exact scaled dot-product attention for AMD Instinct MI355X (gfx950).

A thin Python binding over the C ABI of ``libfa.so`` (include/fa.h).  The
functions here only check and marshal arguments: every step of the
computation runs in the HIP kernels.  PyTorch supplies device memory and the
current stream.

Tensors are [B, H, N, d], contiguous, on the GPU, either all bfloat16 or all
float32 (the float32 path is a slower debug path).  ``scale`` defaults to
1/sqrt(d), as ``softmax_scale=None`` does in the call shown on the page "Flash
Attention 2で打破するローカルLLMの「メモリの壁」：IO最適化の実践的エンジニアリング",
section 「カスタムモデルへの組み込み：コード書き換えのポイント」.
"""
from __future__ import annotations

import ctypes
import math

from ._lib import (  # noqa: F401
    FA_ERR_HIP,
    FA_ERR_INVALID_ARG,
    FA_ERR_TOO_LARGE,
    FA_ERR_UNSUPPORTED,
    FA_OK,
    NOALLOC_SCRATCH_BYTES,
    FaLibraryMissing,
    load,
)

__all__ = [
    "FaError",
    "fa_forward",
    "fa_forward_block_sparse",
    "fa_block_sparse_workspace_size",
    "fa_decode",
    "fa_fp8_buffer_size",
    "fa_fp8_prepare",
    "fa_forward_fp8_prepared",
    "fa_forward_fp8",
    "fa_decode_workspace_size",
    "fa_backward",
    "fa_forward_f32",
    "fa_backward_f32",
    "fa_backward_preprocess",
    "fa_backward_dkdv",
    "fa_backward_dq",
    "fa_backward_dq_delta",
    "fa_backward_workspace_size",
    "fa_backward_noalloc",
    "fa_backward_atomic",
    "fa_backward_atomic_workspace_size",
    "backward_atomic",
    "NOALLOC_SCRATCH_BYTES",
    "fa_status_string",
    "fa_abi_version",
    "forward",
    "forward_block_sparse",
    "decode",
    "prepare_fp8",
    "forward_fp8",
    "DECODE_MAX_QUERIES",
    "backward",
    "BLOCK_SPARSE_BLOCK",
]

BLOCK_SPARSE_BLOCK = 128  # side of a block-sparse mask block (FA_BLOCK_SPARSE_BLOCK)
DECODE_MAX_QUERIES = 8    # FA_DECODE_MAX_QUERIES


class FaError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(fa_status_string(status))


def _call(name: str, *args) -> int:
    return getattr(load(), name)(*args)


# --- raw C-ABI calls (same names as include/fa.h; pointers as ints) ---------

def fa_forward(q, k, v, o, lse, B, H, N, d, causal, scale, stream) -> int:
    return _call("fa_forward", q, k, v, o, lse, B, H, N, d, int(causal), float(scale), stream)


def fa_forward_block_sparse(q, k, v, o, lse, block_mask, B, H, N, d, causal, scale, ws, ws_bytes, stream) -> int:
    return _call("fa_forward_block_sparse", q, k, v, o, lse, block_mask, B, H, N, d, int(causal),
                 float(scale), ws, ws_bytes, stream)


def fa_block_sparse_workspace_size(B, H, N, d) -> int:
    return int(_call("fa_block_sparse_workspace_size", B, H, N, d))


def fa_decode(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, ws, ws_bytes, stream) -> int:
    return _call("fa_decode", q, k, v, o, lse, B, H, Nq, Nk, d, int(causal), float(scale), ws, ws_bytes, stream)


def fa_decode_workspace_size(B, H, Nq, Nk, d) -> int:
    return int(_call("fa_decode_workspace_size", B, H, Nq, Nk, d))


def fa_fp8_buffer_size(B, H, N, d) -> int:
    return int(_call("fa_fp8_buffer_size", B, H, N, d))


def fa_fp8_prepare(q, k, v, signs, B, H, N, d, buf, buf_bytes, stream) -> int:
    return _call("fa_fp8_prepare", q, k, v, signs, B, H, N, d, buf, buf_bytes, stream)


def fa_forward_fp8_prepared(buf, buf_bytes, o, lse, B, H, N, d, causal, scale, rotated, stream) -> int:
    return _call("fa_forward_fp8_prepared", buf, buf_bytes, o, lse, B, H, N, d, int(causal), float(scale),
                 int(rotated), stream)


def fa_forward_fp8(q, k, v, signs, o, lse, B, H, N, d, causal, scale, buf, buf_bytes, stream) -> int:
    return _call("fa_forward_fp8", q, k, v, signs, o, lse, B, H, N, d, int(causal), float(scale), buf,
                 buf_bytes, stream)


def fa_forward_f32(q, k, v, o, lse, B, H, N, d, causal, scale, stream) -> int:
    return _call("fa_forward_f32", q, k, v, o, lse, B, H, N, d, int(causal), float(scale), stream)


def fa_backward(q, k, v, o, lse, do, dq, dk, dv, B, H, N, d, causal, scale, ws, ws_bytes, stream) -> int:
    return _call("fa_backward", q, k, v, o, lse, do, dq, dk, dv, B, H, N, d, int(causal), float(scale),
                 ws, ws_bytes, stream)


def fa_backward_preprocess(o, do, B, H, N, d, ws, ws_bytes, stream) -> int:
    return _call("fa_backward_preprocess", o, do, B, H, N, d, ws, ws_bytes, stream)


def fa_backward_dkdv(q, k, v, lse, do, dk, dv, B, H, N, d, causal, scale, ws, ws_bytes, stream) -> int:
    return _call("fa_backward_dkdv", q, k, v, lse, do, dk, dv, B, H, N, d, int(causal), float(scale), ws,
                 ws_bytes, stream)


def fa_backward_dq(q, k, v, lse, do, dq, B, H, N, d, causal, scale, ws, ws_bytes, stream) -> int:
    return _call("fa_backward_dq", q, k, v, lse, do, dq, B, H, N, d, int(causal), float(scale), ws,
                 ws_bytes, stream)


def fa_backward_dq_delta(q, k, v, o, lse, do, dq, B, H, N, d, causal, scale, ws, ws_bytes, stream) -> int:
    return _call("fa_backward_dq_delta", q, k, v, o, lse, do, dq, B, H, N, d, int(causal), float(scale), ws,
                 ws_bytes, stream)


def fa_backward_f32(q, k, v, o, lse, do, dq, dk, dv, B, H, N, d, causal, scale, ws, ws_bytes, stream) -> int:
    return _call("fa_backward_f32", q, k, v, o, lse, do, dq, dk, dv, B, H, N, d, int(causal),
                 float(scale), ws, ws_bytes, stream)


def fa_backward_workspace_size(B, H, N, d) -> int:
    return int(_call("fa_backward_workspace_size", B, H, N, d))


def fa_backward_atomic_workspace_size(B, H, N, d) -> int:
    return int(_call("fa_backward_atomic_workspace_size", B, H, N, d))


def fa_backward_atomic(q, k, v, o, lse, do, dq, dk, dv, B, H, N, d, causal, scale, ws, ws_bytes, stream) -> int:
    return _call("fa_backward_atomic", q, k, v, o, lse, do, dq, dk, dv, B, H, N, d, int(causal),
                 float(scale), ws, ws_bytes, stream)


def fa_backward_noalloc(q, k, v, o, lse, do, dq, dk, dv, B, H, N, d, causal, scale, stream) -> int:
    return _call("fa_backward_noalloc", q, k, v, o, lse, do, dq, dk, dv, B, H, N, d, int(causal), float(scale),
                 stream)


def fa_status_string(status: int) -> str:
    return _call("fa_status_string", int(status)).decode()


def fa_abi_version() -> int:
    return int(_call("fa_abi_version"))


# --- torch tensor wrappers -------------------------------------------------

def _check(ts, names):
    import torch

    t0 = ts[0]
    if t0.dim() != 4:
        raise ValueError(f"{names[0]} must be [B, H, N, d], got shape {tuple(t0.shape)}")
    if t0.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"unsupported dtype {t0.dtype}; use bfloat16 or float32")
    for t, n in zip(ts, names):
        if t.shape != t0.shape or t.dtype != t0.dtype:
            raise ValueError(f"{n}: shape/dtype {tuple(t.shape)}/{t.dtype} does not match {names[0]}")
        if not t.is_cuda or t.device != t0.device:
            raise ValueError(f"{n} must be on the same GPU as {names[0]}")
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous [B, H, N, d]")
    return t0.dtype == torch.float32


def _stream(device):
    import torch

    return torch.cuda.current_stream(device).cuda_stream


def forward(q, k, v, causal: bool = False, scale: float | None = None):
    """O, LSE = attention(q, k, v).  Returns (o [B,H,N,d], lse [B,H,N] float32)."""
    import torch

    f32 = _check([q, k, v], ["q", "k", "v"])
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fn = fa_forward_f32 if f32 else fa_forward
    st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
            causal, scale, _stream(q.device))
    if st != FA_OK:
        raise FaError(st)
    return o, lse


def forward_block_sparse(q, k, v, block_mask, causal: bool = False, scale: float | None = None,
                         balance: bool = True, workspace=None):
    """Block-sparse attention (bf16): query i sees key j iff
    ``block_mask[i // 128, j // 128]`` is nonzero (and j <= i when causal).

    ``block_mask`` is a [ceil(N/128), ceil(N/128)] uint8 or bool tensor on the
    same GPU.  Rows that see no key get o = 0 and lse = -inf.  With
    ``balance`` heavy mask rows are split over several workgroups (a
    workspace is allocated unless one is passed).
    """
    import torch

    _check([q, k, v], ["q", "k", "v"])
    if q.dtype != torch.bfloat16:
        raise TypeError("forward_block_sparse takes bfloat16 tensors")
    B, H, N, d = q.shape
    nb = -(-N // BLOCK_SPARSE_BLOCK)
    if block_mask.shape != (nb, nb) or block_mask.dtype not in (torch.uint8, torch.bool):
        raise ValueError(f"block_mask must be a uint8/bool [{nb}, {nb}] tensor")
    if not block_mask.is_cuda or block_mask.device != q.device or not block_mask.is_contiguous():
        raise ValueError("block_mask must be contiguous and on the same GPU as q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    ws_ptr, ws_bytes = 0, 0
    if balance:
        need = fa_block_sparse_workspace_size(B, H, N, d)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = fa_forward_block_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                 block_mask.data_ptr(), B, H, N, d, causal, scale, ws_ptr, ws_bytes,
                                 _stream(q.device))
    if st != FA_OK:
        raise FaError(st)
    return o, lse


def decode(q, k, v, causal: bool = True, scale: float | None = None, workspace=None):
    """Decode-phase attention (bf16): ``q`` [B, H, Nq, d] holds the queries of
    the last Nq positions (1 <= Nq <= 8) of a sequence whose keys and values
    ``k``, ``v`` are [B, H, Nk, d].  Returns (o [B, H, Nq, d], lse [B, H, Nq])."""
    import torch

    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if t.dim() != 4 or t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous bfloat16 [B, H, N, d] tensor on the GPU")
        if t.device != q.device:
            raise ValueError(f"{n} must be on the same GPU as q")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != k.shape:
        raise ValueError(f"k and v must be [B, H, Nk, d] = {(B, H, Nk, d)}, got {tuple(k.shape)}, {tuple(v.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_decode_workspace_size(B, H, Nq, Nk, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    st = fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Nq, Nk, d,
                   causal, scale, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                   _stream(q.device))
    if st != FA_OK:
        raise FaError(st)
    return o, lse


def _fp8_args(q, k, v, signs):
    import torch

    _check([q, k, v], ["q", "k", "v"])
    if q.dtype != torch.bfloat16:
        raise TypeError("the FP8 path takes bfloat16 tensors")
    if signs is not None and (signs.dtype != torch.float32 or signs.numel() != q.shape[-1]
                              or not signs.is_cuda or not signs.is_contiguous()):
        raise ValueError("signs must be a contiguous float32 vector of d entries on the GPU")
    return q.shape


def prepare_fp8(q, k, v, signs=None, buf=None):
    """Quantise Q, K (rotated by ``signs`` when given) and V to FP8 into a
    uint8 buffer (layout in include/fa.h) and return it."""
    import torch

    B, H, N, d = _fp8_args(q, k, v, signs)
    need = fa_fp8_buffer_size(B, H, N, d)
    if need == 0:
        raise FaError(-2)
    if buf is None:
        buf = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = fa_fp8_prepare(q.data_ptr(), k.data_ptr(), v.data_ptr(), 0 if signs is None else signs.data_ptr(),
                        B, H, N, d, buf.data_ptr(), buf.numel(), _stream(q.device))
    if st != FA_OK:
        raise FaError(st)
    return buf


def forward_fp8(q, k, v, signs=None, causal: bool = False, scale: float | None = None, buf=None):
    """FP8 forward with incoherent processing (bf16 in/out, d = 128):
    returns (o [B,H,N,d], lse [B,H,N])."""
    import torch

    B, H, N, d = _fp8_args(q, k, v, signs)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_fp8_buffer_size(B, H, N, d)
    if need == 0:
        raise FaError(-2)
    if buf is None:
        buf = torch.empty(need, dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    st = fa_forward_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), 0 if signs is None else signs.data_ptr(),
                        o.data_ptr(), lse.data_ptr(), B, H, N, d, causal, scale, buf.data_ptr(), buf.numel(),
                        _stream(q.device))
    if st != FA_OK:
        raise FaError(st)
    return o, lse


def backward(q, k, v, o, lse, do, causal: bool = False, scale: float | None = None, workspace=None):
    """dQ, dK, dV for the incoming gradient ``do`` of attention(q, k, v)."""
    import torch

    f32 = _check([q, k, v, o, do], ["q", "k", "v", "o", "do"])
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    need = fa_backward_workspace_size(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fn = fa_backward_f32 if f32 else fa_backward
    st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, causal, scale,
            workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q.device))
    if st != FA_OK:
        raise FaError(st)
    return dq, dk, dv


def backward_atomic(q, k, v, o, lse, do, causal: bool = False, scale: float | None = None, workspace=None):
    """dQ, dK, dV from the single-pass backward (bf16 only): dK and dV equal
    ``backward``'s bit for bit; dQ is accumulated with float32 atomics, so its
    last bits depend on their order."""
    import torch

    if _check([q, k, v, o, do], ["q", "k", "v", "o", "do"]):
        raise ValueError("backward_atomic takes bf16 tensors")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    need = fa_backward_atomic_workspace_size(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    st = fa_backward_atomic(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, causal, scale,
                            workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q.device))
    if st != FA_OK:
        raise FaError(st)
    return dq, dk, dv

