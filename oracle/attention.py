"""Oracle for exact scaled dot-product attention: plain, slow, fp64, on the CPU.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
calls it, and it shares no code with the GPU kernels.

What it computes, and where that is defined:

* The result is the scaled dot-product attention formula
  Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V, printed on the page
  "Flash Attention 2で打破するローカルLLMの「メモリの壁」：IO最適化の実践的エンジニアリング",
  section 「標準的なAttention機構のメモリ挙動」.  The same section lays out the
  plain three-pass way to evaluate it: form the score matrix S = Q K^T, turn it
  into the probability matrix P = softmax(S), then form O = P V.  The oracle
  follows those three passes, materialising S and P in full for each
  (batch, head), which is exactly what the fast kernels avoid.
* The softmax scale is an argument (``softmax_scale`` in the call shown in
  section 「カスタムモデルへの組み込み：コード書き換えのポイント」 of the same
  page); the workloads pass 1/sqrt(d).
* ``causal`` masks key j from query i when j > i (top-left aligned square mask,
  so the first query sees only the first key).  The pages name causal
  attention (``causal=True`` in the call above; the causal and non-causal
  benchmark runs in section 「約2倍という数値の対象を確認する」 of
  "FlashAttention-2を読む：長い文脈のアテンションをGPUで効率化する仕組み") but
  do not spell out its alignment; top-left is the reading taken.
* LSE (the log-sum-exp of each row of masked, scaled scores, natural log) is an
  output the pages do not mention.  It is the one number per row that lets a
  backward pass rebuild P without storing it, which the same page describes in
  section 「タイリング（Tiling）と再計算（Recomputation）の仕組み」.
* The backward pass is the exact vector-Jacobian product of O with respect to
  Q, K and V.  The pages print no formula for it; the closed form used here
  follows from the three passes above by the chain rule (softmax Jacobian
  diag(p) - p p^T).

All arithmetic is float64.  Inputs are first widened exactly to float64.
Matrix products use numpy's ``matmul`` (BLAS); no blocking, fusion or
reordering is applied beyond those products.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "scores",
    "softmax_rows",
    "attention_forward",
    "attention_forward_rows",
    "attention_backward",
    "attention_backward_dq_rows",
    "block_visibility",
    "attention_forward_block_sparse",
    "attention_forward_block_sparse_rows",
    "attention_forward_kv",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def scores(q: np.ndarray, k: np.ndarray, causal: bool, scale: float,
           rows: np.ndarray | None = None) -> np.ndarray:
    """First pass: S = scale * Q K^T for one (batch, head), masked.

    ``q`` is [Nq, d] (or the selected ``rows`` of a [N, d] query matrix),
    ``k`` is [Nk, d].  Masked entries are -inf.  ``rows`` gives the query
    positions of the rows of ``q`` (defaults to 0..Nq-1); the causal mask
    hides key j from the query at position i when j > i.
    """
    q = _f64(q)
    k = _f64(k)
    s = float(scale) * (q @ k.T)
    if causal:
        nq, nk = s.shape
        pos = np.arange(nq) if rows is None else np.asarray(rows)
        hidden = np.arange(nk)[None, :] > pos[:, None]
        s = np.where(hidden, -np.inf, s)
    return s


def softmax_rows(s: np.ndarray):
    """Second pass: P = softmax(S) along each row, plus the row log-sum-exp.

    The row maximum is subtracted before exponentiating; in exact arithmetic
    that changes nothing and it keeps exp() from overflowing.  Returns
    (P, LSE) with LSE_i = m_i + log(sum_j exp(S_ij - m_i)).
    """
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = np.sum(e, axis=-1, keepdims=True)
    p = e / z
    lse = (m + np.log(z))[..., 0]
    return p, lse


def attention_forward(q, k, v, causal: bool, scale: float, return_p: bool = False):
    """Exact attention over [B, H, N, d] tensors.

    Returns (O [B,H,N,d], LSE [B,H,N]) in float64, and P [B,H,N,N] when
    ``return_p`` is set (tiny inputs only).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    o = np.empty((B, H, N, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    ps = np.empty((B, H, N, k.shape[2]), dtype=np.float64) if return_p else None
    for b in range(B):
        for h in range(H):
            s = scores(q[b, h], k[b, h], causal, scale)
            p, l = softmax_rows(s)
            o[b, h] = p @ v[b, h]  # third pass: O = P V
            lse[b, h] = l
            if return_p:
                ps[b, h] = p
    if return_p:
        return o, lse, ps
    return o, lse


def attention_forward_rows(q_bh, k_bh, v_bh, rows, causal: bool, scale: float):
    """The forward restricted to some query rows of one (batch, head).

    Row i of O depends only on row i of S, so this is the same definition
    evaluated for the listed rows only.  ``q_bh`` is [N, d]; returns
    (O [len(rows), d], LSE [len(rows)]).
    """
    rows = np.asarray(rows)
    s = scores(_f64(q_bh)[rows], k_bh, causal, scale, rows=rows)
    p, l = softmax_rows(s)
    return p @ _f64(v_bh), l


def attention_backward(q, k, v, do, causal: bool, scale: float):
    """Vector-Jacobian product of O = softmax(scale * Q K^T, masked) V.

    Given dO (the gradient of a scalar loss with respect to O), returns
    (dQ, dK, dV), all [B,H,N,d] float64.  Per (batch, head), with P from the
    forward passes:
        dV = P^T dO
        dP = dO V^T
        dS = P * (dP - rowsum(P * dP))      (softmax Jacobian, row by row)
        dQ = scale * dS K
        dK = scale * dS^T Q
    Masked entries have P = 0, so they contribute nothing.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    B, H = q.shape[:2]
    for b in range(B):
        for h in range(H):
            s = scores(q[b, h], k[b, h], causal, scale)
            p, _ = softmax_rows(s)
            g = do[b, h]
            dv[b, h] = p.T @ g
            dp = g @ v[b, h].T
            rowdot = np.sum(p * dp, axis=-1, keepdims=True)
            ds = p * (dp - rowdot)
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
    return dq, dk, dv


def attention_backward_dq_rows(q_bh, k_bh, v_bh, do_bh, rows, causal: bool, scale: float):
    """dQ of ``attention_backward`` restricted to some query rows of one
    (batch, head).

    Row i of dQ needs only row i of P, dP and dS (dS_i = P_i * (dP_i -
    rowsum(P_i * dP_i)), dQ_i = scale * dS_i K), so this is the same
    definition evaluated for the listed rows.  Inputs are [N, d]; returns
    dQ [len(rows), d].
    """
    rows = np.asarray(rows)
    k, v = _f64(k_bh), _f64(v_bh)
    s = scores(_f64(q_bh)[rows], k, causal, scale, rows=rows)
    p, _ = softmax_rows(s)
    dp = _f64(do_bh)[rows] @ v.T
    ds = p * (dp - np.sum(p * dp, axis=-1, keepdims=True))
    return scale * (ds @ k)


def block_visibility(block_mask: np.ndarray, n: int, block: int) -> np.ndarray:
    """Element visibility [n, n] of a block mask: key j is visible to query i
    when block_mask[i // block, j // block] is nonzero."""
    bm = np.asarray(block_mask) != 0
    idx = np.arange(n) // block
    return bm[idx[:, None], idx[None, :]]


def attention_forward_block_sparse(q, k, v, block_mask, block: int, causal: bool, scale: float):
    """Block-sparse attention: the exact attention of the pages restricted to
    the key blocks a caller-supplied mask marks visible.

    The page "FlashAttention――GPUメモリの読み書きを減らし、注意機構を正確なまま高速・省メモリに"
    (要約, 手法) extends FlashAttention to block-sparse attention without
    spelling out its definition; the reading taken here: key j is visible to
    query i iff block_mask[i // block, j // block] is nonzero (and j <= i when
    causal); the softmax runs over the visible keys only.  A row with no
    visible key has O = 0 and LSE = -inf.

    ``block_mask`` is [ceil(N/block), ceil(N/block)], shared by every (batch,
    head).  Returns (O, LSE) in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    vis = block_visibility(block_mask, N, block)
    o = np.zeros((B, H, N, v.shape[-1]), dtype=np.float64)
    lse = np.full((B, H, N), -np.inf, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s = scores(q[b, h], k[b, h], causal, scale)
            s = np.where(vis, s, -np.inf)
            live = np.isfinite(s).any(axis=1)
            if not live.any():
                continue
            p, l = softmax_rows(s[live])
            o[b, h, live] = p @ v[b, h]
            lse[b, h, live] = l
    return o, lse


def attention_forward_block_sparse_rows(q_bh, k_bh, v_bh, rows, block_mask, block: int,
                                        causal: bool, scale: float):
    """``attention_forward_block_sparse`` for some query rows of one (batch,
    head): the same definition evaluated for the listed rows only.  ``q_bh``
    is [N, d]; returns (O [len(rows), d], LSE [len(rows)]); a row with no
    visible key gets O = 0 and LSE = -inf."""
    rows = np.asarray(rows)
    n = np.asarray(k_bh).shape[0]
    vis = block_visibility(block_mask, n, block)[rows]
    s = scores(_f64(q_bh)[rows], k_bh, causal, scale, rows=rows)
    s = np.where(vis, s, -np.inf)
    o = np.zeros((len(rows), np.asarray(v_bh).shape[-1]), dtype=np.float64)
    lse = np.full(len(rows), -np.inf, dtype=np.float64)
    live = np.isfinite(s).any(axis=1)
    if live.any():
        p, l = softmax_rows(s[live])
        o[live] = p @ _f64(v_bh)
        lse[live] = l
    return o, lse


def attention_forward_kv(q, k, v, causal: bool, scale: float):
    """Attention of Nq new queries over Nk cached keys (the decode phase).

    The page "Flash Attention 2で打破するローカルLLMの「メモリの壁」：IO最適化の実践的
    エンジニアリング" (section 「実装上の差を検証可能な形で残す」) separates the prefill
    phase from the decode phase without defining decode further; the reading
    taken here: ``q`` [B,H,Nq,d] holds the queries of the last Nq positions
    Nk-Nq .. Nk-1 of a sequence whose keys and values ``k``, ``v`` [B,H,Nk,d]
    are all present.  Non-causal, every query sees every key; causal, the
    query at position p sees keys j <= p (the square causal mask aligned at
    the bottom right).  A query that sees no key (possible only when Nq > Nk)
    gets O = 0 and LSE = -inf.  Returns (O [B,H,Nq,d], LSE [B,H,Nq]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, nq, d = q.shape
    nk = k.shape[2]
    pos = np.arange(nk - nq, nk)
    o = np.zeros((B, H, nq, v.shape[-1]), dtype=np.float64)
    lse = np.full((B, H, nq), -np.inf, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s = scores(q[b, h], k[b, h], causal, scale, rows=pos)
            live = np.isfinite(s).any(axis=1)
            if not live.any():
                continue
            p, l = softmax_rows(s[live])
            o[b, h, live] = p @ v[b, h]
            lse[b, h, live] = l
    return o, lse
