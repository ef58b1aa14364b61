"""Oracle for the FP8 forward with incoherent processing: plain, slow, on the CPU.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the GPU kernels.

What it computes, and where that is described:

* The page "FlashAttention-3 — FlashAttention-3", section
  「3. 量子化誤差を低減した低精度（FP8）」, describes FP8 attention with incoherent
  processing: before quantising, the query and key vectors are multiplied by
  a random orthogonal matrix such as a Hadamard matrix, which spreads large
  outlier entries over all coordinates; because the matrix is orthogonal the
  product Q K^T is unchanged, and the FP8 error drops (about 2.6x on the
  page).  The pages fix no FP8 format, no scaling and no matrix; the readings
  taken here are:

  - FP8 is OCP E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
    subnormals, largest finite 448, codes 0x7f/0xff NaN), rounding to nearest
    with ties to even, a sign kept on zero.
  - The random orthogonal matrix is D H / sqrt(d): a diagonal of random
    signs D (an input) followed by the Sylvester Hadamard matrix H (entries
    +-1).  The rotated vectors x D H are formed in float32 by the fast
    Walsh-Hadamard butterfly (stages of width 1, 2, 4, ..., d/2; each pair
    (a, b) becomes (a + b, a - b)); the 1/sqrt(d) of both Q and K is folded
    into the softmax scale as 1/d.
  - Scales are powers of two, one per block of 32 consecutive elements (of a
    row of Q or K; of a column of V over 32 consecutive keys), the smallest
    2^t with amax <= 448 * 2^t, so no value saturates.
  - The attention itself is then exact (float64) on the dequantised values.
    The kernel also rounds P to FP8 before the P V product; that rounding is
    not modelled here, and the tests bound its effect (``p_rounding_bound``,
    derived from the E4M3 format's spacing and pinned against a simulation of
    that rounding).

* The exact attention that the FP8 path approximates is the three-pass
  definition of ``oracle.attention``.
"""
from __future__ import annotations

import numpy as np

from .attention import scores, softmax_rows

__all__ = [
    "E4M3_MAX",
    "e4m3_decode",
    "e4m3_encode",
    "hadamard_matrix",
    "fwht_f32",
    "block_exponent",
    "quantize_rows",
    "quantize_v",
    "attention_forward_fp8",
    "attention_forward_fp8_rows",
    "p_rounding_bound",
]

E4M3_MAX = 448.0
BLOCK = 32
V_TILE = 64


def e4m3_decode(codes) -> np.ndarray:
    """float64 value of each OCP E4M3 code (NaN for 0x7f and 0xff)."""
    c = np.asarray(codes, dtype=np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7))
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


_MAG_CODES = np.arange(0x7F)                   # finite non-negative codes 0x00 .. 0x7e
_MAG_VALUES = e4m3_decode(_MAG_CODES)          # increasing


def e4m3_encode(x) -> np.ndarray:
    """OCP E4M3 code of each value, round to nearest, ties to the even code.

    |x| must not exceed 464 (the midpoint above 448), where the format has no
    finite value; the sign is kept, also on a zero result (-0 -> 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > 464.0) or np.any(np.isnan(a)):
        raise ValueError("value outside the finite E4M3 range")
    i = np.clip(np.searchsorted(_MAG_VALUES, a), 1, len(_MAG_VALUES) - 1)
    lo, hi = _MAG_VALUES[i - 1], _MAG_VALUES[i]
    d_lo, d_hi = a - lo, hi - a
    take_hi = np.where(d_lo == d_hi, (_MAG_CODES[i] & 1) == 0, d_hi < d_lo)
    take_hi = np.where(a >= hi, True, take_hi)
    mag = np.where(take_hi, _MAG_CODES[i], _MAG_CODES[i - 1])
    sign = np.signbit(x).astype(np.int64)
    return (mag | (sign << 7)).astype(np.uint8)


def hadamard_matrix(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (a power of two), entries +-1."""
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht_f32(x) -> np.ndarray:
    """x H along the last axis, in float32, by the butterfly stages in the
    order stated in the module docstring (width 1 first)."""
    y = np.array(x, dtype=np.float32)
    d = y.shape[-1]
    h = 1
    while h < d:
        z = y.reshape(*y.shape[:-1], d // (2 * h), 2, h)
        a, b = z[..., 0, :], z[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(y.shape)
        h *= 2
    return y


def block_exponent(amax) -> np.ndarray:
    """Smallest integer t with amax <= 448 * 2^t (0 when amax is 0)."""
    a = np.asarray(amax, dtype=np.float64)
    m, e = np.frexp(a)                  # a = m 2^e, 0.5 <= m < 1
    t = np.where(m <= 0.875, e - 9, e - 8)   # 448 = 0.875 * 2^9
    return np.where(a > 0, t, 0).astype(np.int64)


def quantize_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """Codes [..., d] and block exponents [..., d/32] of float32 rows."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    xb = x.reshape(*x.shape[:-1], d // BLOCK, BLOCK).astype(np.float64)
    t = block_exponent(np.abs(xb).max(axis=-1))
    codes = e4m3_encode(xb * np.exp2(-t.astype(np.float64))[..., None])
    return codes.reshape(x.shape), t


def quantize_v(v) -> tuple[np.ndarray, np.ndarray]:
    """Codes and exponents of V [..., N, d] in blocks of 32 consecutive keys
    per column: returns codes [..., d, Np] (V transposed, keys in order,
    Np = N rounded up to a multiple of 64, keys past N zero) and exponents
    [..., d, Np/32]."""
    v = np.asarray(v, dtype=np.float64)
    n, d = v.shape[-2:]
    np_ = -(-n // V_TILE) * V_TILE
    vt = np.zeros((*v.shape[:-2], d, np_), dtype=np.float32)
    vt[..., :n] = np.swapaxes(v, -1, -2)
    return quantize_rows(vt)


def _dequant_rows(codes, t):
    d = codes.shape[-1]
    vals = e4m3_decode(codes).reshape(*codes.shape[:-1], d // BLOCK, BLOCK)
    return (vals * np.exp2(t.astype(np.float64))[..., None]).reshape(codes.shape)


def _dequant_v(codes, t, n):
    return np.swapaxes(_dequant_rows(codes, t), -1, -2)[..., :n, :]


def p_rounding_bound(p, vd) -> np.ndarray:
    """Bound on how far rounding the weights to E4M3 can move the output.

    ``p`` [..., M, N] holds normalised weights (rows sum to 1, hidden keys
    0), ``vd`` [..., N, d] the values.  A kernel evaluates the weights
    unnormalised, p'_j = 2^(x_j - m) against a reference m at most 8 (log2
    units) below the row maximum, so the largest p'_j of a row lies in
    [1, 2^8], below the largest finite E4M3 value.  Rounding p'_j to nearest
    E4M3 moves it by at most half a spacing: 2^-4 p'_j where p'_j >= 2^-6 (3
    mantissa bits), and 2^-10 = 2^-4 2^-6 below that (the subnormal spacing
    is 2^-9).  Divided by the row sum l >= max_j p'_j >= 1, the normalised
    weight P_j moves by at most 2^-4 max(P_j, 2^-6 max_j P_j).  So each
    output element O_ic moves by at most 2^-4 times

        sum over visible j of max(P_j, 2^-6 max_j P_j) |v_jc|,

    which this function returns (without the factor 2^-4)."""
    p = np.asarray(p, dtype=np.float64)
    w = np.maximum(p, 2.0 ** -6 * p.max(axis=-1, keepdims=True))
    w = np.where(p > 0, w, 0.0)     # hidden keys carry no weight
    return w @ np.abs(np.asarray(vd, dtype=np.float64))


def attention_forward_fp8(q, k, v, signs, causal: bool, scale: float, return_parts: bool = False):
    """FP8 forward as stated in the module docstring.

    ``q, k, v`` [B, H, N, d] (the exact input values), ``signs`` a length-d
    vector of +-1 (None: no rotation).  Returns (O, LSE) in float64, and with
    ``return_parts`` also a dict with the codes and exponents of Q, K, V,
    the dequantised operands and ``p_error_bound`` [B, H, N, d]: the
    ``p_rounding_bound`` of the weights and the dequantised V, i.e. how far
    rounding the weights to E4M3 can move O, divided by 2^-4."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    if signs is not None:
        sg = np.asarray(signs, dtype=np.float32)
        qr = fwht_f32(q.astype(np.float32) * sg)
        kr = fwht_f32(k.astype(np.float32) * sg)
        s_scale = float(scale) / d
    else:
        qr, kr = q.astype(np.float32), k.astype(np.float32)
        s_scale = float(scale)
    q8, qt = quantize_rows(qr)
    k8, kt = quantize_rows(kr)
    v8, vt = quantize_v(v)
    qd, kd, vd = _dequant_rows(q8, qt), _dequant_rows(k8, kt), _dequant_v(v8, vt, N)
    o = np.empty((B, H, N, d))
    lse = np.empty((B, H, N))
    bound = np.empty((B, H, N, d)) if return_parts else None
    for b in range(B):
        for h in range(H):
            p, l = softmax_rows(scores(qd[b, h], kd[b, h], causal, s_scale))
            o[b, h] = p @ vd[b, h]
            lse[b, h] = l
            if return_parts:
                bound[b, h] = p_rounding_bound(p, vd[b, h])
    if not return_parts:
        return o, lse
    return o, lse, {"q8": q8, "qt": qt, "k8": k8, "kt": kt, "v8": v8, "vt": vt,
                    "qd": qd, "kd": kd, "vd": vd, "p_error_bound": bound}


def attention_forward_fp8_rows(q_bh, k_bh, v_bh, rows, signs, causal: bool, scale: float):
    """``attention_forward_fp8`` for some query rows of one (batch, head):
    ``q_bh``, ``k_bh``, ``v_bh`` are [N, d]; the rows of Q quantise
    independently, so only the listed rows are rotated and quantised, while
    K and V are quantised whole.  Returns (O [len(rows), d], LSE [len(rows)],
    p_error_bound [len(rows), d])."""
    rows = np.asarray(rows)
    q = np.asarray(q_bh, dtype=np.float64)[rows]
    k = np.asarray(k_bh, dtype=np.float64)
    v = np.asarray(v_bh, dtype=np.float64)
    n, d = k.shape
    if signs is not None:
        sg = np.asarray(signs, dtype=np.float32)
        qr, kr = fwht_f32(q.astype(np.float32) * sg), fwht_f32(k.astype(np.float32) * sg)
        s_scale = float(scale) / d
    else:
        qr, kr = q.astype(np.float32), k.astype(np.float32)
        s_scale = float(scale)
    qd = _dequant_rows(*quantize_rows(qr))
    kd = _dequant_rows(*quantize_rows(kr))
    vd = _dequant_v(*quantize_v(v), n)
    p, lse = softmax_rows(scores(qd, kd, causal, s_scale, rows=rows))
    return p @ vd, lse, p_rounding_bound(p, vd)
