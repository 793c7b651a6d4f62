"""Block-scaled FP8 (E4M3 or E5M2 elements, one power-of-two scale per 32 elements) and the expert
FFN on such operands (test infrastructure only; nothing here is shared with the HIP library).

apxml.com page "硬件加速的考量", section "利用稀疏性和量化" / "量化": weights and activations in a
lower precision such as FP8 shrink the experts and the bytes moved, and run on faster matrix
units.  The pages name FP8 but give no element format, scale granularity or rounding.  Readings
taken for the block-scaled variant (the per-row variant is ``oracle.fp8``):

* Element formats: OCP FP8 E4M3 (bias 7, 3 mantissa bits, no infinities, largest finite 448,
  subnormals m 2^-9) and OCP FP8 E5M2 (bias 15, 2 mantissa bits, exponent field 31 for infinity
  and NaN, largest finite 57344, subnormals m 2^-16).  Encoding: the nearest code, ties to the code
  with an even last bit.
* Scales: every row of an operand is cut along its reduction dimension K into blocks of 32
  consecutive elements, and each block gets the smallest power of two s with
  max|block| / s <= the format's largest finite value (s = 1 for an all-zero block), kept within
  what an E8M0 scale byte holds, 2^-127 .. 2^127.  The byte stored is log2(s) + 127.  The rule is
  the per-row reading applied to each block; a power of two makes x / s exact, so the code of each
  element is decided the same way in any binary precision.
* The expert FFN on such operands is the pages' SwiGLU FFN evaluated exactly on the dequantised
  operands: ``G = deq(X_t) deq(Wg[e])^T`` and likewise U, ``A = silu(G) U``; A (rounded to bf16
  by the kernels) is quantised the same way along its width n; ``Y = deq(A) deq(Wd[e])^T``.
"""

import numpy as np

from . import fp8 as _fp8

BLOCK = 32
E5M2_MAX = 57344.0
FORMATS = ("e4m3", "e5m2")


def e5m2_decode(codes):
    """Value of each E5M2 code (+-inf for exponent field 31 with mantissa 0, NaN otherwise)."""
    c = np.asarray(codes, np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 2) & 31
    m = (c & 3).astype(np.float64)
    with np.errstate(over="ignore"):
        mag = np.where(e == 0, m * 2.0 ** -16, (1.0 + m / 4.0) * np.power(2.0, e - 15.0))
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return s * mag


def e5m2_encode(q):
    """Nearest E5M2 code of each finite value with |q| <= 57344, ties to even.

    A non-negative code is monotone in its value: subnormals m 2^-16 have code m (0..3, and 4 is
    the smallest normal 2^-14); a normal value (4 + m) 2^(e-2) has code 4 (e + 15) + m.  The code
    is the value rounded in units of its binade's spacing, offset by the binade's first code."""
    q = np.asarray(q, np.float64)
    if not np.all(np.isfinite(q)) or np.any(np.abs(q) > E5M2_MAX):
        raise ValueError("e5m2_encode needs finite values with |q| <= 57344")
    a = np.abs(q)
    sub = a < 2.0 ** -14
    code = np.zeros(q.shape, np.int64)
    code[sub] = np.rint(a[sub] * 2.0 ** 16).astype(np.int64)  # numpy rint: ties to even
    f, ex = np.frexp(a[~sub])                                 # a = f 2^ex, f in [0.5, 1)
    e = ex - 1
    t = f * 8.0 - 4.0                                         # position inside the binade, [0, 4)
    code[~sub] = (e + 15) * 4 + np.rint(t).astype(np.int64)
    code = code | np.where(np.signbit(q), 0x80, 0)
    assert np.all((code & 0x7F) <= 0x7B)
    return code.astype(np.uint8)


def decode(codes, fmt):
    return _fp8.e4m3_decode(codes) if fmt == "e4m3" else e5m2_decode(codes)


def encode(q, fmt):
    return _fp8.e4m3_encode(q) if fmt == "e4m3" else e5m2_encode(q)


def max_finite(fmt):
    return _fp8.E4M3_MAX if fmt == "e4m3" else E5M2_MAX


def block_scale_exponent(amax, fmt):
    """log2 of the smallest power of two s with amax / s <= max_finite(fmt), clamped to the E8M0
    range [-127, 127]; 0 for amax = 0.  Elementwise over an array of block maxima."""
    a = np.asarray(amax, np.float64)
    f, ex = np.frexp(a)               # amax = f 2^ex; max_finite = 0.875 2^E with E = 9 or 16
    E = 9 if fmt == "e4m3" else 16
    k = ex.astype(np.int64) - E + (f > 0.875).astype(np.int64)
    k = np.where(a == 0.0, 0, np.clip(k, -127, 127))
    return int(k) if k.ndim == 0 else k


def quantize_blocks(X, fmt):
    """Codes [rows, K] (uint8) and scale bytes [rows, K / 32] (uint8, log2(s) + 127) of a 2-D
    array whose K is a multiple of 32; X ~= decode(codes) * 2^(scale - 127) block by block."""
    X = np.asarray(X, np.float64)
    rows, K = X.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = X.reshape(rows, K // BLOCK, BLOCK)
    k = block_scale_exponent(np.max(np.abs(blocks), axis=2), fmt)      # [rows, K / 32]
    codes = encode(blocks / np.power(2.0, k)[:, :, None], fmt).reshape(rows, K)
    return codes, (k + 127).astype(np.uint8)


def dequantize_blocks(codes, scales, fmt):
    codes = np.asarray(codes)
    s = np.power(2.0, np.asarray(scales, np.float64) - 127.0)
    return decode(codes, fmt) * np.repeat(s, BLOCK, axis=1)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def ffn_mx_up(Xq, sx, Wgq, sg, Wuq, su, row_token, expert_off, e, fmt):
    """Expert e's gate/up projection and SwiGLU activation on its rows, exact on the dequantised
    operands: G, U and A = silu(G) U for rows expert_off[e] .. expert_off[e+1]-1."""
    r0, r1 = int(expert_off[e]), int(expert_off[e + 1])
    tok = np.asarray(row_token[r0:r1], np.int64)
    x = dequantize_blocks(np.asarray(Xq)[tok], np.asarray(sx)[tok], fmt)
    wg = dequantize_blocks(Wgq[e], sg[e], fmt)
    wu = dequantize_blocks(Wuq[e], su[e], fmt)
    G = x @ wg.T
    U = x @ wu.T
    return G, U, G * _sigmoid(G) * U


def ffn_mx_down(Aq, sa, Wdq, sd, expert_off, e, fmt):
    """Expert e's down projection on its quantised activation rows, exact: Y rows
    expert_off[e] .. expert_off[e+1]-1."""
    r0, r1 = int(expert_off[e]), int(expert_off[e + 1])
    a = dequantize_blocks(np.asarray(Aq)[r0:r1], np.asarray(sa)[r0:r1], fmt)
    wd = dequantize_blocks(Wdq[e], sd[e], fmt)
    return a @ wd.T
