"""FP8 (OCP E4M3) row quantisation and the FP8 expert FFN (test infrastructure only).

apxml.com page "硬件加速的考量", section "利用稀疏性和量化" / "量化": lowering the precision of
weights and activations (FP16, BF16, INT8 or FP8) shrinks the experts' storage, the bytes moved
when the active experts are loaded, and the time on low-precision matrix units.  The pages give
no number format, scaling rule or placement of the quantisation steps.  Readings taken:

* Element format: OCP FP8 E4M3 -- sign, 4 exponent bits with bias 7, 3 mantissa bits, no
  infinities, codes 0x7F / 0xFF are NaN, largest finite value 448, subnormals m * 2^-9.
  Rounding to the nearest code, ties to the even code (the one with an even last bit).
* Scaling: one scale per row of each operand -- each token row of an activation matrix and each
  output channel (row) of a weight matrix: the smallest power of two ``s`` with
  ``max|row| / s <= 448``; a row of zeros has ``s = 1``.  A power of two makes ``x / s`` exact in
  any binary precision, so the encoding decision is the same here and in a kernel.
* The quantised FFN of expert e for token rows r (x_t = X[t_r]):
  ``G = (s_x[t] sg[e][j]) sum_k q(x)[t][k] q(Wg)[e][j][k]`` and likewise U, the activation
  ``A = silu(G) U`` (stored in bf16 by the kernels), A quantised per row, then
  ``Y[r][c] = (s_a[r] sd[e][c]) sum_j q(A)[r][j] q(Wd)[e][c][j]``.  In words: the SwiGLU FFN of the
  pages evaluated exactly on the dequantised operands.

Plain Python / numpy, float64; nothing here is shared with the HIP library.
"""

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Value of each E4M3 code (NaN for 0x7F and 0xFF).  OCP FP8 E4M3 definition."""
    c = np.asarray(codes, np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.power(2.0, e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return s * mag


def e4m3_encode(q):
    """Nearest E4M3 code of each finite value with |q| <= 448, ties to even.

    As an integer, a non-negative code is monotone in its value: subnormals are m * 2^-9 with
    code m (0..7, and m = 8 is the smallest normal), a normal value (8 + m) 2^(e-10) has code
    8 e + m.  So the code is the rounded value in units of the spacing of its binade, offset by
    the binade's first code.
    """
    q = np.asarray(q, np.float64)
    if not np.all(np.isfinite(q)) or np.any(np.abs(q) > E4M3_MAX):
        raise ValueError("e4m3_encode needs finite values with |q| <= 448")
    a = np.abs(q)
    sub = a < 2.0 ** -6
    code = np.zeros(q.shape, np.int64)
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)  # numpy rint: ties to even
    f, ex = np.frexp(a[~sub])                                # a = f 2^ex, f in [0.5, 1)
    e = ex - 1                                               # a in [2^e, 2^(e+1))
    t = f * 16.0 - 8.0                                       # position inside the binade, [0, 8)
    code[~sub] = (e + 7) * 8 + np.rint(t).astype(np.int64)
    code = code | np.where(np.signbit(q), 0x80, 0)
    assert np.all((code & 0x7F) <= 0x7E)
    return code.astype(np.uint8)


def row_scale(amax):
    """Smallest power of two s with amax / s <= 448 (1 for amax = 0)."""
    amax = float(amax)
    if amax == 0.0:
        return 1.0
    f, ex = np.frexp(amax)           # amax = f 2^ex, f in [0.5, 1): amax / 448 = (2f / 1.75) 2^(ex-9)
    return float(2.0 ** (ex - 9 + (1 if f > 0.875 else 0)))


def quantize_rows(X):
    """Per-row power-of-two scale and E4M3 codes of a 2-D array: codes [rows, K] uint8 and
    scales [rows] float64 with X ~= decode(codes) * scales[:, None]."""
    X = np.asarray(X, np.float64)
    scales = np.array([row_scale(np.max(np.abs(row))) if row.size else 1.0 for row in X])
    codes = e4m3_encode(X / scales[:, None])
    return codes, scales


def dequantize_rows(codes, scales):
    return e4m3_decode(codes) * np.asarray(scales, np.float64)[:, None]


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def ffn_fp8_up(Xq, sx, Wgq, sg, Wuq, su, row_token, expert_off, e):
    """Expert e's gate/up projection and SwiGLU activation on its rows (exact, float64):
    returns G, U and A = silu(G) U for rows expert_off[e] .. expert_off[e+1]-1.
    Weights are indexed one expert at a time (``Wgq[e]`` etc.)."""
    r0, r1 = int(expert_off[e]), int(expert_off[e + 1])
    tok = np.asarray(row_token[r0:r1], np.int64)
    x = e4m3_decode(Xq[tok]) * np.asarray(sx, np.float64)[tok][:, None]
    wg = e4m3_decode(Wgq[e]) * np.asarray(sg[e], np.float64)[:, None]
    wu = e4m3_decode(Wuq[e]) * np.asarray(su[e], np.float64)[:, None]
    G = x @ wg.T
    U = x @ wu.T
    return G, U, G * _sigmoid(G) * U


def ffn_fp8_down(Aq, sa, Wdq, sd, expert_off, e):
    """Expert e's down projection on its (quantised) activation rows, exact: Y rows
    expert_off[e] .. expert_off[e+1]-1."""
    r0, r1 = int(expert_off[e]), int(expert_off[e + 1])
    a = e4m3_decode(Aq[r0:r1]) * np.asarray(sa, np.float64)[r0:r1][:, None]
    wd = e4m3_decode(Wdq[e]) * np.asarray(sd[e], np.float64)[:, None]
    return a @ wd.T
