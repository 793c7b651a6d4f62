"""Pins of the block-scaled FP8 oracle (oracle/mx.py) against the element formats' definitions,
brute force, the per-row quantiser and closed forms."""
import numpy as np
import pytest

from oracle import fp8 as F
from oracle import moe as O
from oracle import mx as M


def test_e5m2_known_codes():
    """Values fixed by the E5M2 definition: bias 15, 2 mantissa bits, subnormals m 2^-16, largest
    finite 57344, exponent field 31 = infinity (mantissa 0) or NaN, sign in bit 7."""
    table = {0x00: 0.0, 0x01: 2.0 ** -16, 0x03: 3 * 2.0 ** -16, 0x04: 2.0 ** -14, 0x07: 1.75 * 2.0 ** -14,
             0x38: 0.5, 0x3C: 1.0, 0x3D: 1.25, 0x3E: 1.5, 0x3F: 1.75, 0x40: 2.0, 0x42: 3.0, 0x78: 32768.0,
             0x7B: 57344.0, 0x80: -0.0, 0xBC: -1.0, 0xFB: -57344.0}
    for c, v in table.items():
        assert M.e5m2_decode(c) == v, hex(c)
    assert np.signbit(M.e5m2_decode(0x80))
    assert M.e5m2_decode(0x7C) == np.inf and M.e5m2_decode(0xFC) == -np.inf
    for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF):
        assert np.isnan(M.e5m2_decode(c))


def test_e5m2_round_trip_order_and_nearest_by_brute_force():
    codes = np.array([c for c in range(256) if (c & 0x7F) <= 0x7B])
    vals = M.e5m2_decode(codes)
    assert np.array_equal(M.e5m2_encode(vals), codes.astype(np.uint8))
    grid = M.e5m2_decode(np.arange(0, 0x7C))
    assert np.all(np.diff(grid) > 0)
    rng = np.random.default_rng(13)
    mids = (grid[1:] + grid[:-1]) / 2
    probe = np.concatenate([rng.uniform(0, 57344, 1000), rng.uniform(0, 2 ** -12, 500), mids,
                            np.nextafter(mids, 0), np.nextafter(mids, 1e6), grid])
    for sgn in (1.0, -1.0):
        got = M.e5m2_encode(sgn * probe).astype(np.int64)
        for v, c in zip(probe, got):
            dd = np.abs(grid - v)
            best = np.flatnonzero(dd == dd.min())
            want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
            assert (c & 0x7F) == want, (v, c, want)
            assert ((c >> 7) == 1) == (sgn < 0)
    assert M.e5m2_encode(1.125) == 0x3C          # tie between 1.0 (0x3C) and 1.25 (0x3D): even
    assert M.e5m2_encode(1.375) == 0x3E          # tie between 0x3D and 0x3E
    with pytest.raises(ValueError):
        M.e5m2_encode(57345.0)


@pytest.mark.parametrize("fmt", M.FORMATS)
def test_block_scale_is_the_smallest_power_of_two(fmt):
    top = M.max_finite(fmt)
    rng = np.random.default_rng(17)
    for amax in np.concatenate([rng.lognormal(0, 8, 400), [top, top * (1 + 2 ** -20), 1.0, 2.0 ** -60]]):
        k = M.block_scale_exponent(amax, fmt)
        assert amax / 2.0 ** k <= top < amax / 2.0 ** (k - 1)
    assert M.block_scale_exponent(0.0, fmt) == 0
    assert M.block_scale_exponent(top, fmt) == 0 and M.block_scale_exponent(np.nextafter(top, 1e9), fmt) == 1
    assert M.block_scale_exponent(2.0 ** -200, fmt) == -127          # E8M0 floor


@pytest.mark.parametrize("fmt", M.FORMATS)
def test_blocks_are_independent_and_rows_reduce_to_the_row_quantiser(fmt):
    """A block's codes and scale depend on that block only; an E4M3 row whose largest magnitude
    occurs in every block gets the per-row quantiser's codes, with the row scale in every block."""
    rng = np.random.default_rng(19)
    X = rng.standard_normal((6, 128)) * rng.lognormal(0, 4, (6, 1))
    c0, s0 = M.quantize_blocks(X, fmt)
    Y = X.copy()
    Y[:, 64:96] *= 1000.0
    c1, s1 = M.quantize_blocks(Y, fmt)
    keep = np.r_[0:64, 96:128]
    assert np.array_equal(c0[:, keep], c1[:, keep]) and np.array_equal(s0[:, [0, 1, 3]], s1[:, [0, 1, 3]])
    assert np.all(s1[:, 2] > s0[:, 2])
    if fmt == "e4m3":
        Z = rng.standard_normal((5, 96))
        for b in range(3):
            Z[:, 32 * b + 5] = 3.0
        Z = np.clip(Z, -2.9, 3.0)
        cz, sz = M.quantize_blocks(Z, fmt)
        cr, sr = F.quantize_rows(Z)
        assert np.array_equal(cz, cr)
        assert np.array_equal(2.0 ** (sz.astype(np.float64) - 127), np.repeat(sr[:, None], 3, axis=1))


@pytest.mark.parametrize("fmt", M.FORMATS)
def test_quantize_blocks_error_bound(fmt):
    """Every element is within half a code spacing (at its magnitude, in its block's scale) of its
    dequantised value; zero blocks give zero codes and scale byte 127."""
    mbits, emin = (3, -6) if fmt == "e4m3" else (2, -14)
    rng = np.random.default_rng(23)
    X = rng.standard_normal((20, 160)) * rng.lognormal(0, 3, (20, 5)).repeat(32, axis=1)
    X[4, 32:64] = 0.0
    codes, sc = M.quantize_blocks(X, fmt)
    D = M.dequantize_blocks(codes, sc, fmt)
    s = np.repeat(2.0 ** (sc.astype(np.float64) - 127), 32, axis=1)
    q = np.abs(X) / s
    e = np.floor(np.log2(np.maximum(q, 2.0 ** emin)))
    spacing = 2.0 ** (e - mbits) * s
    assert np.all(np.abs(D - X) <= spacing / 2 + 1e-300)
    assert sc[4, 1] == 127 and np.all(codes[4, 32:64] == 0)
    assert np.all(np.abs(decoded := M.decode(codes, fmt)) <= M.max_finite(fmt)) and np.all(np.isfinite(decoded))


@pytest.mark.parametrize("fmt", M.FORMATS)
def test_mx_ffn_is_the_ffn_of_the_dequantised_operands(fmt):
    """The block-scaled expert FFN equals the plain SwiGLU FFN of oracle/moe.py evaluated on the
    dequantised operands."""
    rng = np.random.default_rng(29)
    T, d, n, E = 20, 64, 32, 3
    X = rng.standard_normal((T, d))
    Wg = rng.standard_normal((E, n, d)) / 8
    Wu = rng.standard_normal((E, n, d)) / 8
    Wd = rng.standard_normal((E, d, n)) / 6
    plan = O.build_plan(rng.standard_normal((T, E)), 2)
    Xq, sx = M.quantize_blocks(X, fmt)
    q = {k: [M.quantize_blocks(W[e], fmt) for e in range(E)] for k, W in (("g", Wg), ("u", Wu), ("d", Wd))}
    cw = {k: [c for c, _ in v] for k, v in q.items()}
    sw = {k: [s for _, s in v] for k, v in q.items()}
    Xd = M.dequantize_blocks(Xq, sx, fmt)
    R = plan["expert_off"][-1]
    for e in range(E):
        r0, r1 = plan["expert_off"][e], plan["expert_off"][e + 1]
        if r1 == r0:
            continue
        G, U, A = M.ffn_mx_up(Xq, sx, cw["g"], sw["g"], cw["u"], sw["u"], plan["row_token"], plan["expert_off"],
                               e, fmt)
        xe = Xd[plan["row_token"][r0:r1]]
        wg, wu, wd = (M.dequantize_blocks(cw[k][e], sw[k][e], fmt) for k in ("g", "u", "d"))
        assert np.allclose(G, xe @ wg.T, rtol=1e-12, atol=1e-12)
        assert np.allclose(A @ wd.T, O.swiglu_expert_forward(xe, wg, wu, wd)[3], rtol=1e-10, atol=1e-10)
        Aq = np.zeros((R, n), np.uint8)
        sa = np.full((R, n // 32), 127, np.uint8)
        Aq[r0:r1], sa[r0:r1] = M.quantize_blocks(A, fmt)
        Y = M.ffn_mx_down(Aq, sa, cw["d"], sw["d"], plan["expert_off"], e, fmt)
        assert np.allclose(Y, M.dequantize_blocks(Aq[r0:r1], sa[r0:r1], fmt) @ wd.T, rtol=1e-12, atol=1e-12)
