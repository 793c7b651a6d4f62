"""Pins of the FP8 (OCP E4M3) oracle against the format's definition and closed forms."""
import numpy as np
import pytest

from oracle import fp8 as F
from oracle import moe as O


def test_e4m3_known_codes():
    """Values fixed by the E4M3 definition: bias 7, 3 mantissa bits, subnormals m 2^-9, largest
    finite 448, 0x7F / 0xFF NaN, sign in bit 7."""
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6,
             0x30: 0.5, 0x38: 1.0, 0x39: 1.125, 0x40: 2.0, 0x44: 3.0, 0x70: 128.0, 0x78: 256.0, 0x7E: 448.0,
             0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in table.items():
        assert F.e4m3_decode(c) == v, hex(c)
    assert np.signbit(F.e4m3_decode(0x80))
    assert np.isnan(F.e4m3_decode(0x7F)) and np.isnan(F.e4m3_decode(0xFF))


def test_e4m3_round_trip_and_order():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    vals = F.e4m3_decode(codes)
    assert np.array_equal(F.e4m3_encode(vals), codes.astype(np.uint8))
    pos = F.e4m3_decode(np.arange(0, 0x7F))
    assert np.all(np.diff(pos) > 0)  # the positive codes are strictly increasing in value


def test_e4m3_encode_is_nearest_by_brute_force():
    """Against a search over all 127 non-negative codes: the nearest value, ties to the even
    code, for random values, every midpoint and values just beside the midpoints."""
    grid = F.e4m3_decode(np.arange(0, 0x7F))
    rng = np.random.default_rng(3)
    mids = (grid[1:] + grid[:-1]) / 2
    vals = np.concatenate([rng.uniform(0, 448, 2000), rng.uniform(0, 2 ** -5, 500), mids,
                           np.nextafter(mids, 0), np.nextafter(mids, 1000), grid])
    for sgn in (1.0, -1.0):
        got = F.e4m3_encode(sgn * vals).astype(np.int64)
        for v, c in zip(vals, got):
            d = np.abs(grid - v)
            best = np.flatnonzero(d == d.min())
            want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
            assert (c & 0x7F) == want, (v, c, want)
            assert ((c >> 7) == 1) == (sgn < 0)


def test_e4m3_ties_go_to_even():
    assert F.e4m3_encode(1.0625) == 0x38       # between 0x38 (1.0) and 0x39 (1.125)
    assert F.e4m3_encode(1.1875) == 0x3A       # between 0x39 and 0x3A
    assert F.e4m3_encode(1.5 * 2.0 ** -9) == 0x02
    assert F.e4m3_encode(0.5 * 2.0 ** -9) == 0x00
    assert F.e4m3_encode(7.5 * 2.0 ** -9) == 0x08  # rounds up into the first normal binade
    with pytest.raises(ValueError):
        F.e4m3_encode(449.0)


def test_row_scale_is_the_smallest_power_of_two():
    rng = np.random.default_rng(5)
    for amax in np.concatenate([rng.lognormal(0, 6, 500), [448.0, 449.0, 447.0, 1.0, 2.0 ** -20]]):
        s = F.row_scale(amax)
        assert np.log2(s) == np.round(np.log2(s))
        assert amax / s <= 448.0 < amax / (s / 2)
    assert F.row_scale(0.0) == 1.0
    assert F.row_scale(448.0) == 1.0 and F.row_scale(449.0) == 2.0


def test_quantize_rows_error_bound():
    """Each element lies within half a code spacing (at its magnitude) of its dequantised value,
    and the largest element of a row maps to a code of magnitude at most 448."""
    rng = np.random.default_rng(7)
    X = rng.standard_normal((40, 96)) * rng.lognormal(0, 3, (40, 1))
    X[3] = 0.0
    codes, s = F.quantize_rows(X)
    D = F.dequantize_rows(codes, s)
    q = np.abs(X) / s[:, None]
    e = np.floor(np.log2(np.maximum(q, 2.0 ** -6)))
    spacing = np.where(q < 2.0 ** -6, 2.0 ** -9, 2.0 ** (e - 3)) * s[:, None]
    assert np.all(np.abs(D - X) <= spacing / 2 + 1e-300)
    assert np.all(D[3] == 0.0) and s[3] == 1.0


def test_fp8_ffn_is_the_ffn_of_the_dequantised_operands():
    """The quantised expert FFN equals the plain SwiGLU FFN of the oracle evaluated on the
    dequantised inputs (an identity between two independently written statements)."""
    rng = np.random.default_rng(11)
    T, d, n, E = 24, 64, 32, 3
    X = rng.standard_normal((T, d))
    Wg = rng.standard_normal((E, n, d)) / 8
    Wu = rng.standard_normal((E, n, d)) / 8
    Wd = rng.standard_normal((E, d, n)) / 6
    plan = O.build_plan(rng.standard_normal((T, E)), 2)
    Xq, sx = F.quantize_rows(X)
    qg = [F.quantize_rows(Wg[e]) for e in range(E)]
    qu = [F.quantize_rows(Wu[e]) for e in range(E)]
    qd = [F.quantize_rows(Wd[e]) for e in range(E)]
    Wgq, sg = [c for c, _ in qg], [s for _, s in qg]
    Wuq, su = [c for c, _ in qu], [s for _, s in qu]
    Wdq, sd = [c for c, _ in qd], [s for _, s in qd]
    Xd = F.dequantize_rows(Xq, sx)
    for e in range(E):
        r0, r1 = plan["expert_off"][e], plan["expert_off"][e + 1]
        if r1 == r0:
            continue
        G, U, A = F.ffn_fp8_up(Xq, sx, Wgq, sg, Wuq, su, plan["row_token"], plan["expert_off"], e)
        xe = Xd[plan["row_token"][r0:r1]]
        wg, wu = F.dequantize_rows(Wgq[e], sg[e]), F.dequantize_rows(Wuq[e], su[e])
        wd = F.dequantize_rows(Wdq[e], sd[e])
        assert np.allclose(G, xe @ wg.T, rtol=1e-12, atol=1e-12)
        # down on the unquantised activation reproduces the plain expert FFN
        Y_plain = O.swiglu_expert_forward(xe, wg, wu, wd)[3]
        assert np.allclose(A @ wd.T, Y_plain, rtol=1e-10, atol=1e-10)
        Aq = np.zeros((plan["expert_off"][-1], n), np.uint8)
        sa = np.ones(plan["expert_off"][-1])
        Aq[r0:r1], sa[r0:r1] = F.quantize_rows(A)
        Y = F.ffn_fp8_down(Aq, sa, Wdq, sd, plan["expert_off"], e)
        assert np.allclose(Y, F.dequantize_rows(Aq[r0:r1], sa[r0:r1]) @ wd.T, rtol=1e-12, atol=1e-12)
