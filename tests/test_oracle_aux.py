"""Pins of the oracle's directional steering ("【#8】ds4.c 해독하기",
directional-steering section: y - scale * dir * (dir . y)) and activation
wire formats ("【#6】ds4.c 분석하기", distributed-transport passage: f16 and
E4M3 on the wire) against closed forms, numpy's binary16 conversion and a
brute-force search over the E4M3 code table (CPU only)."""
import numpy as np

import oracle
import synth


# ---------------------------------------------------------------- steering

def _unit(rng, n):
    d = rng.standard_normal(n)
    return (d / np.linalg.norm(d)).astype(np.float32)


def test_steer_scale_zero_is_identity():
    rng = np.random.default_rng(1)
    y = rng.standard_normal((3, 64)).astype(np.float32)
    assert np.array_equal(oracle.steer(_unit(rng, 64), 0.0, y), y)


def test_steer_unit_scale_one_removes_the_direction():
    rng = np.random.default_rng(2)
    d = _unit(rng, 256)
    y = rng.standard_normal((4, 256)).astype(np.float32)
    out = oracle.steer(d, 1.0, y).astype(np.float64)
    # the component along dir is gone (up to the f32 rounding of dir and out)
    assert np.max(np.abs(out @ d.astype(np.float64))) < 1e-4
    # the orthogonal part is untouched
    p = y.astype(np.float64) - np.outer(y.astype(np.float64) @ d, d)
    assert np.max(np.abs(out - p)) < 1e-5


def test_steer_parallel_row_scales_by_one_minus_s():
    d = np.zeros(16, np.float32)
    d[3] = 1.0
    y = (np.arange(16, dtype=np.float32) * 0 + 0).reshape(1, 16)
    y[0, 3] = 8.0
    for s in (0.5, -1.5, 2.0):
        out = oracle.steer(d, s, y)
        ref = np.zeros_like(y)
        ref[0, 3] = 8.0 * (1.0 - s)
        assert np.array_equal(out, ref)


def test_steer_hand_example_with_residual():
    # dir = (1, 2), y = (3, 4): dir.y = 11; s = 0.25 -> y - 0.25*11*(1, 2)
    d = np.array([1.0, 2.0], np.float32)
    y = np.array([[3.0, 4.0]], np.float32)
    r = np.array([[10.0, -10.0]], np.float32)
    out = oracle.steer(d, 0.25, y, residual=r)
    assert np.array_equal(out, np.array([[10.0 + 3.0 - 2.75, -10.0 + 4.0 - 5.5]], np.float32))


# ---------------------------------------------------------------- f16

def _f16_cases():
    rng = np.random.default_rng(3)
    specials = np.array([0.0, -0.0, 1.0, -2.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e9, -1e9,
                         2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25,
                         6.1e-5, 1e-8, np.inf, -np.inf], dtype=np.float32)
    # exact ties between adjacent binary16 values (both parities)
    h = rng.integers(0, 0x7BFF, 2000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    ties = ((lo + hi) / 2).astype(np.float32)
    rnd = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000)]).astype(np.float32)
    bits = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    return np.concatenate([specials, ties, -ties, rnd, bits[np.isfinite(bits)]])


def test_f16_rne_matches_numpy():
    x = _f16_cases()
    got = oracle.f16_rne(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_f16_rne_nan_is_canonical_quiet():
    got = oracle.f16_rne(np.array([np.nan, -np.nan], np.float32))
    assert list(got) == [0x7E00, 0xFE00]


# ---------------------------------------------------------------- E4M3

def _e4m3_table():
    # the definition: sign, 4 exponent bits (bias 7), 3 mantissa bits,
    # e = 0 subnormal (m/8 * 2^-6), e = 15 m = 7 NaN, no infinities
    vals = []
    for b in range(256):
        s, e, m = b >> 7, (b >> 3) & 15, b & 7
        if e == 15 and m == 7:
            v = np.nan
        elif e == 0:
            v = m / 8.0 * 2.0 ** -6
        else:
            v = (1 + m / 8.0) * 2.0 ** (e - 7)
        vals.append(-v if s else v)
    return np.array(vals)


def test_e4m3_decode_all_codes():
    t = _e4m3_table()
    got = oracle.e4m3_value(np.arange(256))
    nan = np.isnan(t)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], t[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0


def _e4m3_brute(x: float) -> int:
    """Nearest finite code by exhaustive search; ties to the even mantissa;
    beyond the largest finite value: saturate."""
    t = _e4m3_table()
    if np.isnan(x):
        return 0xFF if np.signbit(x) else 0x7F
    sign = 0x80 if np.signbit(x) else 0
    a = abs(float(x))
    best, bd = None, None
    for b in range(0x7F):  # non-negative finite codes 0x00..0x7E
        d = abs(t[b] - a)
        if bd is None or d < bd or (d == bd and (b & 1) == 0):
            best, bd = b, d
    return sign | best


def test_e4m3_rne_matches_brute_force():
    rng = np.random.default_rng(4)
    t = _e4m3_table()
    fin = np.sort(np.unique(np.abs(t[np.isfinite(t)])))
    mids = ((fin[1:] + fin[:-1]) / 2).astype(np.float32)
    xs = np.concatenate([
        np.array([0.0, -0.0, 448.0, 449.0, 463.99, 464.0, 470.0, 480.0, 1e6, np.inf, -np.inf,
                  2.0 ** -9, 2.0 ** -10, 1.5 * 2.0 ** -10, 2.0 ** -11, 2.0 ** -6, 0.015], np.float32),
        mids, -mids, fin.astype(np.float32) * np.float32(1.0 + 1e-6),
        (rng.standard_normal(3000) * 10.0 ** rng.integers(-4, 3, 3000)).astype(np.float32),
    ])
    got = oracle.e4m3_rne(xs)
    ref = np.array([_e4m3_brute(v) for v in xs], dtype=np.uint8)
    assert np.array_equal(got, ref)
    assert oracle.e4m3_rne(np.array([np.nan], np.float32))[0] == 0x7F


# ---------------------------------------------------------------- steering, fp64 form

def test_steer_f64_hand_example_and_sign():
    # dir = (1, 2), y = (3, 4): dir.y = 11.  s = 0.25 subtracts 0.25*11*(1, 2).
    d = np.array([1.0, 2.0], np.float32)
    y = np.array([[3.0, 4.0]])
    assert np.array_equal(oracle.steer_f64(d, 0.25, y), np.array([[0.25, -1.5]]))
    # a negative scale adds the direction instead (amplification)
    assert np.array_equal(oracle.steer_f64(d, -0.25, y), np.array([[5.75, 9.5]]))
    # the input is left untouched (the binding copies)
    assert np.array_equal(y, np.array([[3.0, 4.0]]))


def test_steer_f64_projection_reflection_and_parallel_rows():
    rng = np.random.default_rng(5)
    dd = rng.standard_normal(512)
    dd /= np.linalg.norm(dd)
    d = dd.astype(np.float32)
    d64 = d.astype(np.float64)
    y = rng.standard_normal((5, 512)) * 3.0
    a = y @ d64
    # scale 1 leaves no component along a unit direction; scale 2 reflects it
    n2 = float(d64 @ d64)                      # 1 up to the f32 rounding of dir
    assert np.max(np.abs(oracle.steer_f64(d, 1.0, y) @ d64 - a * (1.0 - n2))) < 1e-12
    assert np.max(np.abs(oracle.steer_f64(d, 2.0, y) @ d64 - a * (1.0 - 2.0 * n2))) < 1e-12
    # the part orthogonal to dir is unchanged for every scale
    for s in (0.5, 1.0, -0.75):
        out = oracle.steer_f64(d, s, y)
        perp = lambda v: v - np.outer(v @ d64, d64) / n2
        assert np.max(np.abs(perp(out) - perp(y))) < 1e-12
    # a row parallel to dir scales by (1 - s |dir|^2)
    par = np.outer([2.0, -1.0], d64)
    for s in (0.3, 1.0, 1.7):
        assert np.allclose(oracle.steer_f64(d, s, par), par * (1.0 - s * n2), rtol=0, atol=1e-14)


def test_steer_f64_equals_float_form_on_exact_inputs():
    # small integers and a power-of-two scale keep every intermediate exact in
    # both forms, so the fp64 result rounded once equals the float form
    rng = np.random.default_rng(6)
    d = rng.integers(-3, 4, 64).astype(np.float32)
    y = rng.integers(-50, 51, (7, 64)).astype(np.float32)
    for s in (0.0, 0.25, -0.5, 1.0, 2.0):
        f64 = oracle.steer_f64(d, s, y.astype(np.float64))
        ref = y.astype(np.float64) - s * np.outer(y.astype(np.float64) @ d, d)
        assert np.array_equal(f64, ref)
        assert np.array_equal(f64.astype(np.float32), oracle.steer(d, s, y))
