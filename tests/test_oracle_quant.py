"""Pins of the 8-bit KV oracle (oracle/quant_oracle.py) against things other
than itself.  E4M3: the values the OCP FP8 E4M3 format fixes (1.0, 448, 2^-6, 2^-9,
NaN), torch's CPU float8_e4m3fn dtype (decode of all 256 codes, and its
round-to-nearest-even cast in range), brute force over the 254-entry codebook
with ties to an even mantissa, the format's error bound, and attention over
values already on the grid, which must equal the float oracle exactly.
int8: torch's round-half-even cast, brute force at the midpoints, the clamp
and special values, exact round trips and attention on grid values.
Mutations planted in a copy of the module must each fail one of them."""

import inspect
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import quant_oracle as Q

CODES = np.arange(256, dtype=np.uint8)


def _pins(mod):
    """All pins against a module with the quant oracle's functions."""
    # values the format fixes
    dec = mod.e4m3_decode(np.array([0x38, 0x7E, 0x08, 0x01, 0x07, 0x00, 0xB8, 0x40], dtype=np.uint8))
    assert dec.tolist() == [1.0, 448.0, 2.0 ** -6, 2.0 ** -9, 7 * 2.0 ** -9, 0.0, -1.0, 2.0]
    assert np.isnan(mod.e4m3_decode(np.array([0x7F, 0xFF], dtype=np.uint8))).all()
    # torch's float8_e4m3fn reads every code the same way
    ref = torch.from_numpy(CODES.copy()).view(torch.float8_e4m3fn).double().numpy()
    got = mod.e4m3_decode(CODES)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all() and (np.signbit(got) == np.signbit(ref)).all()
    # round trip of every code but NaN
    finite = CODES[~np.isnan(ref)]
    assert (mod.e4m3_quantize(ref[~np.isnan(ref)]) == finite).all()
    # torch's cast (round to nearest even) on random float32 values in range
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 150.0)])
    x = np.clip(x, -448, 448).astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (mod.e4m3_quantize(x.astype(np.float64)) == want).all()
    # brute force: nearest codebook value, ties to the even code (even mantissa)
    vals = ref[:0x7F]                      # +0 .. 448, increasing with the code
    mids = (vals[1:] + vals[:-1]) / 2      # exact midpoints (float64)
    probe = np.concatenate([mids, mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20),
                            rng.uniform(0, 448, 5000), rng.uniform(0, 2.0 ** -5, 2000)])
    for v in probe:
        d = np.abs(vals - v)
        best = np.flatnonzero(d == d.min())
        code = best[0] if len(best) == 1 else best[best % 2 == 0][0]
        assert mod.e4m3_quantize(np.array([v]))[0] == code, v
        assert mod.e4m3_quantize(np.array([-v]))[0] == code | 0x80, -v
    # saturation and NaN
    sat = mod.e4m3_quantize(np.array([448.0, 449.0, 464.0, 479.0, 1e6, -1e30, np.inf, -np.inf]))
    assert sat.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE]
    assert mod.e4m3_quantize(np.array([np.nan]))[0] == 0x7F
    # error bound of the format: half a step of the 3-bit mantissa
    y = rng.uniform(2.0 ** -6, 448, 20000) * rng.choice([-1, 1], 20000)
    err = np.abs(mod.e4m3_decode(mod.e4m3_quantize(y)) - y)
    assert (err <= np.abs(y) * 2.0 ** -4).all()
    z = rng.uniform(-(2.0 ** -6), 2.0 ** -6, 5000)
    assert (np.abs(mod.e4m3_decode(mod.e4m3_quantize(z)) - z) <= 2.0 ** -10).all()
    # the scale divides on the way in and multiplies on the way out
    for scale in (0.0625, 3.0, 0.37):
        on_grid = ref[rng.integers(0, 0x7F, 400)] * rng.choice([-1, 1], 400)
        xs = (on_grid.astype(np.float32) * np.float32(scale)).astype(np.float32)
        codes = mod.quantize_kv(xs, scale)
        back = mod.dequantize(codes, scale)
        if scale != 0.37:  # exact cases: x / scale is on the grid
            assert (mod.e4m3_decode(codes) == on_grid).all()
            assert np.allclose(back, xs, rtol=0, atol=0)
        else:
            assert np.all(np.abs(back - xs) <= np.abs(xs) * 2.0 ** -4 + 2.0 ** -10 * scale)


def test_pins_hold():
    _pins(Q)


def test_attention_on_grid_values_equals_float_oracle():
    """K and V already on the E4M3 grid times the scale: the 8-bit oracle must
    give the float oracle's result on those values, for decode and prefill."""
    rng = np.random.default_rng(3)
    ref = torch.from_numpy(CODES.copy()).view(torch.float8_e4m3fn).double().numpy()
    nb, hkv, d = 12, 2, 16
    kc = rng.integers(0, 0x7E, size=(nb, hkv, 16, d)).astype(np.uint8) | (rng.integers(0, 2, size=(nb, hkv, 16, d)) << 7).astype(np.uint8)
    vc = rng.integers(0, 0x7E, size=(nb, hkv, 16, d)).astype(np.uint8)
    ks, vs = float(np.float32(0.02)), 0.5   # the scales the library takes are float32
    kf, vf = ref[kc] * ks, ref[vc] * vs
    ids = rng.permutation(nb)[:5]
    row = (ids.astype(np.uint32) | (np.array([0, 0, 40, 40, 90], np.uint32) << 16))[None, :]
    q = rng.standard_normal((1, 4, d))
    a = Q.decode_fp8(q, [100], kc, vc, row, [75], 0.25, 1e4, ks, vs)
    b = oracle.decode(q, [100], kf, vf, row, [75], 0.25, 1e4)
    assert np.array_equal(a, b)
    qp = rng.standard_normal((9, 4, d))
    a = Q.prefill_fp8(qp, [0, 9], [70], kc, vc, row, [75], 0.25, 1e4, ks, vs)
    b = oracle.prefill(qp, [0, 9], [70], kf, vf, row, [75], 0.25, 1e4)
    assert np.array_equal(a, b)
    # append: quantises, then writes exactly where the plain append writes
    kg = ref[rng.integers(0, 0x7E, size=(3, hkv, d))]
    vg = ref[rng.integers(0, 0x7E, size=(3, hkv, d))]
    kn, vn = (kg * ks).astype(np.float32), (vg * vs).astype(np.float32)
    k2, v2 = Q.append_fp8(kc, vc, kn, vn, np.array([5, -1, 40]), ks, vs)
    # rows 0 and 2 land in block 0 slot 5 and block 2 slot 8, their grid values
    # recovered exactly; row 1 is padding; nothing else changes
    assert np.array_equal(ref[k2[0, :, 5]], kg[0]) and np.array_equal(ref[v2[2, :, 8]], vg[2])
    assert np.array_equal(ref[k2[2, :, 8]], kg[2]) and np.array_equal(ref[v2[0, :, 5]], vg[0])
    touched = np.zeros(k2.shape, bool)
    touched[0, :, 5] = touched[2, :, 8] = True
    assert np.array_equal(k2[~touched], kc[~touched]) and np.array_equal(v2[~touched], vc[~touched])


MUTATIONS = {
    "exponent_bias_8": [("np.ldexp(1.0 + m / 8.0, e - 7)", "np.ldexp(1.0 + m / 8.0, e - 8)")],
    "subnormal_scale": [("np.ldexp(m / 8.0, -6)", "np.ldexp(m / 8.0, -7)")],
    "nan_code_ignored": [("mag = np.where((e == 15) & (m == 7), np.nan, mag)", "pass")],
    "ties_away_from_zero": [("k = np.rint(a / step).astype(np.int64)",
                             "k = np.floor(a / step + 0.5).astype(np.int64)")],
    "truncation": [("k = np.rint(a / step).astype(np.int64)", "k = np.floor(a / step).astype(np.int64)")],
    "no_saturation": [("code = np.where(a > E4M3_MAX, 0x7E, np.minimum(code, 0x7E))", "pass")],
    "sign_dropped": [("code = code | sign", "pass")],
    "zero_not_special": [("np.where(a > 0, a, 2.0 ** -10)", "np.where(a > 0, a, 1.0)")],
    "scale_multiplies_in": [("np.asarray(x, dtype=np.float32) / np.float32(scale)",
                             "np.asarray(x, dtype=np.float32) * np.float32(scale)")],
    "scale_missing_out": [("return e4m3_decode(codes) * float(np.float32(scale))", "return e4m3_decode(codes)")],
    "mantissa_step": [("step = np.ldexp(1.0, e_unb - 3)", "step = np.ldexp(1.0, e_unb - 2)")],
}


def _mutant(edits):
    src = inspect.getsource(Q)
    for old, new in edits:
        assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("oracle.quant_mutant")
    mod.__package__ = "oracle"
    exec(compile(src, "quant_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    mod = _mutant(MUTATIONS[name])
    with pytest.raises((AssertionError, ValueError, IndexError)):
        _pins(mod)


# ------------------------------------------------------------------ int8 pool
def _int8_pins(mod):
    """int8 codes: torch's round-half-even cast, brute force at midpoints,
    the clamp to +-127, NaN to 0, infinities, exact round trips, and the
    scale's direction."""
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (0.3, 5.0, 60.0, 400.0)]).astype(np.float32)
    want = torch.from_numpy(x).double().round().clamp(-127, 127).to(torch.int8).numpy()
    assert (mod.int8_quantize(x.astype(np.float64)) == want).all()
    # brute force: nearest integer in [-127, 127], ties to the even one
    grid = np.arange(-127, 128, dtype=np.float64)
    probe = np.concatenate([grid[:-1] + 0.5, grid[:-1] + 0.5 + 2.0 ** -20, grid[:-1] + 0.5 - 2.0 ** -20,
                            rng.uniform(-130, 130, 3000)])
    for v in probe:
        d = np.abs(grid - v)
        best = grid[np.flatnonzero(d == d.min())]
        code = best[0] if len(best) == 1 else best[best % 2 == 0][0]
        assert mod.int8_quantize(np.array([v]))[0] == code, v
    ends = mod.int8_quantize(np.array([127.0, 127.5, 128.0, 1e9, -127.5, -128.0, -1e9, np.inf, -np.inf, np.nan,
                                       -0.0, 0.5, -0.5, 1.5, -2.5]))
    assert ends.tolist() == [127, 127, 127, 127, -127, -127, -127, 127, -127, 0, 0, 0, 0, 2, -2]
    codes = np.arange(-127, 128).astype(np.int8)
    assert (mod.int8_decode(codes) == np.arange(-127, 128)).all()
    assert (mod.int8_quantize(mod.int8_decode(codes)) == codes).all()
    assert mod.int8_decode(np.array([0x80], dtype=np.uint8))[0] == -128   # read as two's complement
    for scale in (0.0625, 0.37, 3.0):
        on_grid = rng.integers(-127, 128, 500).astype(np.float64)
        xs = (on_grid.astype(np.float32) * np.float32(scale)).astype(np.float32)
        c = mod.quantize_kv_int8(xs, scale)
        back = mod.dequantize_int8(c, scale)
        if scale != 0.37:
            assert (mod.int8_decode(c) == on_grid).all() and np.array_equal(back, xs)
        else:
            assert np.all(np.abs(back - xs) <= 0.5 * np.float32(scale) + 1e-6 * np.abs(xs))


def test_int8_pins_hold():
    _int8_pins(Q)


def test_int8_attention_on_grid_values_equals_float_oracle():
    """int8 codes times the scale: the int8 oracle gives the float oracle's
    result on those values (decode, prefill), and its append writes the codes
    where the plain append writes rows."""
    rng = np.random.default_rng(8)
    nb, hkv, d = 12, 2, 16
    kc = rng.integers(-127, 128, size=(nb, hkv, 16, d)).astype(np.int8)
    vc = rng.integers(-127, 128, size=(nb, hkv, 16, d)).astype(np.int8)
    ks, vs = float(np.float32(0.02)), 0.5
    kf, vf = kc.astype(np.float64) * ks, vc.astype(np.float64) * vs
    ids = rng.permutation(nb)[:5]
    row = (ids.astype(np.uint32) | (np.array([0, 0, 40, 40, 90], np.uint32) << 16))[None, :]
    q = rng.standard_normal((1, 4, d))
    assert np.array_equal(Q.decode_int8(q, [100], kc, vc, row, [75], 0.25, 1e4, ks, vs),
                          oracle.decode(q, [100], kf, vf, row, [75], 0.25, 1e4))
    qp = rng.standard_normal((9, 4, d))
    assert np.array_equal(Q.prefill_int8(qp, [0, 9], [70], kc, vc, row, [75], 0.25, 1e4, ks, vs),
                          oracle.prefill(qp, [0, 9], [70], kf, vf, row, [75], 0.25, 1e4))
    kg = rng.integers(-127, 128, size=(3, hkv, d)).astype(np.float64)
    vg = rng.integers(-127, 128, size=(3, hkv, d)).astype(np.float64)
    k2, v2 = Q.append_int8(kc, vc, (kg * ks).astype(np.float32), (vg * vs).astype(np.float32),
                           np.array([5, -1, 40]), ks, vs)
    assert np.array_equal(k2[0, :, 5], kg[0]) and np.array_equal(v2[2, :, 8], vg[2])
    touched = np.zeros(k2.shape, bool)
    touched[0, :, 5] = touched[2, :, 8] = True
    assert np.array_equal(k2[~touched], kc[~touched]) and np.array_equal(v2[~touched], vc[~touched])


INT8_MUTATIONS = {
    "ties_away_from_zero": [("r = np.rint(np.clip(np.where(np.isnan(x), 0.0, x), -INT8_MAX, INT8_MAX))",
                             "r = np.trunc(np.clip(np.where(np.isnan(x), 0.0, x), -INT8_MAX, INT8_MAX) "
                             "+ np.copysign(0.5, x))")],
    "truncation": [("r = np.rint(np.clip(", "r = np.trunc(np.clip(")],
    "clamp_to_minus_128": [("-INT8_MAX, INT8_MAX))", "-INT8_MAX - 1, INT8_MAX))")],
    "nan_not_zero": [("np.where(np.isnan(x), 0.0, x)", "np.where(np.isnan(x), 127.0, x)")],
    "unsigned_read": [("np.asarray(codes).view(np.int8).astype(np.float64)",
                       "np.asarray(codes).view(np.uint8).astype(np.float64)")],
    "scale_multiplies_in": [("q = np.asarray(x, dtype=np.float32) / np.float32(scale)\n    return int8_quantize",
                             "q = np.asarray(x, dtype=np.float32) * np.float32(scale)\n    return int8_quantize")],
    "scale_missing_out": [("return int8_decode(codes) * float(np.float32(scale))", "return int8_decode(codes)")],
}


@pytest.mark.parametrize("name", sorted(INT8_MUTATIONS))
def test_int8_mutation_is_caught(name):
    mod = _mutant(INT8_MUTATIONS[name])
    with pytest.raises((AssertionError, ValueError, IndexError)):
        _int8_pins(mod)
