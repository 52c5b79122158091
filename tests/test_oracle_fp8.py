"""Pins of the FP8 (OCP E4M3) oracle: code table, library conversion, ties,
saturation, underflow, round trips, and planted mistakes."""

import math

import numpy as np
import pytest

from oracle import fp8 as F


def table_value(code: int) -> float:
    """The E4M3 value of one code, written out from the format's fields."""
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 15 and mant == 7:
        return math.nan
    if exp_field == 0:
        return sign * mant / 8.0 * 2.0 ** -6
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)


ALL = np.arange(256, dtype=np.uint8)


def test_decode_matches_the_field_formula_for_every_code():
    got = F.decode(ALL)
    ref = np.array([table_value(int(c)) for c in ALL])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_named_codes():
    d = F.decode(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x3C, 0x7E, 0x80, 0xFE, 0x7F, 0xFF],
                          dtype=np.uint8))
    assert d[0] == 0.0 and d[1] == 2.0 ** -9 and d[2] == 7 * 2.0 ** -9 and d[3] == 2.0 ** -6
    assert d[4] == 1.0 and d[5] == 1.5 and d[6] == 448.0 and d[8] == -448.0
    assert d[7] == 0.0 and math.copysign(1.0, d[7]) == -1.0
    assert math.isnan(d[9]) and math.isnan(d[10])


def test_decode_matches_torch_float8_e4m3fn():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch without float8_e4m3fn")
    ref = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).double().numpy()
    got = F.decode(ALL)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_every_finite_code_round_trips():
    finite = ALL[~np.isnan(F.decode(ALL))]
    assert np.array_equal(F.encode(F.decode(finite)), finite)


def test_ties_go_to_the_even_code():
    for c in range(0, 0x7E):                     # consecutive positive codes c, c + 1
        lo, hi = table_value(c), table_value(c + 1)
        mid = (lo + hi) / 2.0
        want = c if c % 2 == 0 else c + 1
        assert int(F.encode(np.array([mid]))[0]) == want, hex(c)
        assert int(F.encode(np.array([-mid]))[0]) == want | 0x80, hex(c)


def test_saturation_nan_and_underflow():
    big = np.array([448.0, 449.0, 463.9, 464.0, 500.0, 1e30, np.inf])
    assert np.all(F.encode(big) == 0x7E) and np.all(F.encode(-big) == 0xFE)
    assert int(F.encode(np.array([np.nan]))[0]) == F.NAN_CODE
    tiny = np.array([2.0 ** -10, 2.0 ** -10 * 1.0001, 3 * 2.0 ** -10, 2.0 ** -12, 0.0])
    assert F.encode(tiny).tolist() == [0x00, 0x01, 0x02, 0x00, 0x00]


def test_encode_matches_torch_in_range():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch without float8_e4m3fn")
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.standard_normal(4000) * s for s in (1e-3, 0.05, 1.0, 30.0, 140.0)])
    x = np.clip(x, -448.0, 448.0).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.encode(x), ref)


def test_quantize_divides_in_float32():
    x = np.array([1.0, 3.0, 100.0], dtype=np.float32)
    s = np.float32(0.3)
    want = F.encode((x / s).astype(np.float32))
    assert np.array_equal(F.quantize(x, s), want)
    np.testing.assert_array_equal(F.dequantize(want, s), F.decode(want) * np.float64(s))


# -- the pins above catch plausible mistakes planted in the oracle ---------------------
def _pins_pass():
    try:
        test_decode_matches_the_field_formula_for_every_code()
        test_every_finite_code_round_trips()
        test_ties_go_to_the_even_code()
        test_saturation_nan_and_underflow()
        return True
    except AssertionError:
        return False


def _decode_bias8(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e, m = (c >> 3) & 0xF, c & 7
    s = np.where(c & 0x80, -1.0, 1.0)
    return np.where(e == 0, s * m * 2.0 ** -10, s * np.ldexp(1.0 + m / 8.0, e - 8))


_orig_encode = F.encode


def _encode_ties_away(x):
    v = np.asarray(x, dtype=np.float64)
    nudged = v * (1 + 1e-12)                      # every tie now rounds up in magnitude
    return _orig_encode(nudged)


def _encode_flush_subnormals(x):
    v = np.asarray(x, dtype=np.float64)
    return _orig_encode(np.where(np.abs(v) < 2.0 ** -6, 0.0, v))


@pytest.mark.parametrize("name", ["bias8", "ties_away", "flush"])
def test_pins_catch_planted_mistakes(monkeypatch, name):
    assert _pins_pass()
    if name == "bias8":
        monkeypatch.setattr(F, "decode", _decode_bias8)
    elif name == "ties_away":
        monkeypatch.setattr(F, "encode", _encode_ties_away)
    else:
        monkeypatch.setattr(F, "encode", _encode_flush_subnormals)
    assert not _pins_pass()


def test_fp8_pool_write_quantises_per_head_and_round_trips_through_the_layout():
    from oracle import cache as OC
    from oracle import layout as OL
    rng = np.random.default_rng(21)
    nb, hkv, d = 4, 2, 64
    kp, vp = OC.empty_pool8(nb, hkv, d)
    k = rng.standard_normal((3, hkv, d)).astype(np.float32) * 5
    v = rng.standard_normal((3, hkv, d)).astype(np.float32)
    ks, vs = np.array([0.5, 2.0], np.float32), np.array([0.25, 1.0], np.float32)
    kp2, vp2 = OC.cache_write8(kp, vp, k, v, [17, -1, 63], ks, vs)
    assert np.array_equal(kp2[1, 0, 1], F.encode((k[0, 0] / ks[0]).astype(np.float32)))
    assert np.array_equal(vp2[3, 1, 15], F.encode((v[2, 1] / vs[1]).astype(np.float32)))
    assert not kp2[0].any() and not kp2[2].any()            # the skipped slot wrote nothing
    assert np.array_equal(OL.k8_to_logical(OL.k8_from_logical(kp2)), kp2)
    kd, vd = OC.dequant_sequence8(kp2, vp2, [0, 1], 18, ks, vs)
    assert np.array_equal(kd[17, 0], F.decode(kp2[1, 0, 1]) * np.float64(ks[0]))
    # dequantised values sit within half a code step of the scaled input
    err = np.abs(kd[17] - k[0]) / ks[:, None]
    assert np.all(err <= np.maximum(np.abs(k[0] / ks[:, None]) * 2.0 ** -4, 2.0 ** -10) + 1e-12)


def test_fp8_layout_hand_worked_offsets():
    """Two elements placed by hand from the layout's definition."""
    from oracle import layout as OL
    x = np.arange(3 * 2 * 16 * 128, dtype=np.int64).reshape(3, 2, 16, 128) % 251
    k = OL.k8_from_logical(x).reshape(3, 2, -1)
    # K (b=1, h=1, t=5, d=77): group 1 of 64, quad (77 % 32) // 8 = 1, half (77 % 64) // 32 = 0, e = 5
    assert k[1, 1, (((1 * 16 + 5) * 4 + 1) * 2 + 0) * 8 + 5] == x[1, 1, 5, 77]
    v = OL.v8_from_logical(x).reshape(3, 2, -1)
    # V (t=6, d=45): token quad 1, group 0, n = (45 % 32) // 2 = 6, half 1, dim parity 1, t % 4 = 2
    assert v[1, 1, ((((1 * 2 + 0) * 16 + 6) * 2 + 1) * 2 + 1) * 4 + 2] == x[1, 1, 6, 45]
