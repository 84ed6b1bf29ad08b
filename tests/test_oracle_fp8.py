"""Pins of the oracle's E4M3 quantiser: the code table against the format's
defining constants, round-to-nearest-even on midpoints, saturation, and a
cross-check of in-range rounding against torch's float8_e4m3fn cast.  CPU."""
import numpy as np
import pytest

from oracle import fp8


def test_code_table_landmarks():
    t = fp8.e4m3_table()
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0          # largest finite
    assert t[0x01] == 2.0 ** -9                             # smallest subnormal
    assert t[0x08] == 2.0 ** -6                             # smallest normal
    assert t[0x07] == 7 * 2.0 ** -9                          # largest subnormal
    assert t[0x38] == 1.0                                   # exponent field 7 = bias
    fin = t[:0x7F]
    assert np.all(np.diff(fin) > 0)                         # codes 0..126 increase
    assert np.array_equal(t[0x80:0xFF], -fin)


def test_encode_roundtrip_all_finite_codes():
    t = fp8.e4m3_table()
    codes = np.array([c for c in range(256) if not np.isnan(t[c])])
    assert np.array_equal(fp8.e4m3_encode(t[codes]), codes.astype(np.uint8))


def test_midpoints_round_to_even_code_and_saturate():
    t = fp8.e4m3_table()
    for c in range(0, 0x7E):
        mid = 0.5 * (t[c] + t[c + 1])
        want = c if c % 2 == 0 else c + 1
        assert fp8.e4m3_encode(np.array([mid]))[0] == want, c
        assert fp8.e4m3_encode(np.array([-mid]))[0] == (want | 0x80), c
    assert fp8.e4m3_encode(np.array([1e6, -500.0]))[0] == 0x7E
    assert fp8.e4m3_encode(np.array([-1e6]))[0] == 0xFE


def test_in_range_rounding_matches_torch_cast():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 120.0)])
    x = x[np.abs(x) <= 440].astype(np.float32)
    ours = fp8.e4m3_encode(x.astype(np.float64))
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_quantize_tensor_scale_and_error_bound():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(4096) * 3
    codes, s = fp8.quantize_tensor(x)
    assert s == np.float32(np.max(np.abs(x.astype(np.float32)))) / np.float32(448)
    deq = fp8.e4m3_values(codes) * np.float64(s)
    # relative error of a 3-bit-mantissa rounding is at most 2^-4 for normals
    big = np.abs(x) > 2.0 ** -6 * s * 2
    assert np.all(np.abs(deq[big] - x[big]) <= np.abs(x[big]) * 2.0 ** -4 + 1e-12)
    z, s0 = fp8.quantize_tensor(np.zeros(10))
    assert s0 == 1.0 and np.all(z == 0)
