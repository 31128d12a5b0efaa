"""Pins for the oracle's rounding: exhaustive over every bf16 / fp16 / e4m3 bit
pattern against torch's CPU casts (library routines), plus random and tie
values, plus the e4m3fn format facts."""
import numpy as np
import torch

from oracle import rounding


def _random_f32(n, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n).astype(np.float32) * np.exp2(rng.integers(-20, 20, n)).astype(np.float32)
    return x


def test_bf16_round_trip_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    fin = np.isfinite(f)
    assert np.array_equal(rounding.f32_to_bf16_bits(f[fin]), bits[fin].astype(np.uint16))


def test_bf16_rounding_matches_torch():
    x = _random_f32(1 << 20, 1)
    # exact ties: a bf16 value plus half an ulp of it
    base = (np.arange(1 << 12, dtype=np.uint32) << 19).view(np.float32)
    base = base[np.isfinite(base)]
    ties = ((base.view(np.uint32) | np.uint32(0x8000))).view(np.float32)
    for arr in (x, ties, -ties):
        ref = torch.from_numpy(arr).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(rounding.f32_to_bf16_bits(arr), ref)


def test_f16_rounding_matches_torch():
    bits = np.arange(1 << 16, dtype=np.uint16)
    f = bits.view(np.float16).astype(np.float32)
    fin = np.isfinite(f)
    assert np.array_equal(rounding.round_f16(f[fin]), f[fin].astype(np.float64))
    x = _random_f32(1 << 20, 2)
    ref = torch.from_numpy(x).to(torch.float16).to(torch.float64).numpy()
    got = rounding.round_f16(x)
    same = (ref == got) | (np.isnan(ref) & np.isnan(got))
    assert same.all()
    fin = np.isfinite(x)
    ref_bits = torch.from_numpy(x[fin]).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(rounding.f32_to_f16_bits(x[fin]), ref_bits)


def test_e4m3_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = rounding.e4m3_bits_to_f64(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    fin = ~np.isnan(ref)
    assert np.array_equal(ref[fin], got[fin])


def test_e4m3_format_facts():
    v = rounding.e4m3_bits_to_f64(np.arange(256, dtype=np.uint8))
    assert np.nanmax(v) == 448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.isnan(v).sum() == 2
    assert v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9     # smallest normal / subnormal
    assert not np.isinf(v).any()


def test_e4m3_rounding_matches_torch_in_range():
    rng = np.random.default_rng(3)
    x = rng.uniform(-448, 448, 1 << 18)
    x = np.concatenate([x, rng.uniform(-1, 1, 1 << 16) * 2.0 ** -6, [0.0, -0.0, 448.0, -448.0]])
    # midpoints between neighbouring codes (ties go to the even code)
    pos = rounding.e4m3_bits_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[1:] + pos[:-1]) / 2
    for arr in (x, mids, -mids):
        ref = torch.from_numpy(arr.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
        got = rounding.round_e4m3(arr.astype(np.float32).astype(np.float64))
        assert np.array_equal(ref, got)


def test_e4m3_grid_rounding_matches_table_search():
    """The binade-grid rounding equals a nearest-value search over the table of
    every finite e4m3 value (ties to the even code)."""
    rng = np.random.default_rng(5)
    pos = rounding.e4m3_bits_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[1:] + pos[:-1]) / 2
    x = np.concatenate([rng.uniform(-500, 500, 1 << 18), rng.standard_normal(1 << 16) * 2.0 ** -7,
                        mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9), pos, -pos,
                        [448.0, 464.0, 1e9, -1e9, 0.0, -0.0]])
    assert np.array_equal(rounding.round_e4m3(x), rounding.e4m3_nearest_by_search(x))
    codes = rounding.f64_to_e4m3_bits(x)
    assert np.array_equal(rounding.e4m3_bits_to_f64(codes), rounding.round_e4m3(x))


def test_e4m3_saturates():
    x = np.array([448.0, 449.0, 463.9, 464.0, 1e6, -1e6, np.inf])
    assert np.array_equal(rounding.round_e4m3(x), [448, 448, 448, 448, 448, -448, 448])
    assert np.isnan(rounding.round_e4m3(np.array([np.nan])))[0]
