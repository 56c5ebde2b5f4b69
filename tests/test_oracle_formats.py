"""Pins of the oracle's storage formats: known values from the format
definitions, exhaustive code round trips and torch's own conversions as an
independent library routine for in-range values."""
import numpy as np
import torch

from oracle.formats import round_bf16, round_e4m3, e4m3_decode, e4m3_encode


def test_bf16_known_values():
    assert round_bf16(1.0) == 1.0
    assert round_bf16(1.0 + 2.0 ** -8) == 1.0                      # tie -> even (mantissa 0)
    assert round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6       # tie -> even (mantissa 2)
    assert round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    assert round_bf16(-3.0) == -3.0
    assert round_bf16(0.0) == 0.0


def test_bf16_matches_torch_on_fp32_inputs():
    g = torch.Generator().manual_seed(0)
    x = torch.randn(200000, generator=g) * torch.exp(torch.randn(200000, generator=g) * 4)
    ref = x.to(torch.bfloat16).to(torch.float64).numpy()
    got = round_bf16(x.to(torch.float64).numpy())
    assert np.array_equal(ref, got)


def test_e4m3_known_values():
    # OCP 8-bit float, E4M3: 0x38 = 1.0, 0x7E = 448 (max), 0x01 = 2^-9 (min subnormal),
    # 0x08 = 2^-6 (min normal), 0x7F = NaN.
    dec = e4m3_decode(np.arange(256))
    assert dec[0x38] == 1.0 and dec[0x7E] == 448.0 and dec[0x01] == 2.0 ** -9
    assert dec[0x08] == 2.0 ** -6 and dec[0x07] == 7 * 2.0 ** -9
    assert np.isnan(dec[0x7F]) and np.isnan(dec[0xFF])
    assert dec[0xB8] == -1.0 and dec[0xFE] == -448.0
    assert np.sum(np.isnan(dec)) == 2
    # saturation and rounding
    assert round_e4m3(1000.0) == 448.0 and round_e4m3(-460.0) == -448.0
    assert round_e4m3(1.0625) == 1.0          # tie between 1.0 and 1.125 -> even
    assert round_e4m3(1.1875) == 1.25         # tie between 1.125 and 1.25 -> even
    assert round_e4m3(2.0 ** -10) == 0.0      # tie between 0 and 2^-9 -> even (0)
    assert round_e4m3(3 * 2.0 ** -10) == 2 * 2.0 ** -9


def test_e4m3_code_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    vals = e4m3_decode(codes)
    assert np.array_equal(e4m3_encode(vals), codes.astype(np.uint8))
    assert np.array_equal(round_e4m3(vals), vals)


def test_e4m3_matches_torch_in_range():
    # torch's float -> float8_e4m3fn conversion rounds to nearest even; inside
    # the finite range it must agree with the oracle's definition.
    g = torch.Generator().manual_seed(1)
    x = (torch.randn(200000, generator=g) * torch.exp(torch.randn(200000, generator=g) * 3))
    x = x[x.abs() < 440]
    ref = x.to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = round_e4m3(x.to(torch.float64).numpy())
    assert np.array_equal(ref, got)
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    dec = e4m3_decode(np.arange(256))
    assert np.array_equal(np.isnan(codes), np.isnan(dec))
    assert np.array_equal(codes[~np.isnan(codes)], dec[~np.isnan(dec)])


def test_e4m3_nearest_by_brute_force():
    vals = np.sort(np.unique(e4m3_decode(np.arange(256))[~np.isnan(e4m3_decode(np.arange(256)))]))
    rng = np.random.default_rng(3)
    x = rng.uniform(-448, 448, 5000) * rng.choice([1, 1e-1, 1e-2, 1e-3], 5000)
    q = round_e4m3(x)
    d = np.abs(vals[None, :] - x[:, None]).min(axis=1)
    assert np.allclose(np.abs(q - x), d, rtol=0, atol=0)
