"""Pins for the oracle's number-format code against torch's own conversions (library routines
written independently of the oracle)."""
import numpy as np
import torch

import oracle


def test_bf16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_bits_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3fn_decode_all_codes():
    bits = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(bits).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3fn_bits_to_f64(bits)
    nan = np.isnan(ref)
    assert nan.sum() == 2                      # 0x7f and 0xff
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # spot values from the format definition
    assert got[0x38] == 1.0 and got[0x7e] == 448.0 and got[0x01] == 2.0 ** -9
    assert got[0xb8] == -1.0 and got[0x08] == 2.0 ** -6


def test_bf16_round_nearest_even():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-39).astype(np.float32),      # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1.0 + 2.0 ** -8,
                  1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20], np.float32),
    ])
    # exact ties: low 16 bits = 0x8000
    u = rng.integers(0, 2 ** 31, 5000, dtype=np.uint64).astype(np.uint32)
    u = (u & np.uint32(0x7F7F0000)) | np.uint32(0x8000)
    x = np.concatenate([x, u.view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f32_to_bf16_bits_rne(x)
    assert np.array_equal(got, ref)
