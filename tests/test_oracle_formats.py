"""Pins for the oracle's storage codecs: every code against torch's own dtype
conversions (a library routine independent of the oracle), plus hand cases
of round-to-nearest-even that a detour through binary32 would get wrong."""

import numpy as np
import torch

from oracle import formats


def test_bf16_decoder_all_codes():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = formats.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_bf16_encoder_matches_torch_on_f32_inputs():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(10000) * 1e-38).astype(np.float32),  # subnormal range
        (rng.standard_normal(10000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 3.3895314e38, -3.3895314e38, 1.0e-45], np.float32),
    ])
    ours = formats.f64_to_bf16_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_encoder_ties_to_even_and_no_double_rounding():
    one = 1.0
    ulp = 2.0 ** -7  # spacing of bf16 values in [1, 2)
    cases = {
        one + ulp / 2: one,  # exact tie -> even (1.0)
        one + 3 * ulp / 2: one + 2 * ulp,  # tie between odd and even -> even
        one + ulp / 2 + 2.0 ** -30: one + ulp,  # just above the tie: rounding once goes up
        -(one + ulp / 2 + 2.0 ** -30): -(one + ulp),
        2.0 ** 128 * (1 - 2.0 ** -9): np.inf,  # rounds past the largest finite value
    }
    for x, want in cases.items():
        got = formats.round_to_bf16(np.array([x]))[0]
        assert got == want, (x, got, want)


def test_e4m3_decoder_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = formats.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2  # S.1111.111 only
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.nanmax(ours) == 448.0
    assert ours[1] == 2.0 ** -9  # smallest subnormal


def test_stored_rows_decodes_subsets():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((10, 4)).astype(np.float32)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    s = formats.Stored(bits, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(s.rows([3, 7]), ref[[3, 7]])
    codes = torch.from_numpy(np.clip(x * 10, -448, 448)).to(torch.float8_e4m3fn)
    sc = np.arange(1, 11, dtype=np.float32)
    s8 = formats.Stored(codes.view(torch.uint8).numpy(), "e4m3", sc)
    ref8 = codes.to(torch.float64).numpy() * sc[:, None]
    assert np.array_equal(s8.rows(slice(2, 5)), ref8[2:5])
